"""The build's inline-assembly guard (no GPU): inline assembly may load only
into LDS; a register-destination load inside an inline-assembly region fails
the build."""
import pytest

from flashattention_attention_variants_amd import build


def _asm(tmp_path, body):
    p = tmp_path / "k.s"
    p.write_text("_Zkernel:\n" + body)
    return str(p)


def test_lds_dma_in_asm_passes(tmp_path):
    build._check_asm_loads(_asm(tmp_path, ";;#ASMSTART\n\ts_mov_b32 s1, m0\n"
                                "\tbuffer_load_dwordx4 v3, s[0:3], 0 offen lds\n;;#ASMEND\n"
                                "\tds_read_b128 v[0:3], v4\n"))


@pytest.mark.parametrize("ins", ["ds_read_b64_tr_b16 v[0:1], v2 offset:16",
                                 "buffer_load_dwordx4 v[0:3], v4, s[0:3], 0 offen",
                                 "global_load_dword v1, v[2:3], off"])
def test_register_load_in_asm_fails(tmp_path, ins):
    with pytest.raises(RuntimeError):
        build._check_asm_loads(_asm(tmp_path, ";;#ASMSTART\n\t%s\n;;#ASMEND\n" % ins))
