"""Host logic of bench.py (no GPU): the amd-smi clock parser."""
import bench

SAMPLE = """GPU: 0
    CLOCK:
        GFX_0:
            CLK: 2346 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 2300 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 2000 MHz
        VCLK_0:
            CLK: 59 MHz
"""


def test_amd_smi_clock_parser():
    gpus = bench._parse_amd_smi_clocks(SAMPLE)
    assert gpus == [dict(sclk_mhz_mean=2323.0, sclk_mhz_min=2300, sclk_mhz_max=2346, mclk_mhz=2000)]
    two = bench._parse_amd_smi_clocks(SAMPLE + SAMPLE.replace("GPU: 0", "GPU: 1"))
    assert len(two) == 2
    assert bench._parse_amd_smi_clocks("no gpu here") == []


def test_multi_gpu_request_exits():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
