"""Summaries of rocprofv3 output for the attention kernels.

    python -m flashattention_attention_variants_amd.profiling stats DIR
        Markdown table of a ``rocprofv3 --kernel-trace --stats --output-format
        csv`` run: calls, average / min / max duration per kernel.

    python -m flashattention_attention_variants_amd.profiling traffic DIR_FETCH DIR_WRITE \\
            --workload NAME --out FILE.json
        HBM bytes per launch from two ``rocprofv3 --pmc FETCH_SIZE`` /
        ``--pmc WRITE_SIZE`` runs of ``bench.py --probe-traffic``.  The probe
        first copies a buffer of known size; the counters of that copy give
        the factor from counter kilobytes to bytes moved (the counters are
        derived from request counts between L2 and the memory fabric, whose
        sizes they assume; the factor absorbs that).  Each variant's launch
        after the copy is scaled by that factor.  The file records a digest
        of the kernel and launcher sources so that a later build can tell the
        figures are stale.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

CMD_VARS = "($REPO is the repository root and $OUT a scratch directory for the profiler's output.)"

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# bytes the traffic probe copies to calibrate the counters
PROBE_COPY_BYTES = 512 << 20


def kernel_digest() -> str:
    """sha256 over the kernel and launcher sources (path order)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hpp")) +
                   glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv_path(dirname: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, dirname))
    return hits[0]


def _csv(dirname: str, suffix: str) -> list[dict]:
    with open(_csv_path(dirname, suffix), newline="") as fh:
        return list(csv.DictReader(fh))


def _file_sha256(path: str) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def record_digest(rec: dict) -> str:
    """sha256 over the fields of a traffic record that its counter runs
    fixed: the kernel digest, the hashes of the counter CSVs read, the
    calibration factors and the per-variant bytes.  A record whose fields
    were edited after the tool wrote it no longer matches."""
    keys = ("kernel_digest", "csv_sha256", "fetch_factor", "write_factor", "per_variant")
    body = json.dumps({k: rec.get(k) for k in keys}, sort_keys=True)
    return hashlib.sha256(body.encode()).hexdigest()[:16]


def traffic_for(path: str, variant: str):
    """HBM bytes per launch of ``variant`` from a traffic record, or None
    when the record is missing, was taken with other kernel sources, or
    does not match its own record digest."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_digest") != kernel_digest() or rec.get("record_digest") != record_digest(rec):
        return None
    v = rec.get("per_variant", {}).get(variant)
    return None if v is None else v["traffic_bytes"]


def short_name(name: str) -> str:
    return name.replace("void ", "").replace("(fl::KernelArgs)", "")


def is_fwd_launch(name: str) -> bool:
    """A forward attention dispatch: the general kernel or the short-row
    Evoformer kernel."""
    return "attn_" in name or "evo_kernel" in name


def is_bwd_kernel(name: str) -> bool:
    return "attn_bwd_kernel" in name


def is_decode_kernel(name: str) -> bool:
    """The decode form of the attention kernel and the merge kernel."""
    return "merge_kernel" in name or (name.rstrip().endswith("(fl::KernelArgs)")
                                      and ", true>" in name.replace(" >", ">"))


def stats_table(dirname: str, keep=None) -> str:
    rows = _csv(dirname, "kernel_stats.csv")
    out = ["| kernel | calls | avg (us) | min (us) | max (us) | share |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        if keep is not None and not keep(r["Name"]):
            continue
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def dispatch_table(dirname: str, keep=None) -> str:
    """Per-dispatch durations from the kernel trace, grouped by kernel and
    launch shape (work-groups = grid / work-group size): a kernel instance
    that serves several workloads of one run gets a row per shape."""
    groups: dict[tuple, list] = {}
    for r in _csv(dirname, "kernel_trace.csv"):
        name = r["Kernel_Name"]
        if keep is not None and not keep(name):
            continue
        nwg = int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1)
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((short_name(name), nwg), []).append(us)
    out = ["| kernel | work-groups | calls | avg (us) | min (us) | max (us) |",
           "|---|---:|---:|---:|---:|---:|"]
    for (name, nwg), v in sorted(groups.items(), key=lambda x: (x[0][0], -x[0][1])):
        out.append("| `%s` | %d | %d | %.1f | %.1f | %.1f |" % (
            name, nwg, len(v), sum(v) / len(v), min(v), max(v)))
    return "\n".join(out)


def _per_dispatch(dirname: str, counter: str) -> list[tuple[int, str, float]]:
    vals: dict[int, list] = {}
    for r in _csv(dirname, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        if d not in vals:
            vals[d] = [r["Kernel_Name"], 0.0]
        vals[d][1] += float(r["Counter_Value"])
    return [(d, v[0], v[1]) for d, v in sorted(vals.items())]


def traffic(dir_fetch: str, dir_write: str, variants: list[str]) -> dict:
    res = {}
    csv_sha = {}
    for key, dirname, counter in (("fetch", dir_fetch, "FETCH_SIZE"), ("write", dir_write, "WRITE_SIZE")):
        csv_sha[key] = _file_sha256(_csv_path(dirname, "counter_collection.csv"))
        disp = _per_dispatch(dirname, counter)
        copies = [(i, v) for i, (_, name, v) in enumerate(disp) if "copy" in name.lower()]
        if not copies:
            raise RuntimeError("%s: no copy dispatch to calibrate against" % dirname)
        ci, cv = max(copies, key=lambda x: x[1])
        attn = [(name, v) for (_, name, v) in disp[ci + 1:] if is_fwd_launch(name)]
        if len(attn) < len(variants):
            raise RuntimeError("%s: %d attention dispatches after the copy, expected %d"
                               % (dirname, len(attn), len(variants)))
        attn = attn[-len(variants):]
        factor = PROBE_COPY_BYTES / (cv * 1024.0)
        res[key] = dict(copy_kib=cv, factor=factor,
                        per_variant={vn: (short_name(nm), kib * 1024.0 * factor)
                                     for vn, (nm, kib) in zip(variants, attn)})
    out = {"kernel_digest": kernel_digest(), "csv_sha256": csv_sha,
           "probe_copy_bytes": PROBE_COPY_BYTES,
           "fetch_factor": res["fetch"]["factor"], "write_factor": res["write"]["factor"],
           "copy_fetch_kib": res["fetch"]["copy_kib"], "copy_write_kib": res["write"]["copy_kib"],
           "per_variant": {}}
    for vn in variants:
        kname, fb = res["fetch"]["per_variant"][vn]
        _, wb = res["write"]["per_variant"][vn]
        out["per_variant"][vn] = dict(kernel=kname, fetch_bytes=round(fb), write_bytes=round(wb),
                                      traffic_bytes=round(fb + wb))
    out["record_digest"] = record_digest(out)
    return out


ALGO_BYTES_NOTE = ("Algorithmic bytes = Q, K, V read once and O written once (bf16).  "
                   "`kernel_digest` names the kernel and launcher sources the counters were "
                   "taken with, `record_digest` the record's own fields as the tool wrote them; "
                   "bench.py reports `traffic` only while both match.")


def stats_markdown(dirname: str, bench_json: str, workload: str) -> str:
    """Kernel-trace summary of the default bench command, with the bench's
    own per-launch timing of the same build beside it."""
    b = json.load(open(bench_json))
    out = ["# attn_mfma_kernel -- %s, all variants" % workload, "",
           "Kernel trace of the default bench command (one step = one call of each variant; "
           "1 s clock settle, %d warmup and %d timed steps), one MI355X." % (b["warmup"], b["steps"]), "", CMD_VARS, "",
           "```",
           "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o run "
           "-- python3 $REPO/bench.py",
           "python3 $REPO/bench.py > $OUT/bench.json",
           "python -m flashattention_attention_variants_amd.profiling stats-md $OUT/kt "
           "--bench $OUT/bench.json --workload %s" % workload,
           "```", "", stats_table(dirname, lambda n: not is_decode_kernel(n) and not is_bwd_kernel(n)), "",
           "Kernel names: `MfmaCfg<D_qk, D_v, streams, QB, MOD, bias, key mask, gate>` with QB the "
           "32-query blocks per wave and MOD 0 = none (vanilla, causal, window, PrefixLM, document), "
           "1 = ALiBi, 2 = softcap with a running reference, 3 = bounded softcap.  One kernel "
           "instance serves several variants when they differ only in the mask interval; its row "
           "then mixes their durations.", "",
           "Bench line of the same build (HIP events on the launch stream, average per launch):", "",
           "| variant | ms / launch | useful TFLOP/s | % of bf16 peak |", "|---|---:|---:|---:|"]
    for k, v in b["per_variant"].items():
        out.append("| %s | %.4f | %.1f | %.1f |" % (k, v["ms"], v["tflops"], 100 * v["frac_bf16_peak"]))
    r = b["roofline"]
    out += ["", "Step value %.1f TFLOP/s.  Dominant kernel: %s, %.4f ms per launch." % (
        b["value"], r["kernel"], r["ms_per_launch"]), "",
            "Per launch shape (the same kernel trace, dispatches grouped by kernel instance and "
            "work-group count): the headline launches are the rows with the headline shape's "
            "work-group count (B H_q ceil(S / rows per work-group): 1024 for the two-block "
            "instances, 2048 for the one-block ones at B 4, H 16, S 4096); the others are the "
            "smaller configurations the same run times.", "",
            dispatch_table(dirname, lambda n: "attn_mfma_kernel" in n and not is_decode_kernel(n)),
            ""]
    return "\n".join(out)


def decode_stats_markdown(dirname: str, bench_json: str) -> str:
    """Kernel-trace summary of the decode kernels in the default bench
    command, with the bench line's decode timing beside it."""
    b = json.load(open(bench_json))
    d = b["decode"]
    out = ["# attn_mfma_kernel (decode form) and merge_kernel -- %s" % d["workload"], "",
           "Kernel trace of the default bench command, which times each decode variant after the "
           "step (per-call HIP events; cold: a 1 GiB buffer read before each call, outside the "
           "events; warm: back-to-back calls; one call = the decode kernel plus the merge "
           "kernel), one MI355X.", "", CMD_VARS, "",
           "```",
           "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o run "
           "-- python3 $REPO/bench.py",
           "python3 $REPO/bench.py > $OUT/bench.json",
           "python -m flashattention_attention_variants_amd.profiling decode-stats-md $OUT/kt "
           "--bench $OUT/bench.json",
           "```", "", stats_table(dirname, is_decode_kernel), "",
           "Kernel names: `MfmaCfg<64, 64, 1, 1, MOD, false, false, false, true>` is the decode form "
           "with MOD 0 = none (causal, window), 1 = ALiBi, 3 = bounded softcap; `merge_kernel<bf16>` "
           "recombines the key ranges.", "",
           "Bench line of the same build (per call, decode + merge; medians; GB/s and the "
           "fraction from the cold median):", "",
           "| variant | cold ms / call | warm ms / call | GB/s (algorithmic) | % of 8 TB/s | "
           "algorithmic MB |",
           "|---|---:|---:|---:|---:|---:|"]
    for k, v in d["per_variant"].items():
        warm = v.get("warm", {}).get("ms_median", float("nan"))
        out.append("| %s | %.4f | %.4f | %.1f | %.1f | %.1f |" % (
            k, v["ms_median"], warm, v["gbs"], 100 * v["frac_hbm"], v["algorithmic_bytes"] / 1e6))
    out.append("")
    return "\n".join(out)


def bwd_stats_markdown(dirname: str, bench_json: str, workload: str) -> str:
    """Kernel-trace summary of the backward launches in the default bench
    command, with the bench line's backward timing beside it."""
    b = json.load(open(bench_json))
    out = ["# attn_bwd_kernel -- %s, all variants" % workload, "",
           "Kernel trace of the default bench command, which times the backward of each variant "
           "after the step (per-call HIP events over back-to-back calls; one call = the dQ "
           "launch plus the dK, dV launch), one MI355X.", "", CMD_VARS, "",
           "```",
           "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o run "
           "-- python3 $REPO/bench.py",
           "python3 $REPO/bench.py > $OUT/bench.json",
           "python -m flashattention_attention_variants_amd.profiling bwd-stats-md $OUT/kt "
           "--bench $OUT/bench.json --workload %s" % workload,
           "```", "", stats_table(dirname, is_bwd_kernel), "",
           "Kernel names: `BwdCfg<role, MOD>` with role 0 = dQ (rows are queries, K and V "
           "streamed), 1 = dK, dV (rows are keys, Q and dO of every query head of the group "
           "streamed); MOD 0 = none, 1 = ALiBi, 2 = softcap.  One instance serves every mask.", "",
           "Bench line of the same build (per call, both launches; median and min; useful FLOPs "
           "= 2.5 x the forward's, TFLOP/s from the median):", "",
           "| variant | ms / call (median) | ms (min) | useful TFLOP/s | % of bf16 peak |",
           "|---|---:|---:|---:|---:|"]
    for k, v in b["backward"]["per_variant"].items():
        out.append("| %s | %.4f | %.4f | %.1f | %.1f |" % (k, v["ms_median"], v["ms_min"], v["tflops"],
                                                          100 * v["frac_bf16_peak"]))
    out.append("")
    return "\n".join(out)


def traffic_markdown(rec: dict) -> str:
    alg = None
    out = ["# HBM traffic per launch -- attn_mfma_kernel, %s" % rec.get("workload", ""), "",
           "Two counter runs of the traffic probe (`bench.py --probe-traffic`: one call of each "
           "variant, a %d-byte device copy, then one more call of each variant), then the summary:"
           % rec["probe_copy_bytes"], "", CMD_VARS, "", "```",
           "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o run "
           "-- python3 $REPO/bench.py --probe-traffic",
           "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o run "
           "-- python3 $REPO/bench.py --probe-traffic",
           "python -m flashattention_attention_variants_amd.profiling traffic $OUT/pmc_fetch "
           "$OUT/pmc_write --workload %s --out profiles/traffic_%s.json --md profiles/traffic_%s.md"
           % (rec.get("workload"), rec.get("workload"), rec.get("workload")), "```", "",
           "Calibration: the copy of %d bytes read %.0f KiB of FETCH_SIZE and %.0f KiB of WRITE_SIZE, "
           "so counter KiB are scaled by %.4f (fetch) and %.4f (write) to bytes."
           % (rec["probe_copy_bytes"], rec["copy_fetch_kib"], rec["copy_write_kib"],
              rec["fetch_factor"], rec["write_factor"]), ""]
    if rec.get("algorithmic_bytes"):
        alg = rec["algorithmic_bytes"]
    out += ["| variant | kernel | fetch MB | write MB | traffic MB | algorithmic MB | ratio |",
            "|---|---|---:|---:|---:|---:|---:|"]
    for k, v in rec["per_variant"].items():
        out.append("| %s | `%s` | %.1f | %.1f | %.1f | %s | %s |" % (
            k, v["kernel"].replace("fl::", ""), v["fetch_bytes"] / 1e6, v["write_bytes"] / 1e6,
            v["traffic_bytes"] / 1e6, "%.1f" % (alg / 1e6) if alg else "-",
            "%.2f" % (v["traffic_bytes"] / alg) if alg else "-"))
    out += ["", ALGO_BYTES_NOTE, "", "kernel_digest: %s" % rec["kernel_digest"],
            "record_digest: %s" % rec["record_digest"],
            "counter CSV sha256: fetch %s, write %s" % (rec["csv_sha256"]["fetch"],
                                                       rec["csv_sha256"]["write"]), ""]
    return "\n".join(out)


EVO_WORKLOAD = "evoformer_bf16_nseq128_nres256_h8_c32"


def evo_traffic_markdown(dir_fetch: str, dir_write: str) -> str:
    """Calibrated HBM bytes of the Evoformer row (pair bias) and column
    launches against their algorithmic bytes."""
    from flashattention_attention_variants_amd import flops, inputs
    wl = inputs.WORKLOADS[EVO_WORKLOAD]
    sh = wl.shape
    rec = traffic(dir_fetch, dir_write, list(wl.variants))
    out = ["# HBM traffic per launch -- Evoformer row and column (evo_kernel), %s"
           % EVO_WORKLOAD, "",
           "Two counter runs of the Evoformer probe (`bench.py --probe-evoformer`: one row call "
           "with the pair bias and one column call, a %d-byte device copy, then both calls "
           "again), then the summary:" % rec["probe_copy_bytes"], "", CMD_VARS, "", "```",
           "cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/evo_fetch -o run "
           "-- python3 $REPO/bench.py --probe-evoformer",
           "cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/evo_write -o run "
           "-- python3 $REPO/bench.py --probe-evoformer",
           "python -m flashattention_attention_variants_amd.profiling evo-traffic $OUT/evo_fetch "
           "$OUT/evo_write", "```", "",
           "Calibration: the copy of %d bytes read %.0f KiB of FETCH_SIZE and %.0f KiB of WRITE_SIZE, "
           "so counter KiB are scaled by %.4f (fetch) and %.4f (write) to bytes."
           % (rec["probe_copy_bytes"], rec["copy_fetch_kib"], rec["copy_write_kib"],
              rec["fetch_factor"], rec["write_factor"]), "",
           "| form | kernel | fetch MB | write MB | traffic MB | algorithmic MB | ratio |",
           "|---|---|---:|---:|---:|---:|---:|"]
    for k, v in rec["per_variant"].items():
        alg = flops.evoformer_bytes(sh["N_seq"], sh["N_res"], sh["H"], sh["C"], k)
        out.append("| %s | `%s` | %.1f | %.1f | %.1f | %.1f | %.2f |" % (
            k, v["kernel"].replace("fl::", ""), v["fetch_bytes"] / 1e6, v["write_bytes"] / 1e6,
            v["traffic_bytes"] / 1e6, alg / 1e6, v["traffic_bytes"] / alg))
    out += ["", "Algorithmic bytes = q, k, v, gate read once, o written once (bf16), the u8 key "
            "mask, and for the row form the pair bias [H, N_res, N_res] read once.", "",
            "kernel_digest: %s" % rec["kernel_digest"], "record_digest: %s" % rec["record_digest"],
            "counter CSV sha256: fetch %s, write %s" % (rec["csv_sha256"]["fetch"],
                                                       rec["csv_sha256"]["write"]), ""]
    return "\n".join(out)


COUNTER_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU "
    "SQ_WAVE_CYCLES SQ_INSTS_SALU GRBM_GUI_ACTIVE",
    "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY "
    "SQ_INSTS_VMEM_RD GRBM_GUI_ACTIVE",
)


def _per_dispatch_all(dirname: str) -> list[dict]:
    disp: dict[int, dict] = {}
    for r in _csv(dirname, "counter_collection.csv"):
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def counters_markdown(dirs: list[str], variants: list[str], workload: str, units: dict) -> str:
    """Per-variant counter table of the probe's last call of each variant.
    MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE / 8 XCDs x
    1024 SIMDs); per-unit figures divide by the number of 32x32 work units."""
    per = {v: {} for v in variants}
    for d in dirs:
        attn = [x for x in _per_dispatch_all(d) if is_fwd_launch(x["name"])][-len(variants):]
        for v, x in zip(variants, attn):
            per[v].update(x)
    out = ["# Counters -- attn_mfma_kernel, %s" % workload, "",
           "One rocprofv3 --pmc run per counter group over the traffic probe (the last call of each "
           "variant is read):", "", CMD_VARS, "", "```"]
    for i, grp in enumerate(COUNTER_PASSES):
        out.append("cd /tmp && rocprofv3 --pmc %s --output-format csv -d $OUT/ctr%d -o run "
                   "-- python3 $REPO/bench.py --probe-traffic" % (grp, i + 1))
    out += ["python -m flashattention_attention_variants_amd.profiling counters-md $OUT/ctr1 "
            "$OUT/ctr2 --workload %s" % workload, "```", "",
            "| variant | MFMA busy | MFMA / unit | VALU / unit | SALU / unit | LDS / unit | "
            "LDS conflict cycles / LDS instr |", "|---|---:|---:|---:|---:|---:|---:|"]
    for v in variants:
        x = per[v]
        simd = x["GRBM_GUI_ACTIVE"] / 8 * 1024
        u = units.get(v)
        f = (lambda c: "%.1f" % (x[c] / u)) if u else (lambda c: "-")
        out.append("| %s | %.1f%% | %s | %s | %s | %s | %.2f |" % (
            v, 100 * x["SQ_VALU_MFMA_BUSY_CYCLES"] / simd, f("SQ_INSTS_MFMA"), f("SQ_INSTS_VALU"),
            f("SQ_INSTS_SALU"), f("SQ_INSTS_LDS"), x["SQ_LDS_BANK_CONFLICT"] / max(x["SQ_INSTS_LDS"], 1)))
    out += ["", "Units (32 queries x 32 keys x one head) are counted only for the dense variants, "
            "where every pair is computed.  VALU counts include the MFMA instructions.", ""]
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    sm = sub.add_parser("stats-md")
    sm.add_argument("dir")
    sm.add_argument("--bench", required=True)
    sm.add_argument("--workload", required=True)
    bm = sub.add_parser("bwd-stats-md")
    bm.add_argument("dir")
    bm.add_argument("--bench", required=True)
    bm.add_argument("--workload", required=True)
    dm = sub.add_parser("decode-stats-md")
    dm.add_argument("dir")
    dm.add_argument("--bench", required=True)
    c = sub.add_parser("counters-md")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--workload", required=True)
    e = sub.add_parser("evo-traffic")
    e.add_argument("dir_fetch")
    e.add_argument("dir_write")
    t = sub.add_parser("traffic")
    t.add_argument("dir_fetch")
    t.add_argument("dir_write")
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--md", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.dir))
    elif a.cmd == "counters-md":
        from flashattention_attention_variants_amd import inputs
        wl = inputs.WORKLOADS[a.workload]
        sh = wl.shape
        dense = sh["B"] * sh["Hq"] * (sh["S"] // 32) ** 2
        units = {v: dense for v in ("vanilla", "alibi", "softcap")}
        path = os.path.join(ROOT, "profiles", "attn_mfma_kernel_%s_counters.md" % a.workload)
        with open(path, "w") as fh:
            fh.write(counters_markdown(a.dirs, list(wl.variants), a.workload, units))
        print("wrote", path)
    elif a.cmd == "bwd-stats-md":
        path = os.path.join(ROOT, "profiles", "attn_bwd_kernel_%s_stats.md" % a.workload)
        with open(path, "w") as fh:
            fh.write(bwd_stats_markdown(a.dir, a.bench, a.workload))
        print("wrote", path)
    elif a.cmd == "decode-stats-md":
        b = json.load(open(a.bench))
        path = os.path.join(ROOT, "profiles", "attn_mfma_kernel_%s_stats.md" % b["decode"]["workload"])
        with open(path, "w") as fh:
            fh.write(decode_stats_markdown(a.dir, a.bench))
        print("wrote", path)
    elif a.cmd == "evo-traffic":
        path = os.path.join(ROOT, "profiles", "traffic_%s.md" % EVO_WORKLOAD)
        with open(path, "w") as fh:
            fh.write(evo_traffic_markdown(a.dir_fetch, a.dir_write))
        print("wrote", path)
    elif a.cmd == "stats-md":
        path = os.path.join(ROOT, "profiles", "attn_mfma_kernel_%s_stats.md" % a.workload)
        with open(path, "w") as fh:
            fh.write(stats_markdown(a.dir, a.bench, a.workload))
        print("wrote", path)
    else:
        from flashattention_attention_variants_amd import flops, inputs
        wl = inputs.WORKLOADS[a.workload]
        rec = traffic(a.dir_fetch, a.dir_write, list(wl.variants))
        rec["workload"] = a.workload
        sh = wl.shape
        rec["algorithmic_bytes"] = flops.attn_bytes(sh["B"], sh["Hq"], sh["Hkv"], sh["S"], sh["S"], sh["D"])
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        if a.md:
            with open(a.md, "w") as fh:
                fh.write(traffic_markdown(rec))
        print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    sys.exit(main())
