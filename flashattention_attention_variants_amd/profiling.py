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


def _csv(dirname: str, suffix: str) -> list[dict]:
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, dirname))
    with open(hits[0], newline="") as fh:
        return list(csv.DictReader(fh))


def short_name(name: str) -> str:
    return name.replace("void ", "").replace("(fl::KernelArgs)", "")


def stats_table(dirname: str) -> str:
    rows = _csv(dirname, "kernel_stats.csv")
    out = ["| kernel | calls | avg (us) | min (us) | max (us) | share |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
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
    for key, dirname, counter in (("fetch", dir_fetch, "FETCH_SIZE"), ("write", dir_write, "WRITE_SIZE")):
        disp = _per_dispatch(dirname, counter)
        copies = [(i, v) for i, (_, name, v) in enumerate(disp) if "copy" in name.lower()]
        if not copies:
            raise RuntimeError("%s: no copy dispatch to calibrate against" % dirname)
        ci, cv = max(copies, key=lambda x: x[1])
        attn = [(name, v) for (_, name, v) in disp[ci + 1:] if "attn_" in name]
        if len(attn) < len(variants):
            raise RuntimeError("%s: %d attention dispatches after the copy, expected %d"
                               % (dirname, len(attn), len(variants)))
        attn = attn[-len(variants):]
        factor = PROBE_COPY_BYTES / (cv * 1024.0)
        res[key] = dict(copy_kib=cv, factor=factor,
                        per_variant={vn: (short_name(nm), kib * 1024.0 * factor)
                                     for vn, (nm, kib) in zip(variants, attn)})
    out = {"kernel_digest": kernel_digest(), "probe_copy_bytes": PROBE_COPY_BYTES,
           "fetch_factor": res["fetch"]["factor"], "write_factor": res["write"]["factor"],
           "copy_fetch_kib": res["fetch"]["copy_kib"], "copy_write_kib": res["write"]["copy_kib"],
           "per_variant": {}}
    for vn in variants:
        kname, fb = res["fetch"]["per_variant"][vn]
        _, wb = res["write"]["per_variant"][vn]
        out["per_variant"][vn] = dict(kernel=kname, fetch_bytes=round(fb), write_bytes=round(wb),
                                      traffic_bytes=round(fb + wb))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("dir_fetch")
    t.add_argument("dir_write")
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.dir))
    else:
        from flashattention_attention_variants_amd import inputs
        wl = inputs.WORKLOADS[a.workload]
        rec = traffic(a.dir_fetch, a.dir_write, list(wl.variants))
        rec["workload"] = a.workload
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    sys.exit(main())
