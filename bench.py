"""Throughput of the fused attention-variant forward on one MI355X.

One step = one forward call of each of the seven FlexAttention-class variants
(vanilla, ALiBi, softcap, causal, causal sliding window 256, PrefixLM 512,
document mask) on the MHA workload B=4, H=16, S=4096, D=64, bf16 (inputs
resident in HBM before timing).  ``value`` is the useful TFLOP/s of the whole
step; per-variant figures, the roofline of the dominant kernel (live HIP
event timing on the launch stream) and the CPU oracle's throughput on a
bounded sample of the same workload are printed on the same JSON line, with
the backward of each variant (TFLOP/s of its five products) and the decode
workload (64 sequences, 32/8 heads, KV caches of 512-8192 tokens, GB/s
against the HBM roofline) timed beside it.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --report        # extra lines: every workload, every variant
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "attention fwd useful TFLOP/s + % bf16 MFMA peak (S=4k, D=64, per variant)"
HEADLINE = "mha_bf16_b4_h16_s4096_d64"
DECODE_WORKLOAD = "decode_bf16_b64_hq32_hkv8_cap8192_d64"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup, so the clocks reach "
                         "their loaded steady state")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--variants", default=None, help="comma list (default: all seven)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward measurement printed beside the step")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode measurement printed beside the step")
    ap.add_argument("--report", action="store_true",
                    help="also print one JSON line per workload and variant")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with HBM bytes per launch measured by rocprofv3 counters "
                         "(default: profiles/traffic_<workload>.json)")
    ap.add_argument("--probe-traffic", action="store_true",
                    help="make only the dispatches the counter runs read: a copy of known "
                         "size, then one call per variant")
    ap.add_argument("--probe-evoformer", action="store_true",
                    help="as --probe-traffic, for the Evoformer workload (row with pair bias, "
                         "then column)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from flashattention_attention_variants_amd import api, flops, inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    api.load_library()
    dev = "cuda"
    if args.probe_evoformer:
        probe_evoformer(torch, api, inputs, dev)
        return
    wl = inputs.WORKLOADS[args.workload]
    assert wl.kind == "attn"
    s = wl.shape
    B, Hq, Hkv, S, D = s["B"], s["Hq"], s["Hkv"], s["S"], s["D"]
    t = inputs.make(wl)
    q, k, v = t["q"].to(dev), t["k"].to(dev), t["v"].to(dev)
    docs = t.get("doc_offsets")
    docs_dev = docs.to(dev) if docs is not None else None
    variants = args.variants.split(",") if args.variants else list(wl.variants)
    pr = wl.params
    outs = {vname: torch.empty_like(q) for vname in variants}

    def kw_for(vname):
        kw = dict(variant=vname)
        for key in ("softcap", "alibi_max_bias", "window", "window_causal", "prefix"):
            if key in pr:
                kw[key] = pr[key]
        if vname == "document":
            kw["doc_offsets"] = docs_dev
        return kw

    kws = {vname: kw_for(vname) for vname in variants}
    fl = {vname: flops.attn_flops(vname, B, Hq, S, S, D, window=pr.get("window", 256),
                                  window_causal=pr.get("window_causal", True),
                                  prefix=pr.get("prefix", 512),
                                  doc_offsets=None if docs is None else docs.numpy())
          for vname in variants}
    nbytes = flops.attn_bytes(B, Hq, Hkv, S, S, D)

    def step(events=None):
        for vname in variants:
            if events is not None:
                events[vname][0].record()
            api.fl_attn_fwd(q, k, v, out=outs[vname], **kws[vname])
            if events is not None:
                events[vname][1].record()

    if args.probe_traffic:
        from flashattention_attention_variants_amd import profiling
        step()
        src = torch.ones(profiling.PROBE_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        print("probe: copy of %d bytes, then one call each of %s"
              % (profiling.PROBE_COPY_BYTES, ",".join(variants)), flush=True)
        return

    t_end = time.perf_counter() + args.settle
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps, every launch bracketed by events on the launch stream
    ev = {vname: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)] for vname in variants}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step({vname: ev[vname][i] for vname in variants})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {vname: sum(a.elapsed_time(b) for a, b in ev[vname]) / args.steps for vname in variants}
    total_flops = sum(fl.values())
    value = total_flops * args.steps / wall / 1e12

    per = {}
    for vname in variants:
        tf = fl[vname] / (ms[vname] * 1e-3) / 1e12
        bound, roof = flops.roofline_tflops(fl[vname], nbytes)
        per[vname] = dict(ms=round(ms[vname], 4), tflops=round(tf, 1),
                          frac_bf16_peak=round(tf / flops.PEAK_BF16_TFLOPS, 4), bound=bound,
                          roofline_tflops=round(roof, 1), frac_roofline=round(tf / roof, 4),
                          useful_gflop=round(fl[vname] / 1e9, 2))
    dom = max(variants, key=lambda vname: ms[vname])
    achieved = fl[dom] / (ms[dom] * 1e-3) / 1e12
    bound, roof = flops.roofline_tflops(fl[dom], nbytes)
    # HBM bytes per launch from the committed counter runs, unless the
    # kernels changed since they were taken
    from flashattention_attention_variants_amd import profiling
    traffic = None
    tpath = args.traffic or os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                         "traffic_%s.json" % wl.name)
    if os.path.exists(tpath):
        rec = json.load(open(tpath))
        if rec.get("kernel_digest") == profiling.kernel_digest() and dom in rec.get("per_variant", {}):
            traffic = rec["per_variant"][dom]["traffic_bytes"]
    roofline = dict(bound=bound, achieved=round(achieved, 1),
                    peak=flops.PEAK_BF16_TFLOPS if bound == "mfma" else flops.PEAK_HBM_GBS,
                    unit="TFLOP/s" if bound == "mfma" else "GB/s",
                    frac=round(achieved / flops.PEAK_BF16_TFLOPS, 4), traffic=traffic,
                    kernel="attn_mfma_kernel (%s)" % dom, ms_per_launch=round(ms[dom], 4),
                    useful_flop_per_launch=fl[dom], algorithmic_bytes_per_launch=nbytes)
    if bound == "hbm":
        gbs = nbytes / (ms[dom] * 1e-3) / 1e9
        roofline.update(achieved=round(gbs, 1), frac=round(gbs / flops.PEAK_HBM_GBS, 4))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(t, variants, kws, wl, args.cpu_seconds)

    # backward of each variant on the same workload (dQ launch + dK, dV
    # launch), timed after the step
    backward = None
    if not args.no_backward:
        d_o = inputs.randn(inputs._gen(wl.seed + 100), tuple(q.shape), wl.dtype).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(B * Hq * S, dtype=torch.float32, device=dev)
        bper = {}
        for vname in variants:
            o_, lse_ = api.fl_attn_fwd(q, k, v, return_lse=True, **kws[vname])
            bms = timeit(torch, lambda: api.fl_attn_bwd(q, k, v, o_, lse_, d_o, dq=dq, dk=dk, dv=dv,
                                                        workspace=ws, **kws[vname]))
            bf = fl[vname] * 5 // 2
            btf = bf / (bms * 1e-3) / 1e12
            bper[vname] = dict(ms=round(bms, 4), tflops=round(btf, 1),
                               frac_bf16_peak=round(btf / flops.PEAK_BF16_TFLOPS, 4))
        backward = dict(per_variant=bper, useful_flop="2.5 x the forward's (five products)",
                        timing="best of 3 batches of back-to-back calls, both launches")

    # decode against a KV cache (split keys + merge), HBM-bound: its own
    # workload, timed after the step, reported beside it
    decode = None
    if not args.no_decode:
        dwl = inputs.WORKLOADS[DECODE_WORKLOAD]
        dt = inputs.make(dwl)
        dg = {k_: v_.to(dev) for k_, v_ in dt.items()}
        dper = {}
        for vname in dwl.variants:
            dms, df, dnb = decode_case(torch, api, flops, dwl, dt, dg, vname, dev)
            gbs = dnb / (dms * 1e-3) / 1e9
            dper[vname] = dict(ms=round(dms, 4), gbs=round(gbs, 1),
                               frac_hbm=round(gbs / flops.PEAK_HBM_GBS, 4),
                               tflops=round(df / (dms * 1e-3) / 1e12, 2),
                               algorithmic_bytes=dnb, bound="hbm")
        decode = dict(workload=dwl.name, per_variant=dper,
                      timing="best of 3 batches of back-to-back calls, decode and merge kernels")
        del dg

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H_q": Hq, "H_kv": Hkv, "S": S, "D": D,
                   "variants": variants, "step": "one forward call per variant",
                   "seed": wl.seed},
        "frac_bf16_peak": round(value / flops.PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "cpu_baseline": cpu, "per_variant": per, "backward": backward,
        "decode": decode,
    }
    print(json.dumps(line), flush=True)
    if args.report:
        report(torch, api, flops, inputs, dev)


def cpu_baseline(t, variants, kws, wl, seconds):
    """Oracle throughput (useful TFLOP/s) on sampled query rows of the same
    workload, all variants, float64, host threads."""
    import numpy as np

    import oracle
    from flashattention_attention_variants_amd import flops

    oracle.build()
    s = wl.shape
    B, Hq, S, D = s["B"], s["Hq"], s["S"], s["D"]
    q64 = t["q"].to(__import__("torch").float64).numpy()
    k64 = t["k"].to(__import__("torch").float64).numpy()
    v64 = t["v"].to(__import__("torch").float64).numpy()
    docs = t.get("doc_offsets")
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)

    def sample(n):
        return np.sort(rng.choice(B * Hq * S, size=n, replace=False))

    def useful(vname, rows):
        # allowed keys of each sampled row, from the same closed forms as the GPU count
        tot = 0
        i = rows % S
        b = rows // (Hq * S)
        kw = kws[vname]
        for ii, bb in zip(i, b):
            if vname in ("vanilla", "alibi", "softcap"):
                n = S
            elif vname == "causal":
                n = ii + 1
            elif vname == "sliding_window":
                n = min(ii + 1, kw["window"])
            elif vname == "prefix_lm":
                n = max(ii + 1, min(kw["prefix"], S))
            else:
                off = docs[bb].numpy()
                d = np.searchsorted(off, ii, side="right") - 1
                n = off[d + 1] - off[d]
            tot += 2 * int(n) * (D + D)
        return tot

    def run(vname, rows):
        kw = {k: v for k, v in kws[vname].items() if k != "doc_offsets"}
        if vname == "document":
            kw["doc_offsets"] = docs.numpy()
        oracle.attn(q64, k64, v64, rows=rows, threads=threads, **kw)

    # calibrate on a small sample, then size the sample to ~seconds of work
    probe = sample(64 * threads)
    t0 = time.perf_counter()
    run("vanilla", probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(max(threads, min(B * Hq * S, seconds / len(variants) / max(per_row, 1e-9))))
    total_flop, total_s = 0, 0.0
    for vname in variants:
        rows = sample(n)
        t0 = time.perf_counter()
        run(vname, rows)
        total_s += time.perf_counter() - t0
        total_flop += useful(vname, rows)
    return {"value": round(total_flop / total_s / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d random query rows per variant (x%d variants) of %s, float64 two-pass, "
                      "%.1f s" % (n, len(variants), wl.name, total_s)}


def timeit(torch, fn, settle=0.3, batches=3, batch_s=0.05):
    """ms per call: a short settle at this case's load, then the fastest of a
    few timed batches of back-to-back calls (events on the current stream,
    which the calls launch on)."""
    t_end = time.perf_counter() + settle
    n = 0
    while time.perf_counter() < t_end or n < 3:
        fn()
        torch.cuda.synchronize()
        n += 1
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    iters = max(5, int(batch_s * 1e3 / max(a.elapsed_time(b), 1e-3)))
    best = float("inf")
    for _ in range(batches):
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) / iters)
    return best


def decode_case(torch, api, flops, wl, t, g, vname, dev):
    """(ms, useful flops, algorithmic bytes) of one decode call of workload wl."""
    s = wl.shape
    kw = dict(variant=vname)
    for key in ("softcap", "alibi_max_bias", "window", "window_causal"):
        if key in wl.params:
            kw[key] = wl.params[key]
    L = t["seqlens"]
    max_len = int(L.max())
    ws_bytes = api.fl_attn_decode_workspace_size(
        s["B"], s["Hq"], s["Hkv"], s["Sq"], max_len, s["D"], variant=vname,
        window=kw.get("window", 256), window_causal=kw.get("window_causal", True))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(g["q"])
    ms = timeit(torch, lambda: api.fl_attn_decode_fwd(
        g["q"], g["k_cache"], g["v_cache"], g["seqlens"], max_seqlen=max_len, workspace=ws,
        out=out, **kw))
    mask = vname if vname in ("causal", "sliding_window", "prefix_lm") else None
    f, nb = flops.decode_work(mask, L.tolist(), s["Hq"], s["Hkv"], s["Sq"], s["D"],
                              window=wl.params.get("window", 256),
                              window_causal=wl.params.get("window_causal", True))
    return ms, f, nb


def report(torch, api, flops, inputs, dev):
    """One JSON line per (workload, variant): time, TFLOP/s, roofline fraction."""

    for name, wl in inputs.WORKLOADS.items():
        t = inputs.make(wl)
        g = {k: v.to(dev) for k, v in t.items()}
        s = wl.shape
        for vname in wl.variants:
            if wl.kind == "attn":
                kw = dict(variant=vname)
                for key in ("softcap", "alibi_max_bias", "window", "window_causal", "prefix"):
                    if key in wl.params:
                        kw[key] = wl.params[key]
                if vname == "document":
                    kw["doc_offsets"] = g["doc_offsets"]
                out = torch.empty_like(g["q"])
                ms = timeit(torch, lambda: api.fl_attn_fwd(g["q"], g["k"], g["v"], out=out, **kw))
                f = flops.attn_flops(vname, s["B"], s["Hq"], s["S"], s["S"], s["D"],
                                     window=wl.params.get("window", 256),
                                     window_causal=wl.params.get("window_causal", True),
                                     prefix=wl.params.get("prefix", 512),
                                     doc_offsets=None if "doc_offsets" not in t else t["doc_offsets"].numpy())
                nb = flops.attn_bytes(s["B"], s["Hq"], s["Hkv"], s["S"], s["S"], s["D"],
                                      elem=2 if wl.dtype == "bf16" else 4)
                peak = flops.PEAK_BF16_TFLOPS if wl.dtype == "bf16" else flops.PEAK_F32_VALU_TFLOPS
            elif wl.kind == "diffattn":
                out = torch.empty(s["B"], s["H"], s["S"], s["Dv"], dtype=torch.bfloat16, device=dev)
                causal = vname == "causal"
                ms = timeit(torch, lambda: api.fl_diffattn_fwd(g["q1"], g["q2"], g["k1"], g["k2"], g["v"],
                                                        lam=wl.params["lam"], causal=causal, out=out))
                f = flops.diffattn_flops(s["B"], s["H"], s["S"], s["Dqk"], s["Dv"], causal)
                nb = flops.diffattn_bytes(s["B"], s["H"], s["S"], s["Dqk"], s["Dv"])
                peak = flops.PEAK_BF16_TFLOPS
            elif wl.kind == "decode":
                ms, f, nb = decode_case(torch, api, flops, wl, t, g, vname, dev)
                peak = flops.PEAK_BF16_TFLOPS
            else:
                out = torch.empty_like(g["q"])
                pb = g["pair_bias"] if vname == "row" else None
                ms = timeit(torch, lambda: api.fl_evoformer_gated_attn_fwd(
                    g["q"], g["k"], g["v"], g["gate"], pair_bias=pb, key_mask=g["key_mask"],
                    axis=vname, out=out))
                f = flops.evoformer_flops(s["N_seq"], s["N_res"], s["H"], s["C"], vname)
                nb = flops.evoformer_bytes(s["N_seq"], s["N_res"], s["H"], s["C"], vname)
                peak = flops.PEAK_BF16_TFLOPS
            tf = f / (ms * 1e-3) / 1e12
            bound, roof = flops.roofline_tflops(f, nb, peak_tflops=peak)
            print(json.dumps({"report": name, "variant": vname, "ms": round(ms, 4),
                              "tflops": round(tf, 2), "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
                              "bound": bound, "roofline_tflops": round(roof, 1),
                              "frac_roofline": round(tf / roof, 4),
                              "frac_peak": round(tf / peak, 4)}), flush=True)


EVO_WORKLOAD = "evoformer_bf16_nseq128_nres256_h8_c32"


def probe_evoformer(torch, api, inputs, dev):
    """The dispatches the Evoformer counter runs read: one row call (pair bias,
    key mask) and one column call, a copy of known size, then the two calls
    again."""
    from flashattention_attention_variants_amd import profiling
    wl = inputs.WORKLOADS[EVO_WORKLOAD]
    t = inputs.make(wl)
    g = {n: t[n].to(dev) for n in ("q", "k", "v", "gate", "pair_bias", "key_mask")}
    out = torch.empty_like(g["q"])

    def calls():
        for axis in wl.variants:
            pb = g["pair_bias"] if axis == "row" else None
            api.fl_evoformer_gated_attn_fwd(g["q"], g["k"], g["v"], g["gate"], pair_bias=pb,
                                            key_mask=g["key_mask"], axis=axis, out=out)

    calls()
    src = torch.ones(profiling.PROBE_COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    calls()
    torch.cuda.synchronize()
    print("probe: copy of %d bytes, then one call each of %s"
          % (profiling.PROBE_COPY_BYTES, ",".join(wl.variants)), flush=True)


if __name__ == "__main__":
    main()
