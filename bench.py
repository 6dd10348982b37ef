"""Throughput of the fused attention-variant forward on one MI355X.

One step = one forward call of each of the seven FlexAttention-class variants
(vanilla, ALiBi, softcap, causal, causal sliding window 256, PrefixLM 512,
document mask) on the MHA workload B=4, H=16, S=4096, D=64, bf16 (inputs
resident in HBM before timing).  ``value`` is the useful TFLOP/s of the whole
step over the wall clock of the timed steps.  The same JSON line carries:

* ``per_variant``: each launch's time in the timed steps (HIP events on the
  launch stream; mean, median, min), TFLOP/s and fraction of peak; the rows
  whose working set would sit in the 256 MB Infinity Cache (sliding window,
  document) are also timed cold, with a 1 GiB buffer read before each call
  outside the events;
* ``roofline`` of the dominant (slowest) launch and ``cpu_baseline``, the
  float64 oracle on a bounded sample of the same workload;
* ``clocks``: shader and memory clocks read with amd-smi while the step runs,
  before and after the timed region;
* ``configs``: every other workload timed per call (10 warm-up calls, then
  at least 30 and about 0.3 s of timed calls; median and min), each with the
  fraction of its own roofline -- the float32 MHA case, the S=2048 variant
  sweep, GQA at S=16384, differential attention, the Evoformer row and
  column forms (cold) and Invariant Point Attention;
* ``backward`` of each headline variant and ``decode`` against a KV cache
  (cold and warm).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
    python bench.py --report        # also one line per config entry
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import shutil
import subprocess
import sys
import time

METRIC = "attention fwd useful TFLOP/s + % bf16 MFMA peak (S=4k, D=64, per variant)"
HEADLINE = "mha_bf16_b4_h16_s4096_d64"
DECODE_WORKLOAD = "decode_bf16_b64_hq32_hkv8_cap8192_d64"
EVO_WORKLOAD = "evoformer_bf16_nseq128_nres256_h8_c32"
# rows whose working set fits the Infinity Cache are timed cold as well
COLD_VARIANTS = ("sliding_window", "document")
FLUSH_BYTES = 1 << 30


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config measurements printed beside the step")
    ap.add_argument("--no-clocks", action="store_true", help="do not read clocks with amd-smi")
    ap.add_argument("--report", action="store_true",
                    help="also print one JSON line per config entry")
    ap.add_argument("--traffic", default=None,
                    help="JSON file with HBM bytes per launch measured by rocprofv3 counters "
                         "(default: profiles/traffic_<workload>.json)")
    ap.add_argument("--probe-traffic", action="store_true",
                    help="make only the dispatches the counter runs read: one call per "
                         "variant, a copy of known size, then one call per variant")
    ap.add_argument("--probe-evoformer", action="store_true",
                    help="as --probe-traffic, for the Evoformer workload (row with pair bias, "
                         "then column)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing helpers


def time_calls(torch, fn, *, warmup=10, min_calls=30, min_s=0.3, max_calls=3000, flush=None):
    """Per-call times in ms of ``fn``: ``warmup`` untimed calls, then n timed
    calls (at least min_calls and about min_s seconds of calls), each
    bracketed by HIP events on the current stream, which the calls launch
    on.  ``flush``, if given, runs before every call outside its events (the
    cold-cache form)."""
    import numpy as np
    for _ in range(warmup):
        if flush is not None:
            flush()
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    t = max(a.elapsed_time(b), 1e-3)
    n = int(min(max_calls, max(min_calls, math.ceil(min_s * 1e3 / t))))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for s, e in evs:
        if flush is not None:
            flush()
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    ts = np.array([s.elapsed_time(e) for s, e in evs])
    return dict(ms_median=round(float(np.median(ts)), 5), ms_min=round(float(ts.min()), 5),
                ms_mean=round(float(ts.mean()), 5), calls=n)


def make_flush(torch, dev):
    """A 1 GiB buffer read (summed) before each cold call: it evicts the L2
    and the 256 MB Infinity Cache.  It is read, not written: lines left
    dirty by a write are written back while the timed call runs (measured
    on the decode workload: 0.186 ms after a 1 GiB write, 0.126 ms after a
    1 GiB read, 0.125 ms with no flush at a 623 MB working set)."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        buf.sum()
    return flush


def _parse_amd_smi_clocks(text):
    """Shader (GFX_n) and memory (MEM_0) clocks in MHz per GPU block of
    ``amd-smi metric -c`` text output."""
    gpus = []
    for block in re.split(r"^GPU:\s*\d+\s*$", text, flags=re.M)[1:]:
        gfx = [int(m) for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", block)]
        mem = [int(m) for m in re.findall(r"MEM_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", block)]
        if gfx:
            gpus.append(dict(sclk_mhz_mean=round(sum(gfx) / len(gfx), 1), sclk_mhz_min=min(gfx),
                             sclk_mhz_max=max(gfx), mclk_mhz=mem[0] if mem else None))
    return gpus


def clocks_under_load(torch, fn, max_s=20.0):
    """Clocks read by ``amd-smi metric -c`` (a child process) while ``fn``
    keeps the GPU busy; None when amd-smi is missing or does not answer."""
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    try:
        p = subprocess.Popen([exe, "metric", "-c"], stdout=subprocess.PIPE,
                             stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t_end = time.perf_counter() + max_s
    while p.poll() is None and time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()
    if p.poll() is None:
        p.kill()
        p.wait()
        return None
    gpus = _parse_amd_smi_clocks(p.stdout.read())
    if not gpus:
        return None
    return gpus[0] if len(gpus) == 1 else dict(per_gpu=gpus)


# ---------------------------------------------------------------------------


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
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
    kws = {vname: attn_kw(vname, pr, docs_dev) for vname in variants}
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

    # settle: the clocks reach their loaded state; then they are read while
    # the step keeps running
    t_end = time.perf_counter() + args.settle
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    clk_before = None if args.no_clocks else clocks_under_load(torch, step)
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
    clk_after = None if args.no_clocks else clocks_under_load(torch, step)
    times = {vname: np.array([a.elapsed_time(b) for a, b in ev[vname]]) for vname in variants}
    ms = {vname: float(times[vname].mean()) for vname in variants}
    total_flops = sum(fl.values())
    value = total_flops * args.steps / wall / 1e12

    flush = make_flush(torch, dev)
    per = {}
    for vname in variants:
        tf = fl[vname] / (ms[vname] * 1e-3) / 1e12
        bound, roof = flops.roofline_tflops(fl[vname], nbytes)
        e = dict(ms=round(ms[vname], 5), ms_median=round(float(np.median(times[vname])), 5),
                 ms_min=round(float(times[vname].min()), 5), tflops=round(tf, 1),
                 frac_bf16_peak=round(tf / flops.PEAK_BF16_TFLOPS, 4), bound=bound,
                 roofline_tflops=round(roof, 1), frac_roofline=round(tf / roof, 4),
                 useful_gflop=round(fl[vname] / 1e9, 2),
                 gbs=round(nbytes / (ms[vname] * 1e-3) / 1e9, 1))
        if vname in COLD_VARIANTS:
            c = time_calls(torch, lambda: api.fl_attn_fwd(q, k, v, out=outs[vname], **kws[vname]),
                           flush=flush, max_calls=1000)
            ctf = fl[vname] / (c["ms_median"] * 1e-3) / 1e12
            e["cold"] = dict(c, tflops=round(ctf, 1), frac_roofline=round(ctf / roof, 4),
                             gbs=round(nbytes / (c["ms_median"] * 1e-3) / 1e9, 1))
        per[vname] = e
    dom = max(variants, key=lambda vname: ms[vname])
    achieved = fl[dom] / (ms[dom] * 1e-3) / 1e12
    bound, roof = flops.roofline_tflops(fl[dom], nbytes)
    # HBM bytes per launch from the committed counter runs, unless the
    # kernels changed since they were taken or the record was edited
    from flashattention_attention_variants_amd import profiling
    tpath = args.traffic or os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                         "traffic_%s.json" % wl.name)
    traffic = profiling.traffic_for(tpath, dom)
    roofline = dict(bound=bound, achieved=round(achieved, 1),
                    peak=flops.PEAK_BF16_TFLOPS if bound == "mfma" else flops.PEAK_HBM_GBS,
                    unit="TFLOP/s" if bound == "mfma" else "GB/s",
                    frac=round(achieved / flops.PEAK_BF16_TFLOPS, 4), traffic=traffic,
                    kernel="attn_mfma_kernel (%s)" % dom, ms_per_launch=round(ms[dom], 5),
                    useful_flop_per_launch=fl[dom], algorithmic_bytes_per_launch=nbytes,
                    timing="mean of the launch's HIP-event durations over the timed steps")
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
        ws = torch.empty(2 * B * Hq * S, dtype=torch.float32, device=dev)
        bper = {}
        for vname in variants:
            o_, lse_ = api.fl_attn_fwd(q, k, v, return_lse=True, **kws[vname])
            r = time_calls(torch, lambda: api.fl_attn_bwd(q, k, v, o_, lse_, d_o, dq=dq, dk=dk, dv=dv,
                                                          workspace=ws, **kws[vname]))
            bf = fl[vname] * 5 // 2
            btf = bf / (r["ms_median"] * 1e-3) / 1e12
            bper[vname] = dict(r, tflops=round(btf, 1),
                               frac_bf16_peak=round(btf / flops.PEAK_BF16_TFLOPS, 4))
        backward = dict(per_variant=bper, useful_flop="2.5 x the forward's (five products)",
                        timing="per call (both launches): median and min of HIP-event times; "
                               "tflops from the median")

    decode = None
    if not args.no_decode:
        decode = measure_decode(torch, api, flops, inputs, dev, flush)

    configs = None
    if not args.no_configs:
        configs = measure_configs(torch, api, flops, inputs, dev, flush)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H_q": Hq, "H_kv": Hkv, "S": S, "D": D,
                   "variants": variants, "step": "one forward call per variant",
                   "seed": wl.seed},
        "frac_bf16_peak": round(value / flops.PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "cpu_baseline": cpu,
        "clocks": dict(before=clk_before, after=clk_after,
                       note="amd-smi metric -c read while the step runs, before and after the "
                            "timed region"),
        "per_variant": per, "configs": configs, "backward": backward, "decode": decode,
    }
    print(json.dumps(line), flush=True)
    if args.report and configs:
        for name, entry in configs.items():
            print(json.dumps({"report": name, **entry}), flush=True)


def attn_kw(vname, pr, docs_dev):
    kw = dict(variant=vname)
    for key in ("softcap", "alibi_max_bias", "window", "window_causal", "prefix"):
        if key in pr:
            kw[key] = pr[key]
    if vname == "document":
        kw["doc_offsets"] = docs_dev
    return kw


def _entry(flops, f, nb, r, cold=None, peak=None, bound_override=None):
    """One measured case: time, TFLOP/s, GB/s and the fraction of its own
    roofline (from the primary timing: cold where given)."""
    peak = peak or flops.PEAK_BF16_TFLOPS
    bound, roof = flops.roofline_tflops(f, nb, peak_tflops=peak)
    prim = cold if cold is not None else r
    ms = prim["ms_median"]
    tf = f / (ms * 1e-3) / 1e12
    gbs = nb / (ms * 1e-3) / 1e9
    e = dict(warm=r, ms_median=ms, tflops=round(tf, 2), frac_bf16_peak=round(tf / peak, 4),
             gbs=round(gbs, 1), bound=bound_override or bound, roofline_tflops=round(roof, 1),
             frac_roofline=round(tf / roof, 4), useful_flop=int(f), algorithmic_bytes=int(nb),
             timing="cold (1 GiB read before each call), median" if cold is not None
             else "warm, median")
    if cold is not None:
        e["cold"] = cold
    if bound == "hbm":
        e["frac_hbm"] = round(gbs / flops.PEAK_HBM_GBS, 4)
    return e


def measure_configs(torch, api, flops, inputs, dev, flush):
    """Every other workload per call, each against its own roofline."""
    out = {}
    # float32 MHA with LSE: latency-bound at this size
    wl = inputs.WORKLOADS["mha_f32_b1_h2_s128_d64"]
    t = inputs.make(wl)
    g = {n: x.to(dev) for n, x in t.items()}
    s = wl.shape
    o = torch.empty_like(g["q"])
    lse = torch.empty(s["B"], s["Hq"], s["S"], dtype=torch.float32, device=dev)
    r = time_calls(torch, lambda: api.fl_attn_fwd(g["q"], g["k"], g["v"], out=o, lse=lse))
    f = flops.attn_flops("vanilla", s["B"], s["Hq"], s["S"], s["S"], s["D"])
    nb = flops.attn_bytes(s["B"], s["Hq"], s["Hkv"], s["S"], s["S"], s["D"], elem=4, lse=True)
    out["%s/vanilla" % wl.name] = _entry(flops, f, nb, r, peak=flops.PEAK_F32_VALU_TFLOPS,
                                         bound_override="latency")
    # bf16 MHA sweep at S=2048 and GQA at S=16384
    for name in ("mha_bf16_b4_h16_s2048_d64", "gqa_bf16_b1_hq32_hkv8_s16384_d64"):
        wl = inputs.WORKLOADS[name]
        t = inputs.make(wl)
        g = {n: x.to(dev) for n, x in t.items()}
        s = wl.shape
        o = torch.empty_like(g["q"])
        for vname in wl.variants:
            kw = attn_kw(vname, wl.params, g.get("doc_offsets"))
            fn = lambda: api.fl_attn_fwd(g["q"], g["k"], g["v"], out=o, **kw)  # noqa: E731
            r = time_calls(torch, fn)
            f = flops.attn_flops(vname, s["B"], s["Hq"], s["S"], s["S"], s["D"],
                                 window=wl.params.get("window", 256),
                                 window_causal=wl.params.get("window_causal", True),
                                 prefix=wl.params.get("prefix", 512),
                                 doc_offsets=None if "doc_offsets" not in t else t["doc_offsets"].numpy())
            nb = flops.attn_bytes(s["B"], s["Hq"], s["Hkv"], s["S"], s["S"], s["D"])
            cold = None
            if vname in COLD_VARIANTS or flops.roofline_tflops(f, nb)[0] == "hbm":
                cold = time_calls(torch, fn, flush=flush, max_calls=1000)
            out["%s/%s" % (name, vname)] = _entry(flops, f, nb, r, cold)
        del g
    # differential attention
    wl = inputs.WORKLOADS["diffattn_bf16_b4_h16_s4096_dqk64_dv128"]
    t = inputs.make(wl)
    g = [t[n].to(dev) for n in ("q1", "q2", "k1", "k2", "v")]
    s = wl.shape
    o = torch.empty(s["B"], s["H"], s["S"], s["Dv"], dtype=torch.bfloat16, device=dev)
    for vname in wl.variants:
        causal = vname == "causal"
        r = time_calls(torch, lambda: api.fl_diffattn_fwd(*g, lam=wl.params["lam"], causal=causal,
                                                          out=o))
        f = flops.diffattn_flops(s["B"], s["H"], s["S"], s["Dqk"], s["Dv"], causal)
        nb = flops.diffattn_bytes(s["B"], s["H"], s["S"], s["Dqk"], s["Dv"])
        out["%s/%s" % (wl.name, vname)] = _entry(flops, f, nb, r)
    del g
    # Evoformer row (pair bias, key mask, gate) and column: HBM-bound, cold
    wl = inputs.WORKLOADS[EVO_WORKLOAD]
    t = inputs.make(wl)
    g = {n: x.to(dev) for n, x in t.items()}
    s = wl.shape
    o = torch.empty_like(g["q"])
    for axis in wl.variants:
        pb = g["pair_bias"] if axis == "row" else None
        fn = lambda: api.fl_evoformer_gated_attn_fwd(  # noqa: E731
            g["q"], g["k"], g["v"], g["gate"], pair_bias=pb, key_mask=g["key_mask"], axis=axis, out=o)
        r = time_calls(torch, fn)
        cold = time_calls(torch, fn, flush=flush, max_calls=1000)
        f = flops.evoformer_flops(s["N_seq"], s["N_res"], s["H"], s["C"], axis)
        nb = flops.evoformer_bytes(s["N_seq"], s["N_res"], s["H"], s["C"], axis)
        out["%s/%s" % (wl.name, axis)] = _entry(flops, f, nb, r, cold)
    del g
    ipa = measure_ipa(torch, api, flops, inputs, dev, flush)
    if ipa:
        out.update(ipa)
    return out


def measure_ipa(torch, api, flops, inputs, dev, flush):
    """Invariant Point Attention core, if the library exports it."""
    if not hasattr(api, "fl_ipa_attn_fwd") or "ipa_bf16_nres256_h12" not in inputs.WORKLOADS:
        return None
    wl = inputs.WORKLOADS["ipa_bf16_nres256_h12"]
    t = inputs.make(wl)
    g = {n: x.to(dev) for n, x in t.items()}
    res = api.fl_ipa_attn_fwd(**g)
    outs = res if isinstance(res, tuple) else (res,)
    fn = lambda: api.fl_ipa_attn_fwd(**g, out=outs)  # noqa: E731
    r = time_calls(torch, fn)
    cold = time_calls(torch, fn, flush=flush, max_calls=1000)
    f, nb = flops.ipa_work(**wl.shape)
    return {"%s/ipa" % wl.name: _entry(flops, f, nb, r, cold)}


def measure_decode(torch, api, flops, inputs, dev, flush):
    """Decode against a KV cache (split keys + merge), HBM-bound: cold
    (primary) and warm per call."""
    dwl = inputs.WORKLOADS[DECODE_WORKLOAD]
    dt = inputs.make(dwl)
    dg = {k_: v_.to(dev) for k_, v_ in dt.items()}
    s = dwl.shape
    dper = {}
    for vname in dwl.variants:
        kw = dict(variant=vname)
        for key in ("softcap", "alibi_max_bias", "window", "window_causal"):
            if key in dwl.params:
                kw[key] = dwl.params[key]
        L = dt["seqlens"]
        max_len = int(L.max())
        ws_bytes = api.fl_attn_decode_workspace_size(
            s["B"], s["Hq"], s["Hkv"], s["Sq"], max_len, s["D"], variant=vname,
            window=kw.get("window", 256), window_causal=kw.get("window_causal", True))
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        out = torch.empty_like(dg["q"])
        fn = lambda: api.fl_attn_decode_fwd(  # noqa: E731
            dg["q"], dg["k_cache"], dg["v_cache"], dg["seqlens"], max_seqlen=max_len, workspace=ws,
            out=out, **kw)
        r = time_calls(torch, fn)
        cold = time_calls(torch, fn, flush=flush, max_calls=1000)
        mask = vname if vname in ("causal", "sliding_window", "prefix_lm") else None
        f, nb = flops.decode_work(mask, L.tolist(), s["Hq"], s["Hkv"], s["Sq"], s["D"],
                                  window=dwl.params.get("window", 256),
                                  window_causal=dwl.params.get("window_causal", True))
        dper[vname] = _entry(flops, f, nb, r, cold)
    return dict(workload=dwl.name, per_variant=dper,
                timing="per call (decode and merge kernels): median and min of HIP-event times, "
                       "cold (1 GiB read before each call) and warm")


def cpu_baseline(t, variants, kws, wl, seconds):
    """Oracle throughput (useful TFLOP/s) on sampled query rows of the same
    workload, all variants, float64, host threads."""
    import numpy as np

    import oracle

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
