"""Host logic of the rocprofv3 summaries (synthetic CSV files, no GPU)."""
import csv
import os

from flashattention_attention_variants_amd import profiling

HEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
        "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value",
        "Start_Timestamp", "End_Timestamp"]


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(HEAD)
        for i, (name, kib) in enumerate(rows, 1):
            w.writerow([i, i, "Agent 1", 1, 1, 1, 64, 1, name, 256, 0, 0, 128, 0, 96, counter,
                        kib, 0, 1])


def test_traffic_calibration(tmp_path):
    variants = ["vanilla", "causal"]
    attn = "void fl::attn_mfma_kernel<fl::MfmaCfg<64, 64, 1, 2, 0> >(fl::KernelArgs)"
    copy_kib = profiling.PROBE_COPY_BYTES / 1024
    # warmup calls, a small unrelated copy, the calibration copy, the measured calls
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(attn, 999.0), (attn, 999.0), ("__amd_rocclr_copyBuffer", 3.0),
                     ("__amd_rocclr_copyBuffer", copy_kib / 2), (attn, 1000.0), (attn, 500.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(attn, 7.0), (attn, 7.0), ("__amd_rocclr_copyBuffer", copy_kib),
                     (attn, 64.0), (attn, 32.0)])
    rec = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"), variants)
    assert abs(rec["fetch_factor"] - 2.0) < 1e-12
    assert abs(rec["write_factor"] - 1.0) < 1e-12
    pv = rec["per_variant"]
    assert pv["vanilla"]["fetch_bytes"] == 1000 * 1024 * 2
    assert pv["causal"]["fetch_bytes"] == 500 * 1024 * 2
    assert pv["vanilla"]["write_bytes"] == 64 * 1024
    assert pv["causal"]["traffic_bytes"] == 500 * 1024 * 2 + 32 * 1024
    assert rec["kernel_digest"] == profiling.kernel_digest()


def test_stats_table(tmp_path):
    d = tmp_path / "kt"
    os.makedirs(d)
    with open(d / "run_kernel_stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow(["void fl::attn_mfma_kernel<X>(fl::KernelArgs)", 3, 3000, 1000.0, 100.0, 900, 1100,
                    10.0])
    t = profiling.stats_table(str(d))
    assert "`fl::attn_mfma_kernel<X>` | 3 | 1.0 | 0.9 | 1.1 | 100.0% |" in t


def test_digest_tracks_sources():
    a = profiling.kernel_digest()
    assert a == profiling.kernel_digest() and len(a) == 16


def test_decode_kernel_names():
    dec = "void fl::attn_mfma_kernel<fl::MfmaCfg<64, 64, 1, 1, 3, false, false, false, true> >(fl::KernelArgs)"
    pre = "void fl::attn_mfma_kernel<fl::MfmaCfg<64, 64, 1, 2, 0, false, false, false, false> >(fl::KernelArgs)"
    evo = "void fl::attn_mfma_kernel<fl::MfmaCfg<32, 32, 1, 2, 0, true, true, true, false> >(fl::KernelArgs)"
    assert profiling.is_decode_kernel(dec)
    assert profiling.is_decode_kernel("_ZN2fl12merge_kernelIDF16bEEvPKfS2_iliPT_Pf")
    assert not profiling.is_decode_kernel(pre) and not profiling.is_decode_kernel(evo)


def test_evoformer_traffic_table(tmp_path):
    from flashattention_attention_variants_amd import flops
    # the row form with its pair bias runs on the short-row kernel
    row = "void fl::evo_kernel<fl::EvoCfg<8, true> >(fl::KernelArgs)"
    col = "void fl::attn_mfma_kernel<fl::MfmaCfg<32, 32, 1, 1, 0, false, true, true, false> >(fl::KernelArgs)"
    copy_kib = profiling.PROBE_COPY_BYTES / 1024
    alg_row = flops.evoformer_bytes(128, 256, 8, 32, "row")
    # the row launch moves exactly its algorithmic bytes, the column twice its own
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(row, 1.0), (col, 1.0), ("__amd_rocclr_copyBuffer", copy_kib),
                     (row, alg_row / 1024), (col, 2 * flops.evoformer_bytes(128, 256, 8, 32, "col") / 1024)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(row, 1.0), (col, 1.0), ("__amd_rocclr_copyBuffer", copy_kib), (row, 0.0),
                     (col, 0.0)])
    md = profiling.evo_traffic_markdown(str(tmp_path / "f"), str(tmp_path / "w"))
    lines = [l for l in md.splitlines() if l.startswith("| row |") or l.startswith("| col |")]
    assert lines[0].endswith("| 1.00 |") and lines[1].endswith("| 2.00 |"), lines


def test_traffic_record_guard(tmp_path):
    """bench.py takes traffic from a record only while the kernel sources and
    the record's own fields are as the tool wrote them."""
    import json
    attn = "void fl::attn_mfma_kernel<fl::MfmaCfg<64, 64, 1, 2, 0> >(fl::KernelArgs)"
    copy_kib = profiling.PROBE_COPY_BYTES / 1024
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [("__amd_rocclr_copyBuffer", copy_kib / 2), (attn, 1000.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib), (attn, 64.0)])
    rec = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"), ["vanilla"])
    assert len(rec["csv_sha256"]["fetch"]) == 64
    path = tmp_path / "t.json"
    path.write_text(json.dumps(rec))
    assert profiling.traffic_for(str(path), "vanilla") == 1000 * 1024 * 2 + 64 * 1024
    assert profiling.traffic_for(str(path), "causal") is None
    # an edited kernel digest (or any other field) voids the record
    for key, val in (("kernel_digest", "0" * 16), ("fetch_factor", 3.0)):
        bad = dict(rec, **{key: val})
        path.write_text(json.dumps(bad))
        assert profiling.traffic_for(str(path), "vanilla") is None, key
    assert profiling.traffic_for(str(tmp_path / "missing.json"), "vanilla") is None


def test_dispatch_table(tmp_path):
    """Dispatches of one kernel instance at two launch shapes get a row each,
    with the average of their own durations."""
    d = tmp_path / "kt"
    os.makedirs(d)
    name = "void fl::attn_mfma_kernel<fl::MfmaCfg<64, 64, 1, 2, 3> >(fl::KernelArgs)"
    head = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
            "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X",
            "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(head)
        # 1024 work-groups: 360 and 362 us; 512 work-groups: 100 us
        for i, (t0, t1, grid) in enumerate([(0, 360000, 262144), (10 ** 6, 10 ** 6 + 362000, 262144),
                                             (2 * 10 ** 6, 2 * 10 ** 6 + 100000, 131072)]):
            w.writerow(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i + 1, 3, name, i + 1, t0, t1, 0, 0,
                        128, 0, 96, 256, 1, 1, grid, 1, 1])
    t = profiling.dispatch_table(str(d))
    rows = [l for l in t.splitlines() if l.startswith("| `")]
    assert rows[0].endswith("| 1024 | 2 | 361.0 | 360.0 | 362.0 |"), rows
    assert rows[1].endswith("| 512 | 1 | 100.0 | 100.0 | 100.0 |"), rows
