"""Host logic of bench.py (CPU only): the rocprofv3 summariser that writes
profiles/, and the traffic lookup that fills the bench line's
roofline.traffic.

- The committed counters must belong to the committed kernel source: every
  entry of profiles/traffic.json carries the source digest it was taken on,
  and the bench reports traffic only while that digest matches.
- The summariser, run on small synthetic rocprofv3 CSV files, must scale
  FETCH_SIZE / WRITE_SIZE by the copy calibration, take medians, and record
  the digest.
"""
import csv
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_committed_counters_match_the_kernel_source():
    b = _bench()
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    digest = b.source_digest()
    assert rec, "profiles/traffic.json is empty"
    for kernel, per in rec.items():
        for workload, ent in per.items():
            assert ent["source_sha256_16"] == digest, (kernel, workload, ent["source_sha256_16"], digest)
            assert ent["bytes_per_launch"] > 0
    # and the lookup the bench line uses returns them
    assert b.load_traffic("row_pass", "c5_mixed") == rec["row_pass"]["c5_mixed"]["bytes_per_launch"]
    assert b.load_traffic("row_pass", "no_such_workload") is None


def test_summariser_scales_and_records(tmp_path):
    b = _bench()
    rdir = tmp_path / "rocprof"
    out = tmp_path / "profiles"
    # kernel trace: three launches each, durations in ns
    trace = []
    t = 1000
    for k in range(3):
        for name, us in (("void row_pass<1, true>(Ctx)", 100 + k), ("void scan_kernel<1>(Ctx)", 6),
                         ("void residual_kernel<1, true>(Ctx)", 15), ("void draw_kernel<1, true>(Ctx)", 6)):
            trace.append([name, t, t + us * 1000])
            t += us * 1000 + 500
    _write(str(rdir / "prof" / "mixed_c5_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           trace)
    pmc = rdir / "pmc"
    cols = ["Kernel_Name", "Counter_Value"]
    # the copy calibration reads 512 MiB and writes 512 MiB; FETCH_SIZE counts half
    _write(str(pmc / "copy_FETCH_SIZE_counter_collection.csv"), cols, [["stream_copy_kernel(x)", 262144.0]] * 3)
    _write(str(pmc / "copy_WRITE_SIZE_counter_collection.csv"), cols, [["stream_copy_kernel(x)", 524288.0]] * 3)
    _write(str(pmc / "bench_FETCH_SIZE_counter_collection.csv"), cols,
           [["row_pass<1, true>(x)", v] for v in (1000.0, 1001.0, 1500.0)] + [["scan_kernel<1>(x)", 10.0]])
    _write(str(pmc / "bench_WRITE_SIZE_counter_collection.csv"), cols,
           [["row_pass<1, true>(x)", 2.0]] * 3 + [["scan_kernel<1>(x)", 1.0]])
    # residual counter passes: two dispatches, per-XCD rows summed per dispatch
    sq = ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"]
    _write(str(pmc / "res_sqA_counter_collection.csv"), sq,
           [["residual_kernel<1, true>(x)", "SQ_INSTS_VALU", d, 100.0] for d in (1, 2) for _ in range(8)]
           + [["residual_kernel<1, true>(x)", "SQ_WAVE_CYCLES", d, 1000.0] for d in (1, 2)])
    _write(str(pmc / "res_sqB_counter_collection.csv"), sq,
           [["residual_kernel<1, true>(x)", "GRBM_GUI_ACTIVE", d, 5.0] for d in (1, 2)])

    assert b.summarize_rocprof(str(rdir), out_dir=str(out)) == 0
    md = (out / "verify_c5_mixed.md").read_text()
    assert "| row_pass | 3 | 101.00 | 101.00 | 100.00 | 102.00 |" in md
    assert "FETCH_SIZE is scaled by 2.0000 and WRITE_SIZE by 1.0000" in md
    assert "| SQ_INSTS_VALU | 800 |" in md                      # eight rows of one dispatch summed
    assert b.source_digest() in md
    traffic = json.loads((out / "traffic.json").read_text())
    ent = traffic["row_pass"]["c5_mixed"]
    assert ent["bytes_per_launch"] == pytest.approx((1001.0 * 2.0 + 2.0 * 1.0) * 1024.0)
    assert ent["source_sha256_16"] == b.source_digest()
    assert traffic["scan"]["c5_mixed"]["bytes_per_launch"] == pytest.approx((10.0 * 2.0 + 1.0) * 1024.0)


def test_gemm_counter_section(tmp_path):
    """Clock and matrix-pipe share from synthetic GEMM counters: 8 XCDs of
    1.8e6 GRBM cycles over 1 ms is 1.8 GHz; the ideal MFMA cycles over that
    clock's 1.8e6 cycles per SIMD give the busy share; the first third of the
    dispatches (the clock ramp) is left out."""
    b = _bench()
    pmc = tmp_path / "pmc"
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    ideal = b.GEMM_FLOPS / b.FLOPS_PER_SIMD_CYCLE
    rows = []
    for d in range(6):
        grbm = (0.9e6 if d < 2 else 1.8e6) * b.XCDS          # the first two: a slow clock
        for name, val in (("GRBM_GUI_ACTIVE", grbm), ("SQ_VALU_MFMA_BUSY_CYCLES", ideal),
                          ("SQ_BUSY_CYCLES", 1.0), ("SQ_WAVES", 32768)):
            rows.append([d, "void lm_head_dl_kernel<0>(LmArgs)", name, val, 0, 1_000_000])
        rows.append([d, "void row_pass<1, true>(Ctx)", "GRBM_GUI_ACTIVE", 1.0, 0, 1000])
    _write(str(pmc / "gemm_sq_counter_collection.csv"), header, rows)
    text = "\n".join(b.gemm_counter_section(str(pmc)))
    busy = ideal / b.SIMDS / 1.8e6
    assert "| clock, GRBM_GUI_ACTIVE / 8 XCDs / duration (GHz) | 1.800 | 1.800-1.800 |" in text
    assert f"| matrix pipe busy at that clock | {busy:.3f} |" in text
    assert b.gemm_counter_section(str(tmp_path / "absent")) == []
