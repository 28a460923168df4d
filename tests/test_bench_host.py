"""Host logic of bench.py (no GPU): the one-GPU guard, kernel-name parsing,
the source check on committed counter summaries, and the rocprofv3 digest
run on synthetic csv files whose expected figures are worked out by hand.
"""
import csv
import os
import subprocess
import sys

import pytest

import bench
from long_context_causal_amd.inputs import HEADLINE, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NS = "cpattn::(anonymous namespace)::"


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_short_kernel_names():
    assert bench._short_kernel(f"void {NS}attn_steps_bf16<128>({NS}StepsParams)") == \
        "attn_steps_bf16<128>"
    assert bench._short_kernel(f"{NS}partition_copy(long, long)") == "partition_copy"
    assert bench._short_kernel("void at::native::vectorized(int)") == "at::native::vectorized"


def test_committed_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """The committed figure counts only while the summary's source hash is
    the hash of the kernel sources in the tree."""
    (tmp_path / "profiles").mkdir()
    prof = tmp_path / "profiles" / "attn_steps_bf16__wl__hbm_traffic.txt"
    digest = bench._kernel_source_digest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_kernel_source_digest", lambda: digest)
    for recorded, want in ((digest, 123456.0), ("0" * 64, None)):
        prof.write_text(f"# kernel source sha256 (x): {recorded}\n"
                        "attention_traffic_bytes_per_launch: 123456\n"
                        "fused_traffic_bytes_per_launch: 789\n")
        assert bench.committed_traffic("wl") == want
        assert bench.committed_traffic("wl", "fused_traffic_bytes_per_launch") == \
            (789.0 if want else None)
    assert bench.committed_traffic("other") is None


def _write(path, fields, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=fields)
        wr.writeheader()
        wr.writerows(rows)


def test_digest_on_synthetic_profiles(tmp_path):
    """Dispatch order: 7 pre-warm and 13 timed launches of the headline
    steps grid, then a per-step launch (the window's end), the headline's
    fused launches, then the backward.  The digest keeps the last 13 steps
    grids (2000 us, so 2.1991e12 FLOP / 2 ms = 1099.5 TFLOP/s), calibrates
    FETCH_SIZE x2 and WRITE_SIZE x1 on the plain copies, and takes the MFMA
    busy fraction per SIMD over the active cycles per XCD."""
    w = WORKLOADS[HEADLINE]
    steps, fused = f"void {NS}attn_steps_bf16<128>({NS}StepsParams)", \
        f"void {NS}attn_fused_bf16<false, 128>({NS}Params)"
    step1, bwd = f"void {NS}attn_step_bf16<false, 128>({NS}Params)", \
        f"void {NS}attn_bwd_dq_share<8, 128>({NS}BwdParams)"
    copy = f"void {NS}partition_copy(long)"
    fl = bench.fused_grid_lanes(w)
    launches = [(1, copy, 65536, 7_000)]
    launches += [(10 + i, steps, 131072, 3_000_000 if i < 7 else 2_000_000) for i in range(20)]
    launches += [(40, step1, 524288, 280_000)]
    launches += [(50 + i, fused, fl, 1_900_000) for i in range(3)]
    launches += [(60, bwd, 524288, 2_800_000)]
    tf = ["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"]
    _write(tmp_path / "prof" / "trace" / "run_kernel_trace.csv", tf,
           [dict(zip(tf, (d, k, g, 1000 * d, 1000 * d + t))) for d, k, g, t in launches])
    cf = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]

    def counters(name, values):
        return [dict(zip(cf, (d, k, g, name, v))) for d, k, g, v in values]
    # a 65536-lane copy moves 65536 * 256 B = 16384 KiB each way
    _write(tmp_path / "prof" / "p1" / "run_counter_collection.csv", cf, counters(
        "FETCH_SIZE", [(1, copy, 65536, 8192), (10, steps, 131072, 500000),
                       (11, steps, 131072, 500000), (40, step1, 524288, 1),
                       (50, fused, fl, 200000), (60, bwd, 524288, 1)]))
    _write(tmp_path / "prof" / "p2" / "run_counter_collection.csv", cf, counters(
        "WRITE_SIZE", [(1, copy, 65536, 16384), (10, steps, 131072, 400000),
                       (11, steps, 131072, 400000), (40, step1, 524288, 1),
                       (50, fused, fl, 100000), (60, bwd, 524288, 1)]))
    sq = []
    for name, value in (("SQ_INSTS_MFMA", 1e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500),
                        ("GRBM_GUI_ACTIVE", 8 * 1000), ("SQ_INSTS_VALU", 6e6),
                        ("SQ_INSTS_LDS", 1.5e6)):
        sq += counters(name, [(10, steps, 131072, value), (40, step1, 524288, 1)])
    _write(tmp_path / "prof" / "p3" / "run_counter_collection.csv", cf, sq)

    out = tmp_path / "out"
    out.mkdir()
    bench.digest(str(tmp_path / "prof"), str(out))
    trace = (out / f"attn_steps_bf16__{w.name}__kernel_trace.txt").read_text()
    assert "attention_avg_launch_us: 2000.000" in trace
    assert f"attention_tflops_from_trace: {w.rank_flops() / 2e6 * 1e-3:.1f}" in trace
    assert "fused_avg_launch_us: 1900.000" in trace
    assert f"kernel source sha256 ({' + '.join(bench.KERNEL_SOURCES)}): " \
        f"{bench._kernel_source_digest()}" in trace
    traffic = (out / f"attn_steps_bf16__{w.name}__hbm_traffic.txt").read_text()
    assert "fetch_scale: 2.0000" in traffic and "write_scale: 1.0000" in traffic
    assert f"attention_traffic_bytes_per_launch: {(500000 * 2 + 400000) * 1024}" in traffic
    assert f"fused_traffic_bytes_per_launch: {(200000 * 2 + 100000) * 1024}" in traffic
    sqt = (out / f"attn_steps_bf16__{w.name}__sq_counters.txt").read_text()
    head = sqt[sqt.index("attn_steps_bf16 (headline share)"):]
    assert "mfma_busy_fraction (busy per SIMD / active cycles per XCD): 0.500" in head
    assert "valu_per_mfma: 6.00" in head and "lds_per_mfma: 1.50" in head


def test_digest_needs_its_csv_files(tmp_path):
    with pytest.raises(FileNotFoundError):
        bench.digest(str(tmp_path / "missing"), str(tmp_path))


def test_host_cpu_model_names_family_and_model():
    import bench
    name = bench.host_cpu_model()
    if name is None:
        pytest.skip("no /proc/cpuinfo model name on this host")
    assert "cpu family" in name and "model" in name, name
