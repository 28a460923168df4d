"""Throughput of one GPU's context-parallel causal attention share.

A step is one pass of the whole path over one batch of synthetic input
already resident in HBM: the zigzag split of Q, K and V (three
cpattn_partition launches), the cp blockwise-attention steps of the
measured rank (at step i the rank reads the K/V block of rank (rank - i)
mod cp; all cp steps as one grid through cpattn_forward_steps, each step
writing its own partial O_i and L_i) and the LSE merge (cpattn_merge).  W
untimed warm-up steps, then K timed steps bracketed by synchronisation.
The same steps launched one by one (cpattn_step_fwd) are reported under
"per_step_launches".

The same share is also timed through the fused form (the split, then one
cpattn_forward_fused launch that carries the online softmax across the cp
key blocks, so there are no partials and no merge) and reported under
"fused", and its backward (cpattn_backward with a seeded bf16 dO and the
forward's merged O and L) under "backward".

value = causal-effective FLOPs of the rank's share (4*d per visible query/
key pair) / the measured time of a step.  Per-kernel times come from HIP
events recorded on the stream the kernels run on.  Also reported: the step
kernels' TFLOP/s for every rank of the share ("ranks", min and max), and
for the other bf16 configurations at their measured rank ("configs").

The CPU baseline times the fp64 oracle on the host cores on a bounded
sample of the same rank share (every k-th local row, all heads).
"""
import argparse
import dataclasses
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-sample-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-rank and per-configuration step timings")
    ap.add_argument("--digest", metavar="DIR", default=None,
                    help="write the profiles/ summaries from rocprofv3 csv output under DIR "
                         "(DIR/trace: kernel trace; DIR/p1, DIR/p2: FETCH_SIZE, WRITE_SIZE; "
                         "DIR/p3: SQ counters; see PROFILE_COMMANDS) and exit")
    return ap.parse_args()


# the sources the forward attention kernels are built from (their digest
# ties a committed counter summary to the code it was measured on)
KERNEL_SOURCES = ("attn_step_bf16.hip", "mfma_tiles.h")


def packing_offsets(s, cp):
    """Sample offsets of the packed leg: eight samples in the length ratio
    1:2:4:1:8:3:5:8 (units of s/32 rows, each a multiple of 2cp)."""
    import numpy as np
    units = [1, 2, 4, 1, 8, 3, 5, 8]
    unit = s // 32
    if unit % (2 * cp) != 0 or unit * 32 != s:
        raise ValueError("the packed leg needs s/32 to be a multiple of 2*cp")
    return np.concatenate([[0], np.cumsum([u * unit for u in units])]).astype(np.int64)


def committed_traffic(workload, key="attention_traffic_bytes_per_launch"):
    """HBM bytes per launch of the attention kernel (key: the step kernel's
    or the fused kernel's line) from the committed counter summary.

    The summary records the sha256 of the kernel sources it was measured
    with (KERNEL_SOURCES, concatenated); if they have changed since, the
    figure no longer describes this kernel and None is returned.
    """
    prof = os.path.join(ROOT, "profiles", f"attn_steps_bf16__{workload}__hbm_traffic.txt")
    if not os.path.exists(prof):
        return None
    digest = _kernel_source_digest()
    recorded, traffic = None, None
    with open(prof) as f:
        for line in f:
            if "kernel source sha256" in line:
                recorded = line.rsplit(":", 1)[1].strip()
            if line.startswith(key + ":"):
                traffic = float(line.split(":", 1)[1])
    return traffic if recorded == digest else None


def cpu_baseline(w, q, k, v, rank, target_s):
    """Oracle (fp64, OpenMP) on every stride-th local row of the rank share."""
    import numpy as np
    from long_context_causal_amd.inputs import as_f32
    from oracle import attention_rows, max_threads
    from oracle import cp as ocp

    pos_all = ocp.zigzag_positions(w.s, w.cp, rank)
    per_row = 4 * w.d * w.hq * w.b * (pos_all + 1)      # FLOPs of each local row
    # calibrate the rate on a few rows, then size the sample to ~target_s
    def run(pos):
        qf = as_f32(q[:, pos]).astype(np.float64)
        hi = int(pos.max()) + 1
        kf = as_f32(k[:, :hi]).astype(np.float64)
        vf = as_f32(v[:, :hi]).astype(np.float64)
        if w.rope_theta is not None:
            qf = ocp.rope(qf, pos, w.rope_theta)
            kf = ocp.rope(kf, np.arange(hi), w.rope_theta)
        t0 = time.perf_counter()
        attention_rows(qf, kf, vf, pos + 1)
        return time.perf_counter() - t0
    probe = pos_all[:: max(1, len(pos_all) // 16)]
    t_probe = run(probe)
    rate = (4 * w.d * w.hq * w.b * (probe + 1)).sum() / max(t_probe, 1e-6)
    stride = max(1, int(np.ceil(per_row.sum() / rate / target_s)))
    sample = pos_all[::stride]
    dt = run(sample)
    flops = float((4 * w.d * w.hq * w.b * (sample + 1)).sum())
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": max_threads(),
            "kind": "oracle", "cpu_model": host_cpu_model(),
            "host_logical_cpus": os.cpu_count(),
            "sample": f"rank {rank}: every {stride}th of its {len(pos_all)} local rows "
                      f"({len(sample)} rows x {w.hq} heads x b={w.b}, all visible keys), "
                      f"{flops / 1e9:.1f} GFLOP in {dt:.1f} s, fp64"}


# The engine clock ramps up over a fraction of a second of load after the
# GPU has idled (e.g. while the host draws the next workload's inputs); a
# leg that timed its kernels right after an idle spell measured them up to
# 25% slow.  Every timed leg first runs its own work for PREWARM_S seconds,
# untimed, then its warm-up steps.
PREWARM_S = 1.0


def prewarm(torch, fn, seconds=PREWARM_S):
    """Runs fn (which enqueues GPU work) repeatedly for about ``seconds``."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo, with its family and
    model numbers and clock (a virtual machine may report only a vendor
    name), or None."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break          # the first processor's block is enough
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    except OSError:
        return None
    name = fields.get("model name")
    if name is None:
        return None
    extra = [f"{k} {fields[k]}" for k in ("cpu family", "model", "cpu MHz") if k in fields]
    return f"{name} ({', '.join(extra)})" if extra else name


def share_fused_tflops(C, torch, P, w, rank, stream, reps=5, warmup=2):
    """TFLOP/s of the fused launch (cpattn_forward_fused) of one rank's
    share, from HIP events on ``stream`` (median)."""
    import numpy as np
    out = P.alloc_out(rank, C.CPATTN_F32)
    with torch.cuda.stream(stream):
        prewarm(torch, lambda: P.forward_fused(out, stream))
        for _ in range(warmup):
            P.forward_fused(out, stream)
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            P.forward_fused(out, stream)
            e[1].record(stream)
            ev.append(e)
        torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del out
    return w.rank_flops() / (ms * 1e-3) / 1e12


def share_step_tflops(C, torch, P, w, rank, stream, reps=5, warmup=2):
    """(attention TFLOP/s of the steps' grid, TFLOP/s over steps + merge) of
    one rank's share, from HIP events on ``stream``."""
    import numpy as np
    buf = P.alloc_rank(rank, C.CPATTN_F32)
    with torch.cuda.stream(stream):
        prewarm(torch, lambda: (P.steps(buf, stream), P.merge(buf, stream)))
        for _ in range(warmup):
            P.steps(buf, stream)
            P.merge(buf, stream)
        torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            P.steps(buf, stream)
            e[1].record(stream)
            P.merge(buf, stream)
            e[2].record(stream)
            ev.append(e)
        torch.cuda.synchronize()
    steps = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    whole = float(np.median([a.elapsed_time(c) for a, _, c in ev]))
    flops = w.rank_flops()
    del buf
    return flops / (steps * 1e-3) / 1e12, flops / (whole * 1e-3) / 1e12


def split_gbps(torch, P, w, stream, reps=5):
    """The split of Q, K and V (RoPE on Q and K where the workload has it)
    in GB/s of algorithmic bytes: in a warm loop, and each launch after a
    512 MB scratch write that evicts the 256 MB last-level cache (medians)."""
    import numpy as np
    es = 2 if w.dtype == "bf16" else 4
    nbytes = 2 * w.b * w.s * (w.hq + 2 * w.hkv) * w.d * es + 4 * w.s
    q_bytes = 2 * w.b * w.s * w.hq * w.d * es
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    hot, cold, q_only = [], [], []
    with torch.cuda.stream(stream):
        prewarm(torch, lambda: P.partition(stream), 0.5)
        for rep in range(2 * reps):
            if rep >= reps:
                scratch.fill_(1)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            P.partition_one("q", stream)
            e[1].record(stream)
            P.partition_one("k", stream)
            P.partition_one("v", stream)
            e[2].record(stream)
            (cold if rep >= reps else hot).append((e[0], e[2]))
            q_only.append((e[0], e[1]))
        torch.cuda.synchronize()
    del scratch
    med = lambda ev: float(np.median([a.elapsed_time(b) for a, b in ev]))
    return {"rope": w.rope_theta is not None, "bytes": nbytes,
            "gbps": round(nbytes / (med(hot) * 1e-3) / 1e9, 1),
            "cold_cache_gbps": round(nbytes / (med(cold) * 1e-3) / 1e9, 1),
            "q_gbps": round(q_bytes / (med(q_only) * 1e-3) / 1e9, 1)}


def peak_check(C, torch, stream, iters=10000, rounds=4):
    """The bf16 MFMA rate this part sustains on a pure matrix stream (random
    operands, two waves per SIMD, one workgroup per CU at a time, 'rounds'
    workgroups per CU), beside the published peak; plus the device's
    compute units and maximum clock."""
    import numpy as np
    cus, khz = C.cpattn_device_info()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    ops = (torch.randn(4096, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    blocks = cus * rounds
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    flops = blocks * 8 * iters * 16 * 32768
    with torch.cuda.stream(stream):
        C.cpattn_probe_mfma(ops, out, blocks, iters, stream)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record(stream)
            C.cpattn_probe_mfma(ops, out, blocks, iters, stream)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
    return {"compute_units": cus, "max_clock_mhz": khz / 1000.0,
            "published_peak_tflops": PEAK_BF16_TFLOPS,
            "peak_at_max_clock_tflops": round(cus * 4 * 1024 * khz * 1e3 / 1e12, 1),
            "mfma_probe_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "probe": "v_mfma_f32_32x32x16_bf16 stream, random bf16 operands, "
                     f"2 waves per SIMD, one workgroup per CU at a time, {rounds} rounds "
                     "(cpattn_probe_mfma)"}


# --- rocprofv3 summaries (python bench.py --digest DIR) ------------------------

# the commands whose csv output --digest reads (run from the repository root)
_BENCH = "python3 bench.py --steps {steps} --warmup {warmup} --cpu-sample-seconds 0"
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {dir}/trace -o run -- "
             + _BENCH.format(steps=10, warmup=3),
    "p1": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {dir}/p1 -o run -- "
          + _BENCH.format(steps=2, warmup=1),
    "p2": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {dir}/p2 -o run -- "
          + _BENCH.format(steps=2, warmup=1),
    "p3": "rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS "
          "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE "
          "--output-format csv -d {dir}/p3 -o run -- " + _BENCH.format(steps=2, warmup=1),
}
# a partition_copy workgroup (256 lanes) moves 4096 16-byte vectors: its
# dispatch reads and writes exactly 256 bytes per lane of its grid (every
# workload here splits into whole workgroups)
COPY_BYTES_PER_LANE = 256


def _short_kernel(name):
    name = name.replace("cpattn::(anonymous namespace)::", "")
    return name[5:].split("(")[0] if name.startswith("void ") else name.split("(")[0]


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def fused_grid_lanes(w):
    return (2 * w.c + 255) // 256 * w.hq * w.b * 512


def _kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "long_context_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def digest(prof_dir, out_dir=None):
    """The three profiles/ summaries of the headline workload from the csv
    output of PROFILE_COMMANDS under prof_dir (written to out_dir, by default
    the repository's profiles/)."""
    import collections
    import statistics
    from long_context_causal_amd.inputs import HEADLINE, WORKLOADS
    w = WORKLOADS[HEADLINE]
    src = _kernel_source_digest()
    cmd = {k: v.format(dir=prof_dir) for k, v in PROFILE_COMMANDS.items()}
    mean = statistics.mean
    out_files = {}

    # Which launches belong to which share, by dispatch order (bench order):
    # the headline's steps grids come before the first per-step launch
    # (attn_step_bf16); the 128k RoPE share's launches come after the first
    # partition_rope (no other workload rotates); the fused launches of the
    # headline share come before the first backward dispatch.  (The steps
    # grid of every share has one resident workgroup per CU, so grid sizes
    # do not tell the shares apart.)
    def windows(rows):
        first = lambda pred: min((int(r["Dispatch_Id"]) for r in rows if pred(r)),
                                 default=1 << 62)
        name = lambda r: _short_kernel(r["Kernel_Name"])
        return {"bwd": first(lambda r: name(r).startswith("attn_bwd")),
                "per_step": first(lambda r: name(r).startswith("attn_step_bf16")),
                "c5": first(lambda r: name(r).startswith("partition_rope"))}

    def steps_of(rows, w_name, value, last=None):
        """Values of the steps-grid dispatches of the headline or the 128k share
        (the last `last` of them: a leg's warm-up and timed launches come after
        its pre-warm)."""
        win = windows(rows)
        lo, hi = (win["c5"], 1 << 62) if w_name == "bf16_gqa_s128k_cp16_rope" else (
            0, win["per_step"])
        # the grid kernel is a template over the head dimension (d = 128 here)
        sel = sorted((r for r in rows
                      if _short_kernel(r["Kernel_Name"]) in ("attn_steps_bf16",
                                                             "attn_steps_bf16<128>")
                      and lo <= int(r["Dispatch_Id"]) < hi), key=lambda r: int(r["Dispatch_Id"]))
        return [value(r) for r in (sel[-last:] if last else sel)]

    def fused_of(rows, grid_key, w_name, value):
        """Values of the fused dispatches of one workload's share."""
        win = windows(rows)
        g = fused_grid_lanes(WORKLOADS[w_name])
        lo, hi = (win["c5"], 1 << 62) if w_name == "bf16_gqa_s128k_cp16_rope" else (0, win["bwd"])
        if w_name not in (HEADLINE, "bf16_gqa_s128k_cp16_rope"):
            lo, hi = 0, 1 << 62
        return [value(r) for r in rows
                if _short_kernel(r["Kernel_Name"]).startswith("attn_fused_bf16")
                and int(r[grid_key]) == g and lo <= int(r["Dispatch_Id"]) < hi]

    # kernel trace: durations per kernel and per (kernel, grid)
    trace = _csv_rows(os.path.join(prof_dir, "trace"), "kernel_trace.csv")
    byg = collections.defaultdict(list)
    dur_of = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    for r in trace:
        byg[(_short_kernel(r["Kernel_Name"]), int(r["Grid_Size_X"]))].append(dur_of(r))
    lines = [f"# rocprofv3 kernel trace (durations in us), {w.name} and the other bf16 workloads",
             f"# command (repository root, MI355X): {cmd['trace']}",
             f"# summary: python3 bench.py --digest {prof_dir}",
             f"# kernel source sha256 ({' + '.join(KERNEL_SOURCES)}): {src}", "",
             f"{'kernel':34s} {'grid_lanes':>11s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
             f"{'max_us':>10s}"]
    for (k, g), v in sorted(byg.items()):
        lines.append(f"{k:34s} {g:11d} {len(v):6d} {mean(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} "
                     f"{max(v) / 1e3:10.2f}")
    lines.append("(launches of several shares on one kernel and grid are split by dispatch "
                 "order below)")
    lines.append("")
    # the headline leg's warm-up and timed launches
    m = re.search(r"--steps (\d+) --warmup (\d+)", cmd["trace"])
    timed = int(m.group(1)) + int(m.group(2))
    for name in (HEADLINE, "bf16_gqa_s8k_cp4", "bf16_mha_s16k_cp4_widelogits",
                 "bf16_gqa_s128k_cp16_rope"):
        wc = WORKLOADS[name]
        v = (steps_of(trace, name, dur_of, timed if name == HEADLINE else None)
             if name in (HEADLINE, "bf16_gqa_s128k_cp16_rope") else [])
        if v:
            lines.append(f"{name} rank {wc.rank}: attn_steps_bf16: {len(v)} launches, "
                         f"mean {mean(v) / 1e3:.2f} us, {wc.rank_flops():.4e} FLOP per launch, "
                         f"{wc.rank_flops() / mean(v) * 1e-3:.1f} TFLOP/s")
        fv = fused_of(trace, "Grid_Size_X", name, dur_of)
        if fv:
            lines.append(f"{name} rank {wc.rank}: attn_fused_bf16 grid {fused_grid_lanes(wc)}: "
                         f"{len(fv)} launches, mean {mean(fv) / 1e3:.2f} us, "
                         f"{wc.rank_flops() / mean(fv) * 1e-3:.1f} TFLOP/s")
    v = steps_of(trace, HEADLINE, dur_of, timed)
    if v:
        lines.append(f"attention_avg_launch_us: {mean(v) / 1e3:.3f}")
        lines.append(f"attention_tflops_from_trace: {w.rank_flops() / mean(v) * 1e-3:.1f}")
    fv = fused_of(trace, "Grid_Size_X", HEADLINE, dur_of)
    if fv:
        lines.append(f"fused_avg_launch_us: {mean(fv) / 1e3:.3f}")
        lines.append(f"fused_tflops_from_trace: {w.rank_flops() / mean(fv) * 1e-3:.1f}")
    out_files[f"attn_steps_bf16__{w.name}__kernel_trace.txt"] = lines

    # HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), scaled by
    # what they read for the plain copies of known size
    def counters(sub):
        d = collections.defaultdict(list)
        rows = _csv_rows(os.path.join(prof_dir, sub), "counter_collection.csv")
        for r in rows:
            d[(_short_kernel(r["Kernel_Name"]), int(r["Grid_Size"]), r["Counter_Name"])].append(
                float(r["Counter_Value"]))
        return d, rows
    (fetch, fetch_rows), (write, write_rows) = counters("p1"), counters("p2")
    cal = []
    for (k, g, c), v in sorted(fetch.items()):
        if k == "partition_copy" and c == "FETCH_SIZE":
            true_kib = g * COPY_BYTES_PER_LANE / 1024
            wv = write.get((k, g, "WRITE_SIZE"))
            if wv:
                cal.append((g, true_kib, mean(v), mean(wv)))
    f_fetch = mean(t / f for _, t, f, _ in cal)
    f_write = mean(t / wr for _, t, _, wr in cal)
    lines = [f"# HBM traffic counters per dispatch (KiB), {w.name}",
             f"# command 1: {cmd['p1']}", f"# command 2: {cmd['p2']}",
             f"# summary: python3 bench.py --digest {prof_dir}",
             f"# kernel source sha256 ({' + '.join(KERNEL_SOURCES)}): {src}",
             "# calibration: every partition_copy dispatch is a plain copy that reads and "
             f"writes {COPY_BYTES_PER_LANE} bytes per lane of its grid",
             f"# {'grid_lanes':>10s} {'true_KiB':>10s} {'FETCH_KiB':>10s} {'WRITE_KiB':>10s} "
             f"{'true/FETCH':>10s} {'true/WRITE':>10s}"]
    for g, t, f, wr in cal:
        lines.append(f"# {g:10d} {t:10.0f} {f:10.0f} {wr:10.0f} {t / f:10.4f} {t / wr:10.4f}")
    lines += [f"fetch_scale: {f_fetch:.4f}", f"write_scale: {f_write:.4f}",
              f"fetch_scale_spread: {min(t / f for _, t, f, _ in cal):.4f}"
              f"..{max(t / f for _, t, f, _ in cal):.4f}",
              f"write_scale_spread: {min(t / wr for _, t, _, wr in cal):.4f}"
              f"..{max(t / wr for _, t, _, wr in cal):.4f}", "",
              f"{'kernel':34s} {'grid_lanes':>11s} {'n':>3s} {'FETCH_KiB':>12s} "
              f"{'WRITE_KiB':>12s} {'scaled_MB':>10s}"]
    scaled_of = {}
    for (k, g, c), v in sorted(fetch.items()):
        if c != "FETCH_SIZE":
            continue
        wv = write.get((k, g, "WRITE_SIZE"))
        if not wv:
            continue
        scaled = (mean(v) * f_fetch + mean(wv) * f_write) * 1024
        scaled_of[(k, g)] = scaled
        lines.append(f"{k:34s} {g:11d} {len(v):3d} {mean(v):12.0f} {mean(wv):12.0f} "
                     f"{scaled / 1e6:10.1f}")
    lines.append("")
    sf = steps_of([r for r in fetch_rows if r["Counter_Name"] == "FETCH_SIZE"], HEADLINE,
                  lambda r: float(r["Counter_Value"]))
    sw = steps_of([r for r in write_rows if r["Counter_Name"] == "WRITE_SIZE"], HEADLINE,
                  lambda r: float(r["Counter_Value"]))
    if sf and sw:
        lines.append(f"attention_traffic_bytes_per_launch: "
                     f"{(mean(sf) * f_fetch + mean(sw) * f_write) * 1024:.0f}")
    ff = fused_of([r for r in fetch_rows if r["Counter_Name"] == "FETCH_SIZE"], "Grid_Size",
                  HEADLINE, lambda r: float(r["Counter_Value"]))
    fw = fused_of([r for r in write_rows if r["Counter_Name"] == "WRITE_SIZE"], "Grid_Size",
                  HEADLINE, lambda r: float(r["Counter_Value"]))
    if ff and fw:
        lines.append(f"fused_traffic_bytes_per_launch: "
                     f"{(mean(ff) * f_fetch + mean(fw) * f_write) * 1024:.0f}")
    out_files[f"attn_steps_bf16__{w.name}__hbm_traffic.txt"] = lines

    # SQ counters: instruction mix and MFMA busy fraction per (kernel, grid)
    sq, sq_rows = counters("p3")
    # the steps grids of the headline share get their own entry
    head = collections.defaultdict(list)
    for r in steps_of(sq_rows, HEADLINE, lambda r: r):
        head[("attn_steps_bf16 (headline share)", 0, r["Counter_Name"])].append(
            float(r["Counter_Value"]))
    sq.update(head)
    lines = [f"# SQ counters per dispatch (sums over the device), bf16 workloads",
             f"# command: {cmd['p3']}", f"# summary: python3 bench.py --digest {prof_dir}",
             f"# kernel source sha256 ({' + '.join(KERNEL_SOURCES)}): {src}"]
    names = sorted({c for (_, _, c) in sq})
    for k, g in sorted({(k, g) for (k, g, _) in sq}):
        lines.append(f"{k} grid={g}" if g else k)
        for c in names:
            v = sq.get((k, g, c))
            if v:
                lines.append(f"   {c:28s} {mean(v):16.0f}")
        mf, busy, gui = (sq.get((k, g, c)) for c in
                         ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
        if mf and busy and gui and mean(mf) > 0:
            # GRBM_GUI_ACTIVE sums the 8 XCDs; MFMA busy sums the 1024 SIMDs
            lines.append(f"   mfma_busy_fraction (busy per SIMD / active cycles per XCD): "
                         f"{mean(busy) / 1024 / (mean(gui) / 8):.3f}")
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS"):
                if sq.get((k, g, c)):
                    lines.append(f"   {c.lower()[9:]}_per_mfma: {mean(sq[(k, g, c)]) / mean(mf):.2f}")
    out_files[f"attn_steps_bf16__{w.name}__sq_counters.txt"] = lines

    out_dir = out_dir or os.path.join(ROOT, "profiles")
    for fname, text in out_files.items():
        with open(os.path.join(out_dir, fname), "w") as f:
            f.write("\n".join(text) + "\n")
        print(f"wrote {os.path.join(out_dir, fname)}")


def main():
    args = parse()
    if args.digest:
        digest(args.digest)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(collectives are out of scope); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from long_context_causal_amd import cpattn as C
    from long_context_causal_amd.inputs import HEADLINE, WORKLOADS, make_inputs
    from long_context_causal_amd.runner import CPProblem

    w = WORKLOADS[args.workload or HEADLINE]
    rank = w.rank
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    buf = P.alloc_rank(rank, C.CPATTN_F32)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def one_step(evs=None):
        def mark(tag):
            if evs is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                evs.append((tag, e))
        mark("start")
        P.partition(stream)
        mark("partition")
        P.steps(buf, stream)
        mark("steps")
        P.merge(buf, stream)
        mark("merge")

    with torch.cuda.stream(stream):
        prewarm(torch, one_step)
        for _ in range(args.warmup):
            one_step()
        torch.cuda.synchronize()
        all_evs = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            evs = []
            one_step(evs)
            all_evs.append(evs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    # the HBM kernels alone with the 256 MB last-level cache evicted first:
    # a 512 MB scratch write between repetitions, outside the timed region
    cold = {"partition": [], "merge": []}
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(max(args.steps // 2, 3)):
            for name, fn in (("partition", lambda: P.partition(stream)),
                             ("merge", lambda: P.merge(buf, stream))):
                scratch.fill_(1)
                e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e0.record(stream)
                fn()
                e1.record(stream)
                cold[name].append((e0, e1))
        torch.cuda.synchronize()
    del scratch
    cold_ms = {k: float(np.median([a.elapsed_time(b) for a, b in v])) for k, v in cold.items()}

    # the same steps launched one by one (cpattn_step_fwd), each timed
    per_step = None
    with torch.cuda.stream(stream):
        prewarm(torch, lambda: [P.step(buf, i, stream) for i in range(w.cp)])
        for _ in range(args.warmup):
            for i in range(w.cp):
                P.step(buf, i, stream)
        torch.cuda.synchronize()
        ps_ev = []
        for _ in range(args.steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(w.cp + 1)]
            e[0].record(stream)
            for i in range(w.cp):
                P.step(buf, i, stream)
                e[i + 1].record(stream)
            ps_ev.append(e)
        torch.cuda.synchronize()
    per_step = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ps_ev]))
                for i in range(w.cp)]

    # the fused form of the same share: split, then one launch
    fused = None
    if w.dtype == "bf16":
        fout = P.alloc_out(rank, C.CPATTN_F32)
        with torch.cuda.stream(stream):
            prewarm(torch, lambda: (P.partition(stream), P.forward_fused(fout, stream)))
            for _ in range(args.warmup):
                P.partition(stream)
                P.forward_fused(fout, stream)
            torch.cuda.synchronize()
            f_total, f_attn = [], []
            for _ in range(args.steps):
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(stream)
                P.partition(stream)
                e1.record(stream)
                P.forward_fused(fout, stream)
                e2.record(stream)
                f_total.append((e0, e2))
                f_attn.append((e1, e2))
            torch.cuda.synchronize()
        fused = {"ms": float(np.mean([a.elapsed_time(b) for a, b in f_total])),
                 "attn_ms": float(np.mean([a.elapsed_time(b) for a, b in f_attn]))}

    # the same dims packed into samples of mixed lengths (each an independent
    # causal sequence split on its own): split, then one varlen launch
    varlen = None
    if w.dtype == "bf16":
        cu = packing_offsets(w.s, w.cp)
        Pv = CPProblem(w, P.q, P.k, P.v, cu_seqlens=cu)
        vout = Pv.alloc_out(rank, C.CPATTN_F32)
        with torch.cuda.stream(stream):
            prewarm(torch, lambda: (Pv.partition(stream), Pv.forward_fused(vout, stream)))
            for _ in range(args.warmup):
                Pv.partition(stream)
                Pv.forward_fused(vout, stream)
            torch.cuda.synchronize()
            v_total, v_attn = [], []
            for _ in range(args.steps):
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(stream)
                Pv.partition(stream)
                e1.record(stream)
                Pv.forward_fused(vout, stream)
                e2.record(stream)
                v_total.append((e0, e2))
                v_attn.append((e1, e2))
            torch.cuda.synchronize()
        # each sample's rank share: 4*d per visible pair, c(2c+1) + (cp-1)*2c^2
        # pairs per (batch, head) with c the sample's chunk length
        v_flops = sum(dataclasses.replace(w, s=int(cu[i + 1] - cu[i])).rank_flops()
                      for i in range(len(cu) - 1))
        # the packed share's backward (seeded bf16 dO, its own O and L)
        gen_v = torch.Generator(device="cuda")
        gen_v.manual_seed(98)
        do_v = torch.randn(vout["o"].shape, generator=gen_v, device="cuda").to(torch.bfloat16)
        gv = Pv.alloc_grads(rank)
        with torch.cuda.stream(stream):
            prewarm(torch, lambda: Pv.backward(gv, vout["o"], vout["lse"], do_v, stream))
            for _ in range(args.warmup):
                Pv.backward(gv, vout["o"], vout["lse"], do_v, stream)
            torch.cuda.synchronize()
            vb_ev = []
            for _ in range(args.steps):
                e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e0.record(stream)
                Pv.backward(gv, vout["o"], vout["lse"], do_v, stream)
                e1.record(stream)
                vb_ev.append((e0, e1))
            torch.cuda.synchronize()
        varlen = {"cu": cu, "flops": v_flops,
                  "ms": float(np.mean([a.elapsed_time(b) for a, b in v_total])),
                  "attn_ms": float(np.mean([a.elapsed_time(b) for a, b in v_attn])),
                  "bwd_ms": float(np.mean([a.elapsed_time(b) for a, b in vb_ev]))}
        del Pv, vout, gv, do_v

    # the backward of the same share: dO seeded bf16, the rank's merged O
    # and L from the forward above
    backward = None
    if w.dtype == "bf16":
        gen = torch.Generator(device="cuda")
        gen.manual_seed(99)
        do_r = torch.randn(buf["o"].shape, generator=gen, device="cuda").to(torch.bfloat16)
        grads = P.alloc_grads(rank)
        with torch.cuda.stream(stream):
            prewarm(torch, lambda: P.backward(grads, buf["o"], buf["lse"], do_r, stream))
            for _ in range(args.warmup):
                P.backward(grads, buf["o"], buf["lse"], do_r, stream)
            torch.cuda.synchronize()
            b_ev = []
            for _ in range(args.steps):
                e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                e0.record(stream)
                P.backward(grads, buf["o"], buf["lse"], do_r, stream)
                e1.record(stream)
                b_ev.append((e0, e1))
            torch.cuda.synchronize()
        backward = float(np.mean([a.elapsed_time(b) for a, b in b_ev]))

    # per-kernel times (ms) from the events, averaged over the timed steps
    part_ms, merge_ms, grid_ms, total_ms = [], [], [], []
    for evs in all_evs:
        d = dict(evs)
        part_ms.append(d["start"].elapsed_time(d["partition"]))
        grid_ms.append(d["partition"].elapsed_time(d["steps"]))
        merge_ms.append(d["steps"].elapsed_time(d["merge"]))
        total_ms.append(d["start"].elapsed_time(d["merge"]))
    mean = lambda xs: float(np.mean(xs))
    ms_step = mean(total_ms)
    attn_ms = mean(grid_ms)
    flops = w.rank_flops()
    value = flops / (ms_step * 1e-3) / 1e12

    es = 2 if w.dtype == "bf16" else 4
    part_bytes = 2 * w.b * w.s * (w.hq + 2 * w.hkv) * w.d * es + 4 * w.s
    merge_rows = sum(st["rows"] for st in buf["steps"])
    merge_bytes = w.b * w.hq * (4 * w.d + 4) * (merge_rows + 2 * w.c)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS

    line = {
        "metric": "causal attention fwd TFLOP/s + % bf16 MFMA peak, per-GPU CP share, s=32k",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded normal Q/K/V, resident in HBM)",
        "config": {"workload": w.name, "b": w.b, "s": w.s, "hq": w.hq, "hkv": w.hkv,
                   "d": w.d, "cp": w.cp, "rank": rank,
                   "rope_theta": w.rope_theta},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": committed_traffic(w.name) if w.dtype == "bf16" else None,
                     "kernel": "attn_steps_bf16" if w.dtype == "bf16" else "attn_step_f32",
                     "flops_per_launch": flops if w.dtype == "bf16" else flops / w.cp,
                     "avg_launch_ms": round(attn_ms if w.dtype == "bf16" else attn_ms / w.cp,
                                            4)},
        "pct_of_peak": round(100 * value / peak, 2),
        "kernels_ms": {"partition_qkv": round(mean(part_ms), 4),
                       "steps": round(attn_ms, 4),
                       "merge": round(mean(merge_ms), 4)},
        "per_step_launches": {"entry_point": "cpattn_step_fwd",
                              "kernel": "attn_step_bf16" if w.dtype == "bf16"
                              else "attn_step_f32",
                              "ms": [round(x, 4) for x in per_step],
                              "attention_tflops": round(flops / (sum(per_step) * 1e-3) / 1e12,
                                                        2)},
        "attention_tflops": round(attn_tflops, 2),
        "steps_plus_merge_tflops": round(flops / ((attn_ms + mean(merge_ms)) * 1e-3) / 1e12, 2),
        "partition_gbps": round(part_bytes / (mean(part_ms) * 1e-3) / 1e9, 1),
        "merge_gbps": round(merge_bytes / (mean(merge_ms) * 1e-3) / 1e9, 1),
        "cold_cache_gbps": {"partition": round(part_bytes / (cold_ms["partition"] * 1e-3) / 1e9, 1),
                            "merge": round(merge_bytes / (cold_ms["merge"] * 1e-3) / 1e9, 1),
                            "note": "each launch after a 512 MB scratch write (last-level "
                                    "cache evicted), median"},
        "rank_flops": flops,
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
    }
    if fused is not None:
        f_tf = flops / (fused["attn_ms"] * 1e-3) / 1e12
        line["fused"] = {
            "entry_point": "cpattn_forward_fused",
            "ms_per_step": round(fused["ms"], 4),
            "value": round(flops / (fused["ms"] * 1e-3) / 1e12, 2),
            "kernel": "attn_fused_bf16",
            "avg_launch_ms": round(fused["attn_ms"], 4),
            "achieved": round(f_tf, 2),
            "frac": round(f_tf / peak, 4),
            "traffic": committed_traffic(w.name, "fused_traffic_bytes_per_launch"),
        }
    if varlen is not None:
        cu = varlen["cu"]
        v_tf = varlen["flops"] / (varlen["attn_ms"] * 1e-3) / 1e12
        line["varlen"] = {
            "entry_point": "cpattn_forward_fused_varlen",
            "sample_lengths": [int(cu[i + 1] - cu[i]) for i in range(len(cu) - 1)],
            "flops": varlen["flops"],
            "ms_per_step": round(varlen["ms"], 4),
            "value": round(varlen["flops"] / (varlen["ms"] * 1e-3) / 1e12, 2),
            "avg_launch_ms": round(varlen["attn_ms"], 4),
            "achieved": round(v_tf, 2),
            "frac": round(v_tf / peak, 4),
            "backward_ms": round(varlen["bwd_ms"], 4),
            "backward_value": round(2.5 * varlen["flops"] / (varlen["bwd_ms"] * 1e-3) / 1e12, 2),
        }
    if backward is not None:
        b_flops = 2.5 * flops
        b_tf = b_flops / (backward * 1e-3) / 1e12
        line["backward"] = {
            "entry_point": "cpattn_backward",
            "ms_per_step": round(backward, 4),
            "flops": b_flops,
            "flops_convention": "10*d per visible (q, k) pair: S, dP, dV, dK, dQ",
            "value": round(b_tf, 2),
            "frac": round(b_tf / peak, 4),
        }
    # every rank of the headline share (the step kernels' TFLOP/s), and the
    # other bf16 configurations at their measured rank
    if w.dtype == "bf16" and not args.no_extra:
        per_rank = [share_step_tflops(C, torch, P, w, r, stream)[0] for r in range(w.cp)]
        line["ranks"] = {"attention_tflops_min": round(min(per_rank), 2),
                         "attention_tflops_max": round(max(per_rank), 2),
                         "attention_tflops": [round(x, 1) for x in per_rank]}
        configs = {}
        for name in ("bf16_gqa_s8k_cp4", "bf16_mha_s16k_cp4_widelogits",
                     "bf16_gqa_s128k_cp16_rope"):
            wc = WORKLOADS[name]
            Pc = CPProblem(wc, *make_inputs(wc))
            with torch.cuda.stream(stream):
                Pc.partition(stream)
            a_tf, w_tf = share_step_tflops(C, torch, Pc, wc, wc.rank, stream)
            configs[name] = {"rank": wc.rank, "attention_tflops": round(a_tf, 2),
                             "frac": round(a_tf / peak, 4),
                             "steps_plus_merge_tflops": round(w_tf, 2),
                             "fused_tflops": round(share_fused_tflops(C, torch, Pc, wc, wc.rank,
                                                                      stream), 2),
                             "partition": split_gbps(torch, Pc, wc, stream)}
            del Pc
            torch.cuda.empty_cache()
        line["configs"] = configs
    if w.dtype == "bf16":
        pc = peak_check(C, torch, stream)
        pc["achieved_over_probe"] = round(attn_tflops / pc["mfma_probe_tflops"], 4)
        line["peak_check"] = pc
    if args.cpu_sample_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, rank, args.cpu_sample_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
