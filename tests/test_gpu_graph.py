"""The device entry points under HIP graph capture.

Each entry point enqueues only kernel launches on the caller's stream (the
zero fills are kernels, not memsets), so a caller can capture it in a HIP
graph.  Each case runs the call eagerly, captures the same call, then
replays the graph three times, with eager work on the same buffers and a
synchronisation between replays, and checks every replay against the eager
result bit for bit (same kernels, same inputs, no atomics on these paths).
"""
import pytest
import torch

from gpu_helpers import C, CPProblem, make_inputs, say, small
from long_context_causal_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu


def _problem():
    w = small(WORKLOADS["bf16_gqa_s8k_cp4"], 2 * 4 * 200)
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    P.partition()
    torch.cuda.synchronize()
    return w, P


def _replays_match(fn, outs, name):
    """Eager call, capture, three replays with the outputs poisoned eagerly
    before each; every replay equals the eager result."""
    fn()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(3):
        for t in outs:                    # eager work between replays
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), f"{name}: replay {i}, output {j}"
        say(f"  {name}: replay {i} equals the eager call")


def test_forward_entry_points_replay():
    w, P = _problem()
    r = w.rank
    buf = P.alloc_rank(r, C.CPATTN_F32)
    _replays_match(lambda: P.forward(buf), [buf["o"], buf["lse"]], "cpattn_forward")
    out = P.alloc_out(r, C.CPATTN_BF16)
    _replays_match(lambda: P.forward_fused(out), [out["o"], out["lse"]], "cpattn_forward_fused")
    na = P.alloc_out(r, C.CPATTN_F32)
    _replays_match(lambda: C.cpattn_forward_noalloc(P.dims, P.dtype, 0.0, r, P.qz, P.kz, P.vz,
                                                    C.CPATTN_F32, na["o"], na["lse"]),
                   [na["o"], na["lse"]], "cpattn_forward_noalloc")
    assert torch.equal(na["o"], buf["o"]) and torch.equal(na["lse"], buf["lse"])


def test_backward_entry_point_replays():
    w, P = _problem()
    r = w.rank
    buf = P.alloc_rank(r, C.CPATTN_F32)
    P.forward(buf)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    do_r = torch.randn(buf["o"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    g = P.alloc_grads(r)
    _replays_match(lambda: P.backward(g, buf["o"], buf["lse"], do_r),
                   [g["dq"], g["dkz"], g["dvz"]], "cpattn_backward")


def test_split_and_packed_entry_points_replay():
    """The split (with RoPE at global positions), and the packed-sample
    split, fused forward and backward: the sample table is copied into the
    kernel arguments during the call, so the captured launches need no host
    memory at replay."""
    import numpy as np
    w = small(WORKLOADS["bf16_gqa_s128k_cp16_rope"], 2 * 16 * 24)
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    _replays_match(lambda: P.partition(), [P.qz, P.kz, P.vz], "cpattn_partition (RoPE)")
    cu = np.array([0, 2 * 16 * 5, 2 * 16 * 6, w.s], dtype=np.int64)
    Pv = CPProblem(w, q, k, v, cu_seqlens=cu)
    _replays_match(lambda: Pv.partition(), [Pv.qz, Pv.kz, Pv.vz], "cpattn_partition_varlen")
    r = w.rank
    out = Pv.alloc_out(r, C.CPATTN_F32)
    _replays_match(lambda: Pv.forward_fused(out), [out["o"], out["lse"]],
                   "cpattn_forward_fused_varlen")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    do_r = torch.randn(out["o"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    g = Pv.alloc_grads(r)
    _replays_match(lambda: Pv.backward(g, out["o"], out["lse"], do_r),
                   [g["dq"], g["dkz"], g["dvz"]], "cpattn_backward_varlen")
