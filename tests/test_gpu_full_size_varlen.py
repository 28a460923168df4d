"""GPU parity of packed samples at full size, over every row or element.

Packed samples are independent causal sequences, each split by the zigzag
rule on its own ("Megatron 面试题（一）" M016: positions reset at sample
boundaries; "Megatron-LM 篇" §3.5: splits finer than a kernel tile).  The
packing is eight samples in the length ratio 1:2:4:1:8:3:5:8 (units of
s/32 rows), the mix the benchmark's packed leg uses.  The reference of
each sample is the oracle's matrix form (oracle/matrix.py) on that
sample's rows alone:

* forward, the 32k GQA headline dims (s = 32768, 64/8 heads, cp = 8): every
  local row of the measured rank (rank 3) through cpattn_forward_fused_varlen;
  O max abs 2e-2, mean abs 2e-3, L max abs 1e-3;
* backward, the 8k GQA dims (s = 8192, 32/8 heads, cp = 4): every rank's
  fused forward and cpattn_backward_varlen share, dK/dV summed per owner,
  every element of dQ, dK and dV; max |err| <= 1e-2 max |ref| and mean
  |err| <= 5e-3 mean |ref| per gradient.
"""
import numpy as np
import pytest

from gpu_helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, C, CPProblem, as_f32, assert_close,
                         assert_grad, host_f32, make_inputs, say, seeded_dout, to_device, torch)
from long_context_causal_amd.inputs import WORKLOADS, f32_to_bf16_bits
from oracle import varlen as ovl
from oracle.matrix import attention_rows_bwd_matrix, attention_rows_matrix

pytestmark = pytest.mark.gpu

UNITS = [1, 2, 4, 1, 8, 3, 5, 8]


def _packing(s, cp):
    unit = s // 32
    assert unit * 32 == s and unit % (2 * cp) == 0
    return np.concatenate([[0], np.cumsum([u * unit for u in UNITS])]).astype(np.int64)


def _f64(x):
    return as_f32(x).astype(np.float64)


def test_fused_varlen_full_size_every_row():
    w = WORKLOADS["bf16_gqa_s32k_cp8"]
    cp, r = w.cp, w.rank
    cu = _packing(w.s, cp)
    say(f"fused varlen full size {w.name} cu={cu.tolist()} rank {r}: every row")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    out = P.alloc_out(r, C.CPATTN_F32)
    P.forward_fused(out)
    torch.cuda.synchronize()
    o, l = host_f32(out["o"]), out["lse"].cpu().numpy()
    del P, out
    torch.cuda.empty_cache()
    rows = ovl.local_rows(cu, cp, r)           # packed row of each local row
    for i in range(len(cu) - 1):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        loc = np.arange(s0 // cp, s1 // cp)    # the rank's local rows of sample i
        g = rows[loc] - s0                     # their in-sample positions
        hi = int(g.max()) + 1
        say(f"  sample {i}: {len(loc)} rows, oracle on up to {hi} keys")
        o_ref, l_ref = attention_rows_matrix(_f64(q[:, rows[loc]]), _f64(k[:, s0:s0 + hi]),
                                             _f64(v[:, s0:s0 + hi]), g + 1, max_elems=1 << 24)
        assert_close(f"sample {i} O", o[:, loc], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
        assert_close(f"sample {i} L", l[:, :, loc], l_ref, 1e-3)


def test_backward_varlen_full_size_every_element():
    w = WORKLOADS["bf16_gqa_s8k_cp4"]
    cu = _packing(w.s, w.cp)
    say(f"backward varlen full size {w.name} cu={cu.tolist()}: every rank, every element")
    q, k, v = make_inputs(w)
    do = seeded_dout(w)
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    doz = ovl.partition(as_f32(do), cu, w.cp)
    tloc = w.s // w.cp
    dq_z = np.zeros((w.cp, w.b, tloc, w.hq, w.d), np.float32)
    dk_z = np.zeros((w.cp, w.b, tloc, w.hkv, w.d))
    dv_z = np.zeros_like(dk_z)
    for r in range(w.cp):
        say(f"  rank {r}: gpu fused forward and backward")
        out = P.alloc_out(r, C.CPATTN_F32)
        P.forward_fused(out)
        g = P.alloc_grads(r)
        P.backward(g, out["o"], out["lse"],
                   to_device(f32_to_bf16_bits(doz[r].astype(np.float32))))
        torch.cuda.synchronize()
        dq_z[r] = g["dq"].cpu().numpy()
        dk_z += g["dkz"].cpu().numpy()         # the reduce-scatter, summed on the owner
        dv_z += g["dvz"].cpu().numpy()
        del out, g
    del P
    torch.cuda.empty_cache()
    dq_g = ovl.unpartition(dq_z, cu).astype(np.float64)
    dk_g, dv_g = ovl.unpartition(dk_z, cu), ovl.unpartition(dv_z, cu)
    dq = np.zeros_like(dq_g)
    dk, dv = np.zeros_like(dk_g), np.zeros_like(dv_g)
    say("  oracle: each sample's causal attention backward, matrix form")
    for i in range(len(cu) - 1):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        dq[:, s0:s1], dk[:, s0:s1], dv[:, s0:s1] = attention_rows_bwd_matrix(
            _f64(q[:, s0:s1]), _f64(k[:, s0:s1]), _f64(v[:, s0:s1]), _f64(do[:, s0:s1]),
            np.arange(1, s1 - s0 + 1), max_elems=1 << 24)
    assert_grad("dQ", dq_g, dq)
    assert_grad("dK", dk_g, dk)
    assert_grad("dV", dv_g, dv)
