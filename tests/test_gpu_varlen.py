"""GPU packed variable-length samples (cpattn_partition_varlen,
cpattn_forward_fused_varlen) vs the packed oracle (``oracle/varlen.py``:
independent causal samples, each split by the zigzag rule on its own, RoPE
at in-sample positions).

* split: bit-exact bytes and in-sample positions for mixed sample lengths
  (chunks of one row up to several tiles), fp32 and bf16; RoPE rows within
  one bf16 rounding of the oracle's fp64 rotation at the in-sample positions;
* fused forward at reduced lengths: every rank, row and head vs the packed
  definition (GQA, MHA with wide logits, RoPE, b = 2), sample mixes whose
  chunks straddle, fill and undershoot the 256-row query tiles;
* one sample is bit-identical to the unpacked cpattn_forward_fused;
* the headline dims packed into samples of 1k..22k rows: sampled rows of
  the measured rank vs the oracle's rows of their sample.
"""
import dataclasses

import numpy as np
import pytest

from gpu_helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, C, CPProblem, as_f32, assert_close,
                         host_f32, make_inputs, say, small, torch)
from long_context_causal_amd.inputs import WORKLOADS
from long_context_causal_amd.runner import bf16_bits
from oracle import attention_rows
from oracle import cp as ocp
from oracle import varlen as ovl

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.cpu().numpy().view(np.uint32)


def _host_bits(x):
    return x if x.dtype == np.uint16 else x.view(np.uint32)


def _cu(cp, chunks):
    """Offsets of samples whose chunk lengths are ``chunks``."""
    return np.concatenate([[0], np.cumsum([2 * cp * c for c in chunks])]).astype(np.int64)


SPLITS = [("fp32_mha_s512_cp2", [3, 60, 1, 64]),
          ("bf16_gqa_s8k_cp4", [100, 1, 37, 256]),
          ("bf16_gqa_s32k_cp8", [3, 17, 1, 40])]


@pytest.mark.parametrize("name,chunks", SPLITS)
def test_partition_varlen_bit_exact(name, chunks):
    base = WORKLOADS[name]
    cu = _cu(base.cp, chunks)
    w = dataclasses.replace(small(base, int(cu[-1])), rope_theta=None)
    say(f"partition varlen {name} cu={cu.tolist()}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    torch.cuda.synchronize()
    for r in range(w.cp):
        assert np.array_equal(P.pos[r].cpu().numpy(), ovl.local_positions(cu, w.cp, r))
    for host, dev in ((k, P.kz), (v, P.vz), (q, P.qz)):
        assert np.array_equal(_bits(dev), ovl.partition(_host_bits(host), cu, w.cp))


def test_partition_varlen_rope_in_sample_positions():
    base = WORKLOADS["bf16_gqa_s128k_cp16_rope"]
    cp = 4
    cu = _cu(cp, [5, 64, 1, 130])
    w = dataclasses.replace(base, s=int(cu[-1]), cp=cp)
    say(f"partition varlen + rope cu={cu.tolist()}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    torch.cuda.synchronize()
    qz, kz = host_f32(P.qz), host_f32(P.kz)
    for r in range(cp):
        rows, pos = ovl.local_rows(cu, cp, r), ovl.local_positions(cu, cp, r)
        for nm, host, dev in (("q", q, qz), ("k", k, kz)):
            want = ocp.rope(as_f32(host[:, rows]).astype(np.float64), pos, w.rope_theta)
            err = np.abs(dev[r] - want)
            bound = np.abs(want) * 2.0 ** -8 + 1e-6
            say(f"  rank {r} {nm}: max err/bound {float((err / bound).max()):.3f}")
            assert np.all(err <= bound)
    assert np.array_equal(_bits(P.vz), ovl.partition(_host_bits(v), cu, cp))


def _packed_ref(w, q, k, v, cu):
    qf, kf, vf = (as_f32(x).astype(np.float64) for x in (q, k, v))
    return ovl.packed_causal_attention(qf, kf, vf, cu, rope_theta=w.rope_theta)


def run_fused(P, rank):
    out = P.alloc_out(rank, C.CPATTN_F32)
    P.forward_fused(out)
    torch.cuda.synchronize()
    return host_f32(out["o"]), out["lse"].cpu().numpy()


FUSED = [("bf16_gqa_s8k_cp4", [100, 1, 37, 256, 64], None),
         ("bf16_gqa_s32k_cp8", [40, 130, 3], 2),
         ("bf16_mha_s16k_cp4_widelogits", [96, 200, 5], None),
         ("bf16_gqa_s128k_cp16_rope", [24, 7, 65], None)]


# 64-wide heads (GQA, and RoPE at in-sample positions)
FUSED_D64 = [("bf16_gqa_s8k_cp4", [100, 1, 37, 256, 64], None, 64),
             ("bf16_gqa_s128k_cp16_rope", [24, 7, 65], None, 64)]


@pytest.mark.parametrize("name,chunks,b,d", [f + (128,) for f in FUSED] + FUSED_D64)
def test_fused_varlen_reduced_all_ranks(name, chunks, b, d):
    base = dataclasses.replace(WORKLOADS[name], d=d)
    cu = _cu(base.cp, chunks)
    w = small(base, int(cu[-1]), b)
    say(f"fused varlen {name} cu={cu.tolist()} b={w.b} d={w.d}")
    q, k, v = make_inputs(w)
    o_ref, l_ref = _packed_ref(w, q, k, v, cu)
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    for r in range(w.cp):
        o, l = run_fused(P, r)
        rows = ovl.local_rows(cu, w.cp, r)
        assert_close(f"rank {r} O", o, o_ref[:, rows], BF16_MAX_ABS, BF16_MEAN_ABS)
        assert_close(f"rank {r} L", l, l_ref[:, :, rows], 1e-3)


def test_fused_varlen_one_sample_is_unpacked():
    w = small(WORKLOADS["bf16_gqa_s32k_cp8"], 2 * 8 * 300)
    say("fused varlen, one sample")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    P.partition()
    Pv = CPProblem(w, q, k, v, cu_seqlens=[0, w.s])
    Pv.partition()
    torch.cuda.synchronize()
    assert torch.equal(P.qz, Pv.qz) and torch.equal(P.kz, Pv.kz)
    for r in (0, w.rank, w.cp - 1):
        o, l = run_fused(P, r)
        ov, lv = run_fused(Pv, r)
        assert np.array_equal(o, ov) and np.array_equal(l, lv)


def test_fused_varlen_full_size_sampled_rows():
    w = WORKLOADS["bf16_gqa_s32k_cp8"]
    cp, r = w.cp, w.rank
    cu = np.array([0, 1024, 9216, 10240, 32768], dtype=np.int64)
    say(f"fused varlen full size {w.name} cu={cu.tolist()} rank {r}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    o, l = run_fused(P, r)
    rows = ovl.local_rows(cu, cp, r)
    rng = np.random.default_rng(3)
    for i in range(len(cu) - 1):
        a, e = cu[i] // cp, cu[i + 1] // cp
        pick = np.unique(np.concatenate([[a, a + (e - a) // 2 - 1, a + (e - a) // 2, e - 1],
                                         rng.integers(a, e, 6)]))
        g = rows[pick]                          # packed rows of the picked local rows
        s0 = int(cu[i])
        qf = as_f32(q[:, g]).astype(np.float64)
        hi = int(g.max()) + 1
        kf = as_f32(k[:, s0:hi]).astype(np.float64)
        vf = as_f32(v[:, s0:hi]).astype(np.float64)
        o_ref, l_ref = attention_rows(qf, kf, vf, g - s0 + 1)
        assert_close(f"sample {i} O", o[:, pick], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
        assert_close(f"sample {i} L", l[:, :, pick], l_ref, 1e-3)


# --- backward of packed samples ---------------------------------------------

from long_context_causal_amd.inputs import f32_to_bf16_bits  # noqa: E402
from long_context_causal_amd.runner import to_device  # noqa: E402

from gpu_helpers import assert_grad as _assert_grad  # noqa: E402  (the unpacked backward's bound)


BWD = [("bf16_gqa_s8k_cp4", [100, 1, 37, 64]),
       ("bf16_gqa_s32k_cp8", [40, 130, 3]),
       ("bf16_mha_s16k_cp4_widelogits", [96, 5, 64]),
       ("bf16_gqa_s128k_cp16_rope", [24, 7, 9])]


@pytest.mark.parametrize("name,chunks,d", [b + (128,) for b in BWD] +
                         [("bf16_gqa_s8k_cp4", [100, 1, 37, 64], 64),
                          ("bf16_gqa_s128k_cp16_rope", [24, 7, 9], 64)])
def test_backward_varlen_all_ranks(name, chunks, d):
    base = dataclasses.replace(WORKLOADS[name], d=d)
    cu = _cu(base.cp, chunks)
    w = small(base, int(cu[-1]))
    say(f"backward varlen {name} cu={cu.tolist()} d={d}")
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(99)
    do = f32_to_bf16_bits(rng.standard_normal((w.b, w.s, w.hq, w.d)).astype(np.float32))
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    doz = ovl.partition(as_f32(do), cu, w.cp)
    tloc = w.s // w.cp
    dq_z = np.zeros((w.cp, w.b, tloc, w.hq, w.d))
    dk_z = np.zeros((w.cp, w.b, tloc, w.hkv, w.d))
    dv_z = np.zeros_like(dk_z)
    for r in range(w.cp):
        out = P.alloc_out(r, C.CPATTN_F32)
        P.forward_fused(out)
        g = P.alloc_grads(r)
        P.backward(g, out["o"], out["lse"],
                   to_device(f32_to_bf16_bits(doz[r].astype(np.float32))))
        torch.cuda.synchronize()
        dq_z[r] = g["dq"].cpu().numpy()
        dk_z += g["dkz"].cpu().numpy()        # the reduce-scatter, summed on the owner
        dv_z += g["dvz"].cpu().numpy()
    qf, kf = as_f32(q).astype(np.float64), as_f32(k).astype(np.float64)
    if w.rope_theta is not None:           # gradients are taken at the rotated Q, K
        pos = ovl.sample_positions(cu)
        qf, kf = ocp.rope(qf, pos, w.rope_theta), ocp.rope(kf, pos, w.rope_theta)
    dq, dk, dv = ovl.packed_causal_attention_bwd(qf, kf, as_f32(v).astype(np.float64),
                                                 as_f32(do).astype(np.float64), cu)
    _assert_grad("dQ", ovl.unpartition(dq_z, cu), dq)
    _assert_grad("dK", ovl.unpartition(dk_z, cu), dk)
    _assert_grad("dV", ovl.unpartition(dv_z, cu), dv)


def test_backward_varlen_one_sample_is_unpacked():
    w = small(WORKLOADS["bf16_gqa_s32k_cp8"], 2 * 8 * 136)
    say("backward varlen, one sample")
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(5)
    P = CPProblem(w, q, k, v)
    P.partition()
    Pv = CPProblem(w, q, k, v, cu_seqlens=[0, w.s])
    Pv.partition()
    r = w.rank
    out = P.alloc_out(r, C.CPATTN_F32)
    P.forward_fused(out)
    do_r = to_device(f32_to_bf16_bits(
        rng.standard_normal(tuple(out["o"].shape)).astype(np.float32)))
    g, gv = P.alloc_grads(r), Pv.alloc_grads(r)
    P.backward(g, out["o"], out["lse"], do_r)
    Pv.backward(gv, out["o"], out["lse"], do_r)
    torch.cuda.synchronize()
    # dq is written by one workgroup per row, and every dK/dV element by one
    # workgroup of the share's grid: the one-sample table is the unpacked
    # call, bit for bit
    for key in ("dq", "dkz", "dvz"):
        assert torch.equal(g[key], gv[key]), key


@pytest.mark.parametrize("rope", [False, True])
def test_varlen_most_samples_all_ranks(rope):
    """The largest packing the ABI takes (CPATTN_MAX_SEQS samples, chunks of
    1 to 3 rows): every rank's fused forward and backward vs the oracle.
    With this many samples the backward's run table falls back to one run
    per step.  With RoPE the split stores the rotated Q and K in bf16, and
    a row of these short samples sees so few keys that the rounding of its
    scores shows in L (up to ~1.2e-3), so the reference takes the oracle's
    rotation rounded to bf16 as its Q and K: the inputs the attention
    actually gets."""
    base = WORKLOADS["bf16_gqa_s128k_cp16_rope" if rope else "bf16_gqa_s8k_cp4"]
    cp = 2
    cu = _cu(cp, [1 + i % 3 for i in range(C.CPATTN_MAX_SEQS)])
    w = small(dataclasses.replace(base, cp=cp, hq=4, hkv=2), int(cu[-1]))
    say(f"varlen {len(cu) - 1} samples, s={w.s}, cp={cp}")
    q, k, v = make_inputs(w)
    qf, kf, vf = (as_f32(x).astype(np.float64) for x in (q, k, v))
    if rope:
        pos = ovl.sample_positions(cu)
        qf, kf = (as_f32(f32_to_bf16_bits(ocp.rope(x, pos, w.rope_theta).astype(np.float32)))
                  .astype(np.float64) for x in (qf, kf))
    o_ref, l_ref = ovl.packed_causal_attention(qf, kf, vf, cu)
    rng = np.random.default_rng(11)
    do = f32_to_bf16_bits(rng.standard_normal((w.b, w.s, w.hq, w.d)).astype(np.float32))
    P = CPProblem(w, q, k, v, cu_seqlens=cu)
    P.partition()
    doz = ovl.partition(as_f32(do), cu, cp)
    tloc = w.s // cp
    dq_z = np.zeros((cp, w.b, tloc, w.hq, w.d))
    dk_z = np.zeros((cp, w.b, tloc, w.hkv, w.d))
    dv_z = np.zeros_like(dk_z)
    for r in range(cp):
        out = P.alloc_out(r, C.CPATTN_F32)
        P.forward_fused(out)
        g = P.alloc_grads(r)
        P.backward(g, out["o"], out["lse"],
                   to_device(f32_to_bf16_bits(doz[r].astype(np.float32))))
        torch.cuda.synchronize()
        rows = ovl.local_rows(cu, cp, r)
        assert_close(f"rank {r} O", out["o"].cpu().numpy(), o_ref[:, rows], BF16_MAX_ABS,
                     BF16_MEAN_ABS)
        assert_close(f"rank {r} L", out["lse"].cpu().numpy(), l_ref[:, :, rows], 1e-3)
        dq_z[r] = g["dq"].cpu().numpy()
        dk_z += g["dkz"].cpu().numpy()
        dv_z += g["dvz"].cpu().numpy()
    dq, dk, dv = ovl.packed_causal_attention_bwd(qf, kf, vf, as_f32(do).astype(np.float64), cu)
    _assert_grad("dQ", ovl.unpartition(dq_z, cu), dq)
    _assert_grad("dK", ovl.unpartition(dk_z, cu), dk)
    _assert_grad("dV", ovl.unpartition(dv_z, cu), dv)
