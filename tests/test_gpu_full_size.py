"""GPU parity at the full sizes of the bf16 workloads, over every row.

Each rank's merged O and L ("Megatron-LM 篇" §3.2, closing paragraph: a
rank's O equals its slice of the non-CP O) through both forward forms:
cpattn_forward (the cp steps' grid, then the merge) and
cpattn_forward_fused (one launch), against the oracle's matrix form of
causal attention (oracle/matrix.py) on the same bf16 bits widened to fp64:

* 8k GQA cp=4 and 16k MHA b=2 cp=4 (wide logits): every rank, every row,
  every head;
* 32k GQA cp=8: every rank, every row;
* 128k GQA cp=16 with RoPE at global positions: the measured rank 7, all
  its 8192 rows, in four blocks of 2048 local rows (one test each, so no
  test runs for long without output);
* 64-wide heads (the same inputs drawn at d = 64): every rank of the 8k GQA
  dims and the measured rank of the 32k dims, every row.

Bounds: O max abs 2e-2, mean abs 2e-3; L max abs 1e-3.
"""
import dataclasses

import numpy as np
import pytest

from gpu_helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, C, CPProblem, assert_close, host_f32,
                         make_inputs, ocp, say, torch)
from long_context_causal_amd.inputs import WORKLOADS, as_f32
from oracle.matrix import attention_at_positions

pytestmark = pytest.mark.gpu

ROPE_BLOCK = 2048
CASES = ([("bf16_gqa_s8k_cp4", r, None, 128) for r in range(4)] +
         [("bf16_mha_s16k_cp4_widelogits", r, None, 128) for r in range(4)] +
         [("bf16_gqa_s32k_cp8", r, None, 128) for r in range(8)] +
         [("bf16_gqa_s128k_cp16_rope", 7, blk, 128) for blk in range(4)] +
         [("bf16_gqa_s8k_cp4", r, None, 64) for r in range(4)] +
         [("bf16_gqa_s32k_cp8", 3, None, 64)])

_state = {}


def _workload(name, d=128):
    """Inputs, their fp32 values and the partitioned device problem of one
    workload (at head dimension d), kept while consecutive tests use it."""
    if _state.get("key") != (name, d):
        _state.clear()
        torch.cuda.empty_cache()
        w = dataclasses.replace(WORKLOADS[name], d=d)
        say(f"{name} d={d}: inputs and split")
        q, k, v = make_inputs(w)
        P = CPProblem(w, q, k, v)
        P.partition()
        torch.cuda.synchronize()
        _state.update(key=(name, d), w=w, P=P, qf=as_f32(q), kf=as_f32(k), vf=as_f32(v), out={})
    return _state


def _gpu_outputs(st, rank):
    """(O, L) of the steps' grid + merge and of the fused launch, fp32."""
    if rank not in st["out"]:
        P = st["P"]
        say(f"  rank {rank}: gpu forward (steps grid + merge, fused)")
        buf = P.alloc_rank(rank, C.CPATTN_F32)
        P.forward(buf)
        fo = P.alloc_out(rank, C.CPATTN_F32)
        P.forward_fused(fo)
        torch.cuda.synchronize()
        st["out"] = {rank: (host_f32(buf["o"]), buf["lse"].cpu().numpy(),
                            host_f32(fo["o"]), fo["lse"].cpu().numpy())}
        del buf, fo
    return st["out"][rank]


def _oracle(st, pos):
    """Oracle O [b, n, hq, d] and L [b, hq, n] of the global rows pos."""
    w = st["w"]
    hi = int(pos.max()) + 1
    qr = st["qf"][:, pos].astype(np.float64)
    kr = st["kf"][:, :hi]
    if w.rope_theta is not None:
        if st.get("k_rope_hi", 0) < hi:
            st["k_rope"] = ocp.rope(st["kf"][:, :hi], np.arange(hi), w.rope_theta)
            st["k_rope_hi"] = hi
        qr = ocp.rope(qr, pos, w.rope_theta)
        kr = st["k_rope"][:, :hi]
    return attention_at_positions(qr, kr, st["vf"][:, :hi], pos)


@pytest.mark.parametrize("name,rank,block,d", CASES)
def test_forward_full_size_every_row(name, rank, block, d):
    st = _workload(name, d)
    w = st["w"]
    o_s, l_s, o_f, l_f = _gpu_outputs(st, rank)
    rows = np.arange(2 * w.c)
    if block is not None:
        rows = rows[block * ROPE_BLOCK:(block + 1) * ROPE_BLOCK]
    pos = ocp.zigzag_positions(w.s, w.cp, rank)[rows]
    say(f"  rank {rank}: oracle on {len(rows)} local rows (global {pos[0]}..{pos[-1]})")
    o_ref, l_ref = _oracle(st, pos)
    assert_close(f"rank {rank} steps O", o_s[:, rows], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    assert_close(f"rank {rank} steps L", l_s[:, :, rows], l_ref, 1e-3)
    assert_close(f"rank {rank} fused O", o_f[:, rows], o_ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    assert_close(f"rank {rank} fused L", l_f[:, :, rows], l_ref, 1e-3)


@pytest.mark.parametrize("name", ["bf16_gqa_s128k_cp16_rope"])
def test_bf16_output_within_one_rounding(name):
    """The bf16 output option of both forms is the fp32 output rounded to
    nearest even (within one bf16 rounding)."""
    st = _workload(name)
    w = st["w"]
    r = w.rank
    o_s, _, o_f, _ = _gpu_outputs(st, r)
    P = st["P"]
    buf = P.alloc_rank(r, C.CPATTN_BF16)
    P.forward(buf)
    fo = P.alloc_out(r, C.CPATTN_BF16)
    P.forward_fused(fo)
    torch.cuda.synchronize()
    for got, ref in ((host_f32(buf["o"]), o_s), (host_f32(fo["o"]), o_f)):
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
