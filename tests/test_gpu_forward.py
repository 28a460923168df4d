"""GPU end-to-end CP forward vs the non-CP oracle, per workload.

* every workload at a reduced length (same heads, head dim, cp, dtype and
  distribution; ragged tiles): every rank, every row, every head;
* the fp32 workload at its full size, every rank and row (1e-5);
* every bf16 workload at its full size, every row: test_gpu_full_size.py.
"""
import dataclasses

import numpy as np
import pytest

from gpu_helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, C, CPProblem, assert_close,
                         make_inputs, ocp, oracle_full, run_rank, say, small, torch)
from long_context_causal_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu

# more steps than one grid launch takes (32): the steps run in two grids
WIDE_CP = dataclasses.replace(WORKLOADS["bf16_gqa_s8k_cp4"], name="bf16_gqa_cp40", s=2 * 40 * 40,
                              hq=4, hkv=2, cp=40)
# one rank: the share is the causal step alone (c = 200, ragged)
ONE_CP = dataclasses.replace(WORKLOADS["bf16_gqa_s8k_cp4"], name="bf16_gqa_cp1", s=400, hq=4,
                             hkv=2, cp=1)
# chunks of one row (c = 1): every rank holds two rows, positions r and
# 2cp - 1 - r; most of its steps see a single key or a single query row
ONE_ROW = dataclasses.replace(WORKLOADS["bf16_gqa_s8k_cp4"], name="bf16_gqa_c1_cp24", s=2 * 24,
                              hq=4, hkv=2, cp=24)
# one query head and one KV head, two batch elements, ragged chunks
ONE_HEAD = dataclasses.replace(WORKLOADS["bf16_gqa_s8k_cp4"], name="bf16_h1_b2_cp4", s=2 * 4 * 50,
                               b=2, hq=1, hkv=1)
EXTRA = {"cp40": WIDE_CP, "cp1": ONE_CP, "c1": ONE_ROW, "h1": ONE_HEAD}

# 64-wide heads (the pages fix no head dimension): GQA, MHA with wide
# logits, RoPE at global positions; ragged chunks
HEAD64 = {
    "gqa": dataclasses.replace(WORKLOADS["bf16_gqa_s8k_cp4"], name="bf16_gqa_d64_cp4",
                               s=2 * 4 * 100, hq=8, hkv=2, d=64),
    "mha_wide": dataclasses.replace(WORKLOADS["bf16_mha_s16k_cp4_widelogits"],
                                    name="bf16_mha_d64_cp4_widelogits", s=2 * 4 * 96, hq=4,
                                    hkv=4, d=64),
    "rope_cp8": dataclasses.replace(WORKLOADS["bf16_gqa_s128k_cp16_rope"],
                                    name="bf16_gqa_d64_cp8_rope", s=2 * 8 * 72, hq=8, hkv=2,
                                    d=64, cp=8),
}


REDUCED = [("fp32_mha_s512_cp2", 2 * 2 * 77, None),
           ("bf16_gqa_s8k_cp4", 2 * 4 * 100, None),
           ("bf16_gqa_s32k_cp8", 2 * 8 * 40, None),
           ("bf16_mha_s16k_cp4_widelogits", 2 * 4 * 96, None),
           ("bf16_gqa_s128k_cp16_rope", 2 * 16 * 24, None),
           ("bf16_gqa_s8k_cp4", 2 * 4 * 256, 3)]


def _bounds(w):
    return (F32_MAX_ABS, None) if w.dtype == "f32" else (BF16_MAX_ABS, BF16_MEAN_ABS)


@pytest.mark.parametrize("name,s,b", REDUCED)
def test_forward_reduced_all_ranks(name, s, b):
    w = small(WORKLOADS[name], s, b)
    say(f"forward reduced {name} s={s} b={w.b}")
    q, k, v = make_inputs(w)
    o_full, l_full = oracle_full(w, q, k, v)
    P = CPProblem(w, q, k, v)
    P.partition()
    mx_abs, mn_abs = _bounds(w)
    for r in range(w.cp):
        o, l = run_rank(P, r)
        pos = ocp.zigzag_positions(w.s, w.cp, r)
        assert_close(f"rank {r} O", o, o_full[:, pos], mx_abs, mn_abs)
        assert_close(f"rank {r} L", l, l_full[:, :, pos], 1e-3 if w.dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("name", sorted(EXTRA))
def test_forward_extreme_cp_all_ranks(name):
    """cp = 40 (more steps than one grid launch takes, ragged chunks c = 40),
    cp = 1 (the causal step alone), chunks of one row (c = 1, cp = 24) and a
    single head (hq = hkv = 1, b = 2), through cpattn_forward and
    cpattn_forward_fused."""
    w = EXTRA[name]
    say(f"forward cp={w.cp} s={w.s}")
    q, k, v = make_inputs(w)
    o_full, l_full = oracle_full(w, q, k, v)
    P = CPProblem(w, q, k, v)
    P.partition()
    for r in range(w.cp):
        o, l = run_rank(P, r)
        pos = ocp.zigzag_positions(w.s, w.cp, r)
        assert_close(f"rank {r} O", o, o_full[:, pos], BF16_MAX_ABS, BF16_MEAN_ABS)
        assert_close(f"rank {r} L", l, l_full[:, :, pos], 1e-3)
        out = P.alloc_out(r, C.CPATTN_F32)
        P.forward_fused(out)
        torch.cuda.synchronize()
        assert_close(f"rank {r} fused O", out["o"].cpu().numpy(), o_full[:, pos], BF16_MAX_ABS,
                     BF16_MEAN_ABS)
        assert_close(f"rank {r} fused L", out["lse"].cpu().numpy(), l_full[:, :, pos], 1e-3)


@pytest.mark.parametrize("name", sorted(HEAD64))
def test_forward_head_dim_64_all_ranks(name):
    """bf16 with d = 64: every rank through cpattn_forward (steps grid and
    merge) and through cpattn_forward_fused, vs the oracle."""
    w = HEAD64[name]
    say(f"forward d=64 {w.name} s={w.s} cp={w.cp}")
    q, k, v = make_inputs(w)
    o_full, l_full = oracle_full(w, q, k, v)
    P = CPProblem(w, q, k, v)
    P.partition()
    for r in range(w.cp):
        pos = ocp.zigzag_positions(w.s, w.cp, r)
        o, l = run_rank(P, r)
        assert_close(f"rank {r} O", o, o_full[:, pos], BF16_MAX_ABS, BF16_MEAN_ABS)
        assert_close(f"rank {r} L", l, l_full[:, :, pos], 1e-3)
        out = P.alloc_out(r, C.CPATTN_F32)
        P.forward_fused(out)
        torch.cuda.synchronize()
        assert_close(f"rank {r} fused O", out["o"].cpu().numpy(), o_full[:, pos], BF16_MAX_ABS,
                     BF16_MEAN_ABS)
        assert_close(f"rank {r} fused L", out["lse"].cpu().numpy(), l_full[:, :, pos], 1e-3)


@pytest.mark.parametrize("cp", [128, 256])
def test_forward_cp_as_fine_as_the_query_tiles(cp):
    """cp as large as the FA2 loop counts ("Megatron-LM 篇" §3.5): at
    s = 32768, cp = 128 and 256 give chunks of 128 and 64 rows, shorter than
    one 256-row query tile.  Every rank through cpattn_forward (steps in
    grids of 32, the merge in passes of 64 partials) and through
    cpattn_forward_fused, vs the oracle (4 query heads, 2 KV heads)."""
    from oracle.matrix import attention_rows_matrix
    from long_context_causal_amd.inputs import as_f32
    w = dataclasses.replace(WORKLOADS["bf16_gqa_s32k_cp8"], name=f"bf16_gqa_s32k_cp{cp}", hq=4,
                            hkv=2, cp=cp)
    say(f"forward cp={cp} s={w.s} c={w.c}")
    q, k, v = make_inputs(w)
    o_full, l_full = attention_rows_matrix(as_f32(q), as_f32(k), as_f32(v), np.arange(1, w.s + 1))
    P = CPProblem(w, q, k, v)
    P.partition()
    worst = 0.0
    for r in range(w.cp):
        pos = ocp.zigzag_positions(w.s, w.cp, r)
        o, l = run_rank(P, r)
        out = P.alloc_out(r, C.CPATTN_F32)
        P.forward_fused(out)
        torch.cuda.synchronize()
        for tag, oo, ll in (("steps", o, l), ("fused", out["o"].cpu().numpy(),
                                              out["lse"].cpu().numpy())):
            err = np.abs(oo - o_full[:, pos])
            worst = max(worst, float(err.max()))
            assert np.isfinite(oo).all(), (tag, r)
            assert err.max() <= BF16_MAX_ABS and err.mean() <= BF16_MEAN_ABS, (tag, r, err.max())
            assert np.abs(ll - l_full[:, :, pos]).max() <= 1e-3, (tag, r)
        if r in (0, w.cp - 1):
            # bf16 output: the running fp32 result of the merge passes lives
            # in the workspace; the output is the fp32 result rounded
            ob, _ = run_rank(P, r, C.CPATTN_BF16)
            assert np.all(np.abs(ob - o) <= np.abs(o) * 2.0 ** -8 + 1e-30), r
    say(f"  every rank within bounds; worst max abs {worst:.3e}")


def test_forward_fp32_full_size():
    w = WORKLOADS["fp32_mha_s512_cp2"]
    say(f"forward full {w.name}")
    q, k, v = make_inputs(w)
    o_full, l_full = oracle_full(w, q, k, v)
    P = CPProblem(w, q, k, v)
    P.partition()
    for r in range(w.cp):
        o, l = run_rank(P, r)
        pos = ocp.zigzag_positions(w.s, w.cp, r)
        assert_close(f"rank {r} O", o, o_full[:, pos], F32_MAX_ABS)
        assert_close(f"rank {r} L", l, l_full[:, :, pos], F32_MAX_ABS)


@pytest.mark.parametrize("name,s", [("bf16_gqa_s32k_cp8", 2 * 8 * 64),
                                    ("bf16_gqa_s32k_cp8", 2 * 8 * 300),
                                    ("bf16_gqa_s128k_cp16_rope", 2 * 16 * 72),
                                    ("fp32_mha_s512_cp2", 512),
                                    ("cp40", WIDE_CP.s), ("cp1", ONE_CP.s)])
def test_stepwise_calls_equal_forward_entry_point(name, s):
    """One launch per step (cpattn_step_fwd), all steps in one grid
    (cpattn_forward_steps) and cpattn_forward give the same bits: every
    partial of every rank, and the merged result.  At s = 2*8*300 the grid
    has 1088-1536 query tiles, more than two per CU, so its workgroups loop
    over their items (ranks 0-2 and 4-6 with a partial last round); the
    per-step launches take one item per workgroup."""
    w = EXTRA[name] if name in EXTRA else small(WORKLOADS[name], s)
    say(f"stepwise vs cpattn_forward_steps vs cpattn_forward: {name} s={s}")
    q, k, v = make_inputs(w)
    P = CPProblem(w, q, k, v)
    P.partition()
    for r in range(w.cp):
        a = P.alloc_rank(r)
        for i in range(w.cp):
            P.step(a, i)
        P.merge(a)
        g = P.alloc_rank(r)
        g["ws"].fill_(255)            # NaN pattern: every partial must be written
        P.steps(g)
        b = P.alloc_rank(r)
        P.forward(b)
        torch.cuda.synchronize()
        for i in range(w.cp):
            assert torch.equal(a["steps"][i]["o"], g["steps"][i]["o"]), (r, i)
            assert torch.equal(a["steps"][i]["lse"], g["steps"][i]["lse"]), (r, i)
        assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"]), r


def test_resident_steps_grid_full_size_equals_stepwise():
    """At the 32k headline share (rank 3: 3072 items on one workgroup per
    CU, each looping over twelve items) the steps' grid writes every step's
    partial O_i and L_i with the same bits as one launch per step, and
    cpattn_forward (the grid and the merge) the same merged result."""
    w = WORKLOADS["bf16_gqa_s32k_cp8"]
    r = w.rank
    say(f"resident steps grid vs per-step launches: {w.name} rank {r}, full size")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    rnd = lambda *sh: (torch.randn(sh, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)  # noqa
    q, k, v = rnd(w.b, w.s, w.hq, w.d), rnd(w.b, w.s, w.hkv, w.d), rnd(w.b, w.s, w.hkv, w.d)
    torch.cuda.synchronize()
    P = CPProblem(w, q, k, v)          # device inputs are used as they are
    P.partition()
    a = P.alloc_rank(r)
    for i in range(w.cp):
        P.step(a, i)
    P.merge(a)
    g = P.alloc_rank(r)
    g["ws"].fill_(255)                # NaN pattern: every partial must be written
    P.steps(g)
    b = P.alloc_rank(r)
    P.forward(b)
    torch.cuda.synchronize()
    for i in range(w.cp):
        assert torch.equal(a["steps"][i]["o"], g["steps"][i]["o"]), i
        assert torch.equal(a["steps"][i]["lse"], g["steps"][i]["lse"]), i
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])
    say("  every partial and the merged result equal bit for bit")
