"""Pins of the oracle's context-parallel emulation (all CPU).

* the split against hand-derived positions (tests/golden, cited there) and
  as a bijection of 0..s-1;
* the step schedule against a hand-derived table;
* exact integer cover: over all ranks and steps every causal pair (i, j),
  j <= i, is computed exactly once and no masked pair ever is.  The pairs
  are read back from the oracle's own step attention (Q = 0 makes the
  weights uniform, one-hot V makes each output row the visible-key
  indicator), so the check exercises the step code, not a retyped mask;
* the reverse ring direction and a wrong step-0 rule both fail that cover;
* equal work on every rank ("one big, one small");
* the invariant of "Megatron-LM 篇" §3.2: every rank's merged output equals
  its slice of the non-CP output, for every cp with 2cp | s;
* merge identities of the two-stage LSE ("Megatron 面试题（一）" M019).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import causal_attention, attention_rows
from oracle import cp as ocp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_positions_golden():
    for case in _load("zigzag_positions.json")["cases"]:
        for r, want in enumerate(case["ranks"]):
            got = ocp.zigzag_positions(case["s"], case["cp"], r)
            assert got.tolist() == want, (case["s"], case["cp"], r)


@pytest.mark.parametrize("s,cp", [(8, 1), (8, 2), (12, 3), (16, 4), (64, 16),
                                  (512, 2), (96, 6), (1024, 8)])
def test_positions_bijection_and_order(s, cp):
    allpos = np.concatenate([ocp.zigzag_positions(s, cp, r) for r in range(cp)])
    assert sorted(allpos.tolist()) == list(range(s))
    for r in range(cp):
        pos = ocp.zigzag_positions(s, cp, r)
        assert np.all(np.diff(pos) > 0)      # local order keeps global order


def test_positions_reject_bad_split():
    with pytest.raises(ValueError):
        ocp.zigzag_positions(10, 3, 0)
    with pytest.raises(ValueError):
        ocp.zigzag_positions(8, 2, 2)


def test_schedule_golden():
    fx = _load("step_schedule.json")
    cp = fx["cp"]
    for r, rows in fx["table"].items():
        for i, (mode, src) in enumerate(rows):
            assert ocp.step_schedule(i, int(r), cp) == (mode, src)


def _cover_counts(s, cp, ring=ocp.step_schedule):
    """counts[r][row, key]: times rank r computes (global row, global key)."""
    q = np.zeros((1, s, 1, s))                       # Q = 0: uniform weights
    k = np.zeros((1, s, 1, s))
    v = np.eye(s)[None, :, None, :]                  # V[j] = e_j, d = s
    qz, kz, vz = ocp.partition(q, cp), ocp.partition(k, cp), ocp.partition(v, cp)
    total = np.zeros((s, s), np.int64)
    per_rank = []
    for r in range(cp):
        pos = ocp.zigzag_positions(s, cp, r)
        counts = np.zeros((s, s), np.int64)
        for i in range(cp):
            mode, src = ring(i, r, cp)
            o, lse, row0 = ocp.step_attention(qz[r], kz[src], vz[src], mode)
            n_vis = np.exp(lse[0, 0])                 # L = ln(#visible keys)
            ind = o[0, :, 0, :] * n_vis[:, None]      # visible-key indicator
            assert np.allclose(ind, np.round(ind), atol=1e-9)
            rows = pos[row0:row0 + o.shape[1]]
            counts[rows] += np.round(ind).astype(np.int64)
        per_rank.append(counts)
        total += counts
    return total, per_rank


@pytest.mark.parametrize("s,cp", [(8, 1), (8, 2), (12, 3), (16, 4), (24, 3),
                                  (32, 8), (40, 5), (64, 16)])
def test_exact_cover_of_causal_triangle(s, cp):
    total, per_rank = _cover_counts(s, cp)
    assert np.array_equal(total, np.tril(np.ones((s, s), np.int64)))
    c = s // (2 * cp)
    want = c * (2 * c + 1) + (cp - 1) * 2 * c * c
    for counts in per_rank:                          # balanced work
        assert counts.sum() == want


def test_reverse_ring_computes_masked_pairs():
    def reverse(i, r, cp):
        mode, _ = ocp.step_schedule(i, r, cp)
        return mode, (r + i) % cp
    total, _ = _cover_counts(16, 4, reverse)
    upper = np.triu(np.ones((16, 16), bool), k=1)
    assert total[upper].sum() > 0


def test_step0_must_be_causal():
    def kv_half_first(i, r, cp):
        mode, src = ocp.step_schedule(i, r, cp)
        return (ocp.KV_FIRST_HALF if i == 0 else mode), src
    total, _ = _cover_counts(16, 4, kv_half_first)
    assert not np.array_equal(total, np.tril(np.ones((16, 16), np.int64)))


def _rand_qkv(seed, b, s, hq, hkv, d, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, s, hq, d)) * scale,
            rng.standard_normal((b, s, hkv, d)) * scale,
            rng.standard_normal((b, s, hkv, d)))


@pytest.mark.parametrize("s,hq,hkv,scale", [(48, 4, 2, 1.0), (96, 2, 2, 2.5),
                                            (120, 6, 3, 1.0)])
def test_cp_merged_equals_non_cp_for_every_cp(s, hq, hkv, scale):
    q, k, v = _rand_qkv(s, 2, s, hq, hkv, 8, scale)
    o_full, l_full = causal_attention(q, k, v)
    for cp in [c for c in range(1, s // 2 + 1) if s % (2 * c) == 0]:
        for r in range(cp):
            o, lse, pos = ocp.cp_forward_rank(q, k, v, cp, r)
            np.testing.assert_allclose(o, o_full[:, pos], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, l_full[:, :, pos], rtol=0, atol=1e-12)


def test_cp_with_rope_at_global_positions():
    s, cp = 64, 4
    q, k, v = _rand_qkv(4, 1, s, 4, 2, 16)
    ar = np.arange(s)
    o_full, l_full = causal_attention(ocp.rope(q, ar), ocp.rope(k, ar), v)
    for r in range(cp):
        o, lse, pos = ocp.cp_forward_rank(q, k, v, cp, r, rope_theta=10000.0)
        np.testing.assert_allclose(o, o_full[:, pos], atol=1e-12)
        np.testing.assert_allclose(lse, l_full[:, :, pos], atol=1e-12)


def test_rope_renumbered_from_zero_is_wrong():
    """Rotating each rank's rows at local indices 0..2c-1 breaks the result
    ("Megatron 面试题（一）" M016: renumbering from 0 breaks the phases)."""
    s, cp, r = 64, 4, 1
    q, k, v = _rand_qkv(6, 1, s, 2, 2, 16)
    ar = np.arange(s)
    o_full, _ = causal_attention(ocp.rope(q, ar), ocp.rope(k, ar), v)
    qz, kz, vz = ocp.partition(q, cp), ocp.partition(k, cp), ocp.partition(v, cp)
    local = np.arange(2 * (s // (2 * cp)))
    qz = np.stack([ocp.rope(x, local) for x in qz])
    kz = np.stack([ocp.rope(x, local) for x in kz])
    parts = []
    for i in range(cp):
        mode, src = ocp.step_schedule(i, r, cp)
        parts.append(ocp.step_attention(qz[r], kz[src], vz[src], mode))
    o, _ = ocp.merge_outputs(parts, 2 * (s // (2 * cp)))
    pos = ocp.zigzag_positions(s, cp, r)
    assert np.abs(o - o_full[:, pos]).max() > 1e-3


# --- merge identities ------------------------------------------------------

@pytest.mark.parametrize("split", [1, 7, 19, 30])
def test_lse_split_identity(split):
    rng = np.random.default_rng(split)
    n, d = 31, 8
    q = rng.standard_normal((1, 5, 2, d)) * 3
    k, v = rng.standard_normal((1, n, 1, d)), rng.standard_normal((1, n, 1, d))
    o_all, l_all = attention_rows(q, k, v, np.full(5, n))
    a = attention_rows(q, k[:, :split], v[:, :split], np.full(5, split))
    b = attention_rows(q, k[:, split:], v[:, split:], np.full(5, n - split))
    o, lse = ocp.merge_outputs([(a[0], a[1], 0), (b[0], b[1], 0)], 5)
    np.testing.assert_allclose(o, o_all, atol=1e-13)
    np.testing.assert_allclose(lse, l_all, atol=1e-13)


def test_merge_empty_partial_is_identity():
    rng = np.random.default_rng(0)
    o1, l1 = rng.standard_normal((1, 3, 2, 4)), rng.standard_normal((1, 2, 3))
    empty = (np.zeros_like(o1), np.full_like(l1, -np.inf), 0)
    o, lse = ocp.merge_outputs([(o1, l1, 0), empty], 3)
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)


def test_merge_of_empty_partials_is_empty_sum():
    """Rows whose partials all see no key merge to the core's own empty
    result (attention over zero keys: O = 0, L = -inf)."""
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((1, 3, 2, 4)), rng.standard_normal((1, 5, 1, 4)), \
        rng.standard_normal((1, 5, 1, 4))
    e1 = attention_rows(q, k, v, [0, 0, 0])
    e2 = attention_rows(q, k[:, :2], v[:, :2], [0, 0, 0])
    o, lse = ocp.merge_outputs([(e1[0], e1[1], 0), (e2[0], e2[1], 0)], 3)
    assert np.array_equal(o, e1[0]) and np.array_equal(lse, e1[1])
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_merge_equal_lse_averages():
    rng = np.random.default_rng(1)
    oa, ob = rng.standard_normal((1, 2, 1, 4)), rng.standard_normal((1, 2, 1, 4))
    l = np.array([[[0.3, -7.0]]])
    o, lse = ocp.merge_outputs([(oa, l, 0), (ob, l.copy(), 0)], 2)
    np.testing.assert_allclose(lse, l + math.log(2.0), atol=1e-15)
    np.testing.assert_allclose(o, (oa + ob) / 2, atol=1e-15)


def test_merge_large_gap_picks_dominant():
    oa, ob = np.ones((1, 1, 1, 2)), -np.ones((1, 1, 1, 2))
    o, lse = ocp.merge_outputs([(oa, np.array([[[30.0]]]), 0),
                                (ob, np.array([[[-30.0]]]), 0)], 1)
    # exact values: tanh(30) = 1 - 1.8e-26 and 30 + ln(1 + e^-60)
    assert abs(o[0, 0, 0, 0] - math.tanh(30.0)) <= 1e-16
    assert abs(lse[0, 0, 0] - (30.0 + math.log1p(math.exp(-60.0)))) <= 1e-15


def test_merge_partial_row_ranges():
    """A partial covering rows c..2c-1 only leaves rows < c to the others."""
    rng = np.random.default_rng(2)
    o1, l1 = rng.standard_normal((1, 4, 1, 2)), rng.standard_normal((1, 1, 4))
    o2, l2 = rng.standard_normal((1, 2, 1, 2)), rng.standard_normal((1, 1, 2))
    o, lse = ocp.merge_outputs([(o1, l1, 0), (o2, l2, 2)], 4)
    assert np.array_equal(o[:, :2], o1[:, :2]) and np.array_equal(lse[..., :2], l1[..., :2])
    want = np.logaddexp(l1[..., 2:], l2)
    np.testing.assert_allclose(lse[..., 2:], want, atol=1e-15)


# --- RoPE ------------------------------------------------------------------

def test_rope_d2_is_plane_rotation_by_position():
    x = np.array([[[[0.6, -1.3]]]]).repeat(5, axis=1)      # [1, 5, 1, 2]
    pos = np.array([0, 1, 2, 100, 131071])
    got = ocp.rope(x, pos)
    for n, p in enumerate(pos):
        c, s = math.cos(p), math.sin(p)
        want = np.array([[c, -s], [s, c]]) @ np.array([0.6, -1.3])
        np.testing.assert_allclose(got[0, n, 0], want, atol=1e-12)


def test_rope_complex_form():
    rng = np.random.default_rng(3)
    d, n = 16, 9
    x = rng.standard_normal((1, n, 2, d))
    pos = rng.integers(0, 10 ** 5, n)
    got = ocp.rope(x, pos, theta=500.0)
    z = x[..., :d // 2] + 1j * x[..., d // 2:]
    freq = np.power(500.0, -np.arange(d // 2) / (d // 2))
    zr = z * np.exp(1j * pos[None, :, None, None] * freq)
    np.testing.assert_allclose(got[..., :d // 2], zr.real, atol=1e-9)
    np.testing.assert_allclose(got[..., d // 2:], zr.imag, atol=1e-9)


def test_rope_dot_depends_on_offset_only():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((1, 1, 1, 32)), rng.standard_normal((1, 1, 1, 32))
    def dot(m, n):
        return float((ocp.rope(q, [m]) * ocp.rope(k, [n])).sum())
    base = dot(10, 3)
    for delta in (1, 1000, 65536):
        assert abs(dot(10 + delta, 3 + delta) - base) < 1e-9
    assert abs(dot(11, 3) - base) > 1e-6
    x = ocp.rope(q, [12345])
    assert abs(np.linalg.norm(x) - np.linalg.norm(q)) < 1e-12


def test_attention_shift_invariant_under_rope():
    rng = np.random.default_rng(8)
    s = 32
    q, k, v = rng.standard_normal((1, s, 2, 8)), rng.standard_normal((1, s, 2, 8)), \
        rng.standard_normal((1, s, 2, 8))
    ar = np.arange(s)
    a = causal_attention(ocp.rope(q, ar), ocp.rope(k, ar), v)
    b = causal_attention(ocp.rope(q, ar + 777), ocp.rope(k, ar + 777), v)
    np.testing.assert_allclose(a[0], b[0], atol=1e-10)
    np.testing.assert_allclose(a[1], b[1], atol=1e-10)


def test_rank_flops_formula_matches_cover_count():
    s, cp = 32, 4
    _, per_rank = _cover_counts(s, cp)
    for r, counts in enumerate(per_rank):
        assert ocp.causal_flops(1, s, 1, 1, cp, r) == 4 * counts.sum()
    assert ocp.causal_flops(1, s, 1, 1, cp) == 4 * s * (s + 1) // 2
