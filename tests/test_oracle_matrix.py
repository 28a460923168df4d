"""Pins of the oracle's matrix form (``oracle/matrix.py``) against things
other than itself.

All on the CPU.  A plausible mistake in the matrix form (a wrong GQA head
map, a mask off by one, a dropped max, rows of one run given another run's
keys, a transposed output) fails at least one of them:

* the row-at-a-time C core (itself pinned to torch SDPA, scipy logsumexp
  and closed forms in test_oracle_attention.py), on random inputs with
  ragged visible-key counts, including rows that see nothing;
* torch's fp64 scaled_dot_product_attention with the causal mask (a
  library attention routine, not the matmul and exp the form uses);
* closed form: Q = 0 and V[j] = j give L[i] = ln(kend_i) and O[i] =
  (kend_i - 1) / 2;
* the run size: tiny and huge score-matrix bounds give the same result.

The backward form (``attention_rows_bwd_matrix``) is pinned the same way:
to the C core's row-at-a-time backward (itself pinned by central finite
differences), to torch autograd through fp64 scaled_dot_product_attention,
to the closed form of dV when Q = 0 (uniform weights: dV[j] sums dO[i] /
kend[i] over the rows that see key j), and to its own run size.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_rows, attention_rows_bwd, causal_attention
from oracle.matrix import attention_at_positions, attention_rows_bwd_matrix, attention_rows_matrix


@pytest.mark.parametrize("b,nq,nk,hq,hkv,d", [(1, 1, 1, 1, 1, 8), (2, 37, 50, 4, 2, 16),
                                              (1, 64, 64, 8, 1, 32), (3, 20, 33, 6, 3, 4)])
def test_matches_c_core_ragged(b, nq, nk, hq, hkv, d):
    rng = np.random.default_rng(nq * 100 + nk)
    q = rng.standard_normal((b, nq, hq, d))
    k = rng.standard_normal((b, nk, hkv, d)) * 2
    v = rng.standard_normal((b, nk, hkv, d))
    kend = rng.integers(0, nk + 1, size=nq)
    kend[0] = 0                                # a row that sees no key
    kend[-1] = nk
    o, l = attention_rows_matrix(q, k, v, kend, max_elems=97)
    o_ref, l_ref = attention_rows(q, k, v, kend)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    np.testing.assert_allclose(l[fin], l_ref[fin], rtol=0, atol=1e-12)
    assert np.all(o[:, kend == 0] == 0.0)


@pytest.mark.parametrize("b,s,hq,hkv,d", [(1, 45, 4, 4, 16), (2, 64, 8, 2, 32)])
def test_matches_torch_sdpa_causal(b, s, hq, hkv, d):
    rng = np.random.default_rng(s)
    q, k, v = (rng.standard_normal((b, s, h, d)) for h in (hq, hkv, hkv))
    o, _ = attention_rows_matrix(q, k, v, np.arange(1, s + 1), max_elems=500)
    g = hq // hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_zero_queries_closed_form():
    nq, nk, d = 40, 40, 8
    q = np.zeros((1, nq, 2, d))
    v = np.broadcast_to(np.arange(nk, dtype=np.float64)[None, :, None, None],
                        (1, nk, 1, d)).copy()
    k = np.random.default_rng(0).standard_normal((1, nk, 1, d))
    kend = np.arange(1, nq + 1)
    o, l = attention_rows_matrix(q, k, v, kend, max_elems=64)
    np.testing.assert_allclose(l, np.log(kend)[None, None, :].repeat(2, 1), atol=1e-13)
    np.testing.assert_allclose(o, np.broadcast_to(((kend - 1) / 2.0)[None, :, None, None],
                                                  o.shape), atol=1e-12)


def test_run_size_does_not_matter_and_positions_form():
    rng = np.random.default_rng(5)
    s, hq, hkv, d = 96, 4, 2, 16
    q, k, v = (rng.standard_normal((1, s, h, d)) for h in (hq, hkv, hkv))
    pos = np.array([0, 3, 4, 50, 51, 90, 95])
    a = attention_at_positions(q[:, pos], k, v, pos, max_elems=1)
    b = attention_at_positions(q[:, pos], k, v, pos, max_elems=1 << 30)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)
    o_full, l_full = causal_attention(q, k, v)
    np.testing.assert_allclose(a[0], o_full[:, pos], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[1], l_full[:, :, pos], rtol=0, atol=1e-12)


def test_explicit_scale():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 12, 2, 8)) for _ in range(3))
    o, l = attention_rows_matrix(q, k, v, np.arange(1, 13), scale=0.3)
    o_ref, l_ref = attention_rows(q, k, v, np.arange(1, 13), scale=0.3)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, atol=1e-12)
    assert not math.isclose(0.3, 1 / math.sqrt(8))


@pytest.mark.parametrize("b,nq,nk,hq,hkv,d", [(1, 1, 1, 1, 1, 8), (2, 37, 50, 4, 2, 16),
                                              (3, 20, 33, 6, 3, 4)])
def test_bwd_matches_c_core_ragged(b, nq, nk, hq, hkv, d):
    rng = np.random.default_rng(nq * 7 + nk)
    q = rng.standard_normal((b, nq, hq, d))
    k = rng.standard_normal((b, nk, hkv, d)) * 2
    v = rng.standard_normal((b, nk, hkv, d))
    do = rng.standard_normal((b, nq, hq, d))
    kend = rng.integers(0, nk + 1, size=nq)
    kend[0] = 0                                # a row that sees no key
    kend[-1] = nk
    got = attention_rows_bwd_matrix(q, k, v, do, kend, max_elems=97)
    ref = attention_rows_bwd(q, k, v, do, kend)
    for x, y in zip(got, ref):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
    assert np.all(got[0][:, kend == 0] == 0.0)


@pytest.mark.parametrize("b,s,hq,hkv,d", [(1, 45, 4, 4, 16), (2, 64, 8, 2, 32)])
def test_bwd_matches_torch_autograd_causal(b, s, hq, hkv, d):
    rng = np.random.default_rng(s + 1)
    q, do = (rng.standard_normal((b, s, hq, d)) for _ in range(2))
    k, v = (rng.standard_normal((b, s, hkv, d)) for _ in range(2))
    dq, dk, dv = attention_rows_bwd_matrix(q, k, v, do, np.arange(1, s + 1), max_elems=700)
    g = hq // hkv
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_(True)
                  for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), is_causal=True)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got, t.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)


def test_bwd_zero_queries_closed_form_dv():
    rng = np.random.default_rng(3)
    nq, nk, hq, d = 30, 41, 4, 8
    q = np.zeros((1, nq, hq, d))
    k, v = (rng.standard_normal((1, nk, 2, d)) for _ in range(2))
    do = rng.standard_normal((1, nq, hq, d))
    kend = rng.integers(1, nk + 1, size=nq)
    _, _, dv = attention_rows_bwd_matrix(q, k, v, do, kend, max_elems=50)
    ref = np.zeros((1, nk, 2, d))
    for i in range(nq):
        for h in range(hq):
            ref[0, :kend[i], h // 2, :] += do[0, i, h, :] / kend[i]
    np.testing.assert_allclose(dv, ref, rtol=0, atol=1e-12)


def test_bwd_run_size_does_not_matter():
    rng = np.random.default_rng(9)
    s, hq, hkv, d = 80, 4, 2, 16
    q, do = (rng.standard_normal((2, s, hq, d)) for _ in range(2))
    k, v = (rng.standard_normal((2, s, hkv, d)) for _ in range(2))
    kend = np.arange(1, s + 1)
    a = attention_rows_bwd_matrix(q, k, v, do, kend, max_elems=1)
    b = attention_rows_bwd_matrix(q, k, v, do, kend, max_elems=1 << 30)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
