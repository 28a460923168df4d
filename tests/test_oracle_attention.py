"""Pins of the oracle's attention core against things other than itself.

Every test here runs on the CPU.  A plausible mistake in ``attention.c``
(a dropped max term, a wrong scale, a transposed operand, a wrong GQA
group, an off-by-one mask) fails at least one of them:

* a library attention routine (torch scaled_dot_product_attention, fp64,
  CPU, causal) and scipy's logsumexp on library-matmul scores;
* closed forms: equal scores give L = a + ln(n) and the mean of V;
  Q = 0 with V[j] = j gives O[i] = i/2 exactly;
* invariants: rows of the weight matrix sum to one, vanish above the
  diagonal; keys after row i never change row i.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention_rows, causal_attention

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


@pytest.mark.parametrize("b,s,hq,hkv,d", [(1, 1, 1, 1, 8), (2, 37, 4, 2, 16),
                                          (1, 64, 8, 1, 32), (3, 20, 6, 3, 4)])
def test_matches_torch_sdpa_fp64(b, s, hq, hkv, d):
    rng = np.random.default_rng(b * 1000 + s)
    q, k, v = _rand(rng, b, s, hq, d), _rand(rng, b, s, hkv, d), _rand(rng, b, s, hkv, d)
    o, lse = causal_attention(q, k, v)
    g = hq // hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)
    # L against scipy's logsumexp of the masked scores
    scores = np.einsum("bihd,bjhd->bhij", q, np.repeat(k, g, axis=2)) / math.sqrt(d)
    mask = np.tril(np.ones((s, s), bool))
    scores = np.where(mask, scores, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(scores, axis=-1),
                               rtol=0, atol=1e-12)


def test_explicit_scale_matches_sdpa_scale():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 1, 12, 2, 8), _rand(rng, 1, 12, 2, 8), _rand(rng, 1, 12, 2, 8)
    o, _ = causal_attention(q, k, v, scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)),
        is_causal=True, scale=0.3)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_equal_scores_closed_form():
    """All keys equal: every visible score is a, so L = a + ln(i+1)."""
    rng = np.random.default_rng(3)
    s, d = 50, 16
    q = _rand(rng, 1, s, 1, d)
    k0 = _rand(rng, d)
    k = np.broadcast_to(k0, (1, s, 1, d)).copy()
    v = _rand(rng, 1, s, 1, d)
    o, lse = causal_attention(q, k, v)
    a = (q[0, :, 0] @ k0) / math.sqrt(d)
    np.testing.assert_allclose(lse[0, 0], a + np.log(np.arange(1, s + 1)), atol=1e-12)
    prefix_mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, s + 1)[:, None]
    np.testing.assert_allclose(o[0, :, 0], prefix_mean, atol=1e-12)


def test_zero_query_ramp_values():
    """Q = 0 and V[j] = j: O[i] = i/2 and L[i] = ln(i+1)."""
    s, d = 300, 4
    q = np.zeros((1, s, 2, d))
    k = np.random.default_rng(0).standard_normal((1, s, 1, d))
    v = np.broadcast_to(np.arange(s, dtype=np.float64)[None, :, None, None],
                        (1, s, 1, d)).copy()
    o, lse = causal_attention(q, k, v)
    want = np.arange(s) / 2.0
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h, :], want[:, None] * np.ones(d), atol=1e-10)
        np.testing.assert_allclose(lse[0, h], np.log(np.arange(1, s + 1)), atol=1e-13)


def test_two_keys_closed_form():
    """Row 1 sees two keys with scores a and b: softmax by hand."""
    d = 2
    q = np.zeros((1, 2, 1, d)); q[0, 1, 0] = [1.0, 0.0]
    k = np.zeros((1, 2, 1, d)); k[0, 0, 0] = [3.0, 0.0]; k[0, 1, 0] = [-1.0, 5.0]
    v = np.zeros((1, 2, 1, d)); v[0, 0, 0] = [1.0, 0.0]; v[0, 1, 0] = [0.0, 1.0]
    o, lse = causal_attention(q, k, v)
    a, b = 3.0 / math.sqrt(2), -1.0 / math.sqrt(2)
    wa = 1.0 / (1.0 + math.exp(b - a))
    assert abs(lse[0, 0, 1] - (a + math.log1p(math.exp(b - a)))) < 1e-14
    np.testing.assert_allclose(o[0, 1, 0], [wa, 1 - wa], atol=1e-15)
    # row 0 sees only key 0
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=0)
    assert lse[0, 0, 0] == 0.0


def test_row_stochastic_weights():
    """With one-hot values V[j] = e_j the output row is the weight row."""
    rng = np.random.default_rng(11)
    s = 24
    q, k = _rand(rng, 2, s, 3, s, scale=2.0), _rand(rng, 2, s, 3, s)
    v = np.broadcast_to(np.eye(s)[None, :, None, :], (2, s, 3, s)).copy()
    w, _ = causal_attention(q, k, v)                    # [b, i, h, j]
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, atol=1e-13)
    upper = np.triu(np.ones((s, s), bool), k=1)
    assert np.all(w.transpose(0, 2, 1, 3)[..., upper] == 0.0)
    assert np.all(w.transpose(0, 2, 1, 3)[..., ~upper] > 0.0)


def test_future_keys_do_not_change_past_rows():
    rng = np.random.default_rng(5)
    s = 40
    q, k, v = _rand(rng, 1, s, 2, 8), _rand(rng, 1, s, 1, 8), _rand(rng, 1, s, 1, 8)
    o, lse = causal_attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[:, 25:] = _rand(rng, 1, s - 25, 1, 8) * 10
    v2[:, 25:] = -v2[:, 25:]
    o2, lse2 = causal_attention(q, k2, v2)
    assert np.array_equal(o[:, :25], o2[:, :25])
    assert np.array_equal(lse[:, :, :25], lse2[:, :, :25])
    assert not np.allclose(o[:, 25:], o2[:, 25:])


def test_gqa_group_is_contiguous():
    """Head h reads KV group h // (hq/hkv): compare with one-head calls."""
    rng = np.random.default_rng(9)
    b, s, hq, hkv, d = 1, 16, 6, 2, 8
    q, k, v = _rand(rng, b, s, hq, d), _rand(rng, b, s, hkv, d), _rand(rng, b, s, hkv, d)
    o, lse = causal_attention(q, k, v)
    for h in range(hq):
        g = h // (hq // hkv)
        oh, lh = causal_attention(q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1])
        assert np.array_equal(o[:, :, h:h + 1], oh)
        assert np.array_equal(lse[:, h:h + 1], lh)


def test_no_visible_key_is_empty_sum():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 1, 3, 1, 4), _rand(rng, 1, 5, 1, 4), _rand(rng, 1, 5, 1, 4)
    o, lse = attention_rows(q, k, v, [0, 5, 1])
    assert np.all(o[0, 0] == 0) and lse[0, 0, 0] == -np.inf
    np.testing.assert_allclose(o[0, 2, 0], v[0, 0, 0], atol=0)


def test_rejects_bad_arguments():
    z = np.zeros((1, 4, 3, 2))
    with pytest.raises(ValueError):
        attention_rows(z, np.zeros((1, 4, 2, 2)), np.zeros((1, 4, 2, 2)), [1, 2, 3, 4])
    with pytest.raises(ValueError):
        attention_rows(np.zeros((1, 2, 2, 2)), np.zeros((1, 4, 2, 2)),
                       np.zeros((1, 4, 2, 2)), [1, 5])


def test_threads_do_not_change_bits():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 2, 64, 4, 16), _rand(rng, 2, 64, 2, 16), _rand(rng, 2, 64, 2, 16)
    a = causal_attention(q, k, v, nthreads=1)
    b = causal_attention(q, k, v, nthreads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
