"""Pins of the packed variable-length oracle (all CPU).

The readings (independent causal samples, per-sample zigzag split, in-sample
positions; "Megatron 面试题（一）" M016 on resetting positions at packed
sample boundaries) are stated in ``oracle/varlen.py``.  Pinned here:

* one sample is the unpacked case: the definition equals the single-sequence
  oracle and the split equals ``cp.partition``;
* the definition against a brute-force masked softmax over the whole packed
  sequence (numpy, one score matrix with the mask "same sample and j <= i"),
  a formulation that never slices by sample;
* the document mask: changing one sample's inputs leaves every other
  sample's outputs bit for bit unchanged;
* the split: a bijection of the packed rows, every rank holding s/cp rows,
  each sample's rows in the single-sequence zigzag order and positions reset
  to the sample start;
* the CP invariant: every rank's merged share equals its rows of the
  definition, with and without RoPE, for mixed lengths down to one-row
  chunks (a split finer than any kernel tile);
* RoPE depends only on position differences, so resetting positions at the
  sample start gives the attention of the unreset (packed-index) positions;
* backward: central differences of a loss through the packed forward, and
  the CP invariant (every rank's dq, and the ranks' dK/dV contributions
  summed per owner, equal the packed gradients).
"""
import numpy as np
import pytest

from oracle import causal_attention
from oracle import cp as ocp
from oracle import varlen as ovl


def _rand(rng, shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _qkv(rng, b, s, hq, hkv, d, scale=1.0):
    return (_rand(rng, (b, s, hq, d), scale), _rand(rng, (b, s, hkv, d), scale),
            _rand(rng, (b, s, hkv, d), scale))


def _brute(q, k, v, cu, scale):
    """Masked softmax over the packed sequence, straight from the mask."""
    b, s, hq, d = q.shape
    g = hq // k.shape[2]
    sample = np.searchsorted(np.asarray(cu)[1:], np.arange(s), side="right")
    idx = np.arange(s)
    mask = (sample[:, None] == sample[None, :]) & (idx[None, :] <= idx[:, None])
    o = np.zeros((b, s, hq, d))
    lse = np.zeros((b, hq, s))
    for n in range(b):
        for h in range(hq):
            z = scale * q[n, :, h] @ k[n, :, h // g].T
            z = np.where(mask, z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            ssum = e.sum(axis=1, keepdims=True)
            o[n, :, h] = (e / ssum) @ v[n, :, h // g]
            lse[n, h] = (m + np.log(ssum))[:, 0]
    return o, lse


def test_single_sample_is_unpacked():
    rng = np.random.default_rng(1)
    b, s, hq, hkv, d, cp = 2, 48, 4, 2, 16, 3
    q, k, v = _qkv(rng, b, s, hq, hkv, d)
    o, lse = ovl.packed_causal_attention(q, k, v, [0, s])
    o_ref, lse_ref = causal_attention(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(ovl.partition(q, [0, s], cp), ocp.partition(q, cp))
    for r in range(cp):
        np.testing.assert_array_equal(ovl.local_positions([0, s], cp, r),
                                      ocp.zigzag_positions(s, cp, r))


@pytest.mark.parametrize("cu", [[0, 8, 12, 36, 40], [0, 4, 8], [0, 28, 32, 60]])
def test_definition_vs_brute_force_mask(cu):
    rng = np.random.default_rng(sum(cu))
    s = cu[-1]
    q, k, v = _qkv(rng, 2, s, 4, 2, 8, 0.7)
    o, lse = ovl.packed_causal_attention(q, k, v, cu, scale=0.4)
    o_b, lse_b = _brute(q, k, v, cu, 0.4)
    np.testing.assert_allclose(o, o_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-12)


def test_document_mask_independence():
    rng = np.random.default_rng(5)
    cu = [0, 12, 20, 44]
    q, k, v = _qkv(rng, 1, 44, 2, 1, 8)
    o, lse = ovl.packed_causal_attention(q, k, v, cu)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 12:20] += 3.0
    k2[:, 12:20] -= 2.0
    v2[:, 12:20] *= -5.0
    o2, lse2 = ovl.packed_causal_attention(q2, k2, v2, cu)
    for a, e in ((0, 12), (20, 44)):
        np.testing.assert_array_equal(o[:, a:e], o2[:, a:e])
        np.testing.assert_array_equal(lse[:, :, a:e], lse2[:, :, a:e])
    assert not np.allclose(o[:, 12:20], o2[:, 12:20])


@pytest.mark.parametrize("cu,cp", [([0, 8, 24, 32], 2), ([0, 6, 12, 30], 3),
                                   ([0, 16, 32, 48, 64, 128], 8)])
def test_split_layout(cu, cp):
    s = cu[-1]
    rows = np.concatenate([ovl.local_rows(cu, cp, r) for r in range(cp)])
    assert sorted(rows.tolist()) == list(range(s))
    for r in range(cp):
        lr = ovl.local_rows(cu, cp, r)
        pos = ovl.local_positions(cu, cp, r)
        assert lr.size == s // cp
        for i in range(len(cu) - 1):
            a, e = cu[i] // cp, cu[i + 1] // cp   # the sample's local rows
            zz = ocp.zigzag_positions(cu[i + 1] - cu[i], cp, r)
            np.testing.assert_array_equal(lr[a:e], cu[i] + zz)
            np.testing.assert_array_equal(pos[a:e], zz)
    x = np.arange(2 * s * 3, dtype=np.float64).reshape(2, s, 3, 1)
    np.testing.assert_array_equal(ovl.unpartition(ovl.partition(x, cu, cp), cu), x)


@pytest.mark.parametrize("cu,cp,theta", [
    ([0, 8, 40, 48], 4, None),            # one-row chunks in two samples
    ([0, 24, 36, 96], 6, None),
    ([0, 16, 64, 80], 2, 10000.0),
    ([0, 4, 8, 12, 16, 44], 2, 500.0),
])
def test_cp_invariant(cu, cp, theta):
    rng = np.random.default_rng(cp * 10 + len(cu))
    s = cu[-1]
    q, k, v = _qkv(rng, 2, s, 4, 2, 16)
    o_ref, lse_ref = ovl.packed_causal_attention(q, k, v, cu, rope_theta=theta)
    for r in range(cp):
        o, lse = ovl.cp_forward_rank(q, k, v, cu, cp, r, rope_theta=theta)
        lr = ovl.local_rows(cu, cp, r)
        np.testing.assert_allclose(o, o_ref[:, lr], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref[:, :, lr], rtol=0, atol=1e-12)


def test_rope_reset_is_relative():
    rng = np.random.default_rng(11)
    cu = [0, 20, 36, 64]
    q, k, v = _qkv(rng, 1, 64, 2, 2, 16)
    o, lse = ovl.packed_causal_attention(q, k, v, cu, rope_theta=1000.0)
    # the same samples rotated at their packed indices instead
    pos = np.arange(64)
    qr, kr = ocp.rope(q, pos, 1000.0), ocp.rope(k, pos, 1000.0)
    o2, lse2 = ovl.packed_causal_attention(qr, kr, v, cu)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-11)
    # while the rotated rows themselves differ after the first sample
    assert not np.allclose(ocp.rope(q[:, 20:36], np.arange(16), 1000.0), qr[:, 20:36])


def test_bad_offsets_rejected():
    with pytest.raises(ValueError):
        ovl.check_cu([0, 6, 16], 16, 2)   # 6 is not a multiple of 2*cp
    with pytest.raises(ValueError):
        ovl.check_cu([0, 8, 8, 16], 16, 2)
    with pytest.raises(ValueError):
        ovl.check_cu([4, 16], 16, 2)
    assert ovl.check_cu([0, 4, 16], 16, 2).dtype == np.int64


# --- backward ----------------------------------------------------------------

def test_bwd_finite_differences_of_packed_definition():
    """Central differences of a scalar loss through the packed forward: a
    check of the gradients that never calls the gradient code's per-sample
    slicing on the forward side."""
    rng = np.random.default_rng(21)
    cu = [0, 4, 12]
    q, k, v = _qkv(rng, 1, 12, 2, 1, 4, 0.8)
    w_o = rng.standard_normal((1, 12, 2, 4))
    dq, dk, dv = ovl.packed_causal_attention_bwd(q, k, v, w_o, cu, scale=0.6)

    def loss(q_, k_, v_):
        o, _ = ovl.packed_causal_attention(q_, k_, v_, cu, scale=0.6)
        return float((o * w_o).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(num - g[idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, g[idx])


@pytest.mark.parametrize("cu,cp", [([0, 8, 40, 48], 4), ([0, 12, 24, 60], 3)])
def test_bwd_cp_invariant(cu, cp):
    """The ranks' dq and their summed dK/dV contributions (what the
    reduce-scatter forms on each owner) equal the packed gradients."""
    rng = np.random.default_rng(cp + len(cu))
    s = cu[-1]
    q, k, v = _qkv(rng, 2, s, 4, 2, 8)
    dout = rng.standard_normal(q.shape)
    dq_ref, dk_ref, dv_ref = ovl.packed_causal_attention_bwd(q, k, v, dout, cu)
    dkz_sum = np.zeros((cp, 2, s // cp, 2, 8))
    dvz_sum = np.zeros_like(dkz_sum)
    for r in range(cp):
        dq_r, dkz, dvz = ovl.cp_backward_rank(q, k, v, dout, cu, cp, r)
        np.testing.assert_allclose(dq_r, dq_ref[:, ovl.local_rows(cu, cp, r)], rtol=0,
                                   atol=1e-11)
        dkz_sum += dkz
        dvz_sum += dvz
    np.testing.assert_allclose(ovl.unpartition(dkz_sum, cu), dk_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(ovl.unpartition(dvz_sum, cu), dv_ref, rtol=0, atol=1e-11)
