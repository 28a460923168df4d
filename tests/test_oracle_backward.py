"""Pins of the backward oracle (``attention_rows_bwd``) and of the CP
backward emulation (``cp.step_attention_bwd``, ``cp.cp_backward_rank``).

The gradients are pinned to things other than their own formulas:
* central finite differences of the forward oracle's loss sum(dO * O);
* the Q = 0 closed forms (uniform attention over the visible prefix);
* GQA equals MHA on replicated K/V with the group's gradients summed;
* linearity in dO;
* the CP scheme: every rank's step contributions, summed per owner (the
  reduce-scatter) and un-permuted, equal the non-CP gradients.
"""
import numpy as np
import pytest

from oracle import attention_rows, attention_rows_bwd, causal_attention, causal_attention_bwd
from oracle import cp as ocp


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("kend", [None, [1, 3, 3, 2, 5]])
def test_finite_differences_every_element(kend):
    b, s, hq, hkv, d = 1, 5, 2, 1, 3
    q, k, v, do = _rand(1, b, s, hq, d), _rand(2, b, s, hkv, d), _rand(3, b, s, hkv, d), \
        _rand(4, b, s, hq, d)
    ke = np.arange(1, s + 1) if kend is None else np.array(kend)

    def loss(q_, k_, v_):
        o, _ = attention_rows(q_, k_, v_, ke)
        return float(np.sum(o * do))

    dq, dk, dv = attention_rows_bwd(q, k, v, do, ke)
    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a, m = arr.copy(), arr.copy()
            a[idx] += eps
            m[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = a, m
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def test_zero_query_closed_form():
    """Q = 0: row i averages v_0..v_i, so dV_j = sum_{i>=j} dO_i / (i+1) and
    dQ_i = scale/(i+1) * sum_{j<=i} (dO_i . (v_j - O_i)) k_j."""
    b, s, hq, d = 1, 9, 1, 4
    scale = 0.3
    q = np.zeros((b, s, hq, d))
    k, v, do = _rand(5, b, s, 1, d), _rand(6, b, s, 1, d), _rand(7, b, s, hq, d)
    dq, dk, dv = causal_attention_bwd(q, k, v, do, scale=scale)
    dv_cf = np.zeros((s, d))
    dq_cf = np.zeros((s, d))
    for i in range(s):
        o_i = v[0, :i + 1, 0].mean(axis=0)
        for j in range(i + 1):
            dv_cf[j] += do[0, i, 0] / (i + 1)
            dq_cf[i] += scale / (i + 1) * np.dot(do[0, i, 0], v[0, j, 0] - o_i) * k[0, j, 0]
    np.testing.assert_allclose(dv[0, :, 0], dv_cf, atol=1e-12)
    np.testing.assert_allclose(dq[0, :, 0], dq_cf, atol=1e-12)


def test_gqa_is_mha_on_replicated_kv_summed_per_group():
    b, s, hq, hkv, d = 2, 7, 4, 2, 5
    q, k, v, do = _rand(8, b, s, hq, d), _rand(9, b, s, hkv, d), _rand(10, b, s, hkv, d), \
        _rand(11, b, s, hq, d)
    dq, dk, dv = causal_attention_bwd(q, k, v, do)
    rep = np.repeat(np.arange(hkv), hq // hkv)
    dq_m, dk_m, dv_m = causal_attention_bwd(q, k[:, :, rep], v[:, :, rep], do)
    np.testing.assert_allclose(dq, dq_m, atol=1e-12)
    np.testing.assert_allclose(dk, dk_m.reshape(b, s, hkv, hq // hkv, d).sum(3), atol=1e-12)
    np.testing.assert_allclose(dv, dv_m.reshape(b, s, hkv, hq // hkv, d).sum(3), atol=1e-12)


def test_linear_in_dout():
    b, s, hq, d = 1, 6, 2, 4
    q, k, v = _rand(12, b, s, hq, d), _rand(13, b, s, hq, d), _rand(14, b, s, hq, d)
    d1, d2 = _rand(15, b, s, hq, d), _rand(16, b, s, hq, d)
    g1 = causal_attention_bwd(q, k, v, d1)
    g2 = causal_attention_bwd(q, k, v, d2)
    g12 = causal_attention_bwd(q, k, v, 2.0 * d1 - 3.0 * d2)
    for a, b_, c in zip(g1, g2, g12):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b_, atol=1e-11)


@pytest.mark.parametrize("s,cp,hq,hkv", [(8, 2, 2, 2), (24, 3, 4, 2), (32, 4, 2, 1),
                                         (16, 1, 2, 2), (48, 4, 4, 4)])
def test_cp_backward_equals_full_backward(s, cp, hq, hkv):
    b, d = 2, 6
    q, k, v, do = _rand(20 + s, b, s, hq, d), _rand(21 + s, b, s, hkv, d), \
        _rand(22 + s, b, s, hkv, d), _rand(23 + s, b, s, hq, d)
    dq_full, dk_full, dv_full = causal_attention_bwd(q, k, v, do)
    two_c = s // cp
    dq_z = np.zeros((cp, b, two_c, hq, d))
    dk_z = np.zeros((cp, b, two_c, hkv, d))
    dv_z = np.zeros((cp, b, two_c, hkv, d))
    for r in range(cp):
        dq_r, dkz, dvz = ocp.cp_backward_rank(q, k, v, do, cp, r)
        dq_z[r] = dq_r
        dk_z += dkz          # the reduce-scatter: every rank's share summed on its owner
        dv_z += dvz
    np.testing.assert_allclose(ocp.unpartition(dq_z, s), dq_full, atol=1e-10)
    np.testing.assert_allclose(ocp.unpartition(dk_z, s), dk_full, atol=1e-10)
    np.testing.assert_allclose(ocp.unpartition(dv_z, s), dv_full, atol=1e-10)


def test_cp_backward_needs_the_final_lse():
    """Using each step's own L instead of the merged one breaks the sum (the
    test would pass for a wrong scheme only if the two coincided)."""
    s, cp, b, hq, d = 16, 2, 1, 1, 4
    q, k, v, do = _rand(30, b, s, hq, d), _rand(31, b, s, hq, d), _rand(32, b, s, hq, d), \
        _rand(33, b, s, hq, d)
    _, dk_full, _ = causal_attention_bwd(q, k, v, do)
    qz, kz, vz, dz = (ocp.partition(x, cp) for x in (q, k, v, do))
    dk_z = np.zeros(kz.shape)
    for r in range(cp):
        o_r, _, _ = ocp.cp_forward_rank(q, k, v, cp, r)
        delta = np.transpose(np.sum(dz[r] * o_r, axis=-1), (0, 2, 1))
        for i in range(cp):
            mode, src = ocp.step_schedule(i, r, cp)
            _, lse_i, row0 = ocp.step_attention(qz[r], kz[src], vz[src], mode)
            lse_wrong = np.full((b, hq, s // cp), np.inf)
            lse_wrong[:, :, row0:row0 + lse_i.shape[2]] = lse_i
            _, dk, _ = ocp.step_attention_bwd(qz[r], kz[src], vz[src], dz[r], lse_wrong, delta,
                                              mode)
            dk_z[src] += dk
    assert np.abs(ocp.unpartition(dk_z, s) - dk_full).max() > 1e-3
