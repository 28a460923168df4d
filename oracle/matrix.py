"""The oracle's attention definition in matrix form, for large inputs.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may call this.  The GPU product never
imports it.

It computes exactly what ``attention.c`` computes (the plain definition of
softmax attention over a visible key prefix; "Megatron-LM 篇", §3.1-§3.3:
the blockwise results are corrected until they equal the unblocked
attention, and §3.2: each rank's O is its slice of the non-CP O), written
as the textbook matrix formula instead of one row at a time:

    S = scale * Q K^T              (library matmul, fp64)
    S[i, j] = -inf  for j >= kend[i]                    (the prefix mask)
    m_i = max_j S[i, j],  E = exp(S - m),  s_i = sum_j E[i, j]
    L_i = m_i + ln s_i,   O = (E V) / s                 (natural log)

with the contiguous GQA grouping (query head h reads KV head h / (hq/hkv),
"Megatron 面试题（一）" M014).  A row with kend = 0 has L = -inf and O = 0,
as in the C core.

The rows are independent, so they are taken in consecutive runs that
bound the size of S in memory; each run multiplies only the keys its rows
can see (up to the run's largest kend).  That bounds memory and skips keys
every row of the run masks; it does not reorder any row's arithmetic
beyond the library's own order of summation inside a matmul.

``attention_rows_bwd_matrix`` is the derivative of the same O for a loss
whose gradient with respect to O is dO, again the textbook formulas in
matrix form (the C core's ``oracle_attention_bwd`` does it row by row):

    P = exp(S - L)  (the softmax weights),  O = P V,  D_i = sum_t dO[i,t] O[i,t]
    dP = dO V^T,  dS = P * (dP - D),  dQ = scale * dS K,
    dK = scale * dS^T Q,  dV = P^T dO

summed over the query heads of a KV head's group for dK and dV.

Why a second form: the row-at-a-time C core streams every visible key of
every row from memory and runs at about 1-2 GFLOP/s per host core; the
parity tests over every row of the full-size workloads need 1e12-1e13
FLOP, which this form (host BLAS, all cores) does in seconds to a minute.
Pins: ``tests/test_oracle_matrix.py`` ties both to the C core, to torch's
fp64 scaled_dot_product_attention (and its autograd gradients) and to
closed forms.
"""
import math

import numpy as np
import torch


def _t64(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


def _row_runs(kend, G, max_elems):
    """Consecutive runs of query rows whose score matrix (rows x G heads x
    the run's largest visible-key count) fits max_elems; a run holds at
    least one row."""
    nq = len(kend)
    runs, i0 = [], 0
    while i0 < nq:
        kmax, i1 = max(int(kend[i0]), 1), i0 + 1
        while i1 < nq:
            grown = max(kmax, int(kend[i1]))
            if (i1 + 1 - i0) * G * grown > max_elems:
                break
            kmax, i1 = grown, i1 + 1
        runs.append((i0, i1))
        i0 = i1
    return runs


def _check(q, k, v, kend):
    b, nq, hq, d = q.shape
    bk, nk, hkv, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d or hq % hkv != 0:
        raise ValueError("q/k/v shapes disagree")
    kend = np.asarray(kend, dtype=np.int64)
    if kend.shape != (nq,) or (kend < 0).any() or (kend > nk).any():
        raise ValueError("kend must hold one count in [0, nk] per query row")
    return kend


def attention_rows_matrix(q, k, v, kend, scale=None, max_elems=1 << 22):
    """Softmax attention of each query row over its visible key prefix.

    q: [b, nq, hq, d]; k, v: [b, nk, hkv, d]; kend: [nq] visible key counts
    (row i sees keys 0 .. kend[i]-1).  Returns (O [b, nq, hq, d], L [b, hq,
    nq]) as fp64 numpy arrays.  max_elems bounds the score matrix of one run
    of rows (rows x keys x heads of a group).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b, nq, hq, d = q.shape
    hkv = k.shape[2]
    kend = _check(q, k, v, kend)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    G = hq // hkv
    o = np.zeros((b, nq, hq, d), np.float64)
    lse = np.full((b, hq, nq), -np.inf, np.float64)
    kend_t = torch.from_numpy(kend)
    runs = _row_runs(kend, G, max_elems)
    for n in range(b):
        for g in range(hkv):
            kt = _t64(k[n, :, g, :].T)           # [d, nk]
            vg = _t64(v[n, :, g, :])             # [nk, d]
            for i0, i1 in runs:
                kk = int(kend[i0:i1].max())
                if kk == 0:
                    continue                     # every row of the run sees nothing
                r = i1 - i0
                qg = _t64(q[n, i0:i1, g * G:(g + 1) * G, :]).reshape(r * G, d)
                s = qg @ kt[:, :kk]              # [r*G, kk], row (i, head) i-major
                s.mul_(scale)
                hidden = torch.arange(kk)[None, :] >= kend_t[i0:i1].repeat_interleave(G)[:, None]
                s.masked_fill_(hidden, -math.inf)
                m = s.max(dim=1).values
                seen = torch.isfinite(m)
                m_safe = torch.where(seen, m, torch.zeros_like(m))
                e = s.sub_(m_safe[:, None]).exp_()   # in place: S becomes exp(S - m)
                tot = e.sum(dim=1)
                out = (e @ vg[:kk]) / torch.where(seen, tot, torch.ones_like(tot))[:, None]
                out[~seen] = 0.0
                l = torch.where(seen, m + torch.log(tot), torch.full_like(m, -math.inf))
                o[n, i0:i1, g * G:(g + 1) * G, :] = out.reshape(r, G, d).numpy()
                lse[n, g * G:(g + 1) * G, i0:i1] = l.reshape(r, G).T.numpy()
    return o, lse


def attention_at_positions(q_rows, k, v, positions, scale=None, max_elems=1 << 22):
    """Causal attention of query rows that sit at global positions
    ``positions`` of a sequence whose keys/values are k, v: row p sees keys
    0 .. p (diagonal included).  q_rows: [b, len(positions), hq, d]."""
    positions = np.asarray(positions, dtype=np.int64)
    return attention_rows_matrix(q_rows, k, v, positions + 1, scale, max_elems)


def attention_rows_bwd_matrix(q, k, v, dout, kend, scale=None, max_elems=1 << 22):
    """Gradients (dQ, dK, dV) of ``attention_rows_matrix``'s O for a loss
    whose gradient with respect to O is ``dout``.

    q, dout: [b, nq, hq, d]; k, v: [b, nk, hkv, d]; kend: [nq].  Returns fp64
    numpy arrays shaped like q, k, v.  dK and dV of a KV head sum the
    contributions of every query head of its group; a row that sees no key
    contributes nothing and gets dQ = 0.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    b, nq, hq, d = q.shape
    hkv = k.shape[2]
    kend = _check(q, k, v, kend)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    G = hq // hkv
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(v.shape, np.float64)
    kend_t = torch.from_numpy(kend)
    runs = _row_runs(kend, G, max_elems)
    for n in range(b):
        for g in range(hkv):
            kg = _t64(k[n, :, g, :])             # [nk, d]
            vg = _t64(v[n, :, g, :])
            dkg = torch.zeros_like(kg)
            dvg = torch.zeros_like(vg)
            for i0, i1 in runs:
                kk = int(kend[i0:i1].max())
                if kk == 0:
                    continue
                r = i1 - i0
                qg = _t64(q[n, i0:i1, g * G:(g + 1) * G, :]).reshape(r * G, d)
                dog = _t64(dout[n, i0:i1, g * G:(g + 1) * G, :]).reshape(r * G, d)
                s = (qg @ kg[:kk].T).mul_(scale)  # [r*G, kk], row (i, head) i-major
                hidden = torch.arange(kk)[None, :] >= kend_t[i0:i1].repeat_interleave(G)[:, None]
                s.masked_fill_(hidden, -math.inf)
                m = s.max(dim=1).values
                seen = torch.isfinite(m)
                m_safe = torch.where(seen, m, torch.zeros_like(m))
                p = s.sub_(m_safe[:, None]).exp_()   # unseen rows: all zeros
                tot = p.sum(dim=1)
                p.div_(torch.where(seen, tot, torch.ones_like(tot))[:, None])
                o = p @ vg[:kk]
                delta = (dog * o).sum(dim=1)
                ds = p * ((dog @ vg[:kk].T) - delta[:, None])
                dq[n, i0:i1, g * G:(g + 1) * G, :] = (scale * (ds @ kg[:kk])).reshape(r, G, d).numpy()
                dkg[:kk] += scale * (ds.T @ qg)
                dvg[:kk] += p.T @ dog
            dk[n, :, g, :] = dkg.numpy()
            dv[n, :, g, :] = dvg.numpy()
    return dq, dk, dv
