"""Packed variable-length sequences under the CP scheme: the oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module (see the package
docstring).

What the pages say.  "Megatron 面试题（一）", M016, in its follow-up on why a
CP rank that holds only local tokens must still know their positions: the
rotary phase of a token is set by its position in its full sequence, and
when samples are packed the positions must be reset (or mapped) at each
sample boundary.  "Megatron-LM 篇" 3.5: the split can be made as fine as
the FA2 loop counts (cp as large as Tr/Tc), so a chunk may be shorter than
one kernel tile.

Readings taken here (the pages leave these open; the GPU path takes the
same ones):
* packed samples are independent causal sequences: a row sees the rows of
  its own sample up to itself, nothing of the other samples;
* each sample's length is a multiple of 2*cp and the sample is split by the
  zigzag rule on its own: rank r holds chunk r, then chunk 2cp-1-r, of every
  sample, samples in packing order.  Rank r's local rows of sample i are
  then local rows [cu[i]/cp, cu[i+1]/cp);
* a row's position (for RoPE) is its index within its sample.

Everything is fp64 and reuses the already pinned single-sequence oracle
(``attention``, ``cp``) sample by sample; the packing layout is the only
new arithmetic.
"""
import numpy as np

from .attention import attention_rows, attention_rows_bwd
from . import cp as ocp


def check_cu(cu, s, cp):
    """The packing offsets as int64: cu[0] = 0, cu[-1] = s, every sample a
    positive multiple of 2*cp long."""
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != s:
        raise ValueError("cu_seqlens must run from 0 to s")
    lens = np.diff(cu)
    if (lens <= 0).any() or (lens % (2 * cp)).any():
        raise ValueError("every sample must be a positive multiple of 2*cp long")
    return cu


def sample_positions(cu):
    """Position of every packed row within its own sample (reset at each
    sample start)."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.concatenate([np.arange(cu[i + 1] - cu[i]) for i in range(cu.size - 1)])


def packed_causal_attention(q, k, v, cu, scale=None, rope_theta=None, nthreads=0):
    """The definition: each sample's causal attention on its own rows.

    q [b, s, hq, d], k/v [b, s, hkv, d].  With ``rope_theta`` Q and K are
    rotated at the in-sample positions first.  Returns (O [b, s, hq, d],
    L [b, hq, s]) in fp64, L the natural-log LSE.
    """
    s = q.shape[1]
    cu = np.asarray(cu, dtype=np.int64)
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros((q.shape[0], q.shape[2], s))
    for i in range(cu.size - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        qi, ki, vi = q[:, a:e], k[:, a:e], v[:, a:e]
        if rope_theta is not None:
            pos = np.arange(e - a)
            qi, ki = ocp.rope(qi, pos, rope_theta), ocp.rope(ki, pos, rope_theta)
        o[:, a:e], lse[:, :, a:e] = attention_rows(qi, ki, vi, np.arange(1, e - a + 1),
                                                   scale, nthreads)
    return o, lse


def local_rows(cu, cp, rank):
    """Packed row index of each of rank ``rank``'s s/cp local rows."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.concatenate([cu[i] + ocp.zigzag_positions(cu[i + 1] - cu[i], cp, rank)
                           for i in range(cu.size - 1)])


def local_positions(cu, cp, rank):
    """In-sample position of each of rank ``rank``'s local rows (what RoPE
    uses on that rank)."""
    cu = np.asarray(cu, dtype=np.int64)
    return np.concatenate([ocp.zigzag_positions(cu[i + 1] - cu[i], cp, rank)
                           for i in range(cu.size - 1)])


def partition(x, cu, cp):
    """[b, s, H, d] -> [cp, b, s/cp, H, d]: every rank's rows, gathered."""
    return np.stack([x[:, local_rows(cu, cp, r)] for r in range(cp)])


def unpartition(xz, cu):
    """Inverse of ``partition`` along the row axis."""
    cp = xz.shape[0]
    s = int(np.asarray(cu)[-1])
    out = np.empty((xz.shape[1], s) + xz.shape[3:], dtype=xz.dtype)
    for r in range(cp):
        out[:, local_rows(cu, cp, r)] = xz[r]
    return out


def cp_forward_rank(q, k, v, cu, cp, rank, scale=None, rope_theta=None, nthreads=0):
    """One rank's CP forward share of a packed batch.

    Sample by sample, the single-sequence CP emulation (split, RoPE at the
    in-sample positions, the cp ring steps, L correction and merge); the
    rank's per-sample results are laid out in its local row order.
    Returns (O [b, s/cp, hq, d], L [b, hq, s/cp]).
    """
    cu = np.asarray(cu, dtype=np.int64)
    os_, ls_ = [], []
    for i in range(cu.size - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        o_i, l_i, _ = ocp.cp_forward_rank(q[:, a:e], k[:, a:e], v[:, a:e], cp, rank, scale,
                                          rope_theta, nthreads=nthreads)
        os_.append(o_i)
        ls_.append(l_i)
    return np.concatenate(os_, axis=1), np.concatenate(ls_, axis=2)


def packed_causal_attention_bwd(q, k, v, dout, cu, scale=None, nthreads=0):
    """Gradients of the packed definition (no RoPE: with respect to the
    attention inputs): each sample's causal-attention gradients on its own
    rows.  Returns (dq [b, s, hq, d], dk, dv [b, s, hkv, d])."""
    cu = np.asarray(cu, dtype=np.int64)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for i in range(cu.size - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        dq[:, a:e], dk[:, a:e], dv[:, a:e] = attention_rows_bwd(
            q[:, a:e], k[:, a:e], v[:, a:e], dout[:, a:e], np.arange(1, e - a + 1), scale,
            nthreads)
    return dq, dk, dv


def cp_backward_rank(q, k, v, dout, cu, cp, rank, scale=None, nthreads=0):
    """One rank's CP backward share of a packed batch (no RoPE).

    Sample by sample, the single-sequence CP backward (the rank's final L and
    D of that sample, the cp ring steps); the rank's dq and its contributions
    to every rank's dK/dV are laid out in local row order.  Returns
    (dq_r [b, s/cp, hq, d], dkz, dvz [cp, b, s/cp, hkv, d]).
    """
    cu = np.asarray(cu, dtype=np.int64)
    dqs, dks, dvs = [], [], []
    for i in range(cu.size - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        dq_i, dk_i, dv_i = ocp.cp_backward_rank(q[:, a:e], k[:, a:e], v[:, a:e], dout[:, a:e],
                                                cp, rank, scale, nthreads=nthreads)
        dqs.append(dq_i)
        dks.append(dk_i)
        dvs.append(dv_i)
    return (np.concatenate(dqs, axis=1), np.concatenate(dks, axis=2),
            np.concatenate(dvs, axis=2))
