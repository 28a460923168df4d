"""Context-parallel emulation of causal attention, step by step, in fp64.

TEST INFRASTRUCTURE: see the package docstring for who may call this.

Follows "Megatron-LM 篇" §3.2 (the five steps of a rank's CP forward) and
§3.4 (load balancing and the three step modes), with the pairing of
"超大规模集群下大语言模型训练实操指南", section "CP 与其他技术结合" (every
device computes one big and one small attention).  The numbered steps of
§3.2 map to functions here:

  1. split the data by cp_size          -> ``zigzag_positions``, ``partition``
  2. blockwise attention of one step    -> ``step_attention``
  3. ring exchange of KV with neighbours -> ``step_schedule`` (which rank's
                                           KV a rank holds at step i)
  4. correct the intermediate L          -> ``correct_lse``
  5. correct and merge O at the end      -> ``merge_outputs``

``cp_forward_rank`` runs them in that order for one rank.  RoPE with
global positions ("Megatron 面试题（一）", M016) is ``rope``.

Readings where the pages leave a step open (each one is pinned by a test):
* rank r holds chunk r followed by chunk 2cp-1-r (chunks of c = s/(2cp)
  tokens); this local order keeps global order, so a causal mask on local
  indices equals the global causal mask;
* at step i rank r holds the KV of rank (r - i) mod cp - the only ring
  direction under which the three modes never touch a masked pair;
* step 0 is the causal step even though "i <= rank" also holds for it;
* the mask is lower-triangular with the diagonal included;
* partial O_i are normalised within their step; L is a natural-log LSE.
"""
import math

import numpy as np

from .attention import attention_rows

CAUSAL = 0
KV_FIRST_HALF = 1
Q_SECOND_HALF = 2
MODE_NAMES = {CAUSAL: "causal", KV_FIRST_HALF: "kv_first_half",
              Q_SECOND_HALF: "q_second_half"}


def chunk_len(s, cp):
    if s % (2 * cp) != 0:
        raise ValueError("sequence length must split into 2*cp equal chunks")
    return s // (2 * cp)


# --- step 1: split the data ---------------------------------------------

def zigzag_positions(s, cp, rank):
    """Global token positions of rank ``rank``'s 2c local rows.

    The sequence is cut into 2*cp chunks of c tokens.  Rank r keeps chunk r
    (a "small" causal workload) and chunk 2cp-1-r (a "big" one), in that
    order ("Megatron-LM 篇" §3.4: rank_0 trades half of its data with
    rank_n-1, rank_1 with rank_n-2, ...).
    """
    c = chunk_len(s, cp)
    if not 0 <= rank < cp:
        raise ValueError("rank out of range")
    small = np.arange(rank * c, (rank + 1) * c, dtype=np.int64)
    big_chunk = 2 * cp - 1 - rank
    big = np.arange(big_chunk * c, (big_chunk + 1) * c, dtype=np.int64)
    return np.concatenate([small, big])


def partition(x, cp):
    """[b, s, H, d] -> [cp, b, 2c, H, d]: every rank's rows, gathered."""
    s = x.shape[1]
    return np.stack([x[:, zigzag_positions(s, cp, r)] for r in range(cp)])


def unpartition(xz, s):
    """Inverse of ``partition`` along the row axis (rows scattered back)."""
    cp = xz.shape[0]
    out = np.empty((xz.shape[1], s) + xz.shape[3:], dtype=xz.dtype)
    for r in range(cp):
        out[:, zigzag_positions(s, cp, r)] = xz[r]
    return out


# --- step 3: ring schedule -------------------------------------------------

def step_schedule(step, rank, cp):
    """(mode, src): the step's attention mode and whose KV the rank holds.

    "Megatron-LM 篇" §3.4: the first step is causal; while the step index
    is at most the rank, the second half of the KV is dropped and no mask
    is applied; after that the first half of Q is dropped, no mask.
    The KV held at step i is the one that travelled i hops along the ring:
    rank (rank - i) mod cp.
    """
    if not 0 <= rank < cp or not 0 <= step < cp:
        raise ValueError("step/rank out of range")
    src = (rank - step) % cp
    if step == 0:
        return CAUSAL, src
    if step <= rank:
        return KV_FIRST_HALF, src
    return Q_SECOND_HALF, src


# --- step 2: one blockwise attention --------------------------------------

def step_attention(q_r, k_src, v_src, mode, scale=None, nthreads=0):
    """One step's blockwise attention on local blocks of 2c rows.

    q_r [b, 2c, hq, d]; k_src, v_src [b, 2c, hkv, d].
    Returns (O_i, L_i, row0): O_i [b, rows, hq, d] normalised within the
    step, L_i [b, hq, rows], covering local query rows row0 .. row0+rows-1.
      causal        : all 2c rows vs all 2c keys, local row j sees keys <= j
      kv_first_half : all 2c rows vs keys 0..c-1, no mask
      q_second_half : rows c..2c-1 vs all 2c keys, no mask
    """
    two_c = q_r.shape[1]
    c = two_c // 2
    if mode == CAUSAL:
        o, lse = attention_rows(q_r, k_src, v_src,
                                np.arange(1, two_c + 1), scale, nthreads)
        return o, lse, 0
    if mode == KV_FIRST_HALF:
        o, lse = attention_rows(q_r, k_src[:, :c], v_src[:, :c],
                                np.full(two_c, c), scale, nthreads)
        return o, lse, 0
    if mode == Q_SECOND_HALF:
        o, lse = attention_rows(q_r[:, c:], k_src, v_src,
                                np.full(c, two_c), scale, nthreads)
        return o, lse, c
    raise ValueError("unknown mode")


# --- steps 4 and 5: corrections -------------------------------------------

def correct_lse(lse_acc, lse_step):
    """Per-step correction of the running L: log(exp(L_acc) + exp(L_i)).

    The two-stage max-then-sum form of "Megatron 面试题（一）" M019:
    subtract the larger value before exponentiating.  -inf means "no keys
    yet" and is the identity.
    """
    m = np.maximum(lse_acc, lse_step)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    total = np.exp(lse_acc - m_safe) + np.exp(lse_step - m_safe)
    with np.errstate(divide="ignore"):
        return np.where(np.isfinite(m), m_safe + np.log(total), m)


def merge_outputs(partials, rows_total):
    """Final correction and merge of the step outputs.

    partials: list of (O_i [b, rows, hq, d], L_i [b, hq, rows], row0).
    The running L is corrected after each step (step 4 of §3.2); after the
    last step every O_i is rescaled by exp(L_i - L) and summed (step 5).
    Returns (O [b, rows_total, hq, d], L [b, hq, rows_total]).
    """
    b, _, hq, d = partials[0][0].shape
    lse = np.full((b, hq, rows_total), -np.inf)
    for _, lse_i, row0 in partials:
        rows = lse_i.shape[2]
        lse[:, :, row0:row0 + rows] = correct_lse(
            lse[:, :, row0:row0 + rows], lse_i)
    o = np.zeros((b, rows_total, hq, d))
    for o_i, lse_i, row0 in partials:
        rows = lse_i.shape[2]
        # a partial with no visible key (L_i = -inf) is an empty sum: weight 0,
        # also on rows where every partial is empty (then O = 0, L = -inf)
        with np.errstate(invalid="ignore"):
            w = np.where(np.isneginf(lse_i), 0.0,
                         np.exp(lse_i - lse[:, :, row0:row0 + rows]))   # [b, hq, rows]
        o[:, row0:row0 + rows] += np.transpose(w, (0, 2, 1))[..., None] * o_i
    return o, lse


# --- RoPE at global positions ---------------------------------------------

def rope(x, positions, theta=10000.0):
    """Rotary position embedding of x [b, n, H, d] at ``positions`` [n].

    RoPE rotates Q and K inside attention, and a CP rank must rotate its
    rows at their global positions ("Megatron 面试题（一）" M016).  The pages
    fix no variant; this is the rotate-half form: for t < d/2 the pair
    (x_t, x_{t+d/2}) is turned by the angle pos * theta**(-2t/d).
    """
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[None, :, None, :]
    sin = np.sin(ang)[None, :, None, :]
    x = np.asarray(x, dtype=np.float64)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# --- a whole rank -----------------------------------------------------------

def cp_forward_rank(q, k, v, cp, rank, scale=None, rope_theta=None,
                    ring=step_schedule, nthreads=0):
    """One rank's CP forward, the five steps of "Megatron-LM 篇" §3.2.

    q [b, s, hq, d], k/v [b, s, hkv, d] unpartitioned.  With ``rope_theta``
    Q and K are rotated after the split, at each row's global position.
    Returns (O [b, 2c, hq, d], L [b, hq, 2c], positions [2c]).
    """
    s = q.shape[1]
    qz, kz, vz = partition(q, cp), partition(k, cp), partition(v, cp)
    if rope_theta is not None:
        for r in range(cp):
            pos = zigzag_positions(s, cp, r)
            qz[r] = rope(qz[r], pos, rope_theta)
            kz[r] = rope(kz[r], pos, rope_theta)
    partials = []
    for i in range(cp):
        mode, src = ring(i, rank, cp)
        partials.append(step_attention(qz[rank], kz[src], vz[src], mode,
                                       scale, nthreads))
    o, lse = merge_outputs(partials, 2 * chunk_len(s, cp))
    return o, lse, zigzag_positions(s, cp, rank)


def causal_flops(b, s, hq, d, cp, rank=None):
    """Causal-effective FLOPs (4*d per visible (q, k) pair).

    rank=None: the whole causal triangle; otherwise one rank's share,
    c(2c+1) + (cp-1)*2c^2 pairs per (batch, head) - the same for every rank.
    """
    if rank is None:
        pairs = s * (s + 1) // 2
    else:
        c = chunk_len(s, cp)
        pairs = c * (2 * c + 1) + (cp - 1) * 2 * c * c
    return 4 * d * b * hq * pairs


def default_scale(d):
    return 1.0 / math.sqrt(d)


# --- backward ---------------------------------------------------------------
# The pages treat the backward only through the communication context
# parallelism adds to it ("超大规模集群…", "CP 与其他技术结合": an all-gather
# of K/V and a reduce-scatter of the K/V gradients).  Each ring step of the
# forward has a backward counterpart on the same blocks; it uses the rank's
# final (merged) L and D = sum_t dO O, so that its softmax weights are the
# final ones, and returns the step's contribution to the source rank's dK
# and dV (what the reduce-scatter sums on that rank).

def step_attention_bwd(q_r, k_src, v_src, dout_r, lse_r, delta_r, mode, scale=None):
    """One step's part of a rank's backward, on local blocks of 2c rows.

    q_r, dout_r [b, 2c, hq, d]; k_src, v_src [b, 2c, hkv, d]; lse_r, delta_r
    [b, hq, 2c] the rank's final L and D.  Rows and keys as in
    ``step_attention``.  Returns (dq [b, 2c, hq, d], zero outside the mode's
    rows; dk, dv [b, 2c, hkv, d], the step's share of the source rank's
    gradients).  For each head h of group g and row i of the mode:
        P_j = exp(scale q_i.k_j - L_i),  dS_j = P_j (dO_i.v_j - D_i),
        dq_i += scale sum_j dS_j k_j,  dk_j += scale dS_j q_i,  dv_j += P_j dO_i.
    """
    q_r, k_src, v_src, dout_r = (np.asarray(x, np.float64) for x in (q_r, k_src, v_src, dout_r))
    b, two_c, hq, d = q_r.shape
    hkv = k_src.shape[2]
    group = hq // hkv
    c = two_c // 2
    if scale is None:
        scale = default_scale(d)
    if mode == CAUSAL:
        rows, nkeys = np.arange(two_c), two_c
    elif mode == KV_FIRST_HALF:
        rows, nkeys = np.arange(two_c), c
    elif mode == Q_SECOND_HALF:
        rows, nkeys = np.arange(c, two_c), two_c
    else:
        raise ValueError("unknown mode")
    visible = np.ones((len(rows), nkeys), bool)
    if mode == CAUSAL:
        visible = np.arange(nkeys)[None, :] <= rows[:, None]
    dq = np.zeros_like(q_r)
    dk = np.zeros((b, two_c, hkv, d))
    dv = np.zeros((b, two_c, hkv, d))
    for n in range(b):
        for h in range(hq):
            g = h // group
            qh = q_r[n, rows, h]                      # [rows, d]
            kh = k_src[n, :nkeys, g]                  # [keys, d]
            vh = v_src[n, :nkeys, g]
            doh = dout_r[n, rows, h]
            z = scale * (qh @ kh.T)
            p = np.where(visible, np.exp(z - lse_r[n, h, rows][:, None]), 0.0)
            dp = doh @ vh.T
            ds = p * (dp - delta_r[n, h, rows][:, None])
            dq[n, rows, h] += scale * (ds @ kh)
            dk[n, :nkeys, g] += scale * (ds.T @ qh)
            dv[n, :nkeys, g] += p.T @ doh
    return dq, dk, dv


def cp_backward_rank(q, k, v, dout, cp, rank, scale=None, ring=step_schedule, nthreads=0):
    """One rank's CP backward (no RoPE).

    q, dout [b, s, hq, d]; k, v [b, s, hkv, d] unpartitioned.  The rank's O
    and L come from ``cp_forward_rank``; D = sum_t dO O per row and head.
    Returns (dq_r [b, 2c, hq, d], dkz, dvz [cp, b, 2c, hkv, d]): the rank's
    query gradient and its contribution to every rank's K/V gradient.
    """
    s = q.shape[1]
    qz, kz, vz, dz = (partition(x, cp) for x in (q, k, v, dout))
    o_r, lse_r, _ = cp_forward_rank(q, k, v, cp, rank, scale, nthreads=nthreads)
    delta_r = np.transpose(np.sum(np.asarray(dz[rank], np.float64) * o_r, axis=-1), (0, 2, 1))
    dq_r = np.zeros(qz[rank].shape)
    dkz = np.zeros(kz.shape)
    dvz = np.zeros(vz.shape)
    for i in range(cp):
        mode, src = ring(i, rank, cp)
        dq, dk, dv = step_attention_bwd(qz[rank], kz[src], vz[src], dz[rank], lse_r, delta_r,
                                        mode, scale)
        dq_r += dq
        dkz[src] += dk
        dvz[src] += dv
    del s
    return dq_r, dkz, dvz
