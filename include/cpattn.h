/*
 * cpattn - context-parallel blockwise causal attention, forward and
 * backward, on one AMD Instinct MI355X (gfx950).
 *
 * The method ("Megatron-LM 篇", Context Parallel, sections 3.1-3.5; with
 * "超大规模集群下大语言模型训练实操指南", section "CP 与其他技术结合"):
 * the sequence is split over cp ranks; each rank computes FA2-style
 * blockwise attention of its queries against one rank's keys and values per
 * ring step, producing a partial output O_i and its log-sum-exp L_i; the L
 * are corrected step by step and the O are rescaled and merged at the end,
 * so each rank's result equals its slice of ordinary causal attention.
 * On one GPU the ring exchange becomes a pointer hand-off: at step i rank r
 * reads the partitioned K/V block of rank (r - i) mod cp.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes (C order, innermost last):
 *   q  [b, s, hq, d]        k, v  [b, s, hkv, d]          (unpartitioned)
 *   xz [cp, b, 2c, h, d]    partitioned: rank r's rows at xz + r*b*2c*h*d
 *   c = s / (2*cp) is the chunk length, 2c the rows a rank holds.
 *   O_i, O  float or bf16 [b, rows, hq, d];  L_i, L  float [b, hq, rows]
 * GQA: query head h reads KV head h / (hq/hkv) (contiguous groups).
 * Softmax scale: 'scale' <= 0 selects 1/sqrt(d).
 * L is the natural-log log-sum-exp of the scaled scores of a row.
 *
 * Ownership: the caller allocates and frees every device buffer; the
 * library allocates no device memory and keeps no state between calls
 * (except the scratch array of cpattn_forward_noalloc, described there).
 * Device pointers must be 16-byte aligned and must not overlap unless a
 * function says otherwise.
 *
 * Streams: 'stream' is a hipStream_t (NULL = the default stream).  Device
 * functions enqueue their kernels on it and return without synchronising;
 * a device fault surfaces at the caller's next synchronisation.
 *
 * Errors: arguments are validated before anything is launched; a rejected
 * call launches nothing and returns a nonzero status (cpattn_status_str
 * names it).  CPATTN_EHIP reports a failed kernel launch.
 *
 * Thread safety: every function is reentrant; calls on different streams
 * may run concurrently.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem dimensions. */
typedef struct cpattn_dims {
    int64_t b;    /* batch size, >= 1                                        */
    int64_t s;    /* full sequence length, a multiple of 2*cp                 */
    int32_t hq;   /* query heads, a multiple of hkv                           */
    int32_t hkv;  /* key/value heads (GQA groups)                              */
    int32_t d;    /* head dimension: 64 or 128                                */
    int32_t cp;   /* context-parallel size (ranks emulated), >= 1: any cp with
                     s % (2*cp) == 0, down to chunks of one row (c = 1)       */
} cpattn_dims;

/* Element types of Q, K, V (and of the merged output). */
enum { CPATTN_F32 = 0, CPATTN_BF16 = 1 };

/* Step modes ("Megatron-LM 篇" section 3.4). */
enum {
    CPATTN_CAUSAL = 0,        /* all 2c rows vs all 2c keys, key j <= row i  */
    CPATTN_KV_FIRST_HALF = 1, /* all 2c rows vs keys 0..c-1, no mask          */
    CPATTN_Q_SECOND_HALF = 2  /* rows c..2c-1 vs all 2c keys, no mask         */
};

/* Status codes. */
enum {
    CPATTN_OK = 0,
    CPATTN_EINVAL = 1,   /* null pointer, bad enum, rank/step out of range   */
    CPATTN_ESHAPE = 2,   /* s % 2cp, hq % hkv, unsupported d, b or s < 1, or
                            a launch that would need more than 2^31-1
                            workgroups                                       */
    CPATTN_EDTYPE = 3,   /* dtype not supported by this entry point          */
    CPATTN_EALIGN = 4,   /* a device pointer is not 16-byte aligned          */
    CPATTN_ENOSPACE = 5, /* workspace too small                              */
    CPATTN_EHIP = 6      /* the HIP runtime reported a launch error          */
};

/* Rotary position embedding applied during the split ("Megatron 面试题（一）",
 * M016: RoPE rotates Q and K inside attention, and a CP rank must use the
 * global position of each row).  Rotate-half form: for t < d/2 the pair
 * (x[t], x[t + d/2]) is turned by pos * theta^(-2t/d) radians. */
typedef struct cpattn_rope {
    double theta;        /* base, > 0 (10000 for the usual RoPE)              */
} cpattn_rope;

/* One partial result of a step, as consumed by cpattn_merge. */
typedef struct cpattn_partial {
    const float *o;      /* [b, rows, hq, d] fp32, normalised within its step */
    const float *lse;    /* [b, hq, rows] fp32 natural-log LSE                */
    int64_t row0;        /* first local row this partial covers              */
    int64_t rows;        /* number of local rows it covers                   */
} cpattn_partial;

/* Packed variable-length samples ("Megatron 面试题（一）", M016 follow-up:
 * positions are reset at each packed sample's boundary).  Every batch
 * element packs the same nseq samples along its sequence axis: sample i is
 * rows [cu_seqlens[i], cu_seqlens[i+1]) of the s rows, an independent
 * causal sequence (no row sees another sample) whose positions restart at
 * 0.  Each sample is split by the zigzag rule on its own: rank r holds its
 * chunk r, then its chunk 2cp-1-r, samples in packing order, so sample i
 * occupies local rows [cu_seqlens[i]/cp, cu_seqlens[i+1]/cp) of every rank.
 * cu_seqlens: caller-owned HOST array of nseq + 1 offsets, cu_seqlens[0] =
 * 0, cu_seqlens[nseq] = s, every sample length a positive multiple of 2*cp
 * (ESHAPE otherwise); 1 <= nseq <= CPATTN_MAX_SEQS.  Read during the call
 * only. */
typedef struct cpattn_varlen {
    int32_t nseq;
    const int64_t *cu_seqlens;
} cpattn_varlen;

#define CPATTN_MAX_SEQS 128

/* Partials one merge pass folds (cpattn_merge). */
#define CPATTN_MERGE_PASS 64

/* Mode and KV source of a step, host only, pure.
 * "Megatron-LM 篇" 3.4: step 0 is causal; steps 1..rank drop the second
 * half of the KV (CPATTN_KV_FIRST_HALF); later steps drop the first half of
 * Q (CPATTN_Q_SECOND_HALF).  3.2 step 3: KV moves one hop along the ring per
 * step, so at step i the rank holds rank (rank - i) mod cp's KV.
 * Writes *mode and *src.  EINVAL if a pointer is NULL or step/rank are not
 * in [0, cp). */
int cpattn_step_mode(int step, int rank, int cp, int *mode, int *src);

/* Global positions of rank 'rank''s 2c local rows, host only, pure.
 * "Megatron-LM 篇" 3.4 and "超大规模集群下大语言模型训练实操指南" "CP 与其他技术
 * 结合": chunk k is paired with chunk 2cp-1-k, rank r holds chunk r then
 * chunk 2cp-1-r: pos[j] = r*c + j for j < c, (2cp-1-r)*c + j - c after.
 * pos: caller-owned host array of 2c int32.  ESHAPE if s % (2cp) != 0 or
 * 2c exceeds INT32_MAX; EINVAL for a NULL pointer or rank out of range. */
int cpattn_partition_positions(int64_t s, int cp, int rank, int32_t *pos);

/* Zigzag split of one tensor ("Megatron-LM 篇" 3.2 step 1), device.
 * x [b, s, h, d] -> xz [cp, b, 2c, h, d] with xz[r, n, j] = x[n, pos_r[j]].
 * dtype: CPATTN_F32 or CPATTN_BF16 (elements are copied bit for bit).
 * pos_dev: optional device array [cp, 2c] int32 receiving every rank's
 * positions (NULL to skip).  rope: optional; when given, each copied row is
 * rotated at its global position (angles in fp64, rotation in fp32, result
 * rounded to the element type).  h is the head count of this tensor (hq for
 * Q, hkv for K and V); dims->hq/hkv are not used here.  x and xz must not
 * overlap. */
int cpattn_partition(const cpattn_dims *dims, int dtype, int h, const void *x,
                     void *xz, int32_t *pos_dev, const cpattn_rope *rope,
                     void *stream);

/* One step's blockwise attention ("Megatron-LM 篇" 3.2 step 2 and 3.4),
 * device.  q_r: rank's partitioned Q block [b, 2c, hq, d]; k_src, v_src:
 * the source rank's partitioned K and V blocks [b, 2c, hkv, d].  All three
 * have element type 'dtype' (CPATTN_BF16: bf16 MFMA with fp32 accumulation;
 * CPATTN_F32: fp32 throughout, the debug path), d = 64 or 128.  mode: CPATTN_CAUSAL,
 * CPATTN_KV_FIRST_HALF or CPATTN_Q_SECOND_HALF.
 * Writes o [b, rows, hq, d] fp32 (normalised within the step) and
 * lse [b, hq, rows] fp32, rows = 2c (first two modes) or c (the last one,
 * holding local rows c..2c-1).  ESHAPE for any other d. */
int cpattn_step_fwd(const cpattn_dims *dims, int dtype, float scale, int mode,
                    const void *q_r, const void *k_src, const void *v_src,
                    float *o, float *lse, void *stream);

/* LSE correction and merge of n partials ("Megatron-LM 篇" 3.2 steps 4 and
 * 5), device.  For each batch n, local row j in [0, 2c) and head h, over the
 * partials that cover j: M = max L_p, L = M + ln sum_p exp(L_p - M),
 * O = sum_p exp(L_p - L) O_p.  A row no partial covers gets L = -inf, O = 0.
 * p: host array of n >= 1 descriptors (device pointers inside), read during
 * the call only; each partial's rows must lie inside [0, 2c) (ESHAPE
 * otherwise).  out_dtype: CPATTN_F32 or CPATTN_BF16 (round to nearest
 * even).  o_out [b, 2c, hq, d]; lse_out [b, hq, 2c] fp32 or NULL.
 * One launch folds up to CPATTN_MERGE_PASS partials; a longer merge runs in
 * passes that carry the running result in o_out and lse_out, so for
 * n > CPATTN_MERGE_PASS out_dtype must be CPATTN_F32 and lse_out non-NULL
 * (ESHAPE otherwise; cpattn_forward has no such limit). */
int cpattn_merge(const cpattn_dims *dims, int n, const cpattn_partial *p,
                 int out_dtype, void *o_out, float *lse_out, void *stream);

/* Bytes of device workspace cpattn_forward needs for 'rank': the fp32
 * partials of all cp steps, plus, when cp > CPATTN_MERGE_PASS, one fp32 O
 * and L of the rank's 2c rows for the running result of the merge passes.
 * Returns 0 on invalid dims or rank. */
size_t cpattn_forward_workspace(const cpattn_dims *dims, int rank);

/* Where cpattn_forward_steps puts each step's partial inside a workspace,
 * host only, pure: parts[i] (i = step, caller-owned host array of cp
 * entries) receives the device addresses of step i's O_i [b, rows, hq, d]
 * and L_i [b, hq, rows] inside ws and the local rows they cover: row0 = 0,
 * rows = 2c for the causal and kv_first_half steps; row0 = c, rows = c
 * for the q_second_half steps (cpattn_step_mode gives the modes).  The
 * descriptors are what cpattn_merge takes.  EINVAL for a NULL pointer or a
 * rank out of range, ESHAPE for bad dims, EALIGN unless ws is 256-byte
 * aligned, ENOSPACE if ws_bytes < cpattn_forward_workspace. */
int cpattn_forward_partials(const cpattn_dims *dims, int rank, void *ws, size_t ws_bytes,
                            cpattn_partial *parts);

/* The cp steps of one rank's forward share ("Megatron-LM 篇" 3.2 step 2,
 * the steps of cpattn_step_mode), device, without the merge: step i reads
 * the source rank's K/V block of the partitioned qz/kz/vz ([cp, b, 2c, h, d]
 * as written by cpattn_partition) and writes its partial O_i and L_i, exactly
 * as cpattn_step_fwd would, into the workspace ws in step order: for each
 * step its O ([b, rows_i, hq, d] fp32), then its L ([b, hq, rows_i] fp32),
 * each starting on a 256-byte boundary (rows_i as for cpattn_step_fwd).
 * CPATTN_BF16 runs all steps as one grid (the steps are independent, so
 * their workgroups overlap one another's loads and stores); CPATTN_F32
 * launches them one by one.  ws: at least cpattn_forward_workspace bytes
 * (ENOSPACE otherwise), 256-byte aligned (EALIGN).  The partials stay in ws
 * for cpattn_merge. */
int cpattn_forward_steps(const cpattn_dims *dims, int dtype, float scale, int rank,
                         const void *qz, const void *kz, const void *vz, void *ws,
                         size_t ws_bytes, void *stream);

/* One rank's whole forward share, device: the cp steps of
 * cpattn_step_mode, each reading the source rank's K/V block of the
 * partitioned qz/kz/vz ([cp, b, 2c, h, d] as written by cpattn_partition),
 * then cpattn_merge into o_out [b, 2c, hq, d] (out_dtype) and lse_out
 * [b, hq, 2c] (may be NULL).  ws: device workspace of at least
 * cpattn_forward_workspace bytes (ENOSPACE otherwise), 256-byte aligned. */
int cpattn_forward(const cpattn_dims *dims, int dtype, float scale, int rank,
                   const void *qz, const void *kz, const void *vz, void *ws,
                   size_t ws_bytes, int out_dtype, void *o_out, float *lse_out,
                   void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc): cpattn_forward
 * without a workspace argument.  The step partials live in a scratch array
 * inside the library, CPATTN_NOALLOC_SCRATCH_BYTES per device, which every
 * GPU the library runs on holds from the library's load until the process
 * ends.  The call allocates nothing; the caller still passes the inputs and
 * outputs, and the stream must belong to the current device.  ENOSPACE if
 * the share's workspace (cpattn_forward_workspace) exceeds the array;
 * otherwise arguments, results and errors as cpattn_forward, bit for bit.
 * Every call on a device shares that device's array and leaves the last
 * call's partials in it: calls that overlap on one device (two streams, or
 * two host threads) race, and the caller must serialise them. */
#define CPATTN_NOALLOC_SCRATCH_BYTES (256u << 20)
int cpattn_forward_noalloc(const cpattn_dims *dims, int dtype, float scale, int rank,
                           const void *qz, const void *kz, const void *vz, int out_dtype,
                           void *o_out, float *lse_out, void *stream);

/* One rank's whole forward share in one launch, device ("超大规模集群…":
 * the rank's big and small attention run concurrently; "Megatron-LM 篇" 3.2
 * step 2 and its per-step LSE correction).  Each query row's online softmax
 * runs on through the key blocks of all cp steps of cpattn_step_mode
 * (kv_first_half halves of ranks r-1..0, q_second_half blocks of ranks
 * cp-1..r+1 for rows c..2c-1, the causal block of rank r), so the per-step
 * correction happens in place: no partials, no merge, no workspace.  The
 * result is the one cpattn_forward gives, up to rounding order.
 * qz, kz, vz: partitioned [cp, b, 2c, h, d] bf16 (CPATTN_BF16 only,
 * EDTYPE otherwise; d = 64 or 128, ESHAPE otherwise).  o_out [b, 2c, hq, d] in
 * out_dtype (CPATTN_F32, or CPATTN_BF16 rounded to nearest even); lse_out
 * [b, hq, 2c] fp32 natural log, or NULL.  Pointers 16-byte aligned (lse_out
 * 4-byte), EALIGN otherwise.  Asynchronous on 'stream'. */
int cpattn_forward_fused(const cpattn_dims *dims, int dtype, float scale, int rank,
                         const void *qz, const void *kz, const void *vz, int out_dtype,
                         void *o_out, float *lse_out, void *stream);

/* Backward, step by step.  The pages name the backward only through the
 * communication context parallelism adds ("超大规模集群…", "CP 与其他技术结合":
 * an all-gather of K/V and a reduce-scatter of their gradients); each ring
 * step of the forward ("Megatron-LM 篇" 3.4: the three modes) has a
 * backward counterpart on the same blocks that uses the rank's FINAL L
 * (the merged lse_out of the forward) and D = sum_t dO O.
 *
 * cpattn_bwd_delta, device: delta_r [b, hq, 2c] fp32 = sum over the head
 * dim of do_r [b, 2c, hq, d] (bf16) times o_r [b, 2c, hq, d] (fp32, the
 * merged forward output).  d = 64 or 128. */
int cpattn_bwd_delta(const cpattn_dims *dims, const float *o_r, const void *do_r,
                     float *delta_r, void *stream);

/* cpattn_step_bwd, device: one step's backward (CPATTN_BF16 only, d = 64 or 128).
 * q_r, do_r [b, 2c, hq, d] bf16; k_src, v_src [b, 2c, hkv, d] bf16 (rank
 * src's blocks); lse_r, delta_r [b, hq, 2c] fp32.  For each row i and head h
 * of the mode and each key j it lets them see, with P = exp(scale q.k - L)
 * and dS = P (dO.v - D):
 *   dq_r [b, 2c, hq, d]  += scale * sum_j dS k_j      (fp32, rows of the mode)
 *   dk_src [b, 2c, hkv, d] += scale * sum dS q_i      (fp32, summed over the
 *   dv_src [b, 2c, hkv, d] += sum P dO_i               group's heads)
 * The three gradient buffers accumulate: the caller zeroes them first. */
int cpattn_step_bwd(const cpattn_dims *dims, int dtype, float scale, int mode,
                    const void *q_r, const void *k_src, const void *v_src,
                    const void *do_r, const float *lse_r, const float *delta_r,
                    float *dq_r, float *dk_src, float *dv_src, void *stream);

/* cpattn_backward, device: one rank's whole backward share.  Zeroes dkz
 * and dvz [cp, b, 2c, hkv, d] (fp32), writes -L/scale and -D (D as in
 * cpattn_bwd_delta) of the rank's rows into delta_ws [2, b, hq, 2c] (the
 * caller's fp32 workspace; the two per-row terms the kernels start the sums
 * of S and dP from), then the cp steps of cpattn_step_mode:
 * dq_r [b, 2c, hq, d] (fp32) is written with the sum over all steps (every
 * row; its previous contents are ignored), and step i adds to rank src's
 * slices of dkz/dvz.  dkz/dvz
 * hold the rank's contributions to every rank's K/V gradient: the inputs
 * of the reduce-scatter that sums them on their owners.  qz, kz, vz:
 * partitioned [cp, b, 2c, h, d] bf16; o_r, lse_r: the rank's merged forward
 * output (fp32) and L; do_r [b, 2c, hq, d] bf16.  No RoPE (gradients are
 * with respect to the rotated Q and K). */
int cpattn_backward(const cpattn_dims *dims, int dtype, float scale, int rank,
                    const void *qz, const void *kz, const void *vz, const float *o_r,
                    const void *do_r, const float *lse_r, float *delta_ws, float *dq_r,
                    float *dkz, float *dvz, void *stream);

/* Packed variable-length forms of the partition and of the fused forward
 * (see cpattn_varlen for the layout).  vl = NULL, or nseq = 1, gives the
 * unpacked call.
 *
 * cpattn_partition_positions_varlen, host, pure: the in-sample positions
 * of rank 'rank''s s/cp local rows into pos (caller-owned host array of
 * s/cp int32).  EINVAL for a NULL pos or offset array or a rank out of
 * range, ESHAPE for bad offsets. */
int cpattn_partition_positions_varlen(int64_t s, int cp, int rank, const cpattn_varlen *vl,
                                      int32_t *pos);

/* cpattn_partition_varlen, device: x [b, s, h, d] -> xz [cp, b, s/cp, h, d],
 * each sample split on its own; pos_dev (optional) [cp, s/cp] receives the
 * in-sample positions; rope (optional) rotates each row at its in-sample
 * position.  Otherwise as cpattn_partition. */
int cpattn_partition_varlen(const cpattn_dims *dims, int dtype, int h, const cpattn_varlen *vl,
                            const void *x, void *xz, int32_t *pos_dev,
                            const cpattn_rope *rope, void *stream);

/* cpattn_forward_fused_varlen, device: rank 'rank''s whole forward share of
 * a packed batch in one launch.  Each sample's rows stream the key blocks
 * of the cp ring steps of that sample only (cpattn_forward_fused on every
 * sample at once).  qz, kz, vz [cp, b, s/cp, h, d] bf16 as written by
 * cpattn_partition_varlen; o_out [b, s/cp, hq, d] (out_dtype); lse_out
 * [b, hq, s/cp] or NULL.  Types, alignment and errors as
 * cpattn_forward_fused. */
int cpattn_forward_fused_varlen(const cpattn_dims *dims, int dtype, float scale, int rank,
                                const cpattn_varlen *vl, const void *qz, const void *kz,
                                const void *vz, int out_dtype, void *o_out, float *lse_out,
                                void *stream);

/* cpattn_backward_varlen, device: cpattn_backward for a packed batch (see
 * cpattn_varlen): every sample's rows take the backward of the cp ring
 * steps of that sample only.  Buffers as cpattn_backward with 2c read as
 * s/cp local rows; o_r and lse_r from cpattn_forward_fused_varlen.  vl =
 * NULL gives cpattn_backward. */
int cpattn_backward_varlen(const cpattn_dims *dims, int dtype, float scale, int rank,
                           const cpattn_varlen *vl, const void *qz, const void *kz,
                           const void *vz, const float *o_r, const void *do_r,
                           const float *lse_r, float *delta_ws, float *dq_r, float *dkz,
                           float *dvz, void *stream);

/* Static name of a status code. */
const char *cpattn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
