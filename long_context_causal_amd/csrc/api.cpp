// C ABI of cpattn: argument validation, the step schedule, workspace
// layout and the launch sequence of one rank's forward share.  See
// include/cpattn.h for the contract of every entry point.
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "cpattn.h"
#include "internal.h"

namespace cpattn {

StepGeom step_geom(const cpattn_dims &dims, int mode, float scale) {
    StepGeom g;
    const int64_t c = dims.s / (2 * dims.cp);
    g.b = dims.b;
    g.two_c = 2 * c;
    g.hq = dims.hq;
    g.hkv = dims.hkv;
    g.d = dims.d;
    g.causal = mode == CPATTN_CAUSAL;
    g.q_row0 = mode == CPATTN_Q_SECOND_HALF ? c : 0;
    g.nq = mode == CPATTN_Q_SECOND_HALF ? c : 2 * c;
    g.nk = mode == CPATTN_KV_FIRST_HALF ? c : 2 * c;
    g.scale = scale > 0.0f ? scale : (float)(1.0 / sqrt((double)dims.d));
    g.scale_log2 = (float)((double)g.scale * 1.4426950408889634);
    return g;
}

}  // namespace cpattn

namespace {

using cpattn::StepGeom;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Grids are 32-bit: a launch of more workgroups than this is refused.
bool fits_grid(int64_t blocks) { return blocks >= 0 && blocks <= (int64_t)INT32_MAX; }

// Shape checks shared by the device entry points.
int check_dims(const cpattn_dims *dims) {
    if (dims == nullptr) return CPATTN_EINVAL;
    if (dims->b < 1 || dims->s < 1 || dims->hq < 1 || dims->hkv < 1 || dims->cp < 1)
        return CPATTN_ESHAPE;
    if (dims->s % (2 * (int64_t)dims->cp) != 0) return CPATTN_ESHAPE;
    if (dims->hq % dims->hkv != 0) return CPATTN_ESHAPE;
    if (dims->d != 64 && dims->d != 128) return CPATTN_ESHAPE;
    // row indices inside the kernels are 32-bit
    if (dims->s / dims->cp > INT32_MAX / 2) return CPATTN_ESHAPE;
    if (dims->b * dims->s > (int64_t)1 << 40) return CPATTN_ESHAPE;
    // element offsets of every tensor fit comfortably in 64 bits
    int64_t elems;
    if (__builtin_mul_overflow(dims->b * dims->s, (int64_t)dims->hq * dims->d, &elems) ||
        elems > (int64_t)1 << 56)
        return CPATTN_ESHAPE;
    return CPATTN_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? CPATTN_OK : CPATTN_EHIP; }

// The packed samples of a batch element as kernel arguments (vl == NULL: one
// sample of s rows).  ESHAPE unless the offsets run from 0 to s in positive
// steps that are multiples of 2cp; EINVAL for a NULL offset array.
int make_table(int64_t s, int cp, const cpattn_varlen *vl, cpattn::SeqTable &t) {
    memset(&t, 0, sizeof(t));
    if (s / cp > INT32_MAX) return CPATTN_ESHAPE;
    if (vl == nullptr) {
        t.nseq = 1;
        t.lcu[1] = (int32_t)(s / cp);
        return CPATTN_OK;
    }
    if (vl->cu_seqlens == nullptr) return CPATTN_EINVAL;
    if (vl->nseq < 1 || vl->nseq > CPATTN_MAX_SEQS) return CPATTN_ESHAPE;
    const int64_t *cu = vl->cu_seqlens;
    if (cu[0] != 0 || cu[vl->nseq] != s) return CPATTN_ESHAPE;
    t.nseq = vl->nseq;
    for (int i = 0; i < vl->nseq; ++i) {
        const int64_t len = cu[i + 1] - cu[i];
        if (len <= 0 || len % (2 * (int64_t)cp) != 0) return CPATTN_ESHAPE;
        t.lcu[i + 1] = (int32_t)(cu[i + 1] / cp);
    }
    return CPATTN_OK;
}

int64_t step_rows(const cpattn_dims &d, int mode) {
    const int64_t c = d.s / (2 * d.cp);
    return mode == CPATTN_Q_SECOND_HALF ? c : 2 * c;
}

// Bytes of one step's partial (O then LSE), each rounded up to 256 bytes.
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t partial_o_bytes(const cpattn_dims &d, int64_t rows) {
    return round256((size_t)d.b * rows * d.hq * d.d * sizeof(float));
}
size_t partial_l_bytes(const cpattn_dims &d, int64_t rows) {
    return round256((size_t)d.b * d.hq * rows * sizeof(float));
}

// The partials of rank's steps inside ws, in step order: each step's O,
// then its L, each region rounded up to 256 bytes.  next() yields them one
// at a time (no host allocation, so the forward path allocates nothing).
struct PartialCursor {
    const cpattn_dims &d;
    int rank, step = 0;
    char *at;
    PartialCursor(const cpattn_dims &dims, int r, void *ws) : d(dims), rank(r), at((char *)ws) {}
    cpattn_partial next(int *mode_out = nullptr, int *src_out = nullptr) {
        int mode, src;
        cpattn_step_mode(step++, rank, d.cp, &mode, &src);
        const int64_t rows = step_rows(d, mode);
        cpattn_partial p;
        p.o = (float *)at;
        at += partial_o_bytes(d, rows);
        p.lse = (float *)at;
        at += partial_l_bytes(d, rows);
        p.row0 = mode == CPATTN_Q_SECOND_HALF ? d.s / (2 * d.cp) : 0;
        p.rows = rows;
        if (mode_out) *mode_out = mode;
        if (src_out) *src_out = src;
        return p;
    }
};

// Bytes of the running fp32 result (O, then L) a merge of more than
// CPATTN_MERGE_PASS partials carries between passes.
size_t running_bytes(const cpattn_dims &d) {
    const int64_t two_c = d.s / d.cp;
    return partial_o_bytes(d, two_c) + partial_l_bytes(d, two_c);
}

// One pass of the merge over n <= CPATTN_MERGE_PASS validated partials:
// the first pass starts from nothing, later ones fold in the running fp32
// result run_o / run_l; every pass but the last writes the running result
// (run_o / run_l may be o_out / lse_out when the output is fp32 with an L).
int merge_pass(const cpattn_dims &d, int n, const cpattn_partial *p, bool first, bool last,
               int out_dtype, void *o_out, float *lse_out, float *run_o, float *run_l,
               hipStream_t stream) {
    cpattn::MergeArgs a;
    a.b = d.b;
    a.two_c = d.s / d.cp;
    a.hq = d.hq;
    a.d = d.d;
    a.n = n;
    a.parts = p;
    a.run_o = first ? nullptr : run_o;
    a.run_l = first ? nullptr : run_l;
    a.out_dtype = last ? out_dtype : CPATTN_F32;
    a.o_out = last ? o_out : (void *)run_o;
    a.lse_out = last ? lse_out : run_l;
    return status_of(cpattn::launch_merge(a, stream));
}
}  // namespace

extern "C" {

const char *cpattn_status_str(int status) {
    switch (status) {
        case CPATTN_OK: return "CPATTN_OK";
        case CPATTN_EINVAL: return "CPATTN_EINVAL: invalid argument";
        case CPATTN_ESHAPE: return "CPATTN_ESHAPE: unsupported shape";
        case CPATTN_EDTYPE: return "CPATTN_EDTYPE: unsupported dtype";
        case CPATTN_EALIGN: return "CPATTN_EALIGN: pointer not 16-byte aligned";
        case CPATTN_ENOSPACE: return "CPATTN_ENOSPACE: workspace too small";
        case CPATTN_EHIP: return "CPATTN_EHIP: HIP launch error";
        default: return "CPATTN_UNKNOWN";
    }
}

int cpattn_step_mode(int step, int rank, int cp, int *mode, int *src) {
    if (mode == nullptr || src == nullptr) return CPATTN_EINVAL;
    if (cp < 1 || rank < 0 || rank >= cp || step < 0 || step >= cp) return CPATTN_EINVAL;
    *src = ((rank - step) % cp + cp) % cp;
    if (step == 0)
        *mode = CPATTN_CAUSAL;
    else if (step <= rank)
        *mode = CPATTN_KV_FIRST_HALF;
    else
        *mode = CPATTN_Q_SECOND_HALF;
    return CPATTN_OK;
}

int cpattn_partition_positions(int64_t s, int cp, int rank, int32_t *pos) {
    if (pos == nullptr || cp < 1 || rank < 0 || rank >= cp) return CPATTN_EINVAL;
    if (s < 1 || s % (2 * (int64_t)cp) != 0) return CPATTN_ESHAPE;
    const int64_t c = s / (2 * (int64_t)cp);
    if (2 * c > INT32_MAX || s > INT32_MAX) return CPATTN_ESHAPE;
    const int64_t big = 2 * (int64_t)cp - 1 - rank;
    for (int64_t j = 0; j < c; ++j) pos[j] = (int32_t)(rank * c + j);
    for (int64_t j = 0; j < c; ++j) pos[c + j] = (int32_t)(big * c + j);
    return CPATTN_OK;
}

int cpattn_partition_varlen(const cpattn_dims *dims, int dtype, int h, const cpattn_varlen *vl,
                            const void *x, void *xz, int32_t *pos_dev, const cpattn_rope *rope,
                            void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (x == nullptr || xz == nullptr) return CPATTN_EINVAL;
    if (h < 1 || h > (1 << 20)) return CPATTN_ESHAPE;
    if (!aligned16(x) || !aligned16(xz) || (pos_dev && ((uintptr_t)pos_dev & 3u)))
        return CPATTN_EALIGN;
    if (rope != nullptr && !(rope->theta > 0.0)) return CPATTN_EINVAL;
    if (dims->s > INT32_MAX) return CPATTN_ESHAPE;
    cpattn::SeqTable t;
    st = make_table(dims->s, dims->cp, vl, t);
    if (st) return st;
    return status_of(cpattn::launch_partition(*dims, dtype, h, t, x, xz, pos_dev, rope,
                                              (hipStream_t)stream));
}

int cpattn_partition(const cpattn_dims *dims, int dtype, int h, const void *x, void *xz,
                     int32_t *pos_dev, const cpattn_rope *rope, void *stream) {
    return cpattn_partition_varlen(dims, dtype, h, nullptr, x, xz, pos_dev, rope, stream);
}

int cpattn_partition_positions_varlen(int64_t s, int cp, int rank, const cpattn_varlen *vl,
                                      int32_t *pos) {
    if (pos == nullptr || cp < 1 || rank < 0 || rank >= cp) return CPATTN_EINVAL;
    if (s < 1 || s % (2 * (int64_t)cp) != 0 || s > INT32_MAX) return CPATTN_ESHAPE;
    cpattn::SeqTable t;
    const int st = make_table(s, cp, vl, t);
    if (st) return st;
    for (int i = 0; i < t.nseq; ++i) {
        const int64_t l0 = t.lcu[i], c = (t.lcu[i + 1] - l0) / 2;
        const int64_t big = 2 * (int64_t)cp - 1 - rank;
        for (int64_t j = 0; j < c; ++j) pos[l0 + j] = (int32_t)(rank * c + j);
        for (int64_t j = 0; j < c; ++j) pos[l0 + c + j] = (int32_t)(big * c + j);
    }
    return CPATTN_OK;
}

int cpattn_step_fwd(const cpattn_dims *dims, int dtype, float scale, int mode,
                    const void *q_r, const void *k_src, const void *v_src, float *o,
                    float *lse, void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (mode != CPATTN_CAUSAL && mode != CPATTN_KV_FIRST_HALF && mode != CPATTN_Q_SECOND_HALF)
        return CPATTN_EINVAL;
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (!q_r || !k_src || !v_src || !o || !lse) return CPATTN_EINVAL;
    if (!aligned16(q_r) || !aligned16(k_src) || !aligned16(v_src) || !aligned16(o) ||
        ((uintptr_t)lse & 3u))
        return CPATTN_EALIGN;
    if (!(scale == scale) || isinf(scale)) return CPATTN_EINVAL;
    const StepGeom g = cpattn::step_geom(*dims, mode, scale);
    // bf16: 256-row query tiles; fp32: 64-row tiles
    if (!fits_grid((g.nq + 63) / 64 * g.hq * g.b)) return CPATTN_ESHAPE;
    hipError_t e = dtype == CPATTN_BF16
                       ? cpattn::launch_step_bf16(g, q_r, k_src, v_src, o, lse, (hipStream_t)stream)
                       : cpattn::launch_step_f32(g, q_r, k_src, v_src, o, lse, (hipStream_t)stream);
    return status_of(e);
}

int cpattn_merge(const cpattn_dims *dims, int n, const cpattn_partial *p, int out_dtype,
                 void *o_out, float *lse_out, void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (p == nullptr || o_out == nullptr) return CPATTN_EINVAL;
    if (n < 1) return CPATTN_ESHAPE;
    if (out_dtype != CPATTN_F32 && out_dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    // more partials than one pass takes: the running result lives in the
    // outputs, so they must be fp32 O and a real L
    if (n > CPATTN_MERGE_PASS && (out_dtype != CPATTN_F32 || lse_out == nullptr))
        return CPATTN_ESHAPE;
    const int64_t two_c = dims->s / dims->cp;
    for (int i = 0; i < n; ++i) {
        if (p[i].o == nullptr || p[i].lse == nullptr) return CPATTN_EINVAL;
        if (p[i].row0 < 0 || p[i].rows < 1 || p[i].row0 + p[i].rows > two_c) return CPATTN_ESHAPE;
        if (!aligned16(p[i].o) || ((uintptr_t)p[i].lse & 3u)) return CPATTN_EALIGN;
    }
    if (!aligned16(o_out) || (lse_out && ((uintptr_t)lse_out & 3u))) return CPATTN_EALIGN;
    if (!fits_grid(dims->b * two_c)) return CPATTN_ESHAPE;
    for (int p0 = 0; p0 < n; p0 += CPATTN_MERGE_PASS) {
        const int np = n - p0 < CPATTN_MERGE_PASS ? n - p0 : CPATTN_MERGE_PASS;
        st = merge_pass(*dims, np, p + p0, p0 == 0, p0 + np == n, out_dtype, o_out, lse_out,
                        (float *)o_out, lse_out, (hipStream_t)stream);
        if (st) return st;
    }
    return CPATTN_OK;
}

size_t cpattn_forward_workspace(const cpattn_dims *dims, int rank) {
    if (check_dims(dims) != CPATTN_OK || rank < 0 || rank >= dims->cp) return 0;
    size_t total = 0;
    for (int i = 0; i < dims->cp; ++i) {
        int mode, src;
        cpattn_step_mode(i, rank, dims->cp, &mode, &src);
        const int64_t rows = step_rows(*dims, mode);
        total += partial_o_bytes(*dims, rows) + partial_l_bytes(*dims, rows);
    }
    if (dims->cp > CPATTN_MERGE_PASS) total += running_bytes(*dims);
    return total;
}

int cpattn_forward_partials(const cpattn_dims *dims, int rank, void *ws, size_t ws_bytes,
                            cpattn_partial *parts) {
    const int st = check_dims(dims);
    if (st) return st;
    if (rank < 0 || rank >= dims->cp || ws == nullptr || parts == nullptr) return CPATTN_EINVAL;
    if (((uintptr_t)ws & 255u) != 0) return CPATTN_EALIGN;
    if (ws_bytes < cpattn_forward_workspace(dims, rank)) return CPATTN_ENOSPACE;
    PartialCursor cur(*dims, rank, ws);
    for (int i = 0; i < dims->cp; ++i) parts[i] = cur.next();
    return CPATTN_OK;
}

int cpattn_forward_steps(const cpattn_dims *dims, int dtype, float scale, int rank,
                         const void *qz, const void *kz, const void *vz, void *ws,
                         size_t ws_bytes, void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (rank < 0 || rank >= dims->cp) return CPATTN_EINVAL;
    if (!qz || !kz || !vz || !ws) return CPATTN_EINVAL;
    if (((uintptr_t)ws & 255u) != 0) return CPATTN_EALIGN;
    if (dtype != CPATTN_F32 && dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (!aligned16(qz) || !aligned16(kz) || !aligned16(vz)) return CPATTN_EALIGN;
    if (!(scale == scale) || isinf(scale)) return CPATTN_EINVAL;
    if (ws_bytes < cpattn_forward_workspace(dims, rank)) return CPATTN_ENOSPACE;

    const size_t es = dtype == CPATTN_BF16 ? 2 : 4;
    const int64_t two_c = dims->s / dims->cp;
    const size_t q_block = (size_t)dims->b * two_c * dims->hq * dims->d * es;
    const size_t kv_block = (size_t)dims->b * two_c * dims->hkv * dims->d * es;
    const char *q_r = (const char *)qz + rank * q_block;
    const int cp = dims->cp;
    constexpr int G = cpattn::STEPS_PER_GRID;
    // 256-row query tiles of every step of a grid, all heads and batches
    if (!fits_grid((two_c + 255) / 256 * dims->hq * dims->b * (cp < G ? cp : G)))
        return CPATTN_ESHAPE;
    // the steps in grids of up to G (fp32: one launch each), their
    // descriptors on the stack
    PartialCursor cur(*dims, rank, ws);
    for (int i0 = 0; i0 < cp; i0 += G) {
        const int n = cp - i0 < G ? cp - i0 : G;
        StepGeom geo[G];
        const void *ks[G], *vs[G];
        float *os[G], *ls[G];
        for (int j = 0; j < n; ++j) {
            int mode, src;
            const cpattn_partial part = cur.next(&mode, &src);
            // ring hand-off: step i0 + j reads rank src's partitioned K/V block
            ks[j] = (const char *)kz + src * kv_block;
            vs[j] = (const char *)vz + src * kv_block;
            os[j] = (float *)part.o;
            ls[j] = (float *)part.lse;
            geo[j] = cpattn::step_geom(*dims, mode, scale);
            if (dtype == CPATTN_F32) {
                st = cpattn_step_fwd(dims, dtype, scale, mode, q_r, ks[j], vs[j], os[j], ls[j],
                                     stream);
                if (st) return st;
            }
        }
        if (dtype == CPATTN_BF16) {
            st = status_of(cpattn::launch_steps_bf16(n, geo, q_r, ks, vs, os, ls,
                                                     (hipStream_t)stream));
            if (st) return st;
        }
    }
    return CPATTN_OK;
}

int cpattn_forward(const cpattn_dims *dims, int dtype, float scale, int rank, const void *qz,
                   const void *kz, const void *vz, void *ws, size_t ws_bytes, int out_dtype,
                   void *o_out, float *lse_out, void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (rank < 0 || rank >= dims->cp) return CPATTN_EINVAL;
    if (!o_out) return CPATTN_EINVAL;
    if (out_dtype != CPATTN_F32 && out_dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (!aligned16(o_out) || (lse_out && ((uintptr_t)lse_out & 3u))) return CPATTN_EALIGN;
    if (!fits_grid(dims->b * (dims->s / dims->cp))) return CPATTN_ESHAPE;
    st = cpattn_forward_steps(dims, dtype, scale, rank, qz, kz, vz, ws, ws_bytes, stream);
    if (st) return st;
    // the merge in passes of CPATTN_MERGE_PASS partials; with more than one
    // pass the running result lives in the fp32 region after the partials
    // (cpattn_forward_workspace counts it)
    PartialCursor cur(*dims, rank, ws);
    const int cp = dims->cp;
    float *run_o = nullptr, *run_l = nullptr;
    if (cp > CPATTN_MERGE_PASS) {
        PartialCursor end(*dims, rank, ws);
        for (int i = 0; i < cp; ++i) end.next();
        run_o = (float *)end.at;
        run_l = (float *)(end.at + partial_o_bytes(*dims, dims->s / cp));
    }
    for (int p0 = 0; p0 < cp; p0 += CPATTN_MERGE_PASS) {
        const int np = cp - p0 < CPATTN_MERGE_PASS ? cp - p0 : CPATTN_MERGE_PASS;
        cpattn_partial parts[CPATTN_MERGE_PASS];
        for (int j = 0; j < np; ++j) parts[j] = cur.next();
        st = merge_pass(*dims, np, parts, p0 == 0, p0 + np == cp, out_dtype, o_out, lse_out,
                        run_o, run_l, (hipStream_t)stream);
        if (st) return st;
    }
    return CPATTN_OK;
}

int cpattn_forward_fused_varlen(const cpattn_dims *dims, int dtype, float scale, int rank,
                                const cpattn_varlen *vl, const void *qz, const void *kz,
                                const void *vz, int out_dtype, void *o_out, float *lse_out,
                                void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    cpattn::SeqTable t;
    st = make_table(dims->s, dims->cp, vl, t);
    if (st) return st;
    // query tiles of 256 rows, sample by sample (the grid is 32-bit)
    if (!fits_grid(((dims->s / dims->cp) / 256 + t.nseq) * dims->hq * dims->b))
        return CPATTN_ESHAPE;
    if (rank < 0 || rank >= dims->cp) return CPATTN_EINVAL;
    if (!qz || !kz || !vz || !o_out) return CPATTN_EINVAL;
    if (!(scale == scale) || isinf(scale)) return CPATTN_EINVAL;
    if (dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (out_dtype != CPATTN_F32 && out_dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (!aligned16(qz) || !aligned16(kz) || !aligned16(vz) || !aligned16(o_out) ||
        (lse_out && ((uintptr_t)lse_out & 3u)))
        return CPATTN_EALIGN;
    const StepGeom g = cpattn::step_geom(*dims, CPATTN_CAUSAL, scale);
    cpattn::FusedGeom f;
    f.b = dims->b;
    f.two_c = g.two_c;
    f.hq = dims->hq;
    f.hkv = dims->hkv;
    f.d = dims->d;
    f.rank = rank;
    f.cp = dims->cp;
    f.scale_log2 = g.scale_log2;
    f.tab = t;
    const hipError_t e = cpattn::launch_fused_bf16(f, qz, kz, vz, o_out,
                                                   out_dtype == CPATTN_BF16, lse_out,
                                                   (hipStream_t)stream);
    return e == hipSuccess ? CPATTN_OK : CPATTN_EHIP;
}

int cpattn_forward_fused(const cpattn_dims *dims, int dtype, float scale, int rank,
                         const void *qz, const void *kz, const void *vz, int out_dtype,
                         void *o_out, float *lse_out, void *stream) {
    return cpattn_forward_fused_varlen(dims, dtype, scale, rank, nullptr, qz, kz, vz, out_dtype,
                                       o_out, lse_out, stream);
}

// Grid bounds of the backward launches (query and key tiles of 128 rows,
// per sample): ESHAPE before anything is launched if one would not fit.
static int check_bwd_grids(const cpattn_dims &d, int nseq) {
    const int64_t two_c = d.s / d.cp;
    const int64_t tiles = two_c / 128 + nseq;
    const int64_t steps_per_grid = d.cp < 32 ? d.cp : 32;
    if (!fits_grid(tiles * d.hq * d.b)) return CPATTN_ESHAPE;                    // dq
    if (!fits_grid(tiles * d.hkv * d.b * (d.hq / d.hkv))) return CPATTN_ESHAPE;  // dK/dV, head splits
    if (!fits_grid(tiles * d.hkv * d.b * steps_per_grid)) return CPATTN_ESHAPE;  // dK/dV, all steps
    if (!fits_grid(d.b * two_c * d.hq / 256 + 1)) return CPATTN_ESHAPE;           // delta
    if (!fits_grid(d.cp * d.b * two_c * d.hkv * d.d / 1024 + 1)) return CPATTN_ESHAPE;  // zero fill
    return CPATTN_OK;
}

int cpattn_bwd_delta(const cpattn_dims *dims, const float *o_r, const void *do_r,
                     float *delta_r, void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (!o_r || !do_r || !delta_r) return CPATTN_EINVAL;
    if (!aligned16(o_r) || !aligned16(do_r) || ((uintptr_t)delta_r & 3u)) return CPATTN_EALIGN;
    const int64_t two_c = dims->s / dims->cp;
    if (!fits_grid(dims->b * two_c * dims->hq / 256 + 1)) return CPATTN_ESHAPE;
    return status_of(cpattn::launch_bwd_delta(dims->b, two_c, dims->hq, dims->d, o_r, do_r,
                                              delta_r, (hipStream_t)stream));
}

int cpattn_step_bwd(const cpattn_dims *dims, int dtype, float scale, int mode, const void *q_r,
                    const void *k_src, const void *v_src, const void *do_r, const float *lse_r,
                    const float *delta_r, float *dq_r, float *dk_src, float *dv_src,
                    void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    if (mode < CPATTN_CAUSAL || mode > CPATTN_Q_SECOND_HALF) return CPATTN_EINVAL;
    if (!q_r || !k_src || !v_src || !do_r || !lse_r || !delta_r || !dq_r || !dk_src || !dv_src)
        return CPATTN_EINVAL;
    if (!(scale == scale) || isinf(scale)) return CPATTN_EINVAL;
    if (dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (!aligned16(q_r) || !aligned16(k_src) || !aligned16(v_src) || !aligned16(do_r) ||
        !aligned16(dq_r) || !aligned16(dk_src) || !aligned16(dv_src) ||
        ((uintptr_t)lse_r & 3u) || ((uintptr_t)delta_r & 3u))
        return CPATTN_EALIGN;
    st = check_bwd_grids(*dims, 1);
    if (st) return st;
    const StepGeom g = cpattn::step_geom(*dims, mode, scale);
    cpattn::SeqTable t;
    st = make_table(dims->s, dims->cp, nullptr, t);
    if (st) return st;
    return status_of(cpattn::launch_step_bwd_bf16(g, t, mode, q_r, k_src, v_src, do_r, lse_r,
                                                  delta_r, dq_r, dk_src, dv_src,
                                                  (hipStream_t)stream));
}

int cpattn_backward_varlen(const cpattn_dims *dims, int dtype, float scale, int rank,
                           const cpattn_varlen *vl, const void *qz, const void *kz,
                           const void *vz, const float *o_r, const void *do_r,
                           const float *lse_r, float *delta_ws, float *dq_r, float *dkz,
                           float *dvz, void *stream) {
    int st = check_dims(dims);
    if (st) return st;
    cpattn::SeqTable t;
    st = make_table(dims->s, dims->cp, vl, t);
    if (st) return st;
    if (rank < 0 || rank >= dims->cp) return CPATTN_EINVAL;
    if (!qz || !kz || !vz || !o_r || !do_r || !lse_r || !delta_ws || !dq_r || !dkz || !dvz)
        return CPATTN_EINVAL;
    if (!(scale == scale) || isinf(scale)) return CPATTN_EINVAL;
    if (dtype != CPATTN_BF16) return CPATTN_EDTYPE;
    if (!aligned16(qz) || !aligned16(kz) || !aligned16(vz) || !aligned16(o_r) ||
        !aligned16(do_r) || !aligned16(dq_r) || !aligned16(dkz) || !aligned16(dvz) ||
        ((uintptr_t)lse_r & 3u) || ((uintptr_t)delta_ws & 3u))
        return CPATTN_EALIGN;
    st = check_bwd_grids(*dims, t.nseq);
    if (st) return st;
    const hipStream_t s = (hipStream_t)stream;
    const int64_t two_c = dims->s / dims->cp;
    const int64_t q_elems = dims->b * two_c * dims->hq * dims->d;
    const int64_t kv_elems = dims->b * two_c * dims->hkv * dims->d;
    const char *q_r = (const char *)qz + rank * q_elems * 2;
    const int cp = dims->cp;
    std::vector<StepGeom> geo(cp);
    std::vector<int> modes(cp);
    std::vector<const void *> ks(cp), vs(cp);
    std::vector<float *> dks(cp), dvs(cp);
    for (int i = 0; i < cp; ++i) {
        int mode, src;
        cpattn_step_mode(i, rank, cp, &mode, &src);
        // ring hand-off: step i reads rank src's K/V and adds to src's dK/dV
        const char *k_src = (const char *)kz + src * kv_elems * 2;
        const char *v_src = (const char *)vz + src * kv_elems * 2;
        geo[i] = cpattn::step_geom(*dims, mode, scale);
        modes[i] = mode;
        ks[i] = k_src;
        vs[i] = v_src;
        dks[i] = dkz + src * kv_elems;
        dvs[i] = dvz + src * kv_elems;
    }
    // the workspace: -L/scale and -D of the rank's rows, the terms the
    // grids start S and dP from
    float *nl = delta_ws, *nd = delta_ws + dims->b * dims->hq * two_c;
    const float inv_scale = (float)(1.0 / (double)geo[0].scale);
    hipError_t e = cpattn::launch_fill_zero(dkz, kv_elems * dims->cp, s);
    if (e == hipSuccess) e = cpattn::launch_fill_zero(dvz, kv_elems * dims->cp, s);
    if (e == hipSuccess)
        e = cpattn::launch_bwd_prep(dims->b, two_c, dims->hq, dims->d, o_r, do_r, lse_r,
                                    inv_scale, nl, nd, s);
    if (e != hipSuccess) return CPATTN_EHIP;
    // every step's dq in one grid (a workgroup streams all steps' keys for
    // its query rows and writes dq once), then every step's dK/dV in one
    // grid (each step owns its source block's contribution)
    e = cpattn::launch_bwd_dq_share_bf16(geo[0], t, rank, cp, q_r, kz, vz, do_r, nl, nd, dq_r,
                                         s);
    if (e != hipSuccess) return CPATTN_EHIP;
    e = cpattn::launch_bwd_dkdv_steps_bf16(cp, geo.data(), t, modes.data(), q_r, ks.data(),
                                           vs.data(), do_r, nl, nd, dks.data(), dvs.data(), s);
    if (e != hipSuccess) return CPATTN_EHIP;
    return CPATTN_OK;
}

int cpattn_backward(const cpattn_dims *dims, int dtype, float scale, int rank, const void *qz,
                    const void *kz, const void *vz, const float *o_r, const void *do_r,
                    const float *lse_r, float *delta_ws, float *dq_r, float *dkz, float *dvz,
                    void *stream) {
    return cpattn_backward_varlen(dims, dtype, scale, rank, nullptr, qz, kz, vz, o_r, do_r,
                                  lse_r, delta_ws, dq_r, dkz, dvz, stream);
}

}  // extern "C"
