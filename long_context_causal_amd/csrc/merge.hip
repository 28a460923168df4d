// LSE correction and merge of a rank's step partials.
//
// "Megatron-LM 篇", Context Parallel 3.2 steps 4 and 5: the intermediate L
// of every step is corrected, then the step outputs O_i are rescaled and
// summed.  With the two-stage max-then-sum form of a log-sum-exp
// ("Megatron 面试题（一）" M019), for one row and head over the partials P
// that cover the row:
//     M = max_p L_p,   L = M + ln sum_p exp(L_p - M),   O = sum_p exp(L_p - L) O_p
// Partials that do not cover the row take no part (they are not zeros with
// L = 0).  All arithmetic is fp32 (exp and log through exp2/log2).
//
// One workgroup per (batch, local row).  For each run of heads whose
// weights fit in LDS it first gathers the row's L_p of those heads and
// turns them into the weights exp(L_p - L), then streams those heads'
// outputs: each lane owns eight 16-byte vectors (consecutive lanes on
// consecutive addresses) and, partial by partial, issues their reads
// together before accumulating, so enough reads are in flight to keep HBM
// busy; one 16-byte (fp32) or 8-byte (bf16) store per vector.
//
// A launch takes at most MAX_PASS partials (the descriptors travel in the
// kernel arguments).  Longer merges run in passes: each later pass folds
// the running result (fp32 O and L of the earlier passes, an ordinary
// partial that covers every row) with the next partials.
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) f32x4 gf32x4;   // global memory

constexpr int NT = 256;
constexpr int MAX_LDS_WEIGHTS = 8192;   // heads of one run x covering partials (32 KiB)
constexpr int MAX_PASS = CPATTN_MERGE_PASS;

struct DevPartial {
    const float *o;
    const float *lse;
    int64_t row0, rows;
};

template <int NP>
struct PartList {
    DevPartial p[NP];
};

// run_o / run_l: the running result of earlier passes (fp32 [b, 2c, hq, d]
// and [b, hq, 2c]) or null; they may alias o_out / lse_out (each lane reads
// its own vectors, and a head's L, before it writes them).
template <int NP, bool BF16_OUT>
__global__ void __launch_bounds__(NT) merge_rows(PartList<NP> pl, int n_parts, int64_t b,
                                                 int64_t two_c, int hq, int d,
                                                 const float *run_o, const float *run_l,
                                                 void *o_out, float *lse_out) {
    __shared__ float w[MAX_LDS_WEIGHTS];   // [n_cover][heads of the run]: L_p, then weights
    __shared__ const float *obase[NP + 1]; // covering partial c: its O at (n, row, head 0)
    __shared__ const float *lbase[NP + 1]; // its L at (n, head 0, row)
    __shared__ int lstride[NP + 1];        // its L elements between heads (its rows)
    __shared__ int n_cover;
    const int64_t rowid = blockIdx.x;      // n * two_c + j
    const int64_t j = rowid % two_c;
    const int64_t n = rowid / two_c;

    if (threadIdx.x == 0) {
        int cnt = 0;
        if (run_o != nullptr) {
            obase[0] = run_o + rowid * (int64_t)hq * d;
            lbase[0] = run_l + n * hq * two_c + j;
            lstride[0] = (int)two_c;
            cnt = 1;
        }
        for (int q = 0; q < n_parts; ++q) {
            const DevPartial &pp = pl.p[q];
            if (j >= pp.row0 && j < pp.row0 + pp.rows) {
                obase[cnt] = pp.o + (n * pp.rows + (j - pp.row0)) * (int64_t)hq * d;
                lbase[cnt] = pp.lse + n * hq * pp.rows + (j - pp.row0);
                lstride[cnt] = (int)pp.rows;
                ++cnt;
            }
        }
        n_cover = cnt;
    }
    __syncthreads();
    const int nc = n_cover;
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.69314718055994531f;
    const int vec_per_head = d / 4;                      // 16 or 32
    const int vph_shift = __builtin_ctz(vec_per_head);
    const int64_t nvec_row = (int64_t)hq * vec_per_head;
    auto store = [&](int i, const f32x4 &a) {
        if (BF16_OUT) {
            u32x2 packed;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                __bf16 lo = (__bf16)a[2 * e], hi = (__bf16)a[2 * e + 1];
                packed[e] = (unsigned)__builtin_bit_cast(uint16_t, lo) |
                            ((unsigned)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            ((u32x2 *)o_out)[rowid * nvec_row + i] = packed;
        } else {
            ((f32x4 *)o_out)[rowid * nvec_row + i] = a;
        }
    };

    // heads per run: as many as fit their weights in LDS
    const int hrun = nc == 0 ? hq : min(hq, MAX_LDS_WEIGHTS / nc);
    for (int h0 = 0; h0 < hq; h0 += hrun) {
        const int nh = min(hrun, hq - h0);
        // every (head, partial) L of the run into LDS, eight loads in flight
        // per lane (lanes past the end re-read the last element, so every
        // read is unconditional and all eight issue before the first wait)
        const int ne = nh * nc;
        for (int e0 = 0; e0 < ne; e0 += 8 * NT) {
            float lv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = min(e0 + k * NT + (int)threadIdx.x, ne - 1);
                const int h = e / nc, c = e - h * nc;
                lv[k] = ((const __attribute__((address_space(1))) float *)lbase[c])
                    [(int64_t)(h0 + h) * lstride[c]];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = e0 + k * NT + threadIdx.x;
                if (e < ne) {
                    const int h = e / nc, c = e - h * nc;
                    w[c * nh + h] = lv[k];
                }
            }
        }
        __syncthreads();
        // one lane per head; partial c of head h at w[c * nh + h], so the
        // lanes of a wave read consecutive words
        for (int h = threadIdx.x; h < nh; h += NT) {
            float *wh = w + h;
            float mx = -INFINITY;
            for (int c = 0; c < nc; ++c) mx = fmaxf(mx, wh[c * nh]);
            float total = -INFINITY;
            if (mx != -INFINITY) {
                float ssum = 0.0f;
                for (int c = 0; c < nc; ++c)
                    ssum += __builtin_amdgcn_exp2f((wh[c * nh] - mx) * LOG2E);
                total = mx + __builtin_amdgcn_logf(ssum) * LN2;
            }
            for (int c = 0; c < nc; ++c)
                wh[c * nh] = (total == -INFINITY)
                                 ? 0.0f
                                 : __builtin_amdgcn_exp2f((wh[c * nh] - total) * LOG2E);
            if (lse_out != nullptr) lse_out[(n * hq + h0 + h) * two_c + j] = total;
        }
        __syncthreads();

        // O of the run's heads: each lane owns KV 16-byte vectors; for every
        // covering partial the KV loads are issued together, then
        // accumulated.  Full chunks of KV * NT vectors run unpredicated; the
        // rest one vector at a time.
        constexpr int KV = 8;
        const int v_begin = h0 * vec_per_head;
        const int nvec = nh * vec_per_head;
        const int full = nvec / (KV * NT) * (KV * NT);
        for (int v0 = v_begin; v0 < v_begin + full; v0 += KV * NT) {
            f32x4 acc[KV];
            int hk[KV];   // the vector's head in the run
#pragma unroll
            for (int k = 0; k < KV; ++k) {
                acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                hk[k] = (v0 - v_begin + k * NT + (int)threadIdx.x) >> vph_shift;
            }
            // two partials per round trip: 2 * KV reads in flight per lane
            int c = 0;
            for (; c + 1 < nc; c += 2) {
                const gf32x4 *s0 = (const gf32x4 *)obase[c] + v0 + threadIdx.x;
                const gf32x4 *s1 = (const gf32x4 *)obase[c + 1] + v0 + threadIdx.x;
                f32x4 x0[KV], x1[KV];
#pragma unroll
                for (int k = 0; k < KV; ++k) x0[k] = s0[k * NT];
#pragma unroll
                for (int k = 0; k < KV; ++k) x1[k] = s1[k * NT];
#pragma unroll
                for (int k = 0; k < KV; ++k) {
                    const int wi = c * nh + hk[k];
                    acc[k] += w[wi] * x0[k] + w[wi + nh] * x1[k];
                }
            }
            if (c < nc) {
                const gf32x4 *s0 = (const gf32x4 *)obase[c] + v0 + threadIdx.x;
                f32x4 x0[KV];
#pragma unroll
                for (int k = 0; k < KV; ++k) x0[k] = s0[k * NT];
#pragma unroll
                for (int k = 0; k < KV; ++k) acc[k] += w[c * nh + hk[k]] * x0[k];
            }
#pragma unroll
            for (int k = 0; k < KV; ++k) store(v0 + k * NT + threadIdx.x, acc[k]);
        }
        for (int i = v_begin + full + threadIdx.x; i < v_begin + nvec; i += NT) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            const int hv = (i - v_begin) >> vph_shift;
            for (int c = 0; c < nc; ++c) acc += w[c * nh + hv] * ((const f32x4 *)obase[c])[i];
            store(i, acc);
        }
        __syncthreads();   // the next run overwrites w
    }
}

template <int NP>
hipError_t launch_np(const MergeArgs &a, hipStream_t stream) {
    PartList<NP> pl;
    for (int q = 0; q < NP; ++q) {
        if (q < a.n) {
            pl.p[q].o = a.parts[q].o;
            pl.p[q].lse = a.parts[q].lse;
            pl.p[q].row0 = a.parts[q].row0;
            pl.p[q].rows = a.parts[q].rows;
        } else {
            pl.p[q] = DevPartial{nullptr, nullptr, 0, 0};
        }
    }
    const int64_t blocks = a.b * a.two_c;
    if (a.out_dtype == CPATTN_BF16)
        hipLaunchKernelGGL((merge_rows<NP, true>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                           pl, a.n, a.b, a.two_c, a.hq, a.d, a.run_o, a.run_l, a.o_out,
                           a.lse_out);
    else
        hipLaunchKernelGGL((merge_rows<NP, false>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                           pl, a.n, a.b, a.two_c, a.hq, a.d, a.run_o, a.run_l, a.o_out,
                           a.lse_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream) {
    if (a.n <= 4) return launch_np<4>(a, stream);
    if (a.n <= 16) return launch_np<16>(a, stream);
    if (a.n <= MAX_PASS) return launch_np<MAX_PASS>(a, stream);
    return hipErrorInvalidValue;   // the caller splits longer merges into passes
}

}  // namespace cpattn
