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
// One workgroup per (batch, local row): it first computes the hq x n
// weights exp(L_p - L) into LDS, then streams the hq*d outputs of the row
// with 16-byte reads of each covering partial (consecutive lanes on
// consecutive addresses) and one 16-byte (fp32) or 8-byte (bf16) store.
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 256;
constexpr int MAX_LDS_WEIGHTS = 8192;   // hq * n must fit (32 KiB)

struct DevPartial {
    const float *o;
    const float *lse;
    int64_t row0, rows;
};

template <int NP>
struct PartList {
    DevPartial p[NP];
};

template <int NP, bool BF16_OUT>
__global__ void __launch_bounds__(NT) merge_rows(PartList<NP> pl, int n_parts, int64_t b,
                                                 int64_t two_c, int hq, int d, void *o_out,
                                                 float *lse_out) {
    __shared__ float w[MAX_LDS_WEIGHTS];   // [hq][n_parts] weights
    __shared__ int cover[NP];              // indices of the covering partials
    __shared__ int n_cover;
    const int64_t rowid = blockIdx.x;      // n * two_c + j
    const int64_t j = rowid % two_c;
    const int64_t n = rowid / two_c;

    if (threadIdx.x == 0) {
        int cnt = 0;
        for (int q = 0; q < n_parts; ++q)
            if (j >= pl.p[q].row0 && j < pl.p[q].row0 + pl.p[q].rows) cover[cnt++] = q;
        n_cover = cnt;
    }
    __syncthreads();
    const int nc = n_cover;
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float LN2 = 0.69314718055994531f;

    for (int h = threadIdx.x; h < hq; h += NT) {
        float mx = -INFINITY;
        for (int c = 0; c < nc; ++c) {
            const DevPartial &pp = pl.p[cover[c]];
            const float l = pp.lse[(n * hq + h) * pp.rows + (j - pp.row0)];
            mx = fmaxf(mx, l);
        }
        float total = -INFINITY;
        if (mx != -INFINITY) {
            float ssum = 0.0f;
            for (int c = 0; c < nc; ++c) {
                const DevPartial &pp = pl.p[cover[c]];
                const float l = pp.lse[(n * hq + h) * pp.rows + (j - pp.row0)];
                ssum += __builtin_amdgcn_exp2f((l - mx) * LOG2E);
            }
            total = mx + __builtin_amdgcn_logf(ssum) * LN2;
        }
        for (int c = 0; c < nc; ++c) {
            const DevPartial &pp = pl.p[cover[c]];
            const float l = pp.lse[(n * hq + h) * pp.rows + (j - pp.row0)];
            w[h * nc + c] = (total == -INFINITY) ? 0.0f
                                                 : __builtin_amdgcn_exp2f((l - total) * LOG2E);
        }
        if (lse_out != nullptr) lse_out[(n * hq + h) * two_c + j] = total;
    }
    __syncthreads();

    const int nvec = hq * d / 4;
    const int vec_per_head = d / 4;
    for (int i = threadIdx.x; i < nvec; i += NT) {
        const int h = i / vec_per_head;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int c = 0; c < nc; ++c) {
            const DevPartial &pp = pl.p[cover[c]];
            const f32x4 *src =
                (const f32x4 *)(pp.o + (n * pp.rows + (j - pp.row0)) * (int64_t)hq * d) + i;
            acc += w[h * nc + c] * (*src);
        }
        if (BF16_OUT) {
            u32x2 packed;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                __bf16 lo = (__bf16)acc[2 * e], hi = (__bf16)acc[2 * e + 1];
                packed[e] = (unsigned)__builtin_bit_cast(uint16_t, lo) |
                            ((unsigned)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            ((u32x2 *)o_out)[rowid * nvec + i] = packed;
        } else {
            ((f32x4 *)o_out)[rowid * nvec + i] = acc;
        }
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
                           pl, a.n, a.b, a.two_c, a.hq, a.d, a.o_out, a.lse_out);
    else
        hipLaunchKernelGGL((merge_rows<NP, false>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                           pl, a.n, a.b, a.two_c, a.hq, a.d, a.o_out, a.lse_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream) {
    if (a.n <= 4) return launch_np<4>(a, stream);
    if (a.n <= 16) return launch_np<16>(a, stream);
    if (a.n <= 64) return launch_np<64>(a, stream);
    return hipErrorInvalidValue;   // api.cpp rejects larger merges first
}

}  // namespace cpattn
