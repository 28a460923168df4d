// Blockwise attention of one CP step in fp32 end to end: the debug path.
//
// Same contract as the bf16 kernel ("Megatron-LM 篇", Context Parallel 3.2
// step 2 and 3.4) but every product, exponential and sum is fp32, so the
// result sits within a few fp32 ulps of the exact softmax.  One lane owns
// one query row; keys stream through LDS in tiles of 32 and each tile's
// scores are reduced with a per-tile max (online softmax with a rescale per
// tile).  Scores use expf/logf from the HIP math library.
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

constexpr int ROWS = 64;   // query rows per workgroup (one wave)
constexpr int TK = 32;     // keys per LDS tile

struct Params {
    const float *q, *k, *v;
    float *o, *lse;
    int64_t two_c, q_row0;
    int nq, nk, hq, hkv, group, num_qtiles;
    float scale;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(ROWS) attn_step_f32(Params p) {
    __shared__ float sK[TK * D];
    __shared__ float sV[TK * D];
    const int tid = threadIdx.x;
    int item = blockIdx.x;
    const int qtile = item % p.num_qtiles;
    item /= p.num_qtiles;
    const int head = item % p.hq;
    const int n = item / p.hq;
    const int g = head / p.group;

    const int row = qtile * ROWS + tid;
    const int rowc = min(row, p.nq - 1);
    float qv[D], acc[D];
    const float *qsrc = p.q + ((n * p.two_c + p.q_row0 + rowc) * (int64_t)p.hq + head) * D;
#pragma unroll
    for (int t = 0; t < D; ++t) {
        qv[t] = qsrc[t];
        acc[t] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;

    const int kend = CAUSAL ? min(p.nk, qtile * ROWS + ROWS) : p.nk;
    const float *kbase = p.k + ((int64_t)n * p.two_c * p.hkv + g) * D;
    const float *vbase = p.v + ((int64_t)n * p.two_c * p.hkv + g) * D;
    const int64_t kstride = (int64_t)p.hkv * D;

    for (int key0 = 0; key0 < kend; key0 += TK) {
        __syncthreads();
        for (int i = tid; i < TK * D; i += ROWS) {
            int j = i / D, t = i % D;
            int key = min(key0 + j, p.nk - 1);
            sK[i] = kbase[key * kstride + t];
            sV[i] = vbase[key * kstride + t];
        }
        __syncthreads();
        float z[TK];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            float dot = 0.0f;
#pragma unroll
            for (int t = 0; t < D; ++t) dot = fmaf(qv[t], sK[j * D + t], dot);
            const int key = key0 + j;
            const bool vis = key < p.nk && (!CAUSAL || key <= row);
            z[j] = vis ? dot * p.scale : -INFINITY;
            tmax = fmaxf(tmax, z[j]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;      // nothing visible yet
        const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < D; ++t) acc[t] *= alpha;
#pragma unroll
        for (int j = 0; j < TK; ++j) {
            const float pj = (z[j] == -INFINITY) ? 0.0f : expf(z[j] - m_new);
            l += pj;
#pragma unroll
            for (int t = 0; t < D; ++t) acc[t] = fmaf(pj, sV[j * D + t], acc[t]);
        }
        m = m_new;
    }

    if (row < p.nq) {
        const float inv = 1.0f / l;
        float *dst = p.o + ((n * (int64_t)p.nq + row) * p.hq + head) * D;
#pragma unroll
        for (int t = 0; t < D; ++t) dst[t] = acc[t] * inv;
        p.lse[((int64_t)n * p.hq + head) * p.nq + row] = m + logf(l);
    }
}

template <int D>
hipError_t launch_d(const StepGeom &g, const void *q, const void *k, const void *v,
                    float *o, float *lse, hipStream_t stream) {
    Params p;
    p.q = (const float *)q;
    p.k = (const float *)k;
    p.v = (const float *)v;
    p.o = o;
    p.lse = lse;
    p.two_c = g.two_c;
    p.q_row0 = g.q_row0;
    p.nq = (int)g.nq;
    p.nk = (int)g.nk;
    p.hq = g.hq;
    p.hkv = g.hkv;
    p.group = g.hq / g.hkv;
    p.num_qtiles = (int)((g.nq + ROWS - 1) / ROWS);
    p.scale = g.scale;
    const int64_t blocks = (int64_t)p.num_qtiles * g.hq * g.b;
    if (g.causal)
        hipLaunchKernelGGL((attn_step_f32<D, true>), dim3((unsigned)blocks), dim3(ROWS), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((attn_step_f32<D, false>), dim3((unsigned)blocks), dim3(ROWS), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_f32(const StepGeom &g, const void *q, const void *k,
                           const void *v, float *o, float *lse, hipStream_t stream) {
    if (g.d == 64) return launch_d<64>(g, q, k, v, o, lse, stream);
    return launch_d<128>(g, q, k, v, o, lse, stream);
}

}  // namespace cpattn
