// Blockwise attention of one CP step, bf16 inputs, fp32 accumulation, on
// gfx950 matrix cores.
//
// What it computes ("Megatron-LM 篇", Context Parallel 3.2 step 2 and 3.4):
// for each query row i of the step and head h, softmax attention over the
// visible keys of the source rank's block, returning the normalised O_i and
// the natural-log LSE L_i.  The mode decides the rows and keys (see
// internal.h: q_row0, nq, nk, causal).
//
// Work decomposition
//   workgroup = 4 waves = BM query rows of one (batch, head); each wave owns
//   QW = 32*NQT consecutive rows.  The KV block is streamed in tiles of
//   BN = 64 keys through LDS; every wave reads every tile.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16; 64 lanes, lane = 32*hi + l)
//   scores are computed transposed, S^T = K Q^T (M = keys, N = queries,
//   K = head dim), so lane l owns query l of a 32-row subtile and 16 key
//   rows of each 32x32 result: register v holds key row 8*(v/4) + 4*hi +
//   v%4.  Row max and row sum of a query are therefore in-lane, plus one
//   exchange with lane l^32.
//   The K rows fed to matrix row m are permuted (bits 2 and 3 of m swapped),
//   so register v of the S^T result holds key 8*hi + v (v < 8) or
//   16 + 8*hi + (v-8): exactly the 8 consecutive keys that lane must supply
//   as the B operand of the next product O^T += V^T P^T (M = head dim,
//   N = queries, K = keys).  P never leaves the lane.
//   V is stored transposed in LDS (V^T [d][key]) so the A operand of that
//   product is one 16-byte read.
//
// Softmax (fp32, log2 domain): x = s * scale * log2(e); p = exp2(x - m).
//   The running max m is only raised when a row's tile max exceeds it by
//   more than 8 (so p <= 256): O and l are rescaled in those rare tiles
//   and left alone otherwise.  The result is the same softmax; exp2 of a
//   bounded argument never overflows.
//   p is rounded to bf16 (nearest even) for the P V product; the row sum l
//   uses the fp32 p.
//
// LDS (64 banks of 4 bytes on gfx950): 16-byte chunks are XOR-swizzled so
// the 16 lanes of each ds_read_b128 phase hit 16 distinct bank groups.
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BN = 64;                 // keys per LDS tile
constexpr float RESCALE_SLACK = 8.0f;  // log2 units a stale max may lag

struct Params {
    const uint16_t *q, *k, *v;
    float *o, *lse;
    int64_t two_c, q_row0;
    int nq, nk, hq, hkv, group, num_qtiles;
    float scale_log2;
};

__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D, int NQT, bool CAUSAL>
__global__ void __launch_bounds__(NTHREADS)
attn_step_bf16(Params p) {
    static_assert(D == 128, "bf16 step kernel is built for head dim 128");
    constexpr int QW = 32 * NQT;          // query rows per wave
    constexpr int BM = QW * NWAVES;       // query rows per workgroup
    constexpr int DCH = D / 8;            // 16-byte chunks per K row
    constexpr int KK = D / 16;            // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;            // 32-wide head-dim tiles of O^T
    constexpr int KCH = BN / 8;           // 16-byte chunks per V^T row
    constexpr int KLOADS = BN * DCH / NTHREADS;

    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * D];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hi = lane >> 5;
    const int l32 = lane & 31;

    // Workgroup -> (batch, kv group, query tile, head in group).  Workgroups
    // are handed to the 8 XCDs round robin; give each XCD a contiguous run of
    // items so the heads sharing a KV group share that XCD's L2.  Within a
    // run, causal steps take their longest query tiles first.
    int item = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) item = (item & 7) * (nblk >> 3) + (item >> 3);
    const int hh = item % p.group;
    item /= p.group;
    const int qt_rank = item % p.num_qtiles;
    item /= p.num_qtiles;
    const int g = item % p.hkv;
    const int n = item / p.hkv;
    const int head = g * p.group + hh;
    const int qtile = CAUSAL ? p.num_qtiles - 1 - qt_rank : qt_rank;

    const int wrow0 = qtile * BM + wave * QW;   // first step row of this wave

    // Q fragments (B operand of S^T): lane holds query l32, dims kk*16+8*hi..
    bf16x8 qf[NQT][KK];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        int row = min(wrow0 + qt * 32 + l32, p.nq - 1);
        const uint16_t *src =
            p.q + ((n * p.two_c + p.q_row0 + row) * (int64_t)p.hq + head) * D + hi * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[qt][kk] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + kk * 16));
    }

    f32x16 acc[NQT][DT];
    float m_run[NQT], l_run[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        m_run[qt] = -INFINITY;
        l_run[qt] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[qt][dt][e] = 0.0f;
    }

    const int kend = CAUSAL ? min(p.nk, qtile * BM + BM) : p.nk;
    const int ntiles = (kend + BN - 1) / BN;

    const uint16_t *kbase = p.k + ((int64_t)n * p.two_c * p.hkv + g) * D;
    const uint16_t *vbase = p.v + ((int64_t)n * p.two_c * p.hkv + g) * D;
    const int64_t kstride = (int64_t)p.hkv * D;   // elements between keys

    // Per-thread load assignment.  K: KLOADS chunks, 16 threads per row.
    // V: 4 consecutive keys x 8 dims, transposed on the way into LDS.
    const int kchunk = tid % DCH;
    const int krow0 = tid / DCH;
    const int vdg = tid % DCH;             // dims 8*vdg .. +7
    const int vkg = tid / DCH;             // keys 4*vkg .. +3
    u32x4 kreg[KLOADS], vreg[4];

    auto load_tile = [&](int key0) {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
            int key = min(key0 + krow0 + u * (NTHREADS / DCH), p.nk - 1);
            kreg[u] = *(const u32x4 *)(kbase + key * kstride + kchunk * 8);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int key = min(key0 + vkg * 4 + j, p.nk - 1);
            vreg[j] = *(const u32x4 *)(vbase + key * kstride + vdg * 8);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < KLOADS; ++u) {
            int row = krow0 + u * (NTHREADS / DCH);
            int phys = kchunk ^ (swap_bits23(row) & (DCH - 1));
            *(u32x4 *)(sK + row * D + phys * 8) = kreg[u];
        }
        // transpose 4 keys x 8 dims -> 8 rows of V^T, 4 keys each
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            unsigned a0 = vreg[0][e2], a1 = vreg[1][e2], a2 = vreg[2][e2], a3 = vreg[3][e2];
            u32x2 lo, hiw;
            lo[0] = (a0 & 0xFFFFu) | (a1 << 16);
            lo[1] = (a2 & 0xFFFFu) | (a3 << 16);
            hiw[0] = (a0 >> 16) | (a1 & 0xFFFF0000u);
            hiw[1] = (a2 >> 16) | (a3 & 0xFFFF0000u);
#pragma unroll
            for (int odd = 0; odd < 2; ++odd) {
                int d = vdg * 8 + e2 * 2 + odd;
                int chunk = vkg >> 1;
                int phys = chunk ^ ((d >> 1) & (KCH - 1));
                *(u32x2 *)(sVt + d * BN + phys * 8 + (vkg & 1) * 4) = odd ? hiw : lo;
            }
        }
    };

    if (ntiles > 0) load_tile(0);

    const int krow_perm = swap_bits23(l32);   // K row fed to matrix row l32

    for (int t = 0; t < ntiles; ++t) {
        const int key0 = t * BN;
        __syncthreads();
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(key0 + BN);

        // Causal: a wave whose rows all precede this tile has nothing to do.
        if (CAUSAL && key0 > wrow0 + QW - 1) continue;
        const bool need_mask =
            (key0 + BN > p.nk) || (CAUSAL && key0 + BN - 1 > wrow0);

        // S^T = K Q^T for the 64-key tile: two 32-key halves
        f32x16 s[NQT][2];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[qt][st][e] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                int row = st * 32 + krow_perm;
                int phys = (kk * 2 + hi) ^ (l32 & (DCH - 1));
                bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sK + row * D + phys * 8));
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
                    s[qt][st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qt][kk], s[qt][st], 0, 0, 0);
            }
        }

        bf16x8 pf[NQT][4];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            const int qrow = wrow0 + qt * 32 + l32;
            float tmax = -INFINITY;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float x = s[qt][st][e] * p.scale_log2;
                    if (need_mask) {
                        int key = key0 + st * 32 + 16 * (e >> 3) + 8 * hi + (e & 7);
                        bool vis = key < p.nk && (!CAUSAL || key <= qrow);
                        x = vis ? x : -INFINITY;
                    }
                    s[qt][st][e] = x;
                    tmax = fmaxf(tmax, x);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run[qt], tmax);
            const bool grow = m_new > m_run[qt] + RESCALE_SLACK;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
                l_run[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[qt][dt] *= alpha;
                m_run[qt] = m_new;
            }
            const float mu = (m_run[qt] == -INFINITY) ? 0.0f : m_run[qt];
            float lsum = 0.0f;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    f32x8 pv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float pe = __builtin_amdgcn_exp2f(s[qt][st][half * 8 + e] - mu);
                        pv[e] = pe;
                        lsum += pe;
                    }
                    pf[qt][st * 2 + half] = __builtin_convertvector(pv, bf16x8);
                }
            }
            l_run[qt] += lsum;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 32 + l32;
#pragma unroll
            for (int kc = 0; kc < BN / 16; ++kc) {
                int phys = (kc * 2 + hi) ^ ((d >> 1) & (KCH - 1));
                bf16x8 vf = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sVt + d * BN + phys * 8));
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
                    acc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qt][kc], acc[qt][dt], 0, 0, 0);
            }
        }
    }

    // Normalise and store O_i (fp32) and L_i (natural log).
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const float lt = l_run[qt] + __shfl_xor(l_run[qt], 32);
        const int row = wrow0 + qt * 32 + l32;
        if (row < p.nq) {
            const float inv = 1.0f / lt;
            float *dst = p.o + ((n * (int64_t)p.nq + row) * p.hq + head) * D + 4 * hi;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = acc[qt][dt][i * 4 + j] * inv;
                    *(f32x4 *)(dst + dt * 32 + i * 8) = w;
                }
            if (hi == 0)
                p.lse[((int64_t)n * p.hq + head) * p.nq + row] =
                    (m_run[qt] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
        }
    }
}

template <int NQT, bool CAUSAL>
hipError_t launch(const StepGeom &g, const void *q, const void *k, const void *v,
                  float *o, float *lse, hipStream_t stream) {
    constexpr int BM = 32 * NQT * NWAVES;
    Params p;
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.o = o;
    p.lse = lse;
    p.two_c = g.two_c;
    p.q_row0 = g.q_row0;
    p.nq = (int)g.nq;
    p.nk = (int)g.nk;
    p.hq = g.hq;
    p.hkv = g.hkv;
    p.group = g.hq / g.hkv;
    p.num_qtiles = (int)((g.nq + BM - 1) / BM);
    p.scale_log2 = g.scale_log2;
    const int64_t blocks = (int64_t)p.num_qtiles * g.hq * g.b;
    hipLaunchKernelGGL((attn_step_bf16<128, NQT, CAUSAL>), dim3((unsigned)blocks),
                       dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepGeom &g, const void *q, const void *k,
                            const void *v, float *o, float *lse, hipStream_t stream) {
    if (g.causal) return launch<1, true>(g, q, k, v, o, lse, stream);
    return launch<1, false>(g, q, k, v, o, lse, stream);
}

}  // namespace cpattn
