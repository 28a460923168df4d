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
//   workgroup = NW waves = BM = 32*NW query rows of one (batch, head); each
//   wave owns 32 consecutive rows.  The KV block streams through LDS in
//   tiles of BN = 64 keys held in a ring of NS stages.  Tiles are copied
//   global -> LDS directly (global_load_lds_dwordx4, no VGPR round trip),
//   NS-1 tiles ahead of the one being computed, so HBM/L2 latency hides
//   behind NS-1 tiles of matrix work; one barrier per tile.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16; lane = 32*hi + l32)
//   Scores are computed transposed, S^T = K Q^T (M = keys, N = queries,
//   K = head dim): lane l32 owns query l32 of its wave and 16 key rows of
//   each 32x32 result; register v holds result row 8*(v/4) + 4*hi + v%4.
//   Row max and row sum are in-lane plus one exchange with lane l32^32.
//   The K row fed to matrix row m is m with bits 2 and 3 swapped, so
//   register v holds key 8*hi + v (v < 8) or 16 + 8*hi + (v-8): the 8
//   consecutive keys the lane supplies as the B operand of the next
//   product O^T += V^T P^T (M = head dim, N = queries, K = keys).  P never
//   leaves the lane.
//   V stays row-major in LDS; the V^T operand (8 consecutive keys of one
//   head-dim column per lane) comes from two ds_read_b64_tr_b16, which
//   hand lane t of each 16-lane group element j of the 4-element block read
//   by lane 4j + t/4 of that group, column t%4.
//
// Softmax (fp32, log2 domain): p = exp2(s*c - m) with c = scale*log2(e).
//   The running max m is raised only when a row's tile max exceeds it by
//   more than 8 (so p <= 256); O and l are rescaled only in those tiles.
//   The result is the same softmax.  p is rounded to bf16 (nearest even) for
//   the P V product; the row sum l accumulates the fp32 p.
//
// LDS (64 banks x 4 bytes on gfx950): rows are 256 bytes; 16-byte chunks
// are XOR-swizzled per row (K: by the matrix row feeding it, V: by key%4)
// so every ds_read_b128 / ds_read_b64_tr_b16 phase hits distinct banks.
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int BN = 64;                 // keys per LDS tile
constexpr int ROWB = D * 2;            // bytes per K/V row in LDS
constexpr int TILEB = BN * ROWB;       // bytes per K (or V) tile
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

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The tile reads are issued from inline assembly: the compiler cannot tell
// the LDS stages apart from the in-flight global->LDS copies and would
// otherwise wait for every copy before each read.  Each block ends with
// lgkmcnt(0), so its outputs are complete when it returns.

// K operands (A of S^T = K Q^T) for k-steps kk0..kk0+3 and both 32-key
// halves of the tile: a[kk] addresses the lane's 16-byte chunk of k-step kk
// in the first half; the second half is 32 rows (8 KiB) further.
__device__ __forceinline__ void read_k4(const unsigned (&a)[4], bf16x8 (&kf)[4][2]) {
    u32x4 r[8];
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:8192\n\t"
        "ds_read_b128 %2, %9\n\t"
        "ds_read_b128 %3, %9 offset:8192\n\t"
        "ds_read_b128 %4, %10\n\t"
        "ds_read_b128 %5, %10 offset:8192\n\t"
        "ds_read_b128 %6, %11\n\t"
        "ds_read_b128 %7, %11 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kf[i][0] = __builtin_bit_cast(bf16x8, r[2 * i]);
        kf[i][1] = __builtin_bit_cast(bf16x8, r[2 * i + 1]);
    }
}

// V^T operands of key chunk kc (16 keys) for the four 32-wide head-dim
// tiles.  Lane L = 16*g + 4*j + q reads, for s in {0, 1}, the 8-byte block at
// V row kc*16 + 8*(g/2) + 4*s + j, head dims dt*32 + 16*(g%2) + 4*q .. +3;
// the transpose hands lane t of group g the column dt*32 + 16*(g%2) + t for
// keys +0..3 of that row block.  a[dt] addresses row 8*(g/2) + j of dims
// tile dt (rows kc*16 and +4 are immediate offsets).
template <int KC>
__device__ __forceinline__ void read_vt(const unsigned (&a)[4], bf16x8 (&vf)[4]) {
    s16x4 r[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(KC * 16 * ROWB),
          "i"(KC * 16 * ROWB + 4 * ROWB));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        vf[dt] = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(r[2 * dt], r[2 * dt + 1], 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int NW, int NS, bool CAUSAL>
struct Kernel {
    static constexpr int BM = 32 * NW;
    static constexpr int NT = 64 * NW;
    // global->LDS instructions per wave per tile (K and V each)
    static constexpr int KI = BN / 4 / NW;    // one instruction fills 4 rows
    static constexpr int LOADS_PER_TILE = 2 * KI;
    static_assert(KI >= 1, "need at most 16 waves");

    // Issue this wave's share of the direct copies of tile `key0` into one
    // LDS stage (sK, sV).
    __device__ __forceinline__ static void issue(const Params &p, char *sK, char *sV,
                                                 const uint16_t *kbase, const uint16_t *vbase,
                                                 int64_t kstride, int key0, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int row = (wave * KI + i) * 4 + (lane >> 4);
            const int phys = lane & 15;
            const int key = min(key0 + row, p.nk - 1);
            const int kchunk = phys ^ (swap_bits23(row) & 15);
            const int vchunk = phys ^ ((row & 3) << 2);
            const int64_t goff = (int64_t)key * kstride;
            char *kdst = sK + (wave * KI + i) * 4 * ROWB;
            char *vdst = sV + (wave * KI + i) * 4 * ROWB;
            __builtin_amdgcn_global_load_lds((const void *)(kbase + goff + kchunk * 8),
                                             (lds_void *)kdst, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(vbase + goff + vchunk * 8),
                                             (lds_void *)vdst, 16, 0, 0);
        }
    }

    // Per-wave state carried from tile to tile.
    struct State {
        bf16x8 qf[D / 16];
        f32x16 acc[D / 32];
        float m_run, l_run;
        unsigned koff[D / 16];   // lane's byte offset of each K chunk in a stage
        unsigned voff[D / 32];   // lane's byte offset of each V^T read in a stage
    };

    // One KV tile: wait for its copies, barrier, refill the stage freed by
    // the previous tile, then S^T = K Q^T, online softmax, O^T += V^T P^T.
    __device__ __forceinline__ static void tile(const Params &p, State &S, int t, int ntiles,
                                                unsigned sK, unsigned sV, char *nK,
                                                char *nV, const uint16_t *kbase,
                                                const uint16_t *vbase, int64_t kstride,
                                                int wrow0, int wave, int lane) {
        const int hi = lane >> 5;
        const int l32 = lane & 31;
        // Own copies of tile t done (the NS-2 tiles issued after it may still
        // be in flight), then all waves' copies: barrier.  The barrier also
        // retires every wave's reads of the stage refilled below (they fed
        // tile t-1's MFMAs).  Copies are issued for every tile index, also
        // past the end (rows clamped, never read), so the number in flight is
        // the same at every wait.
        wait_vmcnt<LOADS_PER_TILE * (NS - 2)>();
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        issue(p, nK, nV, kbase, vbase, kstride, (t + NS - 1) * BN, wave, lane);
        const int key0 = t * BN;
        if (CAUSAL && key0 > wrow0 + 31) return;      // tile after every row of the wave
        // scalar branch: only tiles crossing the diagonal or the end mask
        if ((key0 + BN > p.nk) || (CAUSAL && key0 + BN - 1 > wrow0))
            compute<true>(p, S, sK, sV, key0, wrow0, lane);
        else
            compute<false>(p, S, sK, sV, key0, wrow0, lane);
    }

    // S^T = K Q^T, online softmax and O^T += V^T P^T for one resident tile.
    template <bool MASK>
    __device__ __forceinline__ static void compute(const Params &p, State &S, unsigned sK,
                                                   unsigned sV, int key0, int wrow0, int lane) {
        const int hi = lane >> 5;
        const int l32 = lane & 31;

        // S^T = K Q^T over the 64-key tile: two 32-key halves
        f32x16 s[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 16; ++e) s[h2][e] = 0.0f;
#pragma unroll
        for (int k4 = 0; k4 < D / 64; ++k4) {
            unsigned a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sK + S.koff[k4 * 4 + i];
            bf16x8 kf[4][2];
            read_k4(a, kf);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    s[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i][h2], S.qf[k4 * 4 + i],
                                                                   s[h2], 0, 0, 0);
        }

        // online softmax in the log2 domain
        const int qrow = wrow0 + l32;
        float tmax = -INFINITY;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = s[h2][e];
                if constexpr (MASK) {
                    const int key = key0 + h2 * 32 + 16 * (e >> 3) + 8 * hi + (e & 7);
                    const bool vis = key < p.nk && (!CAUSAL || key <= qrow);
                    x = vis ? x : -INFINITY;
                    s[h2][e] = x;
                }
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * p.scale_log2;
        const float m_new = fmaxf(S.m_run, tmax);
        if (__builtin_amdgcn_ballot_w64(m_new > S.m_run + RESCALE_SLACK)) {
            const float alpha = __builtin_amdgcn_exp2f(S.m_run - m_new);
            S.l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) S.acc[dt] *= alpha;
            S.m_run = m_new;
        }
        const float mu = (S.m_run == -INFINITY) ? 0.0f : S.m_run;
        bf16x8 pf[BN / 16];
        float lsum0 = 0.0f, lsum1 = 0.0f;   // two partial row sums (shorter chains)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(s[h2][half * 8 + e], p.scale_log2, -mu));
                const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
                pf[h2 * 2 + half] = pb;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    lsum0 += pv[e];
                    lsum1 += pv[e + 1];
                }
            }
        S.l_run += lsum0 + lsum1;

        // O^T += V^T P^T; the V^T operand of each MFMA is two transposing reads
        unsigned av[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) av[dt] = sV + S.voff[dt];
        pv_chunk<0>(S, av, pf[0]);
        pv_chunk<1>(S, av, pf[1]);
        pv_chunk<2>(S, av, pf[2]);
        pv_chunk<3>(S, av, pf[3]);
    }

    template <int KC>
    __device__ __forceinline__ static void pv_chunk(State &S, const unsigned (&av)[4],
                                                    const bf16x8 &pfk) {
        bf16x8 vf[4];
        read_vt<KC>(av, vf);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
            S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt], pfk, S.acc[dt], 0, 0, 0);
    }

    __device__ __forceinline__ static void run(const Params &p, char *lds) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        // wave index as a scalar: every per-wave decision below (mask, skip)
        // is then a scalar branch instead of a per-lane select
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int hi = lane >> 5;
        const int l32 = lane & 31;

        // Workgroup -> (batch, kv group, query tile, head in group).  The 8
        // XCDs receive workgroups round robin; give each a contiguous run of
        // items so heads sharing a KV group share that XCD's L2.  Causal
        // steps take their longest query tiles first.
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
        const int wrow0 = qtile * BM + wave * 32;   // first step row of this wave

        const int kend = CAUSAL ? min(p.nk, qtile * BM + BM) : p.nk;
        const int ntiles = (kend + BN - 1) / BN;
        const uint16_t *kbase = p.k + ((int64_t)n * p.two_c * p.hkv + g) * D;
        const uint16_t *vbase = p.v + ((int64_t)n * p.two_c * p.hkv + g) * D;
        const int64_t kstride = (int64_t)p.hkv * D;

        State S;
        // Q fragments (B operand of S^T): lane holds query l32, dims kk*16+8*hi..
        {
            const int row = min(wrow0 + l32, p.nq - 1);
            const uint16_t *src =
                p.q + ((n * p.two_c + p.q_row0 + row) * (int64_t)p.hq + head) * D + hi * 8;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                S.qf[kk] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + kk * 16));
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) S.acc[dt][e] = 0.0f;
        S.m_run = -INFINITY;
        S.l_run = 0.0f;

        // prologue: the first NS-1 tiles in flight (after the Q loads, so the
        // in-order vector-memory counter retires Q first)
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            issue(p, lds + s * 2 * TILEB, lds + s * 2 * TILEB + TILEB, kbase, vbase, kstride,
                  s * BN, wave, lane);

        // lane byte offsets of the tile reads inside a stage (see read_k4/read_vt)
        {
            const int krow = swap_bits23(l32);             // K row fed to matrix row l32
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                S.koff[kk] = krow * ROWB + (((kk * 2 + hi) ^ (l32 & 15)) << 4);
            const int vg = lane >> 4, vj = (lane >> 2) & 3, vq = lane & 3;
            const int x = 2 * (vg & 1) + (vq >> 1);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                S.voff[dt] = (8 * (vg >> 1) + vj) * ROWB + (((dt * 4 + x) ^ (vj << 2)) << 4) +
                             (vq & 1) * 8;
        }
        const unsigned lds_addr =
            (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
        // Q has landed once only the prologue copies are outstanding
        wait_vmcnt<LOADS_PER_TILE * (NS - 1)>();

        // the ring, unrolled by stage so stage offsets are constants
        for (int t0 = 0; t0 < ntiles; t0 += NS) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (t0 + s < ntiles) {
                    const int nxt = (s + NS - 1) % NS;
                    tile(p, S, t0 + s, ntiles, lds_addr + s * 2 * TILEB,
                         lds_addr + s * 2 * TILEB + TILEB, lds + nxt * 2 * TILEB,
                         lds + nxt * 2 * TILEB + TILEB, kbase, vbase, kstride, wrow0, wave, lane);
                }
            }
        }

        // the copies past the end land in stages nobody reads; retire them
        // before the workgroup's LDS is handed to the next workgroup
        wait_vmcnt<0>();

        // Normalise and store O_i (fp32) and L_i (natural log).
        const float lt = S.l_run + __shfl_xor(S.l_run, 32);
        const int row = wrow0 + l32;
        if (row < p.nq) {
            const float inv = 1.0f / lt;
            float *dst = p.o + ((n * (int64_t)p.nq + row) * p.hq + head) * D + 4 * hi;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = S.acc[dt][i * 4 + j] * inv;
                    *(f32x4 *)(dst + dt * 32 + i * 8) = w;
                }
            if (hi == 0)
                p.lse[((int64_t)n * p.hq + head) * p.nq + row] =
                    (S.m_run + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
        }
    }
};

template <int NW, int NS, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW) attn_step_bf16(Params p) {
    // NS stages of (K tile, V tile)
    __shared__ __attribute__((aligned(1024))) char lds[NS * 2 * TILEB];
    Kernel<NW, NS, CAUSAL>::run(p, lds);
}

template <int NW, int NS, bool CAUSAL>
hipError_t launch(const StepGeom &g, const void *q, const void *k, const void *v, float *o,
                  float *lse, hipStream_t stream) {
    constexpr int BM = 32 * NW;
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
    hipLaunchKernelGGL((attn_step_bf16<NW, NS, CAUSAL>), dim3((unsigned)blocks), dim3(64 * NW),
                       0, stream, p);
    return hipGetLastError();
}

constexpr int kWaves = 8;
constexpr int kStages = 3;

}  // namespace

hipError_t launch_step_bf16(const StepGeom &g, const void *q, const void *k, const void *v,
                            float *o, float *lse, hipStream_t stream) {
    if (g.causal) return launch<kWaves, kStages, true>(g, q, k, v, o, lse, stream);
    return launch<kWaves, kStages, false>(g, q, k, v, o, lse, stream);
}

}  // namespace cpattn
