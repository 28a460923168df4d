// Backward of one CP step's blockwise attention, bf16 inputs, fp32
// accumulation, on gfx950 matrix cores.
//
// What it computes: the pages treat the backward only through the
// communication context parallelism adds to it ("超大规模集群…", "CP 与其他
// 技术结合": an all-gather of K/V and a reduce-scatter of their gradients).
// Each forward ring step has a backward counterpart on the same blocks and
// rows ("Megatron-LM 篇" 3.4: the three step modes).  With the rank's final
// (merged) L and D = sum_t dO O of each query row i and head h, and for the
// keys j the mode lets row i see:
//     P_ij  = exp(scale q_i.k_j - L_i)
//     dS_ij = P_ij (dO_i.v_j - D_i)
//     dq_i += scale sum_j dS_ij k_j
//     dk_j += scale sum_{i, h in group} dS_ij q_i
//     dv_j += sum_{i, h in group} P_ij dO_i
// dq is the rank's own query gradient; dk, dv are the step's share of the
// source rank's gradients (summed on their owner by the reduce-scatter).
//
// Two kernels per step, both on v_mfma_f32_32x32x16_bf16 (lane = 32*hi +
// l32; register v of a result holds matrix row 8*(v/4) + 4*hi + v%4):
//   attn_bwd_dq    a wave owns 32 query rows (Q and dO held as B operands)
//                  and streams 32-key tiles of K and V:
//                    S^T = K Q^T, dP^T = V dO^T  (lane l32 owns query l32),
//                    dS^T = P^T (dP^T - D), dQ^T += K^T dS^T;
//   attn_bwd_dkdv  a wave owns 32 keys (K and V held as B operands) and
//                  streams 32-row tiles of Q and dO of every head of the
//                  group:  S = Q K^T, dP = dO V^T  (lane l32 owns key l32),
//                    dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
// The streamed rows are fed to the matrix row swap_bits23(m), so a lane's
// result registers hold 8 consecutive rows: P and dS are the B operand of
// the next product without leaving the lane.
//
// LDS: a streamed tile is contracted over the head dim (row chunks,
// ds_read_b128) and over its rows (8 rows of one column per lane,
// ds_read_b64_tr_b16), so the tiles that need both are written twice, in
// two XOR swizzles: "R" (16-byte chunk c of row r at c ^ (swap_bits23(r) &
// 15)) and "T" (at c ^ ((r & 3) << 2)); each keeps its read pattern free
// of bank conflicts.  Tiles are double-buffered: the next tile's global
// loads are in flight while the current one is computed; one barrier per
// tile.  The MFMAs are compiler builtins, so the compiler pads every hazard.
#include "internal.h"
#include "mfma_tiles.h"

#include <math.h>

namespace cpattn {
namespace {

using namespace tiles;

constexpr int D = 128;
constexpr int NWB = 4;                     // waves per workgroup
constexpr int TR = 32;                     // rows of a streamed tile; rows (keys) per wave
constexpr int RB = ROW_BYTES;              // bytes per tile row
constexpr int TB = TR * RB;                // bytes per tile in one layout
constexpr int CPT = TR * (D / 8) / (64 * NWB);   // 16-byte chunks per thread per tile (= 2)

struct BwdParams {
    const uint16_t *q, *k, *v, *dout;   // q_r, dout_r [b, 2c, hq, d]; k, v [b, 2c, hkv, d]
    const float *lse, *delta;           // the rank's final L (natural log) and D [b, hq, 2c]
    float *dq, *dk, *dv;                // accumulated: dq [b, 2c, hq, d]; dk, dv [b, 2c, hkv, d]
    int64_t two_c, q_row0;
    int nq, nk, hq, hkv, group, ntiles_wg;
    float scale, scale_log2;
    int causal;
};

// Byte offset of chunk c of tile row r in the two layouts.
__device__ __forceinline__ unsigned r_off(int r, int c) {
    return r * RB + ((c ^ (swap_bits23(r) & 15)) << 4);
}
__device__ __forceinline__ unsigned t_off(int r, int c) {
    return r * RB + ((c ^ ((r & 3) << 2)) << 4);
}

// The lane's offsets for the two reads (see the header): row operand of
// k-step kk from an R tile, transposed operand of head-dim tile dt from a T
// tile (plus kc * 16 * RB for the second 16-row chunk).
struct LaneOffsets {
    unsigned roff[D / 16];
    unsigned toff[D / 32];
    __device__ __forceinline__ void init(int lane) {
        const int hi = lane >> 5, l32 = lane & 31;
        const int r = swap_bits23(l32);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) roff[kk] = r * RB + (((kk * 2 + hi) ^ (l32 & 15)) << 4);
        const int vg = lane >> 4, vj = (lane >> 2) & 3, vq = lane & 3;
        const int x = 2 * (vg & 1) + (vq >> 1);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
            toff[dt] = (8 * (vg >> 1) + vj) * RB + (((dt * 4 + x) ^ (vj << 2)) << 4) + (vq & 1) * 8;
    }
};

// The 16-byte chunks a thread copies of a 32-row tile: rows tid/16 and
// tid/16 + 16, chunk tid%16.
__device__ __forceinline__ int tile_row(int tid, int i) { return tid / 16 + 16 * i; }

// B operand of the 8 k-steps for one row (this lane's l32-th row of a
// 32-row block): row chunks kk*16 + 8*hi .. +7.
__device__ __forceinline__ void load_b_rows(const uint16_t *row, int hi, bf16x8 (&f)[D / 16]) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        f[kk] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(row + kk * 16 + hi * 8));
}

#define MFMA __builtin_amdgcn_mfma_f32_32x32x16_bf16

// ---------------------------------------------------------------------------
// dQ: workgroup = 4 waves x 32 query rows of one (batch, head); 32-key tiles
// of K (R and T layouts) and V (R layout) double-buffered in LDS.
__global__ void __launch_bounds__(64 * NWB) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[2 * 3 * TB];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    int item = blockIdx.x;
    const int nqt = p.ntiles_wg;
    const int qt = nqt - 1 - item % nqt;       // longest (causal) tiles first
    item /= nqt;
    const int head = item % p.hq;
    const int n = item / p.hq;
    const int g = head / p.group;
    const int q0 = qt * TR * NWB;
    const int wrow0 = q0 + wave * TR;
    const int kend = p.causal ? min(p.nk, q0 + TR * NWB) : p.nk;
    const int ntiles = (kend + TR - 1) / TR;
    const int wtiles = p.causal ? min(ntiles, (wrow0 + TR - 1) / TR + 1) : ntiles;

    LaneOffsets L;
    L.init(lane);
    const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

    // this lane's query row: Q and dO as B operands, L (log2) and D
    const int qrow = wrow0 + l32;
    const int qr = min(qrow, p.nq - 1);
    const int64_t qoff = ((n * p.two_c + p.q_row0 + qr) * (int64_t)p.hq + head) * D;
    bf16x8 qf[D / 16], df[D / 16];
    load_b_rows(p.q + qoff, hi, qf);
    load_b_rows(p.dout + qoff, hi, df);
    const int64_t lrow = ((int64_t)n * p.hq + head) * p.two_c + p.q_row0 + qr;
    const float lq = p.lse[lrow] * 1.4426950408889634f;
    const float dq_d = p.delta[lrow];
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

    const uint16_t *kb = p.k + ((int64_t)n * p.two_c * p.hkv + g) * D;
    const uint16_t *vb = p.v + ((int64_t)n * p.two_c * p.hkv + g) * D;
    const int64_t ks = (int64_t)p.hkv * D;
    u32x4 kreg[CPT], vreg[CPT];
    auto gload = [&](int t) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int key = min(t * TR + tile_row(tid, i), p.nk - 1);
            kreg[i] = *(const u32x4 *)(kb + key * ks + (tid & 15) * 8);
            vreg[i] = *(const u32x4 *)(vb + key * ks + (tid & 15) * 8);
        }
    };
    auto lstore = [&](int buf) {
        char *base = lds + buf * 3 * TB;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int r = tile_row(tid, i), c = tid & 15;
            *(u32x4 *)(base + r_off(r, c)) = kreg[i];           // K, R layout
            *(u32x4 *)(base + TB + t_off(r, c)) = kreg[i];      // K, T layout
            *(u32x4 *)(base + 2 * TB + r_off(r, c)) = vreg[i];  // V, R layout
        }
    };
    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) gload(t + 1);
        if (t < wtiles) {
            const unsigned sK = lbase + (t & 1) * 3 * TB, sKT = sK + TB, sV = sK + 2 * TB;
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                s = MFMA(k_read(sK + L.roff[kk]), qf[kk], s, 0, 0, 0);
                dp = MFMA(k_read(sV + L.roff[kk]), df[kk], dp, 0, 0, 0);
            }
            const int key0 = t * TR;
            bf16x8 dsb[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                f32x8 ds;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = key0 + 16 * kc + 8 * hi + e;
                    const bool vis = key < p.nk && (!p.causal || key <= qrow);
                    const float pr = vis ? __builtin_amdgcn_exp2f(
                                               __builtin_fmaf(s[kc * 8 + e], p.scale_log2, -lq))
                                         : 0.0f;
                    ds[e] = pr * (dp[kc * 8 + e] - dq_d);
                }
                dsb[kc] = __builtin_convertvector(ds, bf16x8);
            }
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    acc[dt] = MFMA(vt_read(sKT + L.toff[dt] + kc * 16 * RB), dsb[kc], acc[dt], 0,
                                   0, 0);
        }
        if (t + 1 < ntiles) lstore((t + 1) & 1);
        __syncthreads();
    }

    // dq[row] += scale * dQ: lane holds head dims dt*32 + 8*i + 4*hi + j
    if (qrow < p.nq) {
        float *dst = p.dq + qoff + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 *a = (f32x4 *)(dst + dt * 32 + i * 8);
                f32x4 w = *a;
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] += p.scale * acc[dt][i * 4 + j];
                *a = w;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 4 waves x 32 keys of one (batch, KV head); streams
// 32-row tiles of Q and dO (R and T layouts) and their L and D, for every
// query head of the group, double-buffered in LDS.
__global__ void __launch_bounds__(64 * NWB) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dkdv(BwdParams p) {
    constexpr int BUF = 4 * TB + 2 * TR * 4;   // Q R, Q T, dO R, dO T, L, D
    __shared__ __attribute__((aligned(1024))) char lds[2 * BUF];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    int item = blockIdx.x;
    const int nkt = p.ntiles_wg;
    const int kt = item % nkt;                 // causal: early key tiles see the most rows
    item /= nkt;
    const int g = item % p.hkv;
    const int n = item / p.hkv;
    const int k0 = kt * TR * NWB;
    const int wkey0 = k0 + wave * TR;

    LaneOffsets L;
    L.init(lane);
    const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

    // this lane's key: K and V as B operands of S = Q K^T and dP = dO V^T
    const int key = wkey0 + l32;
    const int kr = min(key, p.nk - 1);
    const int64_t koff = ((n * p.two_c + kr) * (int64_t)p.hkv + g) * D;
    bf16x8 kf[D / 16], vf[D / 16];
    load_b_rows(p.k + koff, hi, kf);
    load_b_rows(p.v + koff, hi, vf);
    f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            adk[dt][e] = 0.0f;
            adv[dt][e] = 0.0f;
        }

    // query tiles: every head of the group, rows from the first one that can
    // see this workgroup's keys (causal: row >= key) to the end
    const int qstart = p.causal ? (k0 / TR) : 0;
    const int nqt = (p.nq + TR - 1) / TR;
    const int per_head = max(nqt - qstart, 0);
    const int ntiles = per_head * p.group;
    u32x4 qreg[CPT], dreg[CPT];
    float lreg = 0.0f, dreg1 = 0.0f;
    auto gload = [&](int u) {
        const int head = g * p.group + u / per_head;
        const int qt = qstart + u % per_head;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int row = min(qt * TR + tile_row(tid, i), p.nq - 1);
            const int64_t off = ((n * p.two_c + p.q_row0 + row) * (int64_t)p.hq + head) * D;
            qreg[i] = *(const u32x4 *)(p.q + off + (tid & 15) * 8);
            dreg[i] = *(const u32x4 *)(p.dout + off + (tid & 15) * 8);
        }
        if (tid < TR) {
            const int row = min(qt * TR + tid, p.nq - 1);
            const int64_t lrow = ((int64_t)n * p.hq + head) * p.two_c + p.q_row0 + row;
            lreg = p.lse[lrow] * 1.4426950408889634f;
            dreg1 = p.delta[lrow];
        }
    };
    auto lstore = [&](int buf) {
        char *base = lds + buf * BUF;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int r = tile_row(tid, i), c = tid & 15;
            *(u32x4 *)(base + r_off(r, c)) = qreg[i];
            *(u32x4 *)(base + TB + t_off(r, c)) = qreg[i];
            *(u32x4 *)(base + 2 * TB + r_off(r, c)) = dreg[i];
            *(u32x4 *)(base + 3 * TB + t_off(r, c)) = dreg[i];
        }
        if (tid < TR) {
            ((float *)(base + 4 * TB))[tid] = lreg;
            ((float *)(base + 4 * TB + TR * 4))[tid] = dreg1;
        }
    };
    if (ntiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    for (int u = 0; u < ntiles; ++u) {
        if (u + 1 < ntiles) gload(u + 1);
        const int qt = qstart + u % per_head;
        const int q0 = qt * TR;
        // the wave's keys are visible to some row of the tile
        if (!p.causal || q0 + TR - 1 >= wkey0) {
            const unsigned sQ = lbase + (u & 1) * BUF, sQT = sQ + TB, sD = sQ + 2 * TB,
                           sDT = sQ + 3 * TB;
            const char *lb = lds + (u & 1) * BUF + 4 * TB;
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                s = MFMA(k_read(sQ + L.roff[kk]), kf[kk], s, 0, 0, 0);
                dp = MFMA(k_read(sD + L.roff[kk]), vf[kk], dp, 0, 0, 0);
            }
            bf16x8 pb[2], dsb[2];
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                // L and D of the 8 rows this lane holds: 16*qc + 8*hi .. +7
                const f32x8 lv = *(const f32x8 *)(lb + (16 * qc + 8 * hi) * 4);
                const f32x8 dv8 = *(const f32x8 *)(lb + TR * 4 + (16 * qc + 8 * hi) * 4);
                f32x8 pv, ds;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = q0 + 16 * qc + 8 * hi + e;
                    const bool vis = row < p.nq && key < p.nk && (!p.causal || key <= row);
                    pv[e] = vis ? __builtin_amdgcn_exp2f(
                                      __builtin_fmaf(s[qc * 8 + e], p.scale_log2, -lv[e]))
                                : 0.0f;
                    ds[e] = pv[e] * (dp[qc * 8 + e] - dv8[e]);
                }
                pb[qc] = __builtin_convertvector(pv, bf16x8);
                dsb[qc] = __builtin_convertvector(ds, bf16x8);
            }
#pragma unroll
            for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    adv[dt] = MFMA(vt_read(sDT + L.toff[dt] + qc * 16 * RB), pb[qc], adv[dt], 0,
                                   0, 0);
                    adk[dt] = MFMA(vt_read(sQT + L.toff[dt] + qc * 16 * RB), dsb[qc], adk[dt],
                                   0, 0, 0);
                }
        }
        if (u + 1 < ntiles) lstore((u + 1) & 1);
        __syncthreads();
    }

    if (key < p.nk) {
        float *dk = p.dk + koff + 4 * hi;
        float *dv = p.dv + koff + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 *a = (f32x4 *)(dk + dt * 32 + i * 8);
                f32x4 *b = (f32x4 *)(dv + dt * 32 + i * 8);
                f32x4 wa = *a, wb = *b;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wa[j] += p.scale * adk[dt][i * 4 + j];
                    wb[j] += adv[dt][i * 4 + j];
                }
                *a = wa;
                *b = wb;
            }
    }
}

// ---------------------------------------------------------------------------
// D[n, h, i] = sum_t dO[n, i, h, t] O[n, i, h, t]: one thread per (n, i, h).
__global__ void __launch_bounds__(256) bwd_delta(const float *o, const uint16_t *dout,
                                                 float *delta, int64_t rows, int hq,
                                                 int64_t two_c) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (n*2c + i)*hq + h
    if (idx >= rows) return;
    const float *orow = o + idx * D;
    const uint16_t *drow = dout + idx * D;
    float acc = 0.0f;
#pragma unroll 4
    for (int c = 0; c < D / 8; ++c) {
        const f32x4 o0 = *(const f32x4 *)(orow + c * 8), o1 = *(const f32x4 *)(orow + c * 8 + 4);
        const u32x4 dw = *(const u32x4 *)(drow + c * 8);
        const bf16x8 db = __builtin_bit_cast(bf16x8, dw);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += (float)db[e] * o0[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += (float)db[4 + e] * o1[e];
    }
    const int h = (int)(idx % hq);
    const int64_t ni = idx / hq;
    const int64_t i = ni % two_c, n = ni / two_c;
    delta[(n * hq + h) * two_c + i] = acc;
}

// x[0 .. n) = 0, 16 bytes per thread (n a multiple of 4).
__global__ void __launch_bounds__(256) fill_zero(float *x, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) ((f32x4 *)x)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace

hipError_t launch_bwd_delta(int64_t b, int64_t two_c, int hq, const float *o, const void *dout,
                            float *delta, hipStream_t stream) {
    const int64_t rows = b * two_c * hq;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_delta, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, o,
                       (const uint16_t *)dout, delta, rows, hq, two_c);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *x, int64_t n, hipStream_t stream) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, x,
                       n4);
    return hipGetLastError();
}

hipError_t launch_step_bwd_bf16(const StepGeom &g, const void *q, const void *k, const void *v,
                                const void *dout, const float *lse, const float *delta,
                                float *dq, float *dk, float *dv, hipStream_t stream) {
    BwdParams p = {};
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.dout = (const uint16_t *)dout;
    p.lse = lse;
    p.delta = delta;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.two_c = g.two_c;
    p.q_row0 = g.q_row0;
    p.nq = (int)g.nq;
    p.nk = (int)g.nk;
    p.hq = g.hq;
    p.hkv = g.hkv;
    p.group = g.hq / g.hkv;
    p.scale = g.scale;
    p.scale_log2 = g.scale_log2;
    p.causal = g.causal ? 1 : 0;
    const int rows_wg = TR * NWB;
    p.ntiles_wg = (int)((g.nq + rows_wg - 1) / rows_wg);
    hipLaunchKernelGGL(attn_bwd_dq, dim3((unsigned)((int64_t)p.ntiles_wg * g.hq * g.b)),
                       dim3(64 * NWB), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.ntiles_wg = (int)((g.nk + rows_wg - 1) / rows_wg);
    hipLaunchKernelGGL(attn_bwd_dkdv, dim3((unsigned)((int64_t)p.ntiles_wg * g.hkv * g.b)),
                       dim3(64 * NWB), 0, stream, p);
    return hipGetLastError();
}

}  // namespace cpattn
