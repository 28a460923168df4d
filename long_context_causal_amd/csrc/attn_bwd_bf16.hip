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
    int b, nq, nk, hq, hkv, group, ntiles_wg, head_splits;
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
// dK, dV: workgroup = 8 waves on 128 keys of one (batch, KV head).  Waves
// 0-3 ("P waves") own 32 keys each with K as B operand: S = Q K^T, P, and
// dV^T += dO^T P; each hands its fp32 P to LDS.  Waves 4-7 ("dS waves") own
// the same keys with V as B operand and run one tile behind: dP = dO V^T,
// dS = P (dP - D) with the P handed over, dK^T += Q^T dS.  Every product is
// computed once, and each wave fits in half the register file, so the two
// waves of a key group share a SIMD and overlap their vector and matrix work.
// The workgroup streams 32-row tiles of Q and dO (with L and D) for hpw
// query heads of the group; the group's heads are split over head_splits
// workgroups, which sum into dk, dv with fp32 atomics.
constexpr int NWK = 8;                         // waves per dK/dV workgroup
constexpr int KW = 4;                          // key groups of 32 per workgroup
constexpr int TBUF = 4 * TB + 2 * TR * 4;      // one tile: Q R, Q T, dO R, dO T, L, D
constexpr int PSLAB = 64 * 16 * 4;             // one key group's fp32 P of a tile
constexpr int DKDV_LDS = 3 * TBUF + 2 * KW * PSLAB;

__global__ void __launch_bounds__(64 * NWK) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[DKDV_LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool ds_wave = wave >= KW;           // wave-uniform role
    const int kwave = wave & (KW - 1);
    const int hi = lane >> 5, l32 = lane & 31;
    // longest (causal: first) key blocks are dispatched first
    int item = blockIdx.x;
    const int inner = p.head_splits * p.hkv * p.b;
    const int kt = item / inner;
    item %= inner;
    const int hs = item % p.head_splits;
    item /= p.head_splits;
    const int g = item % p.hkv;
    const int n = item / p.hkv;
    const int hpw = p.group / p.head_splits;   // query heads of this workgroup
    const int h0 = g * p.group + hs * hpw;
    const int k0 = kt * TR * KW;
    const int wkey0 = k0 + kwave * TR;

    LaneOffsets L;
    L.init(lane);
    const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
    float *pslab0 = (float *)(lds + 3 * TBUF + kwave * PSLAB);

    // this lane's key: K (P waves) or V (dS waves) as B operands
    const int key = wkey0 + l32;
    const int kr = min(key, p.nk - 1);
    const int64_t koff = ((n * p.two_c + kr) * (int64_t)p.hkv + g) * D;
    bf16x8 bf[D / 16];
    load_b_rows((ds_wave ? p.v : p.k) + koff, hi, bf);
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

    // query tiles: rows from the first one that can see this workgroup's
    // keys (causal: row >= key) to the end, for each of the hpw heads
    const int qstart = p.causal ? (k0 / TR) : 0;
    const int nqt = (p.nq + TR - 1) / TR;
    const int per_head = max(nqt - qstart, 0);
    const int ntiles = per_head * hpw;
    u32x4 qreg, dreg;
    float lreg = 0.0f, dreg1 = 0.0f;
    auto gload = [&](int u) {
        const int head = h0 + u / per_head;
        const int qt = qstart + u % per_head;
        const int row = min(qt * TR + tid / 16, p.nq - 1);
        const int64_t off = ((n * p.two_c + p.q_row0 + row) * (int64_t)p.hq + head) * D;
        qreg = *(const u32x4 *)(p.q + off + (tid & 15) * 8);
        dreg = *(const u32x4 *)(p.dout + off + (tid & 15) * 8);
        if (tid < TR) {
            const int lrow_q = min(qt * TR + tid, p.nq - 1);
            const int64_t lrow = ((int64_t)n * p.hq + head) * p.two_c + p.q_row0 + lrow_q;
            lreg = p.lse[lrow] * 1.4426950408889634f;
            dreg1 = p.delta[lrow];
        }
    };
    auto lstore = [&](int buf) {
        char *base = lds + buf * TBUF;
        const int r = tid / 16, c = tid & 15;
        *(u32x4 *)(base + r_off(r, c)) = qreg;
        *(u32x4 *)(base + TB + t_off(r, c)) = qreg;
        *(u32x4 *)(base + 2 * TB + r_off(r, c)) = dreg;
        *(u32x4 *)(base + 3 * TB + t_off(r, c)) = dreg;
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
    // iteration it: P waves on tile it, dS waves on tile it - 1; tile u sits
    // in buffer u % 3 and its P in slab u % 2
    int buf_p = 0, buf_ds = 2, buf_next = 1;
    for (int it = 0; ntiles > 0 && it <= ntiles; ++it) {
        if (it + 1 < ntiles) gload(it + 1);
        const int u = ds_wave ? it - 1 : it;
        const int q0 = (qstart + (u < 0 ? 0 : u) % per_head) * TR;
        // the tile exists and some row of it sees the wave's keys
        if (u >= 0 && u < ntiles && (!p.causal || q0 + TR - 1 >= wkey0)) {
            const int buf = ds_wave ? buf_ds : buf_p;
            const unsigned sT = lbase + buf * TBUF;
            const char *lb = lds + buf * TBUF + 4 * TB;
            float *slab = pslab0 + (u & 1) * (KW * PSLAB / 4);
            bf16x8 ob[2];
            if (!ds_wave) {
                f32x16 s = {};
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
                    s = MFMA(k_read(sT + L.roff[kk]), bf[kk], s, 0, 0, 0);
                f32x16 pv;
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    const f32x8 lv = *(const f32x8 *)(lb + (16 * qc + 8 * hi) * 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = q0 + 16 * qc + 8 * hi + e;
                        const bool vis = row < p.nq && key < p.nk && (!p.causal || key <= row);
                        pv[qc * 8 + e] =
                            vis ? __builtin_amdgcn_exp2f(
                                      __builtin_fmaf(s[qc * 8 + e], p.scale_log2, -lv[e]))
                                : 0.0f;
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(f32x4 *)(slab + (j * 64 + lane) * 4) =
                        f32x4{pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]};
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    f32x8 h;
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = pv[qc * 8 + e];
                    ob[qc] = __builtin_convertvector(h, bf16x8);
                }
            } else {
                f32x16 dp = {};
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk)
                    dp = MFMA(k_read(sT + 2 * TB + L.roff[kk]), bf[kk], dp, 0, 0, 0);
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    const f32x8 dv8 = *(const f32x8 *)(lb + TR * 4 + (16 * qc + 8 * hi) * 4);
                    const f32x4 pa = *(const f32x4 *)(slab + ((2 * qc) * 64 + lane) * 4);
                    const f32x4 pb = *(const f32x4 *)(slab + ((2 * qc + 1) * 64 + lane) * 4);
                    f32x8 ds;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ds[e] = pa[e] * (dp[qc * 8 + e] - dv8[e]);
                        ds[4 + e] = pb[e] * (dp[qc * 8 + 4 + e] - dv8[4 + e]);
                    }
                    ob[qc] = __builtin_convertvector(ds, bf16x8);
                }
            }
            // P waves: dV^T += dO^T P;  dS waves: dK^T += Q^T dS
            const unsigned sA = sT + (ds_wave ? TB : 3 * TB);
#pragma unroll
            for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    acc[dt] = MFMA(vt_read(sA + L.toff[dt] + qc * 16 * RB), ob[qc], acc[dt], 0,
                                   0, 0);
        }
        if (it + 1 < ntiles) lstore(buf_next);
        __syncthreads();
        buf_ds = buf_p;
        buf_p = buf_next;
        buf_next = buf_next == 2 ? 0 : buf_next + 1;
    }

    // dv += dV (P waves), dk += scale dK (dS waves); lane holds head dims
    // dt*32 + 8*i + 4*hi + j.  Split heads add with atomics.
    if (key < p.nk && ntiles > 0) {
        float *dst = (ds_wave ? p.dk : p.dv) + koff + 4 * hi;
        const float f = ds_wave ? p.scale : 1.0f;
        if (p.head_splits == 1) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 *a = (f32x4 *)(dst + dt * 32 + i * 8);
                    f32x4 w = *a;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] += f * acc[dt][i * 4 + j];
                    *a = w;
                }
        } else {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        unsafeAtomicAdd(dst + dt * 32 + i * 8 + j, f * acc[dt][i * 4 + j]);
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
    p.b = (int)g.b;
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
    // key tiles of TR * KW keys; the group's heads split so the grid has
    // at least ~2 workgroups per CU (heads per workgroup divides the group)
    p.ntiles_wg = (int)((g.nk + TR * KW - 1) / (TR * KW));
    const int64_t base_wgs = (int64_t)p.ntiles_wg * g.hkv * g.b;
    p.head_splits = 1;
    while (p.head_splits < p.group && p.group % (p.head_splits * 2) == 0 &&
           base_wgs * p.head_splits < 512)
        p.head_splits *= 2;
    hipLaunchKernelGGL(attn_bwd_dkdv, dim3((unsigned)(base_wgs * p.head_splits)),
                       dim3(64 * NWK), 0, stream, p);
    return hipGetLastError();
}

}  // namespace cpattn
