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
// ds_read_b64_tr_b16).  One XOR swizzle keeps both reads free of bank
// conflicts: 16-byte chunk c of tile row r sits at chunk c ^ u_swz(r), with
// u_swz(r) = 4 (r % 4) + (r / 4) % 4 (256-byte rows, d = 128; 128-byte rows,
// d = 64, use h_swz).  Every kernel is a template over the head dimension
// d = 64 or 128.  Tiles are copied global -> LDS
// directly (global_load_lds, no register round trip) several tiles ahead of
// their use into a ring of stages; each lane copies fixed chunks, chosen so
// that the copy's linear LDS order is the swizzled layout.  One barrier per
// tile.  The MFMAs are compiler builtins, so the compiler pads every hazard.
#include "internal.h"
#include "mfma_tiles.h"

#include <math.h>


namespace cpattn {
namespace {

using namespace tiles;

constexpr int TR = 32;                     // rows of a streamed tile; rows (keys) per wave
constexpr float LOG2E = 1.4426950408889634f;
// Tile geometry for head dimension D (bf16 rows of D): bytes per tile row and
// per tile, and the 1 KB copies (64 lanes x 16 bytes) of a tile.
template <int D>
struct TileGeo {
    static_assert(D == 64 || D == 128, "head dimension");
    static constexpr int RB = 2 * D;          // bytes per tile row
    static constexpr int TB = TR * RB;        // bytes per tile
    static constexpr int CPR = RB / 16;       // 16-byte chunks per row
    static constexpr int RPC = 64 / CPR;      // rows per copy
    static constexpr int NCOPY = TR / RPC;    // copies per tile
};

struct BwdParams {
    const uint16_t *q, *k, *v, *dout;   // q_r, dout_r [b, T, hq, d]; k, v [b, T, hkv, d]
    const float *lse, *delta;           // the rank's final L (natural log) and D [b, hq, T]
    float *dq, *dk, *dv;                // accumulated: dq [b, T, hq, d]; dk, dv [b, T, hkv, d]
    int64_t two_c;                      // T: local rows per batch element
    int b, hq, hkv, group, head_splits;
    float scale, scale_log2;
    int mode;                           // the step's mode (same for every sample)
    // the rank's whole share in one grid (dq): k, v are rank 0's blocks of
    // the partitioned K, V, block_elems apart
    int rank, cp;
    int64_t block_elems;
    SeqTable tab;                       // packed samples; tile0: this kernel's tiles
};

// One sample's rows and keys in a step of the given mode: query rows
// [qrow0, qrow0 + nq) and keys [kv0, kv0 + nk) of the local blocks (key j
// visible to row i only if j <= i, both counted from the sample start, when
// causal).
struct Geo {
    int qrow0, kv0, nq, nk;
    bool causal;
};
__device__ __forceinline__ Geo geo_of(const BwdParams &p, int i, int mode) {
    const int l0 = p.tab.lcu[i], c = (p.tab.lcu[i + 1] - l0) >> 1;
    Geo G;
    G.kv0 = l0;
    G.causal = mode == CPATTN_CAUSAL;
    G.qrow0 = mode == CPATTN_Q_SECOND_HALF ? l0 + c : l0;
    G.nq = mode == CPATTN_Q_SECOND_HALF ? c : 2 * c;
    G.nk = mode == CPATTN_KV_FIRST_HALF ? c : 2 * c;
    return G;
}

__device__ __forceinline__ int u_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// The same for 128-byte rows (D = 64: 8 chunks, two rows per pass over the
// 64 banks): chunk c of row r sits at c ^ h_swz(r), h_swz(r) = 4 (r/2 mod 2)
// + (r/4 mod 4).  A row-chunk read's 16 lanes (rows swap_bits23(0..15) or
// 16..31) cover the 8 chunk slots of each row parity once; a transposed
// read's 32 lanes take rows 4s + 0..3 (+8), whose two rows of one parity
// fall in opposite halves of the row.
__device__ __forceinline__ int h_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// The lane's LDS byte offsets in a swizzled tile, kept as a few bases and
// XOR masks (the swizzle is an XOR, so each offset is one v_xad):
//   row operand of k-step kk (row r = swap_bits23(l32), chunk 2 kk + hi):
//     r*RB + 32 ((kk ^ g)) + 16 (hi ^ (f & 1)),  f = u_swz(r), g = f >> 1;
//   transposed read s of head-dim tile dt (row 8 (lane/32) + 4 s + j,
//   chunk 4 dt + x, byte 8 (lane & 1)): tb[s] + 64 (dt ^ (f' >> 2)), where
//   f' = u_swz(row) (rows +0 and +4 differ only in bit 0 of f');
// add kc * 16 * RB for the second 16-row chunk, which has the same swizzle.
template <int D>
struct LaneOffsets {
    static constexpr int RB = TileGeo<D>::RB;
    unsigned rbase, rmask, tb[2], tmask;
    __device__ __forceinline__ void init(int lane) {
        const int hi = lane >> 5, l32 = lane & 31;
        const int r = swap_bits23(l32);
        const int f = u_swz(r);
        rbase = r * RB + 16 * (hi ^ (f & 1));
        rmask = (unsigned)(f >> 1) << 5;
        const int vg = lane >> 4, vj = (lane >> 2) & 3, vq = lane & 3;
        const int x = 2 * (vg & 1) + (vq >> 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = 8 * (vg >> 1) + 4 * s + vj;
            tb[s] = row * RB + (((x ^ u_swz(row)) & 3) << 4) + (vq & 1) * 8;
        }
        tmask = (unsigned)(u_swz(8 * (vg >> 1) + vj) >> 2) << 6;
    }
    __device__ __forceinline__ unsigned roff(int kk) const { return ((kk << 5) ^ rmask) + rbase; }
    __device__ __forceinline__ unsigned toff(int dt, int s) const {
        return ((dt << 6) ^ tmask) + tb[s];
    }
};
// 128-byte rows: the offsets written out (the lane's row and chunk as for
// 256-byte rows, the h_swz swizzle).
template <>
struct LaneOffsets<64> {
    static constexpr int RB = TileGeo<64>::RB;
    int lane_;
    __device__ __forceinline__ void init(int lane) { lane_ = lane; }
    __device__ __forceinline__ unsigned roff(int kk) const {
        const int hi = lane_ >> 5, r = swap_bits23(lane_ & 31);
        return (unsigned)(r * RB + (((2 * kk + hi) ^ h_swz(r)) << 4));
    }
    __device__ __forceinline__ unsigned toff(int dt, int s) const {
        const int vg = lane_ >> 4, vj = (lane_ >> 2) & 3, vq = lane_ & 3;
        const int x = 2 * (vg & 1) + (vq >> 1);
        const int row = 8 * (vg >> 1) + 4 * s + vj;
        return (unsigned)(row * RB + (((4 * dt + x) ^ h_swz(row)) << 4) + (vq & 1) * 8);
    }
};

// Transposed operand from two row blocks (see vt_read).
__device__ __forceinline__ bf16x8 vt_read2(unsigned a0, unsigned a1) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)a0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)a1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copy of 4 tile rows (1 KB: rows 4m .. 4m+3 of a tile, m the copy's index
// in the tile) into the swizzled layout: lane L lands on row 4m + L/16,
// chunk L%16, so it loads chunk (L%16) ^ u_swz(row) of that row.  Returns
// the lane's byte offset from the copy's first row; u_swz(row) depends on m
// only through m % 4.
// With 128-byte rows (D = 64) a copy is 8 rows: lane L lands on row 8m + L/8,
// chunk L%8, and loads chunk (L%8) ^ h_swz(row).
template <int D>
__device__ __forceinline__ unsigned copy_offset(int lane, int m, int64_t row_bytes) {
    if constexpr (D == 64) {
        const int r = lane >> 3;
        return (unsigned)(r * row_bytes) + (((lane & 7) ^ h_swz(8 * m + r)) << 4);
    } else {
        const int r = lane >> 4;
        return (unsigned)(r * row_bytes) + ((((lane & 15) ^ ((r << 2) | (m & 3)))) << 4);
    }
}

// B operand of the D/16 k-steps for one row (this lane's l32-th row of a
// 32-row block): row chunks kk*16 + 8*hi .. +7.
template <int D>
__device__ __forceinline__ void load_b_rows(const uint16_t *row, int hi, bf16x8 (&f)[D / 16]) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        f[kk] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(row + kk * 16 + hi * 8));
}

// Makes the compiler wait for the load of x here, before the tile loop, so
// that no wait for it is left inside the loop.
template <class T>
__device__ __forceinline__ void settle(const T &x) {
    asm volatile("" ::"v"(x));
}
template <class T, int N>
__device__ __forceinline__ void settle(const T (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) settle(x[i]);
}

// x as computed, held in a VGPR: a constant added to it afterwards goes into
// the LDS instruction's offset field instead of a new add of the stage base.
__device__ __forceinline__ unsigned pin(unsigned x) {
    asm volatile("" : "+v"(x));
    return x;
}

#define MFMA __builtin_amdgcn_mfma_f32_32x32x16_bf16

// Issues one wave's copy m of a 32-row tile (rows [RPC m, RPC m + RPC))
// whose first row is row0 (of n rows; rows past n repeat row n-1) from the
// row array base (row stride row_bytes) into the stage tile at sdst.  off:
// the lane's copy_offset for m.
template <int D>
__device__ __forceinline__ void copy_rows(const uint16_t *base, int64_t row_bytes, int row0,
                                          int n, int m, unsigned off, unsigned sdst, int lane) {
    constexpr int RPC = TileGeo<D>::RPC;
    if (row0 + TR <= n) {
        dma16((const char *)base + (row0 + RPC * m) * row_bytes, off, sdst + m * 1024);
    } else {
        // base row b0 <= every row copied, so lane offsets stay >= 0
        const int b0 = max(min(row0, n - TR), 0);
        const int r = lane / (64 / RPC);
        const int row = min(row0 + RPC * m + r, n - 1);
        const unsigned o = off + (unsigned)((row - b0 - r) * row_bytes);
        dma16((const char *)base + b0 * row_bytes, o, sdst + m * 1024);
    }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = NW waves (4 or 8) x 32 query rows of one (batch, head);
// 32-key tiles of K and V stream through NSQ stages, PDQ tiles ahead.  Wave
// w issues copy w (and, with 4 waves at d = 128, copy w + 4) of both tiles;
// a copy is 4 rows at d = 128 and 8 at d = 64.  With 8 waves (d = 128 only)
// a copied tile serves twice the rows (one workgroup per CU instead of
// two); the share's launcher takes 8 when that still leaves two workgroups
// per CU.
constexpr int NWB = 4;                     // waves of the single step's dq
constexpr int NSQ = 4;
constexpr int PDQ = NSQ - 1;
template <int D>
constexpr int stage_dq() { return 2 * TileGeo<D>::TB; }   // K, V

// A cursor over the 32-key tiles a dQ workgroup streams for its query rows,
// one step per tile: the K, V base of the current key block (this batch
// element and KV head, at the sample's first key), the tile's first key, the
// block's keys streamed (rows past them repeat its last), and which rows see
// the block: every row, only rows >= c (the second chunk), or rows >= key
// (causal, both counted from the sample start).
enum : int { SEE_ALL = 0, SEE_SECOND = 1, SEE_CAUSAL = 2 };
struct DqCursor {
    const uint16_t *kb, *vb;
    int key0, nk, see, left;   // left: blocks of this kind after the current one
};

// One step (cpattn_step_bwd's dq launch): the sample's rows and keys of the
// step's mode, one block.
template <int D>
struct DqStepPlan {
    static constexpr int kD = D;
    const uint16_t *kb, *vb;
    int qrow0, nq, nk, ntiles;
    bool causal;
    static constexpr int c = 0;   // no block is seen by the second chunk only
    __device__ __forceinline__ void init(const BwdParams &p, int smp, int q0, int n, int g,
                                         int tile_rows) {
        const Geo G = geo_of(p, smp, p.mode);
        qrow0 = G.qrow0;
        nq = G.nq;
        nk = G.nk;
        causal = G.causal;
        kb = p.k + (((int64_t)n * p.two_c + G.kv0) * p.hkv + g) * D;
        vb = p.v + (((int64_t)n * p.two_c + G.kv0) * p.hkv + g) * D;
        const int kend = causal ? min(nk, q0 + tile_rows) : nk;
        ntiles = (kend + TR - 1) / TR;
    }
    __device__ __forceinline__ DqCursor first() const {
        return DqCursor{kb, vb, 0, nk, causal ? SEE_CAUSAL : SEE_ALL, 0};
    }
    __device__ __forceinline__ void next(DqCursor &C) const { C.key0 += TR; }
};

// A rank's whole share for one query tile (the dq of all cp steps in one
// grid): the sample's 2c local rows, and in streaming order the key
// blocks of its steps -- steps 1 .. r (kv_first_half: keys [0, c) of the
// blocks of ranks r-1 .. 0), steps r+1 .. cp-1 (q_second_half: keys
// [0, 2c) of ranks cp-1 .. r+1, seen by rows c .. 2c-1 only; streamed only
// when the tile has such rows), then step 0 (the rank's own block,
// causal).  dQ of every step sums in the same accumulator.
template <int D>
struct DqSharePlan {
    static constexpr int kD = D;
    const uint16_t *k0, *v0;
    int64_t block;
    int r, cp, c, nAB, kend, ntiles;
    int qrow0, nq;
    __device__ __forceinline__ void init(const BwdParams &p, int smp, int q0, int n, int g,
                                         int tile_rows) {
        const int l0 = p.tab.lcu[smp];
        c = (p.tab.lcu[smp + 1] - l0) >> 1;
        qrow0 = l0;
        nq = 2 * c;
        k0 = p.k + (((int64_t)n * p.two_c + l0) * p.hkv + g) * D;
        v0 = p.v + (((int64_t)n * p.two_c + l0) * p.hkv + g) * D;
        block = p.block_elems;
        r = p.rank;
        cp = p.cp;
        const int cA = (c + TR - 1) / TR, cB = (2 * c + TR - 1) / TR;
        nAB = (q0 + tile_rows > c) ? cp - 1 - r : 0;
        kend = min(2 * c, q0 + tile_rows);
        ntiles = r * cA + nAB * cB + (kend + TR - 1) / TR;
    }
    __device__ __forceinline__ DqCursor block_of(int see) const {
        if (see == SEE_SECOND) {
            const int64_t off = (int64_t)(cp - 1) * block;
            return DqCursor{k0 + off, v0 + off, 0, 2 * c, SEE_SECOND, nAB - 1};
        }
        const int64_t off = (int64_t)r * block;
        return DqCursor{k0 + off, v0 + off, 0, kend, SEE_CAUSAL, 0};
    }
    __device__ __forceinline__ DqCursor first() const {
        if (r > 0) {
            const int64_t off = (int64_t)(r - 1) * block;
            return DqCursor{k0 + off, v0 + off, 0, c, SEE_ALL, r - 1};
        }
        return block_of(nAB > 0 ? SEE_SECOND : SEE_CAUSAL);
    }
    // the next tile (only called while one is left)
    __device__ __forceinline__ void next(DqCursor &C) const {
        C.key0 += TR;
        if (C.key0 < C.nk) return;
        if (C.left > 0) {   // the block of the next lower rank, same kind
            --C.left;
            C.kb -= block;
            C.vb -= block;
            C.key0 = 0;
            return;
        }
        C = block_of(C.see == SEE_ALL && nAB > 0 ? SEE_SECOND : SEE_CAUSAL);
    }
};

// PREP: p.lse and p.delta hold -L/scale and -D (launch_bwd_prep) instead
// of L and D.
template <class Plan, bool ACCUMULATE, bool PREP, int NW>
__device__ __forceinline__ void dq_body(const BwdParams &p, char *lds) {
    constexpr int D = Plan::kD;
    constexpr int RB = TileGeo<D>::RB, TB = TileGeo<D>::TB, RPC = TileGeo<D>::RPC;
    constexpr int STAGE_DQ = stage_dq<D>();
    constexpr int CPW = TileGeo<D>::NCOPY / NW;   // copies per wave and tensor per tile
    static_assert(CPW >= 1 && CPW * NW == TileGeo<D>::NCOPY, "copy split");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hi = lane >> 5, l32 = lane & 31;
    // workgroup -> (head in group, query tile, KV group, batch), fastest
    // first.  The dispatcher deals workgroups to the 8 XCDs round robin;
    // reordered so each XCD takes a contiguous run (the heads of a KV group,
    // which stream the same K/V, share its L2), and inside the run the
    // longest (causal: last) query tiles start first.
    int item = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) item = (item & 7) * (nblk >> 3) + (item >> 3);
    const int nqt = p.tab.tile0[p.tab.nseq];   // query tiles of all samples
    const int hh = item % p.group;
    item /= p.group;
    const int qt_all = nqt - 1 - item % nqt;
    item /= nqt;
    const int g = item % p.hkv;
    const int n = item / p.hkv;
    const int head = g * p.group + hh;
    const int smp = seq_of(p.tab.tile0, p.tab.nseq, qt_all);
    const int qt = qt_all - p.tab.tile0[smp];
    const int q0 = qt * TR * NW;
    const int wrow0 = q0 + wave * TR;
    Plan P;
    P.init(p, smp, q0, n, g, TR * NW);
    const int ntiles = P.ntiles;

    LaneOffsets<D> L;
    L.init(lane);
    const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

    // this lane's query row: Q and dO as B operands, L (log2) and D
    const int qrow = wrow0 + l32;
    const int qr = min(qrow, P.nq - 1);
    const int64_t qoff = ((n * p.two_c + P.qrow0 + qr) * (int64_t)p.hq + head) * D;
    bf16x8 qf[D / 16], df[D / 16];
    load_b_rows<D>(p.q + qoff, hi, qf);
    load_b_rows<D>(p.dout + qoff, hi, df);
    const int64_t lrow = ((int64_t)n * p.hq + head) * p.two_c + P.qrow0 + qr;
    const float lq = PREP ? -p.lse[lrow] * p.scale_log2 : p.lse[lrow] * LOG2E;
    const float dq_d = PREP ? -p.delta[lrow] : p.delta[lrow];
    settle(qf);
    settle(df);
    settle(lq);
    settle(dq_d);
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

    const int64_t row_bytes = (int64_t)p.hkv * D * 2;
    const unsigned coff = copy_offset<D>(lane, wave, row_bytes);   // m = wave (+ NW)
    // copy cursor (tile cu); tiles past the last repeat it, so every wave
    // issues 2 CPW copies per tile
    DqCursor CC = P.first();
    int cu = 0;
    auto issue = [&](int stage) {
        const unsigned sb = lbase + stage * STAGE_DQ;
        if (CC.key0 + TR <= CC.nk) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int m = wave + NW * i;
                dma16((const char *)CC.kb + (CC.key0 + RPC * m) * row_bytes, coff,
                      sb + m * 1024);
                dma16((const char *)CC.vb + (CC.key0 + RPC * m) * row_bytes, coff,
                      sb + TB + m * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                copy_rows<D>(CC.kb, row_bytes, CC.key0, CC.nk, wave + NW * i, coff, sb, lane);
                copy_rows<D>(CC.vb, row_bytes, CC.key0, CC.nk, wave + NW * i, coff, sb + TB,
                             lane);
            }
        }
    };
    auto advance = [&]() {
        if (cu + 1 < ntiles) {
            ++cu;
            P.next(CC);
        }
    };
    if (ntiles > 0) {
#pragma unroll
        for (int i = 0; i < PDQ; ++i) {
            issue(i);
            advance();
        }
        wait_vmcnt<2 * CPW * (PDQ - 1)>();
    }
    lds_barrier();
    // the lane's LDS read offsets in a tile (the stage base is added per read)
    unsigned ro[D / 16], to[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) ro[kk] = L.roff(kk);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        to[dt][0] = L.toff(dt, 0);
        to[dt][1] = L.toff(dt, 1);
    }
    DqCursor T = P.first();   // compute cursor: tile t
    int stage = 0;
    const bool rows_live = wrow0 < P.nq;   // a wave past the sample's rows idles
    const int c_half = P.c;
    for (int t = 0; t < ntiles; ++t) {
        int ns = stage + PDQ;
        if (ns >= NSQ) ns -= NSQ;
        issue(ns);
        advance();
        const bool comp = rows_live && (T.see == SEE_ALL ||
                                        (T.see == SEE_SECOND ? wrow0 + TR - 1 >= c_half
                                                             : T.key0 <= wrow0));
        if (comp) {
            const unsigned sK = lbase + stage * STAGE_DQ;
            // the tile's LDS operands are read ahead of the products
            // (the transposed K^T reads go out behind the S, dP products)
            bf16x8 ak[D / 16], av[D / 16], at[2][D / 32];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const unsigned a = pin(sK + ro[kk]);
                ak[kk] = k_read(a);
                av[kk] = k_read(a + TB);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                s = MFMA(ak[kk], qf[kk], s, 0, 0, 0);
                dp = MFMA(av[kk], df[kk], dp, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            unsigned ta[D / 32][2];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                ta[dt][0] = pin(sK + to[dt][0]);
                ta[dt][1] = pin(sK + to[dt][1]);
            }
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    at[kc][dt] = vt_read2(ta[dt][0] + kc * 16 * RB, ta[dt][1] + kc * 16 * RB);
            __builtin_amdgcn_sched_barrier(0);
            const int key0 = T.key0;
            // tile entirely visible to the wave's rows: no mask
            const bool full = key0 + TR <= T.nk &&
                              (T.see != SEE_CAUSAL || key0 + TR - 1 <= wrow0) &&
                              (T.see != SEE_SECOND || wrow0 >= c_half);
            bf16x8 dsb[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                f32x8 x, ds;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(s[kc * 8 + e], p.scale_log2, -lq);
                if (!full) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int key = key0 + 16 * kc + 8 * hi + e;
                        const bool vis = key < T.nk && (T.see != SEE_CAUSAL || key <= qrow) &&
                                         (T.see != SEE_SECOND || qrow >= c_half);
                        x[e] = vis ? x[e] : -INFINITY;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    ds[e] = __builtin_amdgcn_exp2f(x[e]) * (dp[kc * 8 + e] - dq_d);
                dsb[kc] = __builtin_convertvector(ds, bf16x8);
            }
            // dQ^T += K^T dS^T
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    acc[dt] = MFMA(at[kc][dt], dsb[kc], acc[dt], 0, 0, 0);
        }
        wait_vmcnt<2 * CPW * (PDQ - 1)>();   // tile t + 1 has landed
        lds_barrier();
        stage = stage + 1 == NSQ ? 0 : stage + 1;
        if (t + 1 < ntiles) P.next(T);
    }
    wait_vmcnt<0>();

    // dq[row] (+)= scale * dQ: lane holds head dims dt*32 + 8*i + 4*hi + j
    if (qrow < P.nq) {
        float *dst = p.dq + qoff + 4 * hi;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 *a = (f32x4 *)(dst + dt * 32 + i * 8);
                f32x4 w = ACCUMULATE ? *a : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] += p.scale * acc[dt][i * 4 + j];
                *a = w;
            }
    }
}

// One step's dq (accumulated into dq).
template <int D>
__global__ void __launch_bounds__(64 * NWB) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[NSQ * stage_dq<D>()];
    dq_body<DqStepPlan<D>, true, false, NWB>(p, lds);
}

// The dq of all cp steps of a rank's share in one grid: a workgroup streams
// every step's keys for its query tile and writes dq once.
template <int NW, int D>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_share(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[NSQ * stage_dq<D>()];
    dq_body<DqSharePlan<D>, false, true, NW>(p, lds);
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
// query heads of the group through NSK stages, PDK tiles ahead; the group's
// heads are split over head_splits workgroups, which sum into dk, dv with
// fp32 atomics.  Only the dS waves copy (the P waves carry the exp): dS wave
// 4 + w copies rows 8w .. 8w+7 of Q and dO and the tile's L (lanes 0-31)
// and D (lanes 32-63) into the stage's L/D slot.
constexpr int NWK = 8;                         // waves per dK/dV workgroup
constexpr int KW = 4;                          // key groups of 32 per workgroup
constexpr int NSK = 5;                         // stages: PDK ahead + the two tiles in use
constexpr int PDK = NSK - 2;
constexpr int LD_SLOT = 1024;                  // the tile's L and D (256 bytes used)
constexpr int PSLAB = 64 * 16 * 4;             // one key group's fp32 P of a tile
template <int D>
constexpr int stage_dkdv() { return 2 * TileGeo<D>::TB + LD_SLOT; }   // Q, dO, L/D
template <int D>
constexpr int dkdv_lds() { return NSK * stage_dkdv<D>() + 2 * KW * PSLAB; }

// What a dK/dV workgroup takes from its step: the source block's K and V,
// where its dK and dV go, the mode, and over how many workgroups the
// group's heads are split.
struct KvStep {
    const uint16_t *k, *v;
    float *dk, *dv;
    int mode, head_splits;
    const int32_t *tile0;   // first key tile of each sample in this mode
};

// The dK/dV workgroup 'item' of one step (item as blockIdx.x of that
// step's own launch).
// PREP: p.lse and p.delta hold -L/scale and -D (launch_bwd_prep): they
// start the sums of S and dP, so that S already holds q.k - L/scale and dP
// holds dO.v - D.
template <bool PREP, int D>
__device__ __forceinline__ void dkdv_item(const BwdParams &p, const KvStep &io, int item,
                                          char *lds) {
    constexpr int RB = TileGeo<D>::RB, TB = TileGeo<D>::TB;
    constexpr int STAGE_DKDV = stage_dkdv<D>();
    // dS wave cw copies rows 8 cw .. 8 cw + 7 of Q and of dO: CPT copies of
    // each (two of 4 rows at D = 128, one of 8 at D = 64), and the L/D slot
    constexpr int CPT = 8 / TileGeo<D>::RPC;
    constexpr int NCP = 2 * CPT + 1;           // copies per dS wave per tile
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool ds_wave = wave >= KW;           // wave-uniform role
    const int kwave = wave & (KW - 1);
    const int hi = lane >> 5, l32 = lane & 31;
    // longest (causal: first) key blocks are dispatched first
    const int inner = io.head_splits * p.hkv * p.b;
    const int kt_all = item / inner;
    const int smp = seq_of(io.tile0, p.tab.nseq, kt_all);
    const Geo G = geo_of(p, smp, io.mode);
    const int kt = kt_all - io.tile0[smp];
    item %= inner;
    const int hs = item % io.head_splits;
    item /= io.head_splits;
    const int g = item % p.hkv;
    const int n = item / p.hkv;
    const int hpw = p.group / io.head_splits;   // query heads of this workgroup
    const int h0 = g * p.group + hs * hpw;
    const int k0 = kt * TR * KW;
    const int wkey0 = k0 + kwave * TR;

    LaneOffsets<D> L;
    L.init(lane);
    const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;

    // this lane's key: K (P waves) or V (dS waves) as B operands
    const int key = wkey0 + l32;
    const int kr = min(key, G.nk - 1);
    const int64_t koff = ((n * p.two_c + G.kv0 + kr) * (int64_t)p.hkv + g) * D;
    bf16x8 bf[D / 16];
    load_b_rows<D>((ds_wave ? io.v : io.k) + koff, hi, bf);
    settle(bf);
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

    // query tiles: rows from the first one that can see this workgroup's
    // keys (causal: row >= key) to the end, for each of the hpw heads
    const int qstart = G.causal ? (k0 / TR) : 0;
    const int nqt = (G.nq + TR - 1) / TR;
    const int per_head = max(nqt - qstart, 0);
    const int ntiles = per_head * hpw;
    const int row_first = qstart * TR, row_end = nqt * TR;
    // the lane's LDS read offsets in a tile (the stage base is added per read)
    unsigned ro[D / 16], to[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) ro[kk] = L.roff(kk);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
        to[dt][0] = L.toff(dt, 0);
        to[dt][1] = L.toff(dt, 1);
    }
    const unsigned slab0 = lbase + NSK * STAGE_DKDV + kwave * PSLAB;
    const bool keys_live = wkey0 < G.nk;   // a key group past the last key idles
    // q0: first row of a wave's tile (a compute cursor, one step per tile)
    auto visible = [&](int q0) { return keys_live && (!G.causal || q0 + TR - 1 >= wkey0); };
    auto next_row = [&](int &q0) {
        q0 += TR;
        if (q0 >= row_end) q0 = row_first;
    };

    if (!ds_wave) {
        // P wave, iteration it: tile it (S, P, dV); no copies.
        lds_barrier();
        int st = 0, q0 = row_first;
        for (int it = 0; ntiles > 0 && it <= ntiles; ++it) {
            if (it < ntiles && visible(q0)) {
                const unsigned sT = lbase + st * STAGE_DKDV;
                const unsigned lslot = sT + 2 * TB;
                const unsigned slab = slab0 + (it & 1) * (KW * PSLAB);
                // every LDS operand of the tile is read ahead of its products
                bf16x8 ar[D / 16], at[2][D / 32];
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) ar[kk] = k_read(pin(sT + ro[kk]));
                unsigned ta[D / 32][2];
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    ta[dt][0] = pin(sT + TB + to[dt][0]);
                    ta[dt][1] = pin(sT + TB + to[dt][1]);
                }
#pragma unroll
                for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
                        at[qc][dt] = vt_read2(ta[dt][0] + qc * 16 * RB, ta[dt][1] + qc * 16 * RB);
                // the L terms of the lane's 16 rows
                f32x16 lv;
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    const f32x8 h = *(const __attribute__((address_space(3))) f32x8 *)(
                        uintptr_t)(lslot + (16 * qc + 8 * hi) * 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) lv[qc * 8 + e] = h[e];
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x16 s = {};
                if (PREP) s = lv;   // -L/scale
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) s = MFMA(ar[kk], bf[kk], s, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                const bool full = q0 + TR <= G.nq && wkey0 + TR <= G.nk &&
                                  (!G.causal || wkey0 + TR - 1 <= q0);
                f32x16 x;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    x[i] = PREP ? s[i] * p.scale_log2
                                : __builtin_fmaf(s[i], p.scale_log2, -LOG2E * lv[i]);
                if (!full) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int row = q0 + 16 * (i >> 3) + 8 * hi + (i & 7);
                        const bool vis = row < G.nq && key < G.nk && (!G.causal || key <= row);
                        x[i] = vis ? x[i] : -INFINITY;
                    }
                }
                f32x16 pv;
#pragma unroll
                for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(x[i]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(__attribute__((address_space(3))) f32x4 *)(uintptr_t)(
                        slab + (j * 64 + lane) * 16) =
                        f32x4{pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]};
                bf16x8 ob[2];
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    f32x8 h;
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = pv[qc * 8 + e];
                    ob[qc] = __builtin_convertvector(h, bf16x8);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
                        acc[dt] = MFMA(at[qc][dt], ob[qc], acc[dt], 0, 0, 0);
            }
            lds_barrier();   // (the dS waves have waited for tile it + 1)
            st = st + 1 == NSK ? 0 : st + 1;
            if (it < ntiles) next_row(q0);
        }
    } else {
        // dS wave, iteration it: copies tile it + PDK, computes tile it - 1
        // (dP, dS, dK) with the P the P wave handed over.
        const int cw = kwave;   // copies rows 8 cw .. 8 cw + 7 of Q and dO
        const int64_t row_bytes = (int64_t)p.hq * D * 2;
        const int64_t row_step = TR * row_bytes;
        const unsigned coff0 = copy_offset<D>(lane, CPT * cw, row_bytes);
        const unsigned coff1 = copy_offset<D>(lane, CPT * cw + CPT - 1, row_bytes);
        // Copy cursor: tile cu of the workgroup (heads in turn, rows in
        // 32-row tiles), as byte pointers to its first row in Q and dO and
        // the index of that row's L and D.  Tiles past the last repeat it,
        // so every dS wave issues NCP copies per tile.
        int cu = 0, cr0 = row_first;
        const int64_t hrow0 = (int64_t)n * p.two_c + G.qrow0;   // row of the sample's query 0
        const char *cq = (const char *)(p.q + (hrow0 * p.hq + h0) * D) + row_first * row_bytes;
        const char *cdo = (const char *)(p.dout + (hrow0 * p.hq + h0) * D) + row_first * row_bytes;
        int64_t cli = ((int64_t)n * p.hq + h0) * p.two_c + G.qrow0 + row_first;
        // the L/D slot: lanes 0-31 copy L, lanes 32-63 D (the same layout);
        // the four dS waves write the same bytes.  The per-lane base is
        // settled here so no wait for its load is left inside the tile loop.
        const float *ld_lane = (hi ? p.delta : p.lse) + l32;
        settle(ld_lane);
        auto issue = [&](int stage) {
            const unsigned sb = lbase + stage * STAGE_DKDV;
            if (cr0 + TR <= G.nq) {
                if constexpr (CPT == 2) {
                    dma16(cq + 8 * cw * row_bytes, coff0, sb + 2 * cw * 1024);
                    dma16(cq + (8 * cw + 4) * row_bytes, coff1, sb + (2 * cw + 1) * 1024);
                    dma16(cdo + 8 * cw * row_bytes, coff0, sb + TB + 2 * cw * 1024);
                    dma16(cdo + (8 * cw + 4) * row_bytes, coff1,
                          sb + TB + (2 * cw + 1) * 1024);
                } else {
                    dma16(cq + 8 * cw * row_bytes, coff0, sb + cw * 1024);
                    dma16(cdo + 8 * cw * row_bytes, coff0, sb + TB + cw * 1024);
                }
                dma4(ld_lane + cli, sb + 2 * TB);
            } else {
                // the last tile of a head crosses the sample's last row: rows
                // past it repeat it
                const int64_t back = (int64_t)cr0 * row_bytes;
                const uint16_t *qb = (const uint16_t *)(cq - back);
                const uint16_t *db = (const uint16_t *)(cdo - back);
                copy_rows<D>(qb, row_bytes, cr0, G.nq, CPT * cw, coff0, sb, lane);
                copy_rows<D>(db, row_bytes, cr0, G.nq, CPT * cw, coff0, sb + TB, lane);
                if constexpr (CPT == 2) {
                    copy_rows<D>(qb, row_bytes, cr0, G.nq, 2 * cw + 1, coff1, sb, lane);
                    copy_rows<D>(db, row_bytes, cr0, G.nq, 2 * cw + 1, coff1, sb + TB, lane);
                }
                dma4(ld_lane - l32 + (cli - cr0) + min(cr0 + l32, G.nq - 1), sb + 2 * TB);
            }
        };
        auto advance = [&]() {
            if (cu + 1 >= ntiles) return;
            ++cu;
            cr0 += TR;
            cq += row_step;
            cdo += row_step;
            cli += TR;
            if (cr0 >= row_end) {   // next head
                const int64_t rows = row_end - row_first;
                cr0 = row_first;
                cq += 2 * D - rows * row_bytes;
                cdo += 2 * D - rows * row_bytes;
                cli += p.two_c - rows;
            }
        };
        if (ntiles > 0) {
#pragma unroll
            for (int i = 0; i < PDK; ++i) {
                issue(i);
                advance();
            }
            wait_vmcnt<NCP * (PDK - 1)>();
        }
        lds_barrier();
        int st = NSK - 1, cst = PDK, q0 = row_first;
        for (int it = 0; ntiles > 0 && it <= ntiles; ++it) {
            issue(cst);
            advance();
            cst = cst + 1 == NSK ? 0 : cst + 1;
            if (it > 0 && visible(q0)) {
                const unsigned sT = lbase + st * STAGE_DKDV;
                const unsigned lslot = sT + 2 * TB;
                const unsigned slab = slab0 + ((it - 1) & 1) * (KW * PSLAB);
                bf16x8 ar[D / 16], at[2][D / 32];
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) ar[kk] = k_read(pin(sT + TB + ro[kk]));
                unsigned ta[D / 32][2];
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    ta[dt][0] = pin(sT + to[dt][0]);
                    ta[dt][1] = pin(sT + to[dt][1]);
                }
#pragma unroll
                for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
                        at[qc][dt] = vt_read2(ta[dt][0] + qc * 16 * RB, ta[dt][1] + qc * 16 * RB);
                // the D terms of the lane's 16 rows
                f32x16 dv;
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    const f32x8 h = *(const __attribute__((address_space(3))) f32x8 *)(
                        uintptr_t)(lslot + TR * 4 + (16 * qc + 8 * hi) * 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) dv[qc * 8 + e] = h[e];
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x16 s = {};
                if (PREP) s = dv;   // -D
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) s = MFMA(ar[kk], bf[kk], s, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                bf16x8 ob[2];
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    const f32x4 pa = *(const __attribute__((address_space(3))) f32x4 *)(
                        uintptr_t)(slab + ((2 * qc) * 64 + lane) * 16);
                    const f32x4 pb = *(const __attribute__((address_space(3))) f32x4 *)(
                        uintptr_t)(slab + ((2 * qc + 1) * 64 + lane) * 16);
                    f32x8 ds;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = qc * 8 + e;
                        ds[e] = pa[e] * (PREP ? s[i] : s[i] - dv[i]);
                        ds[4 + e] = pb[e] * (PREP ? s[i + 4] : s[i + 4] - dv[i + 4]);
                    }
                    ob[qc] = __builtin_convertvector(ds, bf16x8);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
                        acc[dt] = MFMA(at[qc][dt], ob[qc], acc[dt], 0, 0, 0);
            }
            wait_vmcnt<NCP * (PDK - 1)>();   // tile it + 1 has landed
            lds_barrier();
            st = st + 1 == NSK ? 0 : st + 1;
            if (it > 0) next_row(q0);
        }
        wait_vmcnt<0>();
    }

    // dv += dV (P waves), dk += scale dK (dS waves); lane holds head dims
    // dt*32 + 8*i + 4*hi + j.  Split heads add with atomics.
    if (key < G.nk && ntiles > 0) {
        float *dst = (ds_wave ? io.dk : io.dv) + koff + 4 * hi;
        const float f = ds_wave ? p.scale : 1.0f;
        if (io.head_splits == 1) {
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

// One step's dK/dV.
template <int D>
__global__ void __launch_bounds__(64 * NWK) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv(BwdParams p) {
    __shared__ __attribute__((aligned(1024))) char lds[dkdv_lds<D>()];
    dkdv_item<false, D>(p, KvStep{p.k, p.v, p.dk, p.dv, p.mode, p.head_splits, p.tab.tile0},
                        blockIdx.x, lds);
}

// The dK/dV of several steps of one rank's share in one grid.  Each step
// reads its own source block and writes that block's dK/dV contribution,
// which no other step of the share touches, so a workgroup takes all query
// heads of its KV group (no head split, no atomics) and the steps'
// workgroups share the machine instead of running in rounds of equal
// workgroups.  The key tiles of packed samples are numbered sample by
// sample: p.tab.tile0 for the modes that see 2c keys of a sample,
// tile0_half for kv_first_half (c keys).  Workgroups come in runs of key
// tiles of one step that see about the same query rows (a non-causal step
// is one run; each key tile of the causal step, which sees rows from its
// first key on, is a run of its own), laid out by the host longest first.
constexpr int MAX_BWD_STEPS = 32;
constexpr int MAX_KV_RUNS = 64;
struct KvStepDesc {
    const uint16_t *k, *v;
    float *dk, *dv;
    int mode;
};
struct KvRun {
    int step, kt0;            // the step (index into st) and its first key tile
    int item0;                // first workgroup of the run in the grid
};
struct DkdvStepsParams {
    BwdParams p;              // the rank's Q side, dims, scale, sample table
    int32_t tile0_half[CPATTN_MAX_SEQS + 1];
    int nruns;
    KvStepDesc st[MAX_BWD_STEPS];
    KvRun run[MAX_KV_RUNS];
};
static_assert(sizeof(DkdvStepsParams) <= 4096, "kernel arguments");

template <int D>
__global__ void __launch_bounds__(64 * NWK) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_steps(DkdvStepsParams sp) {
    __shared__ __attribute__((aligned(1024))) char lds[dkdv_lds<D>()];
    const int item = blockIdx.x;
    int j = 0;
    while (j + 1 < sp.nruns && sp.run[j + 1].item0 <= item) ++j;
    const KvRun &rn = sp.run[j];
    const KvStepDesc &d = sp.st[rn.step];
    const int inner = sp.p.hkv * sp.p.b;   // workgroups per key tile
    const int w = item - rn.item0;
    dkdv_item<true, D>(sp.p,
                    KvStep{d.k, d.v, d.dk, d.dv, d.mode, 1,
                           d.mode == CPATTN_KV_FIRST_HALF ? sp.tile0_half : sp.p.tab.tile0},
                    (rn.kt0 + w / inner) * inner + w % inner, lds);
}

// ---------------------------------------------------------------------------
// D[n, h, i] = sum_t dO[n, i, h, t] O[n, i, h, t]: one thread per (n, i, h).
// PREP: writes -D, and -L[n, h, i] * inv_scale to nl (the terms the share's
// backward grids start S and dP from).
template <bool PREP, int D>
__global__ void __launch_bounds__(256) bwd_delta(const float *o, const uint16_t *dout,
                                                 float *delta, int64_t rows, int hq,
                                                 int64_t two_c, const float *lse,
                                                 float inv_scale, float *nl) {
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
    const int64_t out = (n * hq + h) * two_c + i;
    if (PREP) {
        delta[out] = -acc;
        nl[out] = -lse[out] * inv_scale;
    } else {
        delta[out] = acc;
    }
}

// x[0 .. n) = 0, 16 bytes per thread (n a multiple of 4).
__global__ void __launch_bounds__(256) fill_zero(float *x, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) ((f32x4 *)x)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace

hipError_t launch_bwd_delta(int64_t b, int64_t two_c, int hq, int d, const float *o,
                            const void *dout, float *delta, hipStream_t stream) {
    const int64_t rows = b * two_c * hq;
    if (rows == 0) return hipSuccess;
    auto *fn = d == 64 ? bwd_delta<false, 64> : bwd_delta<false, 128>;
    hipLaunchKernelGGL(fn, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, o,
                       (const uint16_t *)dout, delta, rows, hq, two_c, nullptr, 0.0f, nullptr);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(int64_t b, int64_t two_c, int hq, int d, const float *o,
                           const void *dout, const float *lse, float inv_scale, float *nl,
                           float *nd, hipStream_t stream) {
    const int64_t rows = b * two_c * hq;
    if (rows == 0) return hipSuccess;
    auto *fn = d == 64 ? bwd_delta<true, 64> : bwd_delta<true, 128>;
    hipLaunchKernelGGL(fn, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, o,
                       (const uint16_t *)dout, nd, rows, hq, two_c, lse, inv_scale, nl);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *x, int64_t n, hipStream_t stream) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, x,
                       n4);
    return hipGetLastError();
}

namespace {
BwdParams make_params(const StepGeom &g, const SeqTable &tab, int mode, const void *q,
                      const void *k, const void *v, const void *dout, const float *lse,
                      const float *delta, float *dq, float *dk, float *dv) {
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
    p.hq = g.hq;
    p.hkv = g.hkv;
    p.b = (int)g.b;
    p.group = g.hq / g.hkv;
    p.scale = g.scale;
    p.scale_log2 = g.scale_log2;
    p.mode = mode;
    p.tab = tab;
    return p;
}

// each sample's query rows (dq: tiles of TR * nw rows) or keys (dK/dV:
// tiles of TR * KW keys) in this mode, into p.tab.tile0; returns the total
int64_t fill_tiles(BwdParams &p, const SeqTable &tab, int mode, bool keys, int nw = NWB) {
    const int per_tile = keys ? TR * KW : TR * nw;
    p.tab.tile0[0] = 0;
    for (int i = 0; i < tab.nseq; ++i) {
        const int c = (tab.lcu[i + 1] - tab.lcu[i]) / 2;
        const int n = keys ? (mode == CPATTN_KV_FIRST_HALF ? c : 2 * c)
                           : (mode == CPATTN_Q_SECOND_HALF ? c : 2 * c);
        p.tab.tile0[i + 1] = p.tab.tile0[i] + (n + per_tile - 1) / per_tile;
    }
    return (int64_t)p.tab.tile0[tab.nseq];
}
}  // namespace

hipError_t launch_step_bwd_bf16(const StepGeom &g, const SeqTable &tab, int mode,
                                const void *q, const void *k, const void *v, const void *dout,
                                const float *lse, const float *delta, float *dq, float *dk,
                                float *dv, hipStream_t stream, bool with_dkdv) {
    BwdParams p = make_params(g, tab, mode, q, k, v, dout, lse, delta, dq, dk, dv);
    const int64_t nqt = fill_tiles(p, tab, mode, false);
    auto *dq_fn = g.d == 64 ? attn_bwd_dq<64> : attn_bwd_dq<128>;
    hipLaunchKernelGGL(dq_fn, dim3((unsigned)(nqt * g.hq * g.b)), dim3(64 * NWB), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !with_dkdv) return e;
    // the group's heads split so the grid has at least ~2 workgroups per CU
    // (heads per workgroup divides the group)
    const int64_t base_wgs = fill_tiles(p, tab, mode, true) * g.hkv * g.b;
    p.head_splits = 1;
    while (p.head_splits < p.group && p.group % (p.head_splits * 2) == 0 &&
           base_wgs * p.head_splits < 512)
        p.head_splits *= 2;
    auto *kv_fn = g.d == 64 ? attn_bwd_dkdv<64> : attn_bwd_dkdv<128>;
    hipLaunchKernelGGL(kv_fn, dim3((unsigned)(base_wgs * p.head_splits)), dim3(64 * NWK), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_share_bf16(const StepGeom &g, const SeqTable &tab, int rank, int cp,
                                    const void *q, const void *kz, const void *vz,
                                    const void *dout, const float *lse, const float *delta,
                                    float *dq, hipStream_t stream) {
    BwdParams p = make_params(g, tab, CPATTN_CAUSAL, q, kz, vz, dout, lse, delta, dq, nullptr,
                              nullptr);
    p.rank = rank;
    p.cp = cp;
    p.block_elems = g.b * g.two_c * g.hkv * g.d;
    // query tiles of the 2c local rows of every sample: 256-row tiles (8
    // waves) when they still give two workgroups per CU and no sample is
    // packed (short samples would leave half of a tile's waves idle), else
    // 128-row ones.  With d = 64 a tile is four copies per tensor, one per
    // wave of 4: always 128-row tiles.
    const int64_t nqt8 = fill_tiles(p, tab, CPATTN_CAUSAL, false, 8);
    if (g.d == 128 && tab.nseq == 1 && nqt8 * g.hq * g.b >= 2 * (int64_t)device_cu_count()) {
        auto *fn8 = attn_bwd_dq_share<8, 128>;
        hipLaunchKernelGGL(fn8, dim3((unsigned)(nqt8 * g.hq * g.b)), dim3(64 * 8), 0, stream, p);
        return hipGetLastError();
    }
    const int64_t nqt = fill_tiles(p, tab, CPATTN_CAUSAL, false, 4);
    auto *fn4 = g.d == 64 ? attn_bwd_dq_share<4, 64> : attn_bwd_dq_share<4, 128>;
    hipLaunchKernelGGL(fn4, dim3((unsigned)(nqt * g.hq * g.b)), dim3(64 * 4), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_steps_bf16(int n, const StepGeom *g, const SeqTable &tab,
                                      const int *mode, const void *q, const void *const *k,
                                      const void *const *v, const void *dout,
                                      const float *lse, const float *delta, float *const *dk,
                                      float *const *dv, hipStream_t stream) {
    for (int j0 = 0; j0 < n; j0 += MAX_BWD_STEPS) {
        const int nb = n - j0 < MAX_BWD_STEPS ? n - j0 : MAX_BWD_STEPS;
        DkdvStepsParams sp = {};
        sp.p = make_params(g[0], tab, CPATTN_CAUSAL, q, nullptr, nullptr, dout, lse, delta,
                           nullptr, nullptr, nullptr);
        const int64_t kt_full = fill_tiles(sp.p, tab, CPATTN_CAUSAL, true);
        BwdParams half = sp.p;
        const int64_t kt_half = fill_tiles(half, tab, CPATTN_KV_FIRST_HALF, true);
        for (int i = 0; i <= tab.nseq; ++i) sp.tile0_half[i] = half.tab.tile0[i];
        // runs: (step, first key tile, key tiles, query rows each key tile sees)
        int rs[MAX_KV_RUNS], rk[MAX_KV_RUNS], rc[MAX_KV_RUNS];
        int64_t rl[MAX_KV_RUNS];
        int nr = 0, ncausal = 0;
        for (int jj = 0; jj < nb; ++jj) ncausal += mode[j0 + jj] == CPATTN_CAUSAL ? 1 : 0;
        const int64_t two_c = g[0].two_c;
        // packed samples: a run per (step, sample) when the table holds them
        const bool per_sample = tab.nseq > 1 && nb * tab.nseq <= MAX_KV_RUNS;
        for (int jj = 0; jj < nb; ++jj) {
            const int i = j0 + jj;
            sp.st[jj] = KvStepDesc{(const uint16_t *)k[i], (const uint16_t *)v[i], dk[i], dv[i],
                                   mode[i]};
            const int nkt = (int)(mode[i] == CPATTN_KV_FIRST_HALF ? kt_half : kt_full);
            if (per_sample) {
                // the sample's key tiles (causal: first tile first) see at
                // most its 2c rows (q_second_half: its second c)
                const int32_t *t0 =
                    mode[i] == CPATTN_KV_FIRST_HALF ? sp.tile0_half : sp.p.tab.tile0;
                for (int q = 0; q < tab.nseq; ++q) {
                    const int64_t two_cq = tab.lcu[q + 1] - tab.lcu[q];
                    rs[nr] = jj;
                    rk[nr] = t0[q];
                    rc[nr] = t0[q + 1] - t0[q];
                    rl[nr++] = mode[i] == CPATTN_Q_SECOND_HALF ? two_cq / 2 : two_cq;
                }
                continue;
            }
            if (mode[i] != CPATTN_CAUSAL || tab.nseq > 1) {
                // every key tile sees the same rows (kv_first_half: all 2c,
                // q_second_half: the second c; packed samples: one run)
                rs[nr] = jj;
                rk[nr] = 0;
                rc[nr] = nkt;
                rl[nr++] = mode[i] == CPATTN_Q_SECOND_HALF ? two_c / 2 : two_c;
                continue;
            }
            // causal: key tile kt sees the rows from its first key on
            const int room = (MAX_KV_RUNS - (nb - ncausal)) / ncausal;
            const int per = (nkt + room - 1) / room;   // key tiles per run
            for (int kt = 0; kt < nkt; kt += per) {
                rs[nr] = jj;
                rk[nr] = kt;
                rc[nr] = nkt - kt < per ? nkt - kt : per;
                rl[nr++] = two_c - (int64_t)kt * TR * KW;
            }
        }
        // longest first (stable: ties keep step order)
        for (int a = 1; a < nr; ++a)
            for (int b2 = a; b2 > 0 && rl[b2 - 1] < rl[b2]; --b2) {
                int t = rs[b2]; rs[b2] = rs[b2 - 1]; rs[b2 - 1] = t;
                t = rk[b2]; rk[b2] = rk[b2 - 1]; rk[b2 - 1] = t;
                t = rc[b2]; rc[b2] = rc[b2 - 1]; rc[b2 - 1] = t;
                const int64_t tl = rl[b2]; rl[b2] = rl[b2 - 1]; rl[b2 - 1] = tl;
            }
        const int64_t inner = (int64_t)g[0].hkv * g[0].b;
        int64_t items = 0;
        for (int a = 0; a < nr; ++a) {
            sp.run[a] = KvRun{rs[a], rk[a], (int)items};
            items += rc[a] * inner;
        }
        sp.nruns = nr;
        auto *fn = g[0].d == 64 ? attn_bwd_dkdv_steps<64> : attn_bwd_dkdv_steps<128>;
        hipLaunchKernelGGL(fn, dim3((unsigned)items), dim3(64 * NWK), 0, stream, sp);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace cpattn
