// Blockwise attention of one CP step, and of a rank's whole share in one
// launch, bf16 inputs, fp32 accumulation, on gfx950 matrix cores.
//
// What it computes ("Megatron-LM 篇", Context Parallel 3.2 step 2 and 3.4):
// for each query row i of the step and head h, softmax attention over the
// visible keys of the source rank's block, returning the normalised O_i and
// the natural-log LSE L_i.  The mode decides the rows and keys (see
// internal.h: q_row0, nq, nk, causal).
//
// The fused form ("超大规模集群…", the big and small attention of one rank
// run concurrently; "Megatron-LM 篇" 3.2 step 2, the per-step LSE
// correction): one workgroup streams, for its query rows, the key blocks of
// all cp steps of the rank one after another -- the first halves of the
// blocks of ranks r-1 .. 0, then (rows of the second chunk only) the whole
// blocks of ranks cp-1 .. r+1, then the rank's own block under the causal
// mask -- and keeps one running max, sum and accumulator across them.
// Carrying the online softmax from one block to the next is the per-step
// L/O correction done in place, so the result is the merged O and L with
// no per-step partials.
//
// Work decomposition
//   workgroup = 8 waves = 256 query rows of one (batch, head); each wave
//   owns 32 consecutive rows.  The KV block streams through LDS in tiles of
//   BN = 64 keys held in a ring of 4 stages, copied global -> LDS directly
//   (global_load_lds_dwordx4, no VGPR round trip) two tiles ahead.
//
// Schedule ("ping-pong"): a wave alternates a matrix phase G(t) = {S^T(t) =
//   K(t) Q^T, O^T += V(t-1)^T P(t-1)} and a vector phase V(t) = {online
//   softmax of S(t) into P(t)}.  Waves 4-7 run one phase behind waves 0-3,
//   and one workgroup barrier separates phases, so on every SIMD (one wave
//   of each group) one wave issues matrix instructions while the other
//   issues the softmax: the exp/max/sum work hides under the MFMAs.  Inside
//   a matrix phase the LDS reads of the next group of four MFMAs are in
//   flight while the current four execute.
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
// LDS (64 banks x 4 bytes on gfx950): rows are 2d bytes (256 for d = 128,
// 128 for d = 64, one template per head dimension); 16-byte chunks are
// XOR-swizzled per row (see Kernel::k_swz / v_swz) so every ds_read_b128 /
// ds_read_b64_tr_b16 phase hits distinct banks.  With d = 64 a matrix phase
// has four steps of four MFMAs instead of eight; it is then the shorter
// half of the ping-pong, so the tile's row max and the step of the LDS
// addresses to the next stages run at its end rather than in the vector
// half (the same instructions on the same values).
// The global -> LDS copies are issued from inline assembly, so the compiler
// does not track them (it would otherwise wait for every copy in flight
// before each LDS read, as it cannot tell the stages apart); explicit vmcnt
// waits before the barrier that publishes a tile complete them.  Each copy
// takes the tile's base address in SGPRs and a per-lane byte offset fixed
// for the whole kernel, so issuing a tile costs no vector address math.
// LDS reads are ordinary loads and transposing-read builtins the compiler
// schedules.
#include "internal.h"
#include "mfma_tiles.h"

#include <math.h>

#include <atomic>

namespace cpattn {
namespace {

using namespace tiles;

constexpr int BN = 64;                 // keys per LDS tile
constexpr int NW = 8;                  // waves per workgroup
constexpr int BM = 32 * NW;            // query rows per workgroup
constexpr int NS = 4;                  // LDS stages
constexpr float RESCALE_SLACK = 8.0f;  // log2 units a stale max may lag
// bytes of one K (or V) tile in LDS for head dimension D (bf16 rows of D)
constexpr int tile_bytes(int D) { return BN * D * 2; }

struct Params {
    const uint16_t *q, *k, *v;
    void *o;                 // fp32, or bf16 for the fused form's bf16 output
    float *lse;
    int64_t two_c, q_row0;
    int nq, nk, hq, hkv, group, num_qtiles;
    float scale_log2;
    // fused form: the rank, the ring size, the element stride between the
    // partitioned blocks of consecutive ranks, and the packed samples
    int rank, cp;
    int64_t block_elems;
    SeqTable tab;
};

// One tile of the key sequence a workgroup streams: the block it comes from
// (K and V bases of the workgroup's batch and KV head), its first key in the
// block, the keys of the block visible in this segment, whether the causal
// mask applies, and the first query row that sees the segment at all.
struct TileRef {
    const uint16_t *kb, *vb;
    int key0, nk;
    bool causal;
    int min_row;
};

// One CP step: the source rank's block, the mode's keys.
// Every plan also names the workgroup's query tile: qtile (its index in its
// sequence), qrow0 and nq (the local row of the sequence's query row 0 and
// its query rows), orow0 and orows (the output row of query row 0 and the
// output rows per batch element).
template <bool CAUSAL, int D>
struct StepPlan {
    static constexpr bool kLongestFirst = CAUSAL;   // later causal tiles see more keys
    static constexpr int kD = D;
    const uint16_t *kb, *vb;
    int nk, ntiles;
    int qtile, qrow0, nq, orow0, orows;
    __device__ __forceinline__ void init(const Params &p, int qt, int n, int g) {
        qtile = qt;
        qrow0 = (int)p.q_row0;
        nq = p.nq;
        orow0 = 0;
        orows = p.nq;
        kb = p.k + ((int64_t)n * p.two_c * p.hkv + g) * D;
        vb = p.v + ((int64_t)n * p.two_c * p.hkv + g) * D;
        nk = p.nk;
        const int kend = CAUSAL ? min(p.nk, qtile * BM + BM) : p.nk;
        ntiles = (kend + BN - 1) / BN;
    }
    // tiles past the last (copied ahead, never computed) repeat the last
    __device__ __forceinline__ TileRef tile(int u) const {
        return TileRef{kb, vb, min(u, ntiles - 1) * BN, nk, CAUSAL, 0};
    }
    // tile u from tile u - 1 (the same as tile(u), without its arithmetic)
    __device__ __forceinline__ TileRef next(const TileRef &a, int u) const {
        if (u >= ntiles) return a;
        TileRef t = a;
        t.key0 += BN;
        return t;
    }
    // whether the wave whose rows start at wrow0 computes tile t: causal
    // waves stop after their diagonal
    __device__ __forceinline__ bool comp(int t, int wrow0) const {
        if (t < 0 || wrow0 >= nq) return false;   // a wave past the last row idles
        return CAUSAL ? t < min(ntiles, (wrow0 + 31) / BN + 1) : t < ntiles;
    }
};

// A rank's whole share of one sequence (one packed sample: c is its chunk
// length, and its rows start at local row lcu of every rank's block).
// Segments in streaming order: ranks r-1 .. 0, keys
// [0, c) (steps 1 .. r, kv_first_half); ranks cp-1 .. r+1, keys [0, 2c)
// (steps r+1 .. cp-1, q_second_half: only rows c .. 2c-1 see them, and the
// segments are streamed only when some row of the workgroup is one of
// those); rank r, keys [0, min(2c, q0 + BM)) causal (step 0).  A segment
// whose length is not a multiple of BN ends in a masked tile.
// floor(u / d) for 0 <= u, 1 <= d < 2^31, with m = floor((2^32 - 1) / d): the
// high product is floor(u / d) or one less, and one compare settles it (so the
// per-tile segment lookups cost a few scalar instructions, not a division).
__device__ __forceinline__ int div_by(int u, unsigned m, int d) {
    int q = (int)__umulhi((unsigned)u, m);
    if (u - q * d >= d) ++q;
    return q;
}

template <int D>
struct FusedPlan {
    static constexpr bool kLongestFirst = true;     // later tiles: second chunk, causal
    static constexpr int kD = D;
    const uint16_t *k0, *v0;      // rank 0's block, this batch and KV head
    int64_t block;                // elements between consecutive ranks' blocks
    int r, cp, c, cA, nAB, cB, ta, tb, kend, ntiles, q0;
    unsigned mA, mB;              // div_by multipliers of cA and cB
    int qtile, qrow0, nq, orow0, orows;
    __device__ __forceinline__ void init(const Params &p, int qt, int n, int g) {
        const int i = seq_of(p.tab.tile0, p.tab.nseq, qt);
        const int l0 = p.tab.lcu[i];
        qtile = qt - p.tab.tile0[i];
        c = (p.tab.lcu[i + 1] - l0) >> 1;
        qrow0 = l0;
        nq = 2 * c;
        orow0 = l0;
        orows = (int)p.two_c;
        k0 = p.k + (((int64_t)n * p.two_c + l0) * p.hkv + g) * D;
        v0 = p.v + (((int64_t)n * p.two_c + l0) * p.hkv + g) * D;
        block = p.block_elems;
        r = p.rank;
        cp = p.cp;
        q0 = qtile * BM;
        cA = (c + BN - 1) / BN;
        cB = (2 * c + BN - 1) / BN;
        mA = 0xFFFFFFFFu / (unsigned)cA;
        mB = 0xFFFFFFFFu / (unsigned)cB;
        nAB = (q0 + BM > c) ? cp - 1 - r : 0;
        ta = r * cA;
        tb = ta + nAB * cB;
        kend = min(2 * c, q0 + BM);
        ntiles = tb + (kend + BN - 1) / BN;
    }
    __device__ __forceinline__ TileRef tile(int u) const {
        u = min(u, ntiles - 1);
        if (u < ta) {
            const int seg = div_by(u, mA, cA);
            const int64_t off = (int64_t)(r - 1 - seg) * block;
            return TileRef{k0 + off, v0 + off, (u - seg * cA) * BN, c, false, 0};
        }
        if (u < tb) {
            const int seg = div_by(u - ta, mB, cB);
            const int64_t off = (int64_t)(cp - 1 - seg) * block;
            return TileRef{k0 + off, v0 + off, (u - ta - seg * cB) * BN, 2 * c, false, c};
        }
        const int64_t off = (int64_t)r * block;
        return TileRef{k0 + off, v0 + off, (u - tb) * BN, kend, true, 0};
    }
    // tile u from tile u - 1 (the same as tile(u), without the segment
    // lookup): the next tile of the segment, or the first of the next one
    __device__ __forceinline__ TileRef next(const TileRef &a, int u) const {
        if (u >= ntiles) return a;
        if (u == tb) {
            const int64_t off = (int64_t)r * block;
            return TileRef{k0 + off, v0 + off, 0, kend, true, 0};
        }
        if (u == ta) {
            const int64_t off = (int64_t)(cp - 1) * block;
            return TileRef{k0 + off, v0 + off, 0, 2 * c, false, c};
        }
        TileRef t = a;
        if (a.key0 + BN < a.nk) {
            t.key0 += BN;
        } else {   // next block of the same kind: one rank lower
            t.kb -= block;
            t.vb -= block;
            t.key0 = 0;
        }
        return t;
    }
    __device__ __forceinline__ bool comp(int t, int wrow0) const {
        if (t < 0 || wrow0 >= nq) return false;   // a wave past the sample's rows idles
        if (t < ta) return true;
        if (t < tb) return wrow0 + 31 >= c;
        return t - tb < min(ntiles - tb, (wrow0 + 31) / BN + 1);
    }
};

// Workgroup index in the order that gives each XCD a contiguous run (the
// dispatcher deals workgroups to the 8 XCDs round robin).
__device__ __forceinline__ int xcd_order(int blk, int nblk) {
    return (nblk & 7) == 0 ? (blk & 7) * (nblk >> 3) + (blk >> 3) : blk;
}

template <class Plan, bool OUT_BF16>
struct Kernel {
    static constexpr int D = Plan::kD;
    static constexpr int ROWB = D * 2;            // bytes per K/V row in LDS
    static constexpr int TILEB = tile_bytes(D);   // bytes per K (or V) tile
    static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    static constexpr int RPC = 64 / CPR;          // tile rows per copy (64 lanes x 16 bytes)
    static constexpr int KI = BN / RPC / NW;      // copy instructions per wave per tile (each)
    static constexpr int LPT = 2 * KI;            // copies per wave per tile (K and V)
    static constexpr int NSTEP = D / 16;          // matrix steps per phase (four MFMAs each)
    static_assert(D == 64 || D == 128, "head dimension");
    static_assert(KI >= 1 && BN % (RPC * NW) == 0, "copy split");
    // LDS chunk c of tile row r holds chunk c ^ k_swz(r) of the K row and
    // chunk c ^ v_swz(r) of the V row.  256-byte rows (D = 128): K by the
    // matrix row that reads it, V by r % 4.  128-byte rows (D = 64; two rows
    // share one pass over the 64 banks): K by r / 2, V by (r / 2) % 2.
    __device__ __forceinline__ static int k_swz(int r) {
        return D == 128 ? swap_bits23(r) & 15 : (r >> 1) & 7;
    }
    __device__ __forceinline__ static int v_swz(int r) {
        return D == 128 ? (r & 3) << 2 : ((r >> 1) & 1) << 2;
    }
    // Per-wave state.
    struct State {
        bf16x8 qf[D / 16];       // Q as the B operand of S^T
        f32x16 acc[D / 32];      // O^T
        f32x16 s[2];             // S^T of the tile between its two phases
        bf16x8 pf[BN / 16];      // P of the tile between its two phases
        float m_run, l_run;
        // lane's LDS address of each K chunk / V^T read in the current
        // stages (advanced once per tile, so matrix phases add immediates only)
        unsigned koff[D / 16];
        unsigned voff[D / 32];
        unsigned gk[KI], gv[KI]; // lane's byte offsets of its K and V copies in a tile
        int krow[KI];            // tile row of each of the lane's copies
        int64_t kstride;         // elements between consecutive keys
    };

    // Issue this wave's share of the direct copies of one tile into an LDS
    // stage (K at sK, V at sK + TILEB): a scalar tile base plus the lane's
    // fixed offsets.  A tile crossing its segment end repeats row nk-1.
    __device__ __forceinline__ static void issue(const State &S, unsigned sK, const TileRef &tr,
                                                 int wave) {
        if (tr.key0 + BN <= tr.nk) {
            const uint16_t *kb = tr.kb + (int64_t)tr.key0 * S.kstride;
            const uint16_t *vb = tr.vb + (int64_t)tr.key0 * S.kstride;
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const unsigned dst = sK + (wave * KI + i) * RPC * ROWB;
                dma16(kb, S.gk[i], dst);
                dma16(vb, S.gv[i], dst + TILEB);
            }
        } else {
            // base row b0 <= every row copied, so lane offsets stay >= 0
            const int b0 = max(min(tr.key0, tr.nk - BN), 0);
            const uint16_t *kb = tr.kb + (int64_t)b0 * S.kstride;
            const uint16_t *vb = tr.vb + (int64_t)b0 * S.kstride;
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const int key = min(tr.key0 + S.krow[i], tr.nk - 1);
                // gk holds krow rows; move the lane to row key - b0
                const unsigned adj = (unsigned)((key - b0 - S.krow[i]) * (int)S.kstride * 2);
                const unsigned dst = sK + (wave * KI + i) * RPC * ROWB;
                dma16(kb, S.gk[i] + adj, dst);
                dma16(vb, S.gv[i] + adj, dst + TILEB);
            }
        }
    }

    // The O^T products of matrix step i: products 2i and 2i+1 of the
    // (key chunk, head-dim tile) pairs in chunk-major order.
    __device__ __forceinline__ static constexpr int o_chunk(int i, int j) {
        return (2 * i + j) / (D / 32);
    }
    __device__ __forceinline__ static constexpr int o_tile(int i, int j) {
        return (2 * i + j) % (D / 32);
    }
    // LDS operands of matrix step i (see matrix_phase): the two K chunks of
    // k-step i and the V^T blocks of its two O^T products.
    __device__ __forceinline__ static void step_reads(const State &S, int i, bf16x8 (&kf)[2],
                                                      bf16x8 (&vf)[2]) {
        kf[0] = k_read(S.koff[i]);
        kf[1] = k_read(S.koff[i] + 32 * ROWB);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            vf[j] = vt_read<ROWB>(S.voff[o_tile(i, j)] + o_chunk(i, j) * 16 * ROWB);
    }

    // The operands of the first two matrix steps, read ahead: a wave issues
    // them at the end of its vector half so that their LDS latency passes
    // while it waits at the barrier, and its matrix phase starts on resident
    // operands.
    struct Ahead {
        bf16x8 kf[2][2], vf[2][2];
    };
    __device__ __forceinline__ static void read_ahead(const State &S, Ahead &A) {
        step_reads(S, 0, A.kf[0], A.vf[0]);
        step_reads(S, 1, A.kf[1], A.vf[1]);
    }

    // Matrix phase: S^T(t) = K(t) Q^T and O^T += V(t-1)^T P(t-1), from the
    // stages S.koff / S.voff point at, its first two steps' operands in A.
    // One code path for every phase: the first phase multiplies a zeroed V
    // tile by P = 0, and the S^T of the phase after a wave's last tile is
    // computed on resident rows and dropped.
    __device__ __forceinline__ static void matrix_phase(State &S, const Ahead &A) {
        // D/16 steps of four MFMAs: step i does k-step i of S^T (both 32-key
        // halves) and O^T products 2i and 2i+1 (chunk-major order: for D = 128
        // head-dim tiles 2(i%2), 2(i%2)+1 of key chunk i/2; for D = 64 both
        // tiles of key chunk i).
        // The LDS reads of step i+2 are issued before the MFMAs of step i, so
        // two steps of matrix work cover each read's latency (the fences keep
        // the compiler from hoisting every read, which would exhaust registers).
        bf16x8 kf[3][2], vf[3][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            kf[0][j] = A.kf[0][j];
            vf[0][j] = A.vf[0][j];
            kf[1][j] = A.kf[1][j];
            vf[1][j] = A.vf[1][j];
        }
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            const int cur = i % 3;
            if (i + 2 < NSTEP) step_reads(S, i + 2, kf[(i + 2) % 3], vf[(i + 2) % 3]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
                S.s[h2] = i == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                       kf[cur][h2], S.qf[i], f32x16{}, 0, 0, 0)
                                 : __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                       kf[cur][h2], S.qf[i], S.s[h2], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                S.acc[o_tile(i, j)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    vf[cur][j], S.pf[o_chunk(i, j)], S.acc[o_tile(i, j)], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Row max of the tile's raw scores; the masked variant first sets the
    // invisible scores to -inf (keys past the block, or after the row).
    template <bool MASK>
    __device__ __forceinline__ static float tile_max(const TileRef &tr, State &S, int qrow,
                                                     int hi) {
        const int key0 = tr.key0;
        float tmax = -INFINITY;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = S.s[h2][e];
                if constexpr (MASK) {
                    const int key = key0 + h2 * 32 + 16 * (e >> 3) + 8 * hi + (e & 7);
                    const bool vis =
                        key < tr.nk && (!tr.causal || key <= qrow) && qrow >= tr.min_row;
                    x = vis ? x : -INFINITY;
                    S.s[h2][e] = x;
                }
                tmax = fmaxf(tmax, x);
            }
        return tmax;
    }

    // Vector phase: online softmax of S(t) into P(t), rescaling O and l
    // first when the running max moves by more than the slack.
    // The tile's row max in log2 units (masking the invisible scores first
    // on tiles that need it).
    __device__ __forceinline__ static float scaled_tile_max(const Params &p, State &S,
                                                            const TileRef &tr, int wrow0,
                                                            int lane) {
        const int hi = lane >> 5;
        const int qrow = wrow0 + (lane & 31);
        // scalar: only tiles crossing the diagonal or the segment end, and
        // waves that straddle a segment's first row, mask
        const bool mask = (tr.key0 + BN > tr.nk) || (tr.causal && tr.key0 + BN - 1 > wrow0) ||
                          wrow0 < tr.min_row;
        const float tmax =
            mask ? tile_max<true>(tr, S, qrow, hi) : tile_max<false>(tr, S, qrow, hi);
        return halves_max(tmax) * p.scale_log2;
    }

    __device__ __forceinline__ static void softmax_phase(const Params &p, State &S,
                                                         float tmax) {
        const float m_new = fmaxf(S.m_run, tmax);
        if (__builtin_amdgcn_ballot_w64(m_new > S.m_run + RESCALE_SLACK)) {
            // a row that has seen no visible key yet (m = -inf) keeps alpha 1
            const float alpha =
                m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(S.m_run - m_new);
            S.l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) S.acc[dt] *= alpha;
            S.m_run = m_new;
        }
        const float mu = (S.m_run == -INFINITY) ? 0.0f : S.m_run;
        float lsum0 = 0.0f, lsum1 = 0.0f;   // two partial row sums (shorter chains)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f32x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(S.s[h2][half * 8 + e], p.scale_log2, -mu));
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    lsum0 += pv[e];
                    lsum1 += pv[e + 1];
                }
                S.pf[h2 * 2 + half] = __builtin_convertvector(pv, bf16x8);
            }
        S.l_run += lsum0 + lsum1;
    }

    // The barrier opening half-iteration h.  Before it this wave's copies of
    // tile (h+1)/2 are complete (only the copies of the tile after may still
    // fly), so tile u is resident from barrier 2u-1 on; after it, at even
    // h = 2u, the copies of tile u+2 are issued.  No LDS wait: a matrix phase
    // consumes its own reads, and the reads a wave issues ahead of the
    // barrier touch stages that no copy in flight or issued here overwrites.
    __device__ __forceinline__ static void sync(const Plan &P, State &S, int h,
                                                unsigned lds_addr, int wave, TileRef &cpy) {
        const bool even = (h & 1) == 0;
        wait_vmcnt<LPT>();
        asm volatile("s_barrier" ::: "memory");
        if (even) {
            const int u = (h >> 1) + 2;
            cpy = P.next(cpy, u);
            issue(S, lds_addr + (u % NS) * 2 * TILEB, cpy, wave);
        }
    }

    // Workgroup -> (batch, kv group, query tile, head in group).  The 8
    // XCDs receive workgroups round robin; give each a contiguous run of
    // items so heads sharing a KV group share that XCD's L2.  Causal steps
    // take their longest query tiles first.
    __device__ __forceinline__ static void run(const Params &p, char *lds) {
        int item = xcd_order(blockIdx.x, gridDim.x);
        const int hh = item % p.group;
        item /= p.group;
        const int qt_rank = item % p.num_qtiles;
        item /= p.num_qtiles;
        const int g = item % p.hkv;
        const int n = item / p.hkv;
        run_item(p, lds, n, g, hh, Plan::kLongestFirst ? p.num_qtiles - 1 - qt_rank : qt_rank);
    }

    // The query tile qt of head g * group + hh of batch element n.
    __device__ __forceinline__ static void run_item(const Params &p, char *lds, int n, int g,
                                                    int hh, int qt) {
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        // wave index as a scalar: every per-wave decision below is a scalar
        // branch instead of a per-lane select
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int grp = wave >> 2;                   // 0: leading, 1: trailing group
        const int hi = lane >> 5;
        const int l32 = lane & 31;
        const int head = g * p.group + hh;
        Plan P;
        P.init(p, qt, n, g);
        const int wrow0 = P.qtile * BM + wave * 32;   // first row of this wave in its sequence
        const int ntiles = P.ntiles;
        State S;
        S.kstride = (int64_t)p.hkv * D;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int row = (wave * KI + i) * RPC + lane / CPR;
            const int phys = lane % CPR;
            S.krow[i] = row;
            S.gk[i] = (unsigned)(row * S.kstride * 2 + ((phys ^ k_swz(row)) << 4));
            S.gv[i] = (unsigned)(row * S.kstride * 2 + ((phys ^ v_swz(row)) << 4));
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) S.acc[dt][e] = 0.0f;
        S.m_run = -INFINITY;
        S.l_run = 0.0f;
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e) S.pf[kc][e] = (__bf16)0.0f;
        // the V tile the first matrix phase reads (stage NS-1) starts as zeros;
        // its first copy is issued two barriers later
        {
            u32x4 *z = (u32x4 *)(lds + (NS - 1) * 2 * TILEB + TILEB);
            const u32x4 zero = {0u, 0u, 0u, 0u};
            for (int i = tid; i < TILEB / 16; i += 64 * NW) z[i] = zero;
        }

        {
            const int krow = swap_bits23(l32);             // K row fed to matrix row l32
            const int ksw = D == 128 ? (l32 & 15) : k_swz(krow);   // k_swz(krow)
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                S.koff[kk] = krow * ROWB + (((kk * 2 + hi) ^ ksw) << 4);
            const int vg = lane >> 4, vj = (lane >> 2) & 3, vq = lane & 3;
            const int x = 2 * (vg & 1) + (vq >> 1);
            const int vrow = 8 * (vg >> 1) + vj;
            const int vsw = D == 128 ? vj << 2 : v_swz(vrow);         // v_swz(vrow)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                S.voff[dt] = vrow * ROWB + (((dt * 4 + x) ^ vsw) << 4) + (vq & 1) * 8;
        }
        const unsigned lds_addr =
            (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) S.koff[kk] += lds_addr;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) S.voff[dt] += lds_addr + (NS - 1) * 2 * TILEB + TILEB;
        // prologue: tiles 0 and 1 in flight, then Q; one full wait before the
        // loop (tile 0 has to land first anyway) also tells the compiler that
        // Q is resident, so it puts no memory wait inside the loop
        // tile cursors: cpy is the last tile copied (tiles 0 and 1 here, then
        // tile u + 2 after barrier 2u), cur the tile of the softmax phase
        TileRef cpy = P.tile(1), cur = P.tile(0);
        issue(S, lds_addr, cur, wave);
        issue(S, lds_addr + 2 * TILEB, cpy, wave);
        {
            const int row = min(wrow0 + l32, P.nq - 1);
            const uint16_t *src =
                p.q + ((n * p.two_c + P.qrow0 + row) * (int64_t)p.hq + head) * D + hi * 8;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                S.qf[kk] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(src + kk * 16));
        }
        wait_vmcnt<0>();

        // Half-iterations h = 0 .. 2T+1, one barrier each.  The leading group
        // runs phase h, the trailing group phase h-1: phase 2t is the matrix
        // phase G(t), phase 2t+1 the softmax of tile t.  Tile u is resident
        // from barrier 2u-1 on (its K is read ahead in phase 2u-1 by the
        // leading group, its V two phases after its K), and after barrier 2u
        // tile u+2 is copied into the stage tile u-2 left (its last readers,
        // the matrix phases of tile u-1 and the reads ahead of them, ran
        // before that barrier).  The trailing group's first and the leading
        // group's last half-iteration are idle.
        // A wave computes tile t when P.comp(t): the matrix phase G(t) runs
        // when it needs S(t) or adds P(t-1); after a tile the wave skips, P is
        // zero, so a following G adds nothing for it.
        // The zero stage's writes complete before the first barrier.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        sync(P, S, 0, lds_addr, wave, cpy);
        Ahead A;
        read_ahead(S, A);
        if (grp == 1) sync(P, S, 1, lds_addr, wave, cpy);
        // With 64-wide heads the matrix phase is the shorter half (half the
        // MFMAs of d = 128 for the same softmax), so the tile max and the
        // step to the next stages run at its end instead of in the vector
        // half; the two halves of a SIMD's ping-pong then take about as long
        // as each other.  The same instructions run in the same order on the
        // same values either way.
        constexpr bool EARLY = D == 64;
        auto advance = [&](int t) {
            // next tile: the K stage moves from t % NS to (t+1) % NS and the V
            // stage from (t-1) % NS to t % NS
            const unsigned kstep = ((t + 1) % NS == 0) ? (unsigned)(-(NS - 1) * 2 * TILEB)
                                                       : (unsigned)(2 * TILEB);
            const unsigned vstep = (t % NS == 0) ? (unsigned)(-(NS - 1) * 2 * TILEB)
                                                 : (unsigned)(2 * TILEB);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) S.koff[kk] += kstep;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) S.voff[dt] += vstep;
        };
        for (int t = 0; t <= ntiles; ++t) {
            const int hg = 2 * t + grp;    // the barrier this wave last passed
            if (P.comp(t, wrow0) || P.comp(t - 1, wrow0))
                matrix_phase(S, A);
            if (t == ntiles) break;
            if (t > 0) cur = P.next(cur, t);
            const bool comp = P.comp(t, wrow0);
            float tmax = 0.0f;
            if constexpr (EARLY) {
                if (comp) tmax = scaled_tile_max(p, S, cur, wrow0, lane);
                advance(t);
            }
            sync(P, S, hg + 1, lds_addr, wave, cpy);
            if (comp) {
                if constexpr (!EARLY) tmax = scaled_tile_max(p, S, cur, wrow0, lane);
                softmax_phase(p, S, tmax);
            } else {
#pragma unroll
                for (int kc = 0; kc < BN / 16; ++kc)
#pragma unroll
                    for (int e = 0; e < 8; ++e) S.pf[kc][e] = (__bf16)0.0f;
            }
            if constexpr (!EARLY) advance(t);
            // K(t+1) is resident since barrier 2t+1, V(t) since barrier 2t
            read_ahead(S, A);
            sync(P, S, hg + 2, lds_addr, wave, cpy);
        }
        if (grp == 0) sync(P, S, 2 * ntiles + 1, lds_addr, wave, cpy);
        // copies issued past the end land in stages nobody reads; retire them
        // before the workgroup's LDS is handed to the next workgroup
        wait_vmcnt<0>();

        // Normalise and store O (fp32, or bf16 rounded to nearest even) and
        // L (natural log).
        const float lt = halves_sum(S.l_run);
        const int row = wrow0 + l32;
        if (row < P.nq) {
            const float inv = 1.0f / lt;
            const int64_t orow = (int64_t)n * P.orows + P.orow0 + row;
            const int64_t base = (orow * p.hq + head) * D + 4 * hi;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = S.acc[dt][i * 4 + j] * inv;
                    if constexpr (OUT_BF16) {
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        *(bf16x4 *)((__bf16 *)p.o + base + dt * 32 + i * 8) =
                            __builtin_convertvector(w, bf16x4);
                    } else {
                        *(f32x4 *)((float *)p.o + base + dt * 32 + i * 8) = w;
                    }
                }
            if (hi == 0 && p.lse != nullptr)
                p.lse[((int64_t)n * p.hq + head) * P.orows + P.orow0 + row] =
                    (S.m_run + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
        }
    }
};

// One CP step (fp32 partial output).
template <bool CAUSAL, int D>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_step_bf16(Params p) {
    __shared__ __attribute__((aligned(1024))) char lds[NS * 2 * tile_bytes(D)];
    Kernel<StepPlan<CAUSAL, D>, false>::run(p, lds);
}

// Several CP steps of one rank in one launch (fp32 partial outputs).  The
// steps are independent: step j reads its source block and writes its own
// partial, exactly as its own launch of attn_step_bf16 would.  One grid
// lets the workgroup scheduler start a step's query tiles while another
// step's workgroups are still storing their outputs, where separate
// launches make every CU load and store at the same moments.
struct StepDesc {
    const uint16_t *k, *v;   // the source rank's block
    float *o, *lse;          // the step's partial
    int q_row0, nq, nk, causal, num_qtiles;
};
// Query tiles of one step that stream the same number of key tiles (every
// tile of a non-causal step; one tile, or a run of neighbouring tiles, of the
// causal step), in workgroup order: tile qt0, qt0 + dir, ...
struct WorkRun {
    int step, qt0, dir;
    int item0;               // first workgroup of the run within one (batch, KV head)
};
constexpr int MAX_STEPS = 32;   // steps per launch (kernel argument space)
constexpr int MAX_RUNS = 64;
struct StepsParams {
    const uint16_t *q;
    int64_t two_c;
    int hq, hkv, group, nruns, items;   // items: workgroups per (batch, KV head)
    int total;                          // items of the grid; > gridDim.x: workgroups loop
    float scale_log2;
    StepDesc st[MAX_STEPS];
    WorkRun run[MAX_RUNS];
};
static_assert(sizeof(StepsParams) <= 4096, "kernel arguments");

template <int D>
__device__ __forceinline__ void steps_item(const StepsParams &sp, int item, char *lds) {
    const int ng = item / sp.items;
    int w = item - ng * sp.items;
    int j = 0;
    while (j + 1 < sp.nruns && sp.run[j + 1].item0 <= w) ++j;
    const WorkRun &r = sp.run[j];
    w -= r.item0;
    const StepDesc &d = sp.st[r.step];
    Params p = {};
    p.q = sp.q;
    p.k = d.k;
    p.v = d.v;
    p.o = d.o;
    p.lse = d.lse;
    p.two_c = sp.two_c;
    p.q_row0 = d.q_row0;
    p.nq = d.nq;
    p.nk = d.nk;
    p.hq = sp.hq;
    p.hkv = sp.hkv;
    p.group = sp.group;
    p.num_qtiles = d.num_qtiles;
    p.scale_log2 = sp.scale_log2;
    const int hh = w % sp.group, qt = r.qt0 + r.dir * (w / sp.group);
    const int g = ng % sp.hkv, n = ng / sp.hkv;
    if (d.causal)
        Kernel<StepPlan<true, D>, false>::run_item(p, lds, n, g, hh, qt);
    else
        Kernel<StepPlan<false, D>, false>::run_item(p, lds, n, g, hh, qt);
}

template <int D>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_steps_bf16(StepsParams sp) {
    __shared__ __attribute__((aligned(1024))) char lds[NS * 2 * tile_bytes(D)];
    // workgroup -> (batch, KV head), then the run, then (query tile, head in
    // group) inside it; the runs are laid out longest first across all steps
    if (sp.total == (int)gridDim.x) {
        steps_item<D>(sp, xcd_order(blockIdx.x, gridDim.x), lds);
        return;
    }
    // Fewer workgroups than items (one per CU, a multiple of 8 of each):
    // workgroup b serves the items of XCD b % 8's contiguous range (longest
    // first) round by round, in alternating directions, so each CU's items
    // add up to about the same work.  A workgroup that stays resident skips
    // the launch of a new one and its last item's stores drain while the
    // next item starts.
    const int xq = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
    const int range = sp.total >> 3;
    for (int r = 0; r * nslot < range; ++r) {
        const int li = r * nslot + ((r & 1) ? nslot - 1 - slot : slot);
        if (li >= range) continue;
        if (r > 0) lds_barrier();   // every wave is done with the LDS of the last item
        steps_item<D>(sp, xq * range + li, lds);
    }
}

// A rank's whole share (merged output, fp32 or bf16).
template <bool OUT_BF16, int D>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fused_bf16(Params p) {
    __shared__ __attribute__((aligned(1024))) char lds[NS * 2 * tile_bytes(D)];
    Kernel<FusedPlan<D>, OUT_BF16>::run(p, lds);
}

template <class KernelFn>
hipError_t launch_kernel(KernelFn fn, const Params &p, int64_t b, int hq, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.num_qtiles * hq * b;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepGeom &g, const void *q, const void *k, const void *v,
                            float *o, float *lse, hipStream_t stream) {
    Params p = {};
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
    if (g.d == 64) {
        if (g.causal) return launch_kernel(attn_step_bf16<true, 64>, p, g.b, g.hq, stream);
        return launch_kernel(attn_step_bf16<false, 64>, p, g.b, g.hq, stream);
    }
    if (g.causal) return launch_kernel(attn_step_bf16<true, 128>, p, g.b, g.hq, stream);
    return launch_kernel(attn_step_bf16<false, 128>, p, g.b, g.hq, stream);
}

int device_cu_count() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of the steps grid that fit at once (one per CU: the LDS ring
// takes 128 KiB), a multiple of 8.
static int resident_slots() { return device_cu_count() & ~7; }

hipError_t launch_steps_bf16(int n, const StepGeom *g, const void *q, const void *const *k,
                             const void *const *v, float *const *o, float *const *lse,
                             hipStream_t stream) {
    static_assert(MAX_STEPS == STEPS_PER_GRID, "one grid takes the steps of one call");
    if (n < 1 || n > MAX_STEPS) return hipErrorInvalidValue;
    StepsParams sp = {};
    sp.q = (const uint16_t *)q;
    sp.two_c = g[0].two_c;
    sp.hq = g[0].hq;
    sp.hkv = g[0].hkv;
    sp.group = g[0].hq / g[0].hkv;
    sp.scale_log2 = g[0].scale_log2;
    // runs of query tiles with their key-tile counts: a non-causal step is
    // one run; the causal step's tiles (query tile qt sees keys up to
    // 256(qt+1)) are one run each, or runs of neighbours when there are
    // more tiles than the run table holds
    int len[MAX_RUNS], cnt[MAX_RUNS], nr = 0, ncausal = 0;
    for (int i = 0; i < n; ++i) ncausal += g[i].causal ? 1 : 0;
    for (int i = 0; i < n; ++i) {
        StepDesc &d = sp.st[i];
        d.k = (const uint16_t *)k[i];
        d.v = (const uint16_t *)v[i];
        d.o = o[i];
        d.lse = lse[i];
        d.q_row0 = (int)g[i].q_row0;
        d.nq = (int)g[i].nq;
        d.nk = (int)g[i].nk;
        d.causal = g[i].causal ? 1 : 0;
        d.num_qtiles = (int)((g[i].nq + BM - 1) / BM);
        if (!d.causal) {
            sp.run[nr] = WorkRun{i, 0, 1, 0};
            len[nr] = (d.nk + BN - 1) / BN;
            cnt[nr++] = d.num_qtiles;
            continue;
        }
        const int room = (MAX_RUNS - (n - ncausal)) / ncausal;   // runs this step may take
        const int per = (d.num_qtiles + room - 1) / room;        // tiles per run
        for (int qt = d.num_qtiles - 1; qt >= 0; qt -= per) {
            sp.run[nr] = WorkRun{i, qt, -1, 0};
            len[nr] = (min(d.nk, (qt + 1) * BM) + BN - 1) / BN;
            cnt[nr++] = min(per, qt + 1);
        }
    }
    // longest first (stable: ties keep step order)
    for (int a = 1; a < nr; ++a)
        for (int b2 = a; b2 > 0 && len[b2 - 1] < len[b2]; --b2) {
            const WorkRun tr = sp.run[b2];
            sp.run[b2] = sp.run[b2 - 1];
            sp.run[b2 - 1] = tr;
            const int tl = len[b2], tc = cnt[b2];
            len[b2] = len[b2 - 1];
            cnt[b2] = cnt[b2 - 1];
            len[b2 - 1] = tl;
            cnt[b2 - 1] = tc;
        }
    int items = 0;
    for (int a = 0; a < nr; ++a) {
        sp.run[a].item0 = items;
        items += cnt[a] * sp.group;
    }
    sp.nruns = nr;
    sp.items = items;
    const int64_t total = (int64_t)items * sp.hkv * g[0].b;
    sp.total = (int)total;
    // one resident workgroup per CU when there are more than two items per
    // CU and the items split evenly over the 8 XCD ranges
    const int64_t slots = resident_slots();
    const int64_t blocks = (slots >= 8 && total % 8 == 0 && total > 2 * slots) ? slots : total;
    if (g[0].d == 64)
        hipLaunchKernelGGL(attn_steps_bf16<64>, dim3((unsigned)blocks), dim3(64 * NW), 0, stream,
                           sp);
    else
        hipLaunchKernelGGL(attn_steps_bf16<128>, dim3((unsigned)blocks), dim3(64 * NW), 0, stream,
                           sp);
    return hipGetLastError();
}

hipError_t launch_fused_bf16(const FusedGeom &f, const void *qz, const void *kz, const void *vz,
                             void *o, bool out_bf16, float *lse, hipStream_t stream) {
    Params p = {};
    const int64_t block_q = f.b * f.two_c * f.hq * f.d;   // one rank's Q block, elements
    p.q = (const uint16_t *)qz + f.rank * block_q;
    p.k = (const uint16_t *)kz;
    p.v = (const uint16_t *)vz;
    p.o = o;
    p.lse = lse;
    p.two_c = f.two_c;
    p.q_row0 = 0;
    p.nq = (int)f.two_c;
    p.nk = (int)f.two_c;
    p.hq = f.hq;
    p.hkv = f.hkv;
    p.group = f.hq / f.hkv;
    p.scale_log2 = f.scale_log2;
    p.rank = f.rank;
    p.cp = f.cp;
    p.block_elems = f.b * f.two_c * f.hkv * f.d;
    // query tiles sample by sample
    p.tab = f.tab;
    p.tab.tile0[0] = 0;
    for (int i = 0; i < p.tab.nseq; ++i)
        p.tab.tile0[i + 1] = p.tab.tile0[i] + (p.tab.lcu[i + 1] - p.tab.lcu[i] + BM - 1) / BM;
    p.num_qtiles = p.tab.tile0[p.tab.nseq];
    if (f.d == 64) {
        if (out_bf16) return launch_kernel(attn_fused_bf16<true, 64>, p, f.b, f.hq, stream);
        return launch_kernel(attn_fused_bf16<false, 64>, p, f.b, f.hq, stream);
    }
    if (out_bf16) return launch_kernel(attn_fused_bf16<true, 128>, p, f.b, f.hq, stream);
    return launch_kernel(attn_fused_bf16<false, 128>, p, f.b, f.hq, stream);
}

}  // namespace cpattn
