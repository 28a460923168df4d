// Zigzag split of Q, K or V over the cp emulated ranks, with global
// position ids and optional RoPE at those positions.
//
// "Megatron-LM 篇", Context Parallel 3.2 step 1 (split by cp_size) and 3.4
// (rank_0 trades half its data with rank_n-1, rank_1 with rank_n-2, ...);
// "超大规模集群下大语言模型训练实操指南", "CP 与其他技术结合" (one big and one
// small attention per device).  The sequence is cut into 2cp chunks of c
// rows; rank r holds chunk r, then chunk 2cp-1-r:
//     xz[r, n, j] = x[n, pos_r(j)],  pos_r(j) = r*c + j            (j < c)
//                                             (2cp-1-r)*c + j - c  (j >= c)
// RoPE ("Megatron 面试题（一）", M016): every copied row is rotated at its
// global position pos_r(j), never at its local index.
//
// Packed samples (same page, M016's follow-up: positions reset at packed
// sample boundaries): each sample is split by the rule above on its own,
// with c its own chunk length, and occupies local rows [cu/cp, cu'/cp) of
// every rank; pos_r(j) is then the position within the sample.  An
// unpacked batch is the one-sample case.
//
// Without RoPE the kernel is a pure HBM copy: each workgroup moves a run of
// whole output rows with 16-byte loads and stores, consecutive lanes on
// consecutive addresses.  With RoPE each workgroup takes a run of rows too:
// it builds the run's cos/sin table in LDS (angles pos * theta^(-2t/d) in
// fp64, sincos in fp64, rounded to fp32), then rotates the pairs (t, t +
// d/2) of every head in fp32, 16-byte vectors at a time, and rounds the
// result to the element type (bf16: nearest even).
#include "internal.h"

#include <math.h>

namespace cpattn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;

constexpr int MAX_ROWS_PER_BLOCK = 512;   // copy kernel: rows handled per workgroup

struct CopyParams {
    const char *x;
    char *xz;
    int32_t *pos;
    int64_t s, tloc, b, rows_total;   // tloc = s / cp local rows; rows_total = cp * b * tloc
    int cp;
    int vecs_per_row;                 // 16-byte vectors per row (h*d*es/16)
    int rows_per_block;
    SeqTable tab;
};

// Local row j of rank r -> its row in the batch element's packed sequence
// (src) and its position within its sample (pos).
__device__ __forceinline__ void source_row(const SeqTable &t, int cp, int64_t r, int64_t j,
                                           int64_t &src, int64_t &pos) {
    const int i = seq_of(t.lcu, t.nseq, (int)j);
    const int64_t c = (t.lcu[i + 1] - t.lcu[i]) / 2;
    const int64_t jj = j - t.lcu[i];
    pos = jj < c ? r * c + jj : (2 * cp - 1 - r) * c + (jj - c);
    src = (int64_t)t.lcu[i] * cp + pos;
}

// Output row index -> (rank, batch, local row)
__device__ __forceinline__ void split_row(int64_t row, int64_t b, int64_t tloc,
                                          int64_t &r, int64_t &n, int64_t &j) {
    j = row % tloc;
    int64_t rn = row / tloc;
    n = rn % b;
    r = rn / b;
}

// positions of every rank: pos[r * tloc + j]
__device__ __forceinline__ void write_positions(const SeqTable &t, int cp, int64_t tloc,
                                                int32_t *pos) {
    const int64_t total = (int64_t)cp * tloc;
    for (int64_t i = threadIdx.x; i < total; i += NT) {
        int64_t src, ps;
        source_row(t, cp, i / tloc, i % tloc, src, ps);
        pos[i] = (int32_t)ps;
    }
}

__global__ void __launch_bounds__(NT) partition_copy(CopyParams p) {
    __shared__ int64_t srow[MAX_ROWS_PER_BLOCK];   // source row of each row of the block
    const int64_t row0 = (int64_t)blockIdx.x * p.rows_per_block;
    for (int rr = threadIdx.x; rr < p.rows_per_block; rr += NT) {
        const int64_t row = row0 + rr;
        if (row < p.rows_total) {
            int64_t r, n, j, src, ps;
            split_row(row, p.b, p.tloc, r, n, j);
            source_row(p.tab, p.cp, r, j, src, ps);
            srow[rr] = n * p.s + src;
        }
    }
    __syncthreads();
    // Eight 16-byte reads in flight per lane before the eight writes: one
    // read at a time (a write between them) leaves HBM latency-bound.
    // Full blocks run unpredicated; the last block one vector at a time.
    constexpr int U = 8;
    const int nvec = p.rows_per_block * p.vecs_per_row;
    const int64_t rows_here = p.rows_total - row0;
    const int full = rows_here >= p.rows_per_block ? nvec / (U * NT) * (U * NT) : 0;
    const __attribute__((address_space(1))) u32x4 *xg =
        (const __attribute__((address_space(1))) u32x4 *)p.x;
    __attribute__((address_space(1))) u32x4 *zg = (__attribute__((address_space(1))) u32x4 *)p.xz;
    for (int i0 = 0; i0 < full; i0 += U * NT) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int i = i0 + k * NT + threadIdx.x;
            const int rr = i / p.vecs_per_row;
            v[k] = xg[srow[rr] * p.vecs_per_row + (i - rr * p.vecs_per_row)];
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int i = i0 + k * NT + threadIdx.x;
            zg[row0 * p.vecs_per_row + i] = v[k];
        }
    }
    for (int i = full + threadIdx.x; i < nvec; i += NT) {
        const int rr = i / p.vecs_per_row;
        const int vv = i - rr * p.vecs_per_row;
        const int64_t row = row0 + rr;
        if (row >= p.rows_total) break;
        zg[row * p.vecs_per_row + vv] = xg[srow[rr] * p.vecs_per_row + vv];
    }
    if (p.pos != nullptr && blockIdx.x == 0) write_positions(p.tab, p.cp, p.tloc, p.pos);
}

template <typename T>
struct RopeParams {
    const T *x;
    T *xz;
    int32_t *pos;
    int64_t s, tloc, b, rows_total;
    int cp, h, d;
    int rows_per_block;
    double theta;
    SeqTable tab;
};

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
    return __uint_as_float((unsigned)v << 16);
}
template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
    __bf16 b = (__bf16)v;   // round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

constexpr int MAX_ROPE_ROWS = 64;      // rows per workgroup
constexpr int MAX_HALF = 64;           // d / 2

// A run of whole output rows per workgroup, as the copy kernel.  The
// workgroup first finds each row's source row and position, then fills a
// table of the run's cos and sin (angles in fp64, rounded to fp32; the
// inverse frequencies theta^(-2t/d) once per workgroup), then rotates: a
// lane takes the 16-byte vector at dims [e, e + EV) of one head together
// with its partner at [e + d/2, e + d/2 + EV) (the rotate-half pairs),
// both read with 16-byte loads, four pairs in flight, and writes both
// rotated vectors with 16-byte stores.
template <typename T>
__global__ void __launch_bounds__(NT) partition_rope(RopeParams<T> p) {
    constexpr int EV = 16 / sizeof(T);          // elements per 16-byte vector
    __shared__ int64_t srow[MAX_ROPE_ROWS];     // source element offset of each row
    __shared__ double inv_freq[MAX_HALF];
    __shared__ float cs[MAX_ROPE_ROWS][MAX_HALF];
    __shared__ float sn[MAX_ROPE_ROWS][MAX_HALF];
    __shared__ int32_t rpos[MAX_ROPE_ROWS];
    const int half = p.d / 2;
    const int64_t row0 = (int64_t)blockIdx.x * p.rows_per_block;
    const int nrows = (int)min((int64_t)p.rows_per_block, p.rows_total - row0);
    for (int rr = threadIdx.x; rr < nrows; rr += NT) {
        int64_t r, n, j, sp, gp;
        split_row(row0 + rr, p.b, p.tloc, r, n, j);
        source_row(p.tab, p.cp, r, j, sp, gp);
        srow[rr] = (n * p.s + sp) * (int64_t)p.h * p.d;
        rpos[rr] = (int32_t)gp;
    }
    for (int t = threadIdx.x; t < half; t += NT)
        inv_freq[t] = pow(p.theta, -2.0 * (double)t / (double)p.d);
    __syncthreads();
    for (int e = threadIdx.x; e < nrows * half; e += NT) {
        const int rr = e / half, t = e - rr * half;
        double sv, cv;
        sincos((double)rpos[rr] * inv_freq[t], &sv, &cv);
        cs[rr][t] = (float)cv;
        sn[rr][t] = (float)sv;
    }
    __syncthreads();

    // tasks: (row of the run, head, vector pair) with the pair fastest
    const int pairs = half / EV;
    const int per_row = p.h * pairs;
    const int ntask = nrows * per_row;
    const __attribute__((address_space(1))) u32x4 *xg =
        (const __attribute__((address_space(1))) u32x4 *)p.x;
    __attribute__((address_space(1))) u32x4 *zg = (__attribute__((address_space(1))) u32x4 *)p.xz;
    constexpr int U = 4;
    for (int i0 = 0; i0 < ntask; i0 += U * NT) {
        u32x4 lo[U], hi[U];
        int64_t dst[U];
        int rrow[U], tt[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            // lanes past the last task repeat it (their stores are skipped)
            const int task = min(i0 + k * NT + (int)threadIdx.x, ntask - 1);
            const int rr = task / per_row;
            const int rem = task - rr * per_row;
            const int hh = rem / pairs, jp = rem - hh * pairs;
            const int64_t off = (int64_t)hh * p.d + jp * EV;   // element offset in the row
            lo[k] = xg[(srow[rr] + off) / EV];
            hi[k] = xg[(srow[rr] + off + half) / EV];
            dst[k] = ((row0 + rr) * (int64_t)p.h * p.d + off) / EV;
            rrow[k] = rr;
            tt[k] = jp * EV;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            if (i0 + k * NT + (int)threadIdx.x >= ntask) continue;
            const T *a = (const T *)&lo[k];
            const T *bq = (const T *)&hi[k];
            u32x4 olo, ohi;
            T *ya = (T *)&olo;
            T *yb = (T *)&ohi;
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const float x1 = to_f32(a[e]), x2 = to_f32(bq[e]);
                const float cn = cs[rrow[k]][tt[k] + e], s1 = sn[rrow[k]][tt[k] + e];
                ya[e] = from_f32<T>(x1 * cn - x2 * s1);
                yb[e] = from_f32<T>(x2 * cn + x1 * s1);
            }
            zg[dst[k]] = olo;
            zg[dst[k] + half / EV] = ohi;
        }
    }
    if (p.pos != nullptr && blockIdx.x == 0) write_positions(p.tab, p.cp, p.tloc, p.pos);
}

}  // namespace

hipError_t launch_partition(const cpattn_dims &dims, int dtype, int h, const SeqTable &tab,
                            const void *x, void *xz, int32_t *pos, const cpattn_rope *rope,
                            hipStream_t stream) {
    const int es = dtype == CPATTN_BF16 ? 2 : 4;
    const int64_t tloc = dims.s / dims.cp;
    const int64_t rows_total = (int64_t)dims.cp * dims.b * tloc;
    if (rope == nullptr) {
        CopyParams p;
        p.x = (const char *)x;
        p.xz = (char *)xz;
        p.pos = pos;
        p.s = dims.s;
        p.tloc = tloc;
        p.b = dims.b;
        p.rows_total = rows_total;
        p.cp = dims.cp;
        p.vecs_per_row = (int)((int64_t)h * dims.d * es / 16);
        p.tab = tab;
        // about 64 KiB per workgroup (d >= 64 and es >= 2 give at least 8
        // vectors per row, so at most MAX_ROWS_PER_BLOCK rows)
        p.rows_per_block = p.vecs_per_row >= 4096 ? 1 : 4096 / p.vecs_per_row;
        if (p.rows_per_block > MAX_ROWS_PER_BLOCK) return hipErrorInvalidValue;
        const int64_t blocks = (rows_total + p.rows_per_block - 1) / p.rows_per_block;
        hipLaunchKernelGGL(partition_copy, dim3((unsigned)blocks), dim3(NT), 0, stream, p);
        return hipGetLastError();
    }
    // runs of whole rows, about 64 KiB of input per workgroup
    const int64_t row_bytes = (int64_t)h * dims.d * es;
    int rpb = (int)(65536 / row_bytes);
    rpb = rpb < 1 ? 1 : (rpb > MAX_ROPE_ROWS ? MAX_ROPE_ROWS : rpb);
    if (dims.d / 2 > MAX_HALF || (dims.d / 2) % (16 / es) != 0) return hipErrorInvalidValue;
    const int64_t blocks = (rows_total + rpb - 1) / rpb;
    if (dtype == CPATTN_BF16) {
        RopeParams<uint16_t> p{(const uint16_t *)x, (uint16_t *)xz, pos, dims.s, tloc, dims.b,
                               rows_total, dims.cp, h, dims.d, rpb, rope->theta, tab};
        hipLaunchKernelGGL(partition_rope<uint16_t>, dim3((unsigned)blocks), dim3(NT), 0,
                           stream, p);
    } else {
        RopeParams<float> p{(const float *)x, (float *)xz, pos, dims.s, tloc, dims.b,
                            rows_total, dims.cp, h, dims.d, rpb, rope->theta, tab};
        hipLaunchKernelGGL(partition_rope<float>, dim3((unsigned)blocks), dim3(NT), 0,
                           stream, p);
    }
    return hipGetLastError();
}

}  // namespace cpattn
