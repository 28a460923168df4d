// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by api.cpp and
// returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#ifdef __HIPCC__
#include <hip/hip_runtime.h>
#endif

#include "cpattn.h"

namespace cpattn {

// Geometry of one step, derived from the dims and the mode.
struct StepGeom {
    int64_t b;
    int64_t two_c;      // rows of a rank's local block
    int32_t hq, hkv, d;
    int64_t q_row0;     // first local query row read
    int64_t nq;         // query rows computed (= rows of O_i)
    int64_t nk;         // keys visible to the step (0..nk-1 of the block)
    bool causal;        // key j visible to row i only if j <= q_row0 + i
    float scale;        // softmax scale
    float scale_log2;   // softmax scale * log2(e)
};

StepGeom step_geom(const cpattn_dims &dims, int mode, float scale);

// The samples packed in each batch element, as kernel arguments: sample i
// occupies local rows [lcu[i], lcu[i+1]) of every rank (lcu = cu_seqlens /
// cp); tile0[i] is the first query tile of sample i in a fused launch (set
// by that launcher).  An unpacked batch is one sample of s rows.
struct SeqTable {
    int32_t nseq;
    int32_t lcu[CPATTN_MAX_SEQS + 1];
    int32_t tile0[CPATTN_MAX_SEQS + 1];
};

#ifdef __HIPCC__
// Largest i in [0, n) with a[i] <= x (a ascending, a[0] <= x); device code
// only (the host side of the library also builds with a plain C++ compiler
// for its sanitizer tests).
__device__ inline int seq_of(const int32_t *a, int n, int x) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}
#endif

hipError_t launch_partition(const cpattn_dims &dims, int dtype, int h, const SeqTable &tab,
                            const void *x, void *xz, int32_t *pos,
                            const cpattn_rope *rope, hipStream_t stream);

hipError_t launch_step_bf16(const StepGeom &g, const void *q, const void *k,
                            const void *v, float *o, float *lse,
                            hipStream_t stream);
// Steps 0 .. n-1 of one rank's share (bf16) in one grid: step i reads
// k[i]/v[i] and writes o[i]/lse[i], as launch_step_bf16 would.  At most
// STEPS_PER_GRID steps per call (their descriptors travel in the kernel
// arguments); hipErrorInvalidValue otherwise.
constexpr int STEPS_PER_GRID = 32;
hipError_t launch_steps_bf16(int n, const StepGeom *g, const void *q, const void *const *k,
                             const void *const *v, float *const *o, float *const *lse,
                             hipStream_t stream);

// Geometry of one rank's fused share (cpattn_forward_fused[_varlen]).
struct FusedGeom {
    int64_t b;
    int64_t two_c;      // local rows per batch element (s / cp)
    int32_t hq, hkv, d, rank, cp;
    float scale_log2;
    SeqTable tab;       // the packed samples (tile0 filled by the launcher)
};

// qz, kz, vz: the partitioned tensors of all ranks [cp, b, s/cp, h, d]
// bf16 (d = 64 or 128).  o: [b, s/cp, hq, d] fp32, or bf16 when out_bf16;
// lse: [b, hq, s/cp] or null.
hipError_t launch_fused_bf16(const FusedGeom &f, const void *qz, const void *kz,
                             const void *vz, void *o, bool out_bf16, float *lse,
                             hipStream_t stream);

// Backward of one step (bf16, d = 64 or 128) for every packed sample of 'tab' in
// step mode 'mode': dq += , dk += , dv += (fp32).  g supplies b, two_c (the
// local rows), the heads and the scale.
hipError_t launch_step_bwd_bf16(const StepGeom &g, const SeqTable &tab, int mode,
                                const void *q, const void *k, const void *v, const void *dout,
                                const float *lse, const float *delta, float *dq, float *dk,
                                float *dv, hipStream_t stream, bool with_dkdv = true);
// The dq of all cp steps of rank's share in one grid (bf16): kz, vz are the
// partitioned K, V of all ranks; every row of dq is written (not added to).
// nl, nd: -L/scale and -D of the rank's rows (launch_bwd_prep).
hipError_t launch_bwd_dq_share_bf16(const StepGeom &g, const SeqTable &tab, int rank, int cp,
                                    const void *q, const void *kz, const void *vz,
                                    const void *dout, const float *nl, const float *nd,
                                    float *dq, hipStream_t stream);
// The dK/dV of steps 0 .. n-1 of one rank's share in one grid: step i
// reads k[i]/v[i] and adds to dk[i]/dv[i] (distinct blocks, zeroed by the
// caller), mode[i] its mode; g[0] supplies the dims and scale, tab the
// packed samples; nl, nd as for the dq grid.
hipError_t launch_bwd_dkdv_steps_bf16(int n, const StepGeom *g, const SeqTable &tab,
                                      const int *mode,
                                      const void *q, const void *const *k,
                                      const void *const *v, const void *dout,
                                      const float *nl, const float *nd, float *const *dk,
                                      float *const *dv, hipStream_t stream);

// delta[n, h, i] = sum_t dout[n, i, h, t] o[n, i, h, t]; o fp32, dout bf16;
// t < d (64 or 128).
hipError_t launch_bwd_delta(int64_t b, int64_t two_c, int hq, int d, const float *o,
                            const void *dout, float *delta, hipStream_t stream);
// The per-row terms the share's backward grids start their sums from:
// nl[n, h, i] = -lse[n, h, i] * inv_scale and nd[n, h, i] = -delta[n, h, i].
hipError_t launch_bwd_prep(int64_t b, int64_t two_c, int hq, int d, const float *o,
                           const void *dout, const float *lse, float inv_scale, float *nl,
                           float *nd, hipStream_t stream);

// Compute units of the current device (cached per device), 0 if it cannot
// be queried.
int device_cu_count();

// x[0 .. n) = 0 (n a multiple of 4, x 16-byte aligned).
hipError_t launch_fill_zero(float *x, int64_t n, hipStream_t stream);

hipError_t launch_step_f32(const StepGeom &g, const void *q, const void *k,
                           const void *v, float *o, float *lse,
                           hipStream_t stream);

// One launch of the merge: n <= CPATTN_MERGE_PASS partials, plus (when
// run_o is not null) the running fp32 result of earlier passes, folded in as
// a partial that covers every row; run_o / run_l may alias o_out / lse_out.
struct MergeArgs {
    int64_t b, two_c;
    int32_t hq, d;
    int n;
    const cpattn_partial *parts;   // host array, n entries
    const float *run_o;            // [b, 2c, hq, d] fp32, or null
    const float *run_l;            // [b, hq, 2c] fp32 (with run_o)
    int out_dtype;
    void *o_out;
    float *lse_out;
};

hipError_t launch_merge(const MergeArgs &a, hipStream_t stream);

}  // namespace cpattn
