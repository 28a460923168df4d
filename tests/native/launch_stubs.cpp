// Host stand-ins for the kernel launchers of libcpattn (csrc/internal.h),
// for the sanitizer build of the C ABI's host code (api.cpp) on a machine
// with no GPU.  Each stub reads every host-side argument the real launcher
// reads (so AddressSanitizer checks the arrays api.cpp hands over), checks
// the invariants the kernels rely on, and counts its calls; a broken
// invariant aborts.  Device pointers are never dereferenced.
#include <stdio.h>
#include <stdlib.h>

#include "internal.h"

namespace stubs {
int launches[16];
enum { PARTITION, STEP_BF16, STEPS_BF16, FUSED, STEP_BWD, DQ_SHARE, DKDV_STEPS, DELTA, FILL,
       STEP_F32, MERGE };
}

#define REQUIRE(c)                                                              \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "launch stub: %s failed at line %d\n", #c, __LINE__); \
            abort();                                                            \
        }                                                                       \
    } while (0)

namespace cpattn {

static void check_geom(const StepGeom &g) {
    REQUIRE(g.b >= 1 && g.two_c >= 2 && g.hq >= g.hkv && g.hq % g.hkv == 0);
    REQUIRE(g.q_row0 + g.nq <= g.two_c && g.nk <= g.two_c && g.nq >= 1 && g.nk >= 1);
    REQUIRE(g.scale > 0.0f);
}

static void check_table(const SeqTable &t) {
    REQUIRE(t.nseq >= 1 && t.nseq <= CPATTN_MAX_SEQS && t.lcu[0] == 0);
    for (int i = 0; i < t.nseq; ++i) REQUIRE(t.lcu[i + 1] > t.lcu[i]);
}

hipError_t launch_partition(const cpattn_dims &dims, int dtype, int h, const SeqTable &tab,
                            const void *x, void *xz, int32_t *, const cpattn_rope *rope,
                            hipStream_t) {
    check_table(tab);
    REQUIRE(x && xz && h >= 1 && (dtype == CPATTN_F32 || dtype == CPATTN_BF16));
    REQUIRE((int64_t)tab.lcu[tab.nseq] * dims.cp == dims.s);
    if (rope) REQUIRE(rope->theta > 0.0);
    ++stubs::launches[stubs::PARTITION];
    return hipSuccess;
}

hipError_t launch_step_bf16(const StepGeom &g, const void *q, const void *k, const void *v,
                            float *o, float *lse, hipStream_t) {
    check_geom(g);
    REQUIRE(q && k && v && o && lse && (g.d == 64 || g.d == 128));
    ++stubs::launches[stubs::STEP_BF16];
    return hipSuccess;
}

hipError_t launch_steps_bf16(int n, const StepGeom *g, const void *q, const void *const *k,
                             const void *const *v, float *const *o, float *const *lse,
                             hipStream_t) {
    REQUIRE(n >= 1 && n <= STEPS_PER_GRID && q);
    for (int i = 0; i < n; ++i) {
        check_geom(g[i]);
        REQUIRE(k[i] && v[i] && o[i] && lse[i]);
    }
    ++stubs::launches[stubs::STEPS_BF16];
    return hipSuccess;
}

hipError_t launch_fused_bf16(const FusedGeom &f, const void *qz, const void *kz, const void *vz,
                             void *o, bool, float *, hipStream_t) {
    check_table(f.tab);
    REQUIRE(qz && kz && vz && o && f.rank >= 0 && f.rank < f.cp && (f.d == 64 || f.d == 128));
    ++stubs::launches[stubs::FUSED];
    return hipSuccess;
}

hipError_t launch_step_bwd_bf16(const StepGeom &g, const SeqTable &tab, int mode, const void *q,
                                const void *k, const void *v, const void *dout, const float *lse,
                                const float *delta, float *dq, float *dk, float *dv, hipStream_t,
                                bool) {
    check_geom(g);
    check_table(tab);
    REQUIRE(mode >= CPATTN_CAUSAL && mode <= CPATTN_Q_SECOND_HALF);
    REQUIRE(q && k && v && dout && lse && delta && dq && dk && dv);
    ++stubs::launches[stubs::STEP_BWD];
    return hipSuccess;
}

hipError_t launch_bwd_dq_share_bf16(const StepGeom &g, const SeqTable &tab, int rank, int cp,
                                    const void *q, const void *kz, const void *vz,
                                    const void *dout, const float *lse, const float *delta,
                                    float *dq, hipStream_t) {
    check_geom(g);
    check_table(tab);
    REQUIRE(rank >= 0 && rank < cp && q && kz && vz && dout && lse && delta && dq);
    ++stubs::launches[stubs::DQ_SHARE];
    return hipSuccess;
}

hipError_t launch_bwd_dkdv_steps_bf16(int n, const StepGeom *g, const SeqTable &tab,
                                      const int *mode, const void *q, const void *const *k,
                                      const void *const *v, const void *dout, const float *lse,
                                      const float *delta, float *const *dk, float *const *dv,
                                      hipStream_t) {
    check_table(tab);
    REQUIRE(n >= 1 && q && dout && lse && delta);
    for (int i = 0; i < n; ++i) {
        check_geom(g[i]);
        REQUIRE(mode[i] >= CPATTN_CAUSAL && mode[i] <= CPATTN_Q_SECOND_HALF);
        REQUIRE(k[i] && v[i] && dk[i] && dv[i]);
        for (int j = 0; j < i; ++j) REQUIRE(dk[j] != dk[i]);   // each step owns its block
    }
    stubs::launches[stubs::DKDV_STEPS] += (n + 31) / 32;
    return hipSuccess;
}

hipError_t launch_bwd_delta(int64_t b, int64_t two_c, int hq, int d, const float *o,
                            const void *dout, float *delta, hipStream_t) {
    REQUIRE(b >= 1 && two_c >= 2 && hq >= 1 && (d == 64 || d == 128) && o && dout && delta);
    ++stubs::launches[stubs::DELTA];
    return hipSuccess;
}

hipError_t launch_bwd_prep(int64_t b, int64_t two_c, int hq, int d, const float *o,
                           const void *dout, const float *lse, float inv_scale, float *nl,
                           float *nd, hipStream_t) {
    REQUIRE(b >= 1 && two_c >= 2 && hq >= 1 && (d == 64 || d == 128) && o && dout && lse && nl &&
            nd);
    REQUIRE(inv_scale > 0.0f && nd == nl + b * hq * two_c);
    ++stubs::launches[stubs::DELTA];
    return hipSuccess;
}

hipError_t launch_fill_zero(float *x, int64_t n, hipStream_t) {
    REQUIRE(x && n >= 0 && n % 4 == 0);
    ++stubs::launches[stubs::FILL];
    return hipSuccess;
}

hipError_t launch_step_f32(const StepGeom &g, const void *q, const void *k, const void *v,
                           float *o, float *lse, hipStream_t) {
    check_geom(g);
    REQUIRE(q && k && v && o && lse && (g.d == 64 || g.d == 128));
    ++stubs::launches[stubs::STEP_F32];
    return hipSuccess;
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t) {
    REQUIRE(a.n >= 1 && a.n <= CPATTN_MERGE_PASS && a.o_out);
    REQUIRE((a.run_o == nullptr) == (a.run_l == nullptr));
    for (int i = 0; i < a.n; ++i) {
        REQUIRE(a.parts[i].o && a.parts[i].lse);
        REQUIRE(a.parts[i].row0 >= 0 && a.parts[i].rows >= 1);
        REQUIRE(a.parts[i].row0 + a.parts[i].rows <= a.two_c);
    }
    ++stubs::launches[stubs::MERGE];
    return hipSuccess;
}

}  // namespace cpattn
