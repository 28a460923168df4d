// Host driver for the sanitizer build of the C ABI (api.cpp linked with the
// launch stubs): every entry point with valid arguments (the stubs check
// what reaches them) and with each kind of invalid argument (refused before
// any launch), the pure host functions over many shapes, and the shapes
// that stress the host arithmetic (cp up to 512, packed tables of 128
// samples, grids at the 32-bit limit).  Device addresses are fake aligned
// integers the stubs never dereference.  Exit status 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "cpattn.h"

namespace stubs {
extern int launches[16];
enum { PARTITION, STEP_BF16, STEPS_BF16, FUSED, STEP_BWD, DQ_SHARE, DKDV_STEPS, DELTA, FILL,
       STEP_F32, MERGE };
}

static int failures = 0;
#define EXPECT(c)                                                               \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "abi driver: %s failed at line %d\n", #c, __LINE__); \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

static void *dev(uintptr_t i) { return (void *)((uintptr_t)1 << 32 | i << 12); }

static cpattn_dims dims(int64_t b, int64_t s, int hq, int hkv, int d, int cp) {
    cpattn_dims x;
    x.b = b;
    x.s = s;
    x.hq = hq;
    x.hkv = hkv;
    x.d = d;
    x.cp = cp;
    return x;
}

static int count(int k) { return stubs::launches[k]; }

static void pure_functions() {
    for (int cp = 1; cp <= 512; cp = cp < 8 ? cp + 1 : cp * 2) {
        // every (step, rank): src and mode; every rank's positions cover 0..s-1 once
        const int64_t c = 3, s = 2 * cp * c;
        std::vector<int> seen(s, 0);
        for (int r = 0; r < cp; ++r) {
            for (int i = 0; i < cp; ++i) {
                int mode, src;
                EXPECT(cpattn_step_mode(i, r, cp, &mode, &src) == CPATTN_OK);
                EXPECT(src == ((r - i) % cp + cp) % cp);
                EXPECT(mode == (i == 0 ? CPATTN_CAUSAL
                                       : i <= r ? CPATTN_KV_FIRST_HALF : CPATTN_Q_SECOND_HALF));
            }
            std::vector<int32_t> pos(2 * c);
            EXPECT(cpattn_partition_positions(s, cp, r, pos.data()) == CPATTN_OK);
            for (int32_t p : pos) ++seen[p];
            cpattn_dims d = dims(1, s, 4, 2, 128, cp);
            const size_t ws = cpattn_forward_workspace(&d, r);
            std::vector<cpattn_partial> parts(cp);
            EXPECT(ws > 0);
            EXPECT(cpattn_forward_partials(&d, r, dev(1), ws, parts.data()) == CPATTN_OK);
            EXPECT(cpattn_forward_partials(&d, r, dev(1), ws - 1, parts.data()) ==
                   CPATTN_ENOSPACE);
            for (int i = 0; i < cp; ++i)
                EXPECT(parts[i].row0 + parts[i].rows <= 2 * c && (uintptr_t)parts[i].o % 256 == 0);
        }
        for (int64_t p = 0; p < s; ++p) EXPECT(seen[p] == 1);
    }
    int mode, src;
    EXPECT(cpattn_step_mode(0, 0, 0, &mode, &src) == CPATTN_EINVAL);
    EXPECT(cpattn_step_mode(3, 0, 3, &mode, &src) == CPATTN_EINVAL);
    EXPECT(cpattn_step_mode(0, 0, 1, nullptr, &src) == CPATTN_EINVAL);
    int32_t pos[8];
    EXPECT(cpattn_partition_positions(10, 2, 0, pos) == CPATTN_ESHAPE);
    EXPECT(cpattn_partition_positions(8, 2, 2, pos) == CPATTN_EINVAL);
    EXPECT(cpattn_partition_positions(8, 2, 0, nullptr) == CPATTN_EINVAL);
    // packed tables: the longest one, and every kind of bad offset
    std::vector<int64_t> cu(CPATTN_MAX_SEQS + 2);
    for (int i = 0; i <= CPATTN_MAX_SEQS + 1; ++i) cu[i] = 8 * i;
    cpattn_varlen vl = {CPATTN_MAX_SEQS, cu.data()};
    std::vector<int32_t> vpos(8 * CPATTN_MAX_SEQS);
    EXPECT(cpattn_partition_positions_varlen(8 * CPATTN_MAX_SEQS, 4, 1, &vl, vpos.data()) ==
           CPATTN_OK);
    vl.nseq = CPATTN_MAX_SEQS + 1;
    EXPECT(cpattn_partition_positions_varlen(8 * (CPATTN_MAX_SEQS + 1), 4, 1, &vl,
                                             vpos.data()) == CPATTN_ESHAPE);
    int64_t bad[3] = {0, 6, 16};
    cpattn_varlen vb = {2, bad};
    EXPECT(cpattn_partition_positions_varlen(16, 2, 0, &vb, vpos.data()) == CPATTN_ESHAPE);
    cpattn_varlen vn = {2, nullptr};
    EXPECT(cpattn_partition_positions_varlen(16, 2, 0, &vn, vpos.data()) == CPATTN_EINVAL);
}

static void device_entry_points() {
    void *stream = nullptr;
    cpattn_dims d = dims(2, 4096, 8, 2, 128, 4);
    const int before_part = count(stubs::PARTITION);
    cpattn_rope rope = {10000.0};
    EXPECT(cpattn_partition(&d, CPATTN_BF16, 8, dev(1), dev(2), (int32_t *)dev(3), &rope,
                            stream) == CPATTN_OK);
    EXPECT(count(stubs::PARTITION) == before_part + 1);
    rope.theta = -1.0;
    EXPECT(cpattn_partition(&d, CPATTN_BF16, 8, dev(1), dev(2), nullptr, &rope, stream) ==
           CPATTN_EINVAL);
    EXPECT(cpattn_partition(&d, 7, 8, dev(1), dev(2), nullptr, nullptr, stream) ==
           CPATTN_EDTYPE);
    EXPECT(count(stubs::PARTITION) == before_part + 1);

    // one step of each mode, both element types
    for (int mode = 0; mode < 3; ++mode) {
        EXPECT(cpattn_step_fwd(&d, CPATTN_BF16, 0.0f, mode, dev(1), dev(2), dev(3),
                               (float *)dev(4), (float *)dev(5), stream) == CPATTN_OK);
        EXPECT(cpattn_step_fwd(&d, CPATTN_F32, 0.25f, mode, dev(1), dev(2), dev(3),
                               (float *)dev(4), (float *)dev(5), stream) == CPATTN_OK);
    }
    EXPECT(cpattn_step_fwd(&d, CPATTN_BF16, 0.0f, 3, dev(1), dev(2), dev(3), (float *)dev(4),
                           (float *)dev(5), stream) == CPATTN_EINVAL);
    // 64-wide heads, forward and backward
    cpattn_dims d64 = dims(2, 4096, 8, 2, 64, 4);
    EXPECT(cpattn_step_fwd(&d64, CPATTN_BF16, 0.0f, 0, dev(1), dev(2), dev(3), (float *)dev(4),
                           (float *)dev(5), stream) == CPATTN_OK);
    EXPECT(cpattn_step_bwd(&d64, CPATTN_BF16, 0.0f, 0, dev(1), dev(2), dev(3), dev(4),
                           (float *)dev(5), (float *)dev(6), (float *)dev(7), (float *)dev(8),
                           (float *)dev(9), stream) == CPATTN_OK);
    cpattn_dims d96 = dims(2, 4096, 8, 2, 96, 4);
    EXPECT(cpattn_step_fwd(&d96, CPATTN_BF16, 0.0f, 0, dev(1), dev(2), dev(3), (float *)dev(4),
                           (float *)dev(5), stream) == CPATTN_ESHAPE);

    // whole shares: cp below, at and above one merge pass and one steps grid
    for (int cp : {1, 4, 33, 64, 65, 128, 256}) {
        cpattn_dims dc = dims(1, 2 * cp * 40, 4, 2, 128, cp);
        for (int r : {0, cp / 2, cp - 1}) {
            const size_t ws = cpattn_forward_workspace(&dc, r);
            const int m0 = count(stubs::MERGE), g0 = count(stubs::STEPS_BF16);
            for (int out : {CPATTN_F32, CPATTN_BF16})
                EXPECT(cpattn_forward(&dc, CPATTN_BF16, 0.0f, r, dev(1), dev(2), dev(3), dev(4),
                                      ws, out, dev(5), out == CPATTN_F32 ? (float *)dev(6)
                                                                         : nullptr,
                                      stream) == CPATTN_OK);
            EXPECT(count(stubs::MERGE) - m0 == 2 * ((cp + CPATTN_MERGE_PASS - 1) /
                                                   CPATTN_MERGE_PASS));
            EXPECT(count(stubs::STEPS_BF16) - g0 == 2 * ((cp + 31) / 32));
            EXPECT(cpattn_forward(&dc, CPATTN_BF16, 0.0f, r, dev(1), dev(2), dev(3), dev(4),
                                  ws - 1, CPATTN_F32, dev(5), nullptr, stream) == CPATTN_ENOSPACE);
            EXPECT(cpattn_forward_fused(&dc, CPATTN_BF16, 0.0f, r, dev(1), dev(2), dev(3),
                                        CPATTN_BF16, dev(5), nullptr, stream) == CPATTN_OK);
            EXPECT(cpattn_backward(&dc, CPATTN_BF16, 0.0f, r, dev(1), dev(2), dev(3),
                                   (const float *)dev(4), dev(5), (const float *)dev(6),
                                   (float *)dev(7), (float *)dev(8), (float *)dev(9),
                                   (float *)dev(10), stream) == CPATTN_OK);
        }
    }
    // merge: one pass, several passes in place, and the refusals
    std::vector<cpattn_partial> parts(200);
    for (int i = 0; i < 200; ++i) {
        parts[i].o = (const float *)dev(100 + i);
        parts[i].lse = (const float *)dev(400 + i);
        parts[i].row0 = i % 2 ? 512 : 0;   // 2c = 1024 local rows
        parts[i].rows = i % 2 ? 512 : 1024;
    }
    const int m0 = count(stubs::MERGE);
    EXPECT(cpattn_merge(&d, 200, parts.data(), CPATTN_F32, dev(1), (float *)dev(2), stream) ==
           CPATTN_OK);
    EXPECT(count(stubs::MERGE) - m0 == 4);
    EXPECT(cpattn_merge(&d, 200, parts.data(), CPATTN_BF16, dev(1), (float *)dev(2), stream) ==
           CPATTN_ESHAPE);
    EXPECT(cpattn_merge(&d, 64, parts.data(), CPATTN_BF16, dev(1), nullptr, stream) == CPATTN_OK);
    parts[7].rows = 1025;
    EXPECT(cpattn_merge(&d, 64, parts.data(), CPATTN_F32, dev(1), nullptr, stream) ==
           CPATTN_ESHAPE);

    // backward of packed samples: the longest table
    cpattn_dims dv = dims(1, 8 * 4 * CPATTN_MAX_SEQS, 4, 2, 128, 4);
    std::vector<int64_t> cu(CPATTN_MAX_SEQS + 1);
    for (int i = 0; i <= CPATTN_MAX_SEQS; ++i) cu[i] = 32 * i;
    cpattn_varlen vl = {CPATTN_MAX_SEQS, cu.data()};
    EXPECT(cpattn_backward_varlen(&dv, CPATTN_BF16, 0.0f, 3, &vl, dev(1), dev(2), dev(3),
                                  (const float *)dev(4), dev(5), (const float *)dev(6),
                                  (float *)dev(7), (float *)dev(8), (float *)dev(9),
                                  (float *)dev(10), stream) == CPATTN_OK);
    EXPECT(cpattn_forward_fused_varlen(&dv, CPATTN_BF16, 0.0f, 3, &vl, dev(1), dev(2), dev(3),
                                       CPATTN_F32, dev(4), (float *)dev(5), stream) == CPATTN_OK);
    EXPECT(cpattn_partition_varlen(&dv, CPATTN_BF16, 4, &vl, dev(1), dev(2), (int32_t *)dev(3),
                                   nullptr, stream) == CPATTN_OK);
    for (int mode = 0; mode < 3; ++mode)
        EXPECT(cpattn_step_bwd(&d, CPATTN_BF16, 0.0f, mode, dev(1), dev(2), dev(3), dev(4),
                               (const float *)dev(5), (const float *)dev(6), (float *)dev(7),
                               (float *)dev(8), (float *)dev(9), stream) == CPATTN_OK);
    EXPECT(cpattn_bwd_delta(&d, (const float *)dev(1), dev(2), (float *)dev(3), stream) ==
           CPATTN_OK);

    // shapes past the limits of the host arithmetic
    cpattn_dims huge = dims(1, (int64_t)1 << 30, 512, 512, 128, 1);
    EXPECT(cpattn_backward(&huge, CPATTN_BF16, 0.0f, 0, dev(1), dev(2), dev(3),
                           (const float *)dev(4), dev(5), (const float *)dev(6), (float *)dev(7),
                           (float *)dev(8), (float *)dev(9), (float *)dev(10),
                           stream) == CPATTN_ESHAPE);
    cpattn_dims wide = dims((int64_t)1 << 20, (int64_t)1 << 20, 1 << 30, 1, 128, 1);
    EXPECT(cpattn_forward_fused(&wide, CPATTN_BF16, 0.0f, 0, dev(1), dev(2), dev(3), CPATTN_F32,
                                dev(4), nullptr, stream) == CPATTN_ESHAPE);
    EXPECT(cpattn_forward_workspace(&wide, 0) == 0);
}

int main() {
    pure_functions();
    device_entry_points();
    if (failures) {
        fprintf(stderr, "abi sanitizer driver: %d failures\n", failures);
        return 1;
    }
    printf("abi sanitizer driver: ok\n");
    return 0;
}
