// Peak check for the roofline: the bf16 matrix-core rate this part sustains
// on a stream of v_mfma_f32_32x32x16_bf16 with no memory traffic, the
// denominator that sits beside the published dense peak.  Also an LDS fill
// that the memory-safety tests run before each attention launch.
//
// Every wave keeps eight independent accumulators and feeds each MFMA a
// different pair of its eight operand registers (loaded once from the
// caller's random bf16 values), so successive MFMAs see changing data as in
// the attention kernels: matrix throughput on this part depends on the
// operand bits.  Workgroups of 8 waves, two waves per SIMD, like the
// attention kernels: each workgroup reserves 96 KiB of LDS it does not
// use, so one workgroup runs per CU at a time and the grid runs in rounds.
// One float per lane (the sum of its accumulators) is written so nothing
// is optimised away.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "cpattn_probe.h"
#include "mfma_tiles.h"

namespace cpattn {
namespace {

using namespace tiles;

constexpr int NT = 512;
constexpr unsigned LDS_RESERVE = 96 * 1024;   // one workgroup per CU

__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_probe(const uint16_t *operands, float *out, int iters) {
    const int lane = threadIdx.x & 63;
    // eight bf16x8 operands per lane from a 4096-value table
    bf16x8 r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint16_t *src = operands + ((j * 64 + lane) * 8) % 4096;
        r[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)src);
    }
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    r[(j + u) & 7], r[(j + 2 * u + 3) & 7], acc[j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[j][e];
    out[(int64_t)blockIdx.x * NT + threadIdx.x] = sum;
}

// Every 16-byte word of the LDS a workgroup can hold (160 KiB on gfx950) set
// to one pattern, so one workgroup runs per CU at a time.  The LDS keeps
// its contents after a kernel ends, so a kernel that ran on a CU before
// another can leave values the later one might read if it used LDS it had
// not written.  The asm statement takes the array's address and clobbers
// memory, so the stores are not removed as dead.
constexpr int LDS_FILL_WORDS = 160 * 1024 / 16;
constexpr int LDS_FILL_NT = 256;

__global__ void __launch_bounds__(LDS_FILL_NT) lds_fill(uint32_t pattern) {
    __shared__ u32x4 words[LDS_FILL_WORDS];
    const u32x4 v = {pattern, pattern, pattern, pattern};
    for (int i = threadIdx.x; i < LDS_FILL_WORDS; i += LDS_FILL_NT) words[i] = v;
    asm volatile("s_waitcnt lgkmcnt(0)" ::"v"((unsigned)(uintptr_t)words) : "memory");
}

}  // namespace
}  // namespace cpattn

extern "C" {

int cpattn_probe_mfma(const void *operands, float *out, int blocks, int iters, void *stream) {
    if (operands == nullptr || out == nullptr || blocks < 1 || iters < 1) return 1;
    if (((uintptr_t)operands & 15u) != 0) return 1;
    hipLaunchKernelGGL(cpattn::mfma_probe, dim3((unsigned)blocks), dim3(cpattn::NT),
                       cpattn::LDS_RESERVE, (hipStream_t)stream, (const uint16_t *)operands, out,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int cpattn_probe_fill_lds(unsigned pattern, int blocks, void *stream) {
    if (blocks < 1) return 1;
    hipLaunchKernelGGL(cpattn::lds_fill, dim3((unsigned)blocks), dim3(cpattn::LDS_FILL_NT), 0,
                       (hipStream_t)stream, (uint32_t)pattern);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int cpattn_device_info(int *compute_units, int *max_clock_khz) {
    if (compute_units == nullptr || max_clock_khz == nullptr) return 1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, dev) !=
        hipSuccess)
        return 1;
    if (hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess)
        return 1;
    return 0;
}

}  // extern "C"
