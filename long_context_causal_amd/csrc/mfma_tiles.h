// Operand tiles of v_mfma_f32_32x32x16_bf16 on gfx950: vector types, the
// row permutation that makes an MFMA result the next MFMA's operand, the
// two LDS reads that feed the matrix cores, and the direct global -> LDS
// copies that fill them.  Shared by the forward and backward attention
// kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {
namespace tiles {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Matrix row m of an MFMA operand is fed tile row swap_bits23(m) (bits 2 and
// 3 swapped): then register v of a 32x32 result, which holds matrix row
// 8*(v/4) + 4*hi + v%4, holds tile row 8*hi + v (v < 8) or 16 + 8*hi + v-8,
// i.e. the 8 consecutive rows a lane supplies along K of the next MFMA.
__device__ __forceinline__ int swap_bits23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Bytes of one LDS tile row: a bf16 row of a 128-wide head.
constexpr int ROW_BYTES = 256;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Row operand of one k-step (16 consecutive head dims of one tile row): the
// lane's 16-byte chunk, one ds_read_b128.
__device__ __forceinline__ bf16x8 k_read(unsigned addr) {
    return __builtin_bit_cast(bf16x8, *(const lds_u32x4 *)(uintptr_t)addr);
}

// Transposed operand (8 consecutive tile rows of one head-dim column per
// lane) of row chunk kc (16 rows) for one 32-wide head-dim tile.  Lane
// L = 16*g + 4*j + q reads, for s in {0, 1}, the 8-byte block at tile row
// kc*16 + 8*(g/2) + 4*s + j, head dims dt*32 + 16*(g%2) + 4*q .. +3; the
// transpose hands lane t of group g the column dt*32 + 16*(g%2) + t for rows
// +0..3 of that row block.  addr: row 8*(g/2) + j of the tile's dims block;
// RB: bytes per tile row.
template <int RB = ROW_BYTES>
__device__ __forceinline__ bf16x8 vt_read(unsigned addr) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)addr);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4 *)(uintptr_t)(addr + 4 * RB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Reductions across the two 32-lane halves of a wave (lane l with l ^ 32)
// by one v_permlane32_swap: it exchanges the upper half of its first operand
// with the lower half of its second, so with x in both every lane ends up
// holding {x[l], x[l ^ 32]} in the pair, in some order.  A plain VALU
// instruction: unlike a lane shuffle it does not go through the LDS queue.
__device__ __forceinline__ void swap_halves(float &a, float &b) {
    // two wait states on each side cover the VALU-write and result-read
    // hazards that the compiler does not see through inline asm
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float halves_max(float x) {
    float y = x;
    swap_halves(x, y);
    return fmaxf(x, y);
}
__device__ __forceinline__ float halves_sum(float x) {
    float y = x;
    swap_halves(x, y);
    return x + y;
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One direct global -> LDS copy of 16 bytes per lane from base + off (base
// wave-uniform, in SGPRs; off a per-lane byte offset); lane L writes
// lds_base + 16*L.  m0 carries the LDS base (declared clobbered, so the
// compiler keeps nothing of its own there across the copy); one wait state
// separates its write from the copy that reads it.
__device__ __forceinline__ void dma16(const void *base, unsigned off, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds_base)
                 : "memory", "m0");
}

// One direct global -> LDS copy of 4 bytes per lane from the lane's own
// address; lane L writes lds_base + 4*L.
__device__ __forceinline__ void dma4(const void *addr, unsigned lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(addr), "s"(lds_base)
                 : "memory", "m0");
}

// Waits for the wave's LDS operations, then for every wave of the workgroup.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace tiles
}  // namespace cpattn
