// Device-side definitions shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wsl.h"

namespace wsl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte streaming load: weights are read once per call, so they are loaded
// non-temporally and do not displace the small, reused operands from cache.
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The 16 NF4 levels as binary32 bit patterns, ascending: normal quantiles with
// an exact zero, scaled so that the extremes are -1 and +1 (NF4 as introduced
// in QLoRA; deep-fold README, "Метод").  Built once on the host and frozen
// here as literals, so that every kernel multiplies by exactly these bits.
constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

__device__ __forceinline__ float level(int code) { return __builtin_bit_cast(float, kLevelBits[code]); }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Round-to-nearest-even binary32 -> bf16 of two values, lo in bits 0..15 (one
// v_cvt_pk_bf16_f32; finite inputs).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// Index (in fp16 elements) of scale (row n, group g) in the device layout:
// rows in blocks of 16, [group][row] inside a block; the last block has rb rows.
__device__ __forceinline__ int64_t scale_index(int64_t n, int64_t g, int64_t groups, int64_t n_out) {
    const int64_t blk = n >> 4;
    const int64_t rem = n_out - (blk << 4);
    const int64_t rb = rem < 16 ? rem : 16;
    return blk * 16 * groups + g * rb + (n & 15);
}

__device__ __forceinline__ uint32_t rotl32(uint32_t v, int s) { return (v << s) | (v >> (32 - s)); }
__device__ __forceinline__ uint32_t rotr32(uint32_t v, int s) { return (v >> s) | (v << (32 - s)); }

// Pair table (64 KB, one ds_read_b64 per two codes).  Entry of byte value b (the
// codes of two consecutive k, even k in the low nibble) = (level(b & 15),
// level(b >> 4)), replicated 32 times: lane l reads copy l % 32 at byte offset
// b * 256 + (l % 32) * 8, so the 32 lanes served together touch 32 distinct
// 8-byte bank pairs whatever the codes are.  The address is one SDWA move that
// writes byte B of the (un-rotated) code word into bits 8..15 of a register whose
// low byte already holds the lane's copy offset.
constexpr int kPairTableBytes = 256 * 32 * 8;

template <int B>
__device__ __forceinline__ void pair_addr(uint32_t &a, uint32_t w) {
    if constexpr (B == 0)
        asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0" : "+v"(a) : "v"(w));
    else if constexpr (B == 1)
        asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1" : "+v"(a) : "v"(w));
    else if constexpr (B == 2)
        asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_2" : "+v"(a) : "v"(w));
    else
        asm("v_mov_b32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3" : "+v"(a) : "v"(w));
}

// The 16 levels into lut[0..15] (LDS).  Lane c < 16 selects its level from the
// literals with compare-selects, so no memory load sits in a kernel prologue.
__device__ __forceinline__ void write_levels(float *lut) {
    if (threadIdx.x < 16) {
        uint32_t v = kLevelBits[0];
#pragma unroll
        for (int c = 1; c < 16; ++c) v = (threadIdx.x == static_cast<unsigned>(c)) ? kLevelBits[c] : v;
        lut[threadIdx.x] = __builtin_bit_cast(float, v);
    }
}

// Fill the pair table (kPairTableBytes of LDS at `tab`) cooperatively; the caller
// synchronizes the workgroup before the first lookup.
// Entries by low nibble: a wave takes the byte values with low nibble L or L + 1 (L even;
// lanes 0..31 write copy l of L, lanes 32..63 copy l - 32 of L + 1) for all 16 high
// nibbles.  Each lane selects level(L + its half) once from the literals; level(high) is
// a literal of the unrolled loop and the high nibble an immediate offset of the LDS
// write, so the fill issues no memory load and needs no wait of its own: 16 writes per
// wave for the 8 values of L (waves beyond 8 have nothing to do; fewer waves take several
// L each).  blockDim.x must be a multiple of 64.
__device__ __forceinline__ void fill_pair_table(char *tab) {
    const int wave = static_cast<int>(threadIdx.x >> 6);
    const int nw = static_cast<int>(blockDim.x >> 6);
    const int lane = static_cast<int>(threadIdx.x & 63);
    for (int l2 = wave; l2 < 8; l2 += nw) {
        const int lo = 2 * l2 + (lane >> 5);
        uint32_t v = kLevelBits[0];
#pragma unroll
        for (int c = 1; c < 16; ++c) v = (lo == c) ? kLevelBits[c] : v;
        const float lvl = __builtin_bit_cast(float, v);
        float2 *t2 = reinterpret_cast<float2 *>(tab + lo * 256 + (lane & 31) * 8);
#pragma unroll
        for (int hi = 0; hi < 16; ++hi) t2[hi * 512] = make_float2(lvl, level(hi));
    }
}

// Workgroup barrier that orders LDS accesses only: waits for this wave's LDS
// operations, not for its global loads still in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum across the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace wsl
