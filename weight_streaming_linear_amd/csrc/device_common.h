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

// Round-to-nearest-even binary32 -> bf16 (hardware conversion, finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = static_cast<__bf16>(lo);
    __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
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

// Sum across the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace wsl
