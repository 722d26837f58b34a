// NF4 group-64 encoder (nf4_pack) and tile restorer (nf4_dequant_tile) for gfx950.
//
// deep-fold README, "Метод": every group of 64 weights carries 4-bit NF4 codes
// and one FP16 scale; kernels restore only the fragment of the current tile,
// into BF16.  The encoder there is an offline CPU tool; here it is a device
// kernel so a weight matrix never has to leave HBM, and it is bit-exact by
// construction: the scale is a correctly rounded fp16, and every code decision
// is an exact comparison in fp64 (w > m_i * s with both factors exactly
// representable and their product exact).
#include "device_common.h"

namespace wsl {

// IEEE binary16 round-to-nearest-even of a non-negative finite binary32 value,
// in integer arithmetic (independent of the hardware conversion's modes).
__device__ __forceinline__ uint32_t f16_rne_bits(float a) {
    const uint32_t u = __builtin_bit_cast(uint32_t, a);
    const uint32_t e = u >> 23;
    const uint32_t m = u & 0x7fffffu;
    if (e == 0) return 0;                         // below 2^-126: rounds to +0
    const int E = static_cast<int>(e) - 127;
    if (E >= 16) return 0x7c00;                   // >= 65536: +inf
    if (E >= -14) {                               // normal range of binary16
        uint32_t h = (static_cast<uint32_t>(E + 15) << 10) | (m >> 13);
        const uint32_t rem = m & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;   // a carry may give +inf
        return h;
    }
    const int sh = -(E + 1);                      // subnormal: units of 2^-24
    if (sh > 24) return 0;
    const uint32_t full = m | 0x800000u;
    uint32_t q = full >> sh;
    const uint32_t rem = full & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    return q;
}

// One thread per (row, group).  Reads 64 bf16 (128 B), writes 32 code bytes
// and one fp16 scale in the device layout.
__global__ __launch_bounds__(256) void nf4_pack_kernel(const uint16_t *__restrict__ w, int64_t n_out,
                                                       int64_t k, uint8_t *__restrict__ packed,
                                                       uint32_t *__restrict__ status) {
    const int64_t groups = k >> 6;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= n_out * groups) return;
    const int64_t n = t / groups;
    const int64_t g = t - n * groups;

    const uint4 *src = reinterpret_cast<const uint4 *>(w + n * k + g * 64);
    uint32_t v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 q = src[i];
        v[4 * i + 0] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
    uint32_t amax = 0;
    bool nonfinite = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t lo = v[i] & 0x7fffu, hi = (v[i] >> 16) & 0x7fffu;
        nonfinite |= (lo >= 0x7f80u) | (hi >= 0x7f80u);
        amax = lo > amax ? lo : amax;
        amax = hi > amax ? hi : amax;
    }
    uint32_t sbits = f16_rne_bits(__builtin_bit_cast(float, amax << 16));
    uint32_t st = 0;
    if (nonfinite) st |= WSL_STATUS_NONFINITE;
    else if (sbits >= 0x7c00u) st |= WSL_STATUS_OVERFLOW;

    uint32_t words[8];
    if (st != 0 || sbits == 0) {
        sbits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) words[i] = 0x77777777u;   // every code 7 (the exact zero)
    } else {
        const double s = static_cast<double>(f16_to_f32(sbits));
        double thr[15];
#pragma unroll
        for (int i = 0; i < 15; ++i)
            thr[i] = ((static_cast<double>(level(i)) + static_cast<double>(level(i + 1))) * 0.5) * s;
#pragma unroll
        for (int wi = 0; wi < 8; ++wi) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t pair = v[wi * 4 + (j >> 1)];
                const uint32_t hbits = (j & 1) ? (pair >> 16) : (pair & 0xffffu);
                const double x = static_cast<double>(__builtin_bit_cast(float, hbits << 16));
                uint32_t code = 0;
#pragma unroll
                for (int i = 0; i < 15; ++i) code += (x > thr[i]) ? 1u : 0u;
                word |= code << (4 * j);
            }
            words[wi] = word;
        }
    }
    if (st != 0 && status != nullptr) atomicOr(status, st);

    uint4 *dst = reinterpret_cast<uint4 *>(packed + n * (k >> 1) + g * 32);
    dst[0] = make_uint4(rotl32(words[0], 2), rotl32(words[1], 2), rotl32(words[2], 2), rotl32(words[3], 2));
    dst[1] = make_uint4(rotl32(words[4], 2), rotl32(words[5], 2), rotl32(words[6], 2), rotl32(words[7], 2));
    uint16_t *scales = reinterpret_cast<uint16_t *>(packed + n_out * (k >> 1));
    scales[scale_index(n, g, groups, n_out)] = static_cast<uint16_t>(sbits);
}

// One thread per tile element (a diagnostic path; the linear kernels restore
// weights in registers instead).
__global__ __launch_bounds__(256) void nf4_dequant_tile_kernel(const uint8_t *__restrict__ packed, int64_t n_out,
                                                               int64_t k, int64_t row0, int64_t k0,
                                                               int64_t rows, int64_t cols,
                                                               uint16_t *__restrict__ tile, int64_t ld) {
    const int64_t groups = k >> 6;
    const uint32_t *words = reinterpret_cast<const uint32_t *>(packed);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * (k >> 1));
    const int64_t total = rows * cols;
    for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
         idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t r = idx / cols, c = idx - r * cols;
        const int64_t n = row0 + r, kk = k0 + c;
        const uint32_t canon = rotr32(words[n * (k >> 3) + (kk >> 3)], 2);
        const int code = static_cast<int>((canon >> (4 * (kk & 7))) & 15u);
        const float s = f16_to_f32(scales[scale_index(n, kk >> 6, groups, n_out)]);
        const float p = level(code) * s;
        tile[r * ld + c] = static_cast<uint16_t>(pack_bf16x2(p, 0.0f) & 0xffffu);
    }
}

int launch_pack(const void *w, int64_t n_out, int64_t k, void *packed, uint32_t *status, hipStream_t s) {
    const int64_t work = n_out * (k >> 6);
    const int64_t blocks = (work + 255) / 256;
    if (blocks > 0x7fffffff) return WSL_E_SHAPE;
    hipLaunchKernelGGL(nf4_pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(w), n_out, k, static_cast<uint8_t *>(packed), status);
    return WSL_OK;
}

int launch_dequant_tile(const void *packed, int64_t n_out, int64_t k, int64_t row0, int64_t k0, int64_t rows,
                        int64_t cols, void *tile, int64_t ld, hipStream_t s) {
    const int64_t total = rows * cols;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(nf4_dequant_tile_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint8_t *>(packed), n_out, k, row0, k0, rows, cols,
                       static_cast<uint16_t *>(tile), ld);
    return WSL_OK;
}

}  // namespace wsl
