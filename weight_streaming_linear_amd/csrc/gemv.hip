// Decode GEMV y = W x for gfx950: bf16 weights or packed NF4 weights.
//
// deep-fold README, "Метод" table: decode runs an N=1 NF4 GEMV, with codes and
// scales resident in video memory and restored in registers only for the
// fragment being multiplied.  TCPP README: bf16 weights are used as stored.
// The work is a pure weight stream (each weight byte is read exactly once and
// used for one multiply-add), so both kernels are built around HBM:
//   * a wavefront covers 1 KB of one row per step (64 lanes x 16-byte loads,
//     fully coalesced) and keeps R rows in flight at once;
//   * the waves of a workgroup split the k range of the same R rows, and the
//     partial sums are combined through LDS in a fixed order (deterministic,
//     no atomics);
//   * x is tiny (<= 64 KB) and is read through the cache hierarchy;
//   * NF4 codes are turned into levels through a 16-entry fp32 table in LDS
//     (16 distinct banks, so lanes reading the same entry broadcast and lanes
//     reading different entries never conflict).  The device layout rotates
//     each 32-bit code word left by 2 bits so that one AND with 0x3C on a byte
//     (and, for the odd codes, on the word rotated right by 4) gives the byte
//     address code*4 of the table entry directly.
#include "device_common.h"

namespace wsl {

constexpr int kMaxWaves = 8;

template <int R>
__device__ __forceinline__ void block_reduce_store(float (&acc)[R], float *red, int lane, int wave, int waves,
                                                   int64_t row0, int64_t n_out, float *__restrict__ y) {
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
    if (waves == 1) {
        if (lane < R) {
            float v = acc[0];
#pragma unroll
            for (int r = 1; r < R; ++r) v = (lane == r) ? acc[r] : v;
            if (row0 + lane < n_out) y[row0 + lane] = v;
        }
        return;
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) red[wave * R + r] = acc[r];
    }
    __syncthreads();
    if (wave == 0 && lane < R) {
        float v = red[lane];
        for (int w = 1; w < waves; ++w) v += red[w * R + lane];
        if (row0 + lane < n_out) y[row0 + lane] = v;
    }
}

// ---------------------------------------------------------------- bf16
// Lane slice: 8 consecutive bf16 (16 B); a wave step covers 512 k.
template <int R, int U>
__global__ __launch_bounds__(512) void gemv_bf16_kernel(const uint16_t *__restrict__ w, int64_t n_out, int64_t k,
                                                        const uint16_t *__restrict__ x, float *__restrict__ y) {
    __shared__ float red[kMaxWaves * R];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;

    const uint16_t *rowp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = (row0 + r < n_out) ? row0 + r : n_out - 1;
        rowp[r] = w + row * k;
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    const int64_t step = static_cast<int64_t>(512) * waves;
    for (int64_t kb = static_cast<int64_t>(wave) * 512 + lane * 8; kb < k; kb += step * U) {
        uint4 xv[U];
        uint4 wv[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kk = kb + u * step;
            const bool ok = kk < k;
            xv[u] = ok ? *reinterpret_cast<const uint4 *>(x + kk) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[u][r] = ok ? load_stream16(rowp[r] + kk)
                              : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float x0 = bf16_lo(xv[u].x), x1 = bf16_hi(xv[u].x), x2 = bf16_lo(xv[u].y), x3 = bf16_hi(xv[u].y);
            const float x4 = bf16_lo(xv[u].z), x5 = bf16_hi(xv[u].z), x6 = bf16_lo(xv[u].w), x7 = bf16_hi(xv[u].w);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint4 q = wv[u][r];
                float a = acc[r];
                a = __builtin_fmaf(bf16_lo(q.x), x0, a);
                a = __builtin_fmaf(bf16_hi(q.x), x1, a);
                a = __builtin_fmaf(bf16_lo(q.y), x2, a);
                a = __builtin_fmaf(bf16_hi(q.y), x3, a);
                a = __builtin_fmaf(bf16_lo(q.z), x4, a);
                a = __builtin_fmaf(bf16_hi(q.z), x5, a);
                a = __builtin_fmaf(bf16_lo(q.w), x6, a);
                a = __builtin_fmaf(bf16_hi(q.w), x7, a);
                acc[r] = a;
            }
        }
    }
    block_reduce_store<R>(acc, red, lane, wave, waves, row0, n_out, y);
}

// ---------------------------------------------------------------- NF4
// Dot product of 32 codes (one 16-byte device-layout load) with 32 fp32 x.
__device__ __forceinline__ float nf4_dot32(const uint4 q, const float (&xf)[32], const char *lut) {
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t we = wd[i];
        const uint32_t wo = rotr32(we, 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float le = *reinterpret_cast<const float *>(lut + ((we >> (8 * b)) & 0x3cu));
            const float lo = *reinterpret_cast<const float *>(lut + ((wo >> (8 * b)) & 0x3cu));
            p0 = __builtin_fmaf(le, xf[8 * i + 2 * b], p0);
            p1 = __builtin_fmaf(lo, xf[8 * i + 2 * b + 1], p1);
        }
    }
    return p0 + p1;
}

// Lane slice: 32 consecutive codes (16 B, half a group); a wave step covers 2048 k.
template <int R>
__global__ __launch_bounds__(512) void gemv_nf4_kernel(const uint8_t *__restrict__ packed, int64_t n_out, int64_t k,
                                                       const uint16_t *__restrict__ x, float *__restrict__ y) {
    __shared__ float lut[16];
    __shared__ float red[kMaxWaves * R];
    if (threadIdx.x < 16) lut[threadIdx.x] = level(threadIdx.x);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
    const int64_t groups = k >> 6;
    const int64_t rowbytes = k >> 1;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);

    int64_t rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = (row0 + r < n_out) ? row0 + r : n_out - 1;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    const char *lutp = reinterpret_cast<const char *>(lut);
    const int64_t step = static_cast<int64_t>(2048) * waves;
    for (int64_t kk = static_cast<int64_t>(wave) * 2048 + lane * 32; kk < k; kk += step) {
        uint4 q[R];
        float s[R];
        const int64_t g = kk >> 6;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            q[r] = load_stream16(packed + rows[r] * rowbytes + (kk >> 1));
            s[r] = f16_to_f32(scales[scale_index(rows[r], g, groups, n_out)]);
        }
        float xf[32];
        const uint4 *xp = reinterpret_cast<const uint4 *>(x + kk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = xp[i];
            xf[8 * i + 0] = bf16_lo(v.x);
            xf[8 * i + 1] = bf16_hi(v.x);
            xf[8 * i + 2] = bf16_lo(v.y);
            xf[8 * i + 3] = bf16_hi(v.y);
            xf[8 * i + 4] = bf16_lo(v.z);
            xf[8 * i + 5] = bf16_hi(v.z);
            xf[8 * i + 6] = bf16_lo(v.w);
            xf[8 * i + 7] = bf16_hi(v.w);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(s[r], nf4_dot32(q[r], xf, lutp), acc[r]);
    }
    block_reduce_store<R>(acc, red, lane, wave, waves, row0, n_out, y);
}

// ---------------------------------------------------------------- launch
// Waves per workgroup: up to 4, splitting the k steps of the workgroup's rows,
// as long as every wave gets at least two steps.
static int gemv_waves(int64_t steps) {
    int waves = 1;
    while (waves < 4 && waves * 2 <= steps) waves *= 2;
    return waves;
}

constexpr int kRowsBf16 = 4;
constexpr int kRowsNf4 = 4;

int launch_gemv_bf16(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s) {
    const int waves = gemv_waves((k + 511) / 512);
    const int64_t grid = (n_out + kRowsBf16 - 1) / kRowsBf16;
    if (grid > 0x7fffffff) return WSL_E_SHAPE;
    hipLaunchKernelGGL((gemv_bf16_kernel<kRowsBf16, 2>), dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0, s,
                       static_cast<const uint16_t *>(w), n_out, k, static_cast<const uint16_t *>(x), y);
    return WSL_OK;
}

int launch_gemv_nf4(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s) {
    const int waves = gemv_waves((k + 2047) / 2048);
    const int64_t grid = (n_out + kRowsNf4 - 1) / kRowsNf4;
    if (grid > 0x7fffffff) return WSL_E_SHAPE;
    hipLaunchKernelGGL((gemv_nf4_kernel<kRowsNf4>), dim3(static_cast<unsigned>(grid)), dim3(64 * waves), 0, s,
                       static_cast<const uint8_t *>(w), n_out, k, static_cast<const uint16_t *>(x), y);
    return WSL_OK;
}

}  // namespace wsl
