// Decode GEMV y = W x for gfx950: bf16 weights or packed NF4 weights.
//
// deep-fold README, "Метод" table: decode runs an N=1 NF4 GEMV, with codes and
// scales resident in video memory and restored in registers only for the
// fragment being multiplied.  TCPP README, "What exact means here": bf16 weights
// are used as stored.  The work is a pure weight stream (each weight byte is
// read once and feeds one multiply-add), so both kernels are built around HBM:
//   * a wavefront reads 1 KB of one row per step (64 lanes x 16-byte
//     non-temporal loads) and keeps several rows in flight;
//   * the waves of a workgroup split the k range of the same rows; each wave
//     folds its per-row sums across lanes with a transposed reduction
//     (v_permlane32_swap, v_permlane16_swap, then DPP inside 16 or 8 lanes),
//     and the per-wave partials meet in LDS in a fixed order -- deterministic,
//     no atomics;
//   * x (<= 64 KB) is read through the cache hierarchy;
//   * NF4 codes become levels through a 16-entry fp32 table in LDS (16
//     distinct banks: lanes reading one entry broadcast, lanes reading
//     different entries never conflict).  The device layout rotates each
//     32-bit code word left by 2 bits, so one AND with 0x3C on a byte (and,
//     for the odd codes, on the word rotated right by 4) is already the byte
//     address code*4 of the table entry.
#include "device_common.h"

namespace wsl {

constexpr int kMaxWaves = 8;

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float as_f(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ uint32_t as_u(float v) { return __builtin_bit_cast(uint32_t, v); }

// DPP controls (gfx9): quad_perm(1,0,3,2) = 0xB1, quad_perm(2,3,0,1) = 0x4E,
// row_half_mirror = 0x141, row_ror:8 = 0x128.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f(__builtin_amdgcn_update_dpp(0u, as_u(v), CTRL, 0xF, 0xF, false));
}

// Sum inside groups of 8 consecutive lanes (every lane of the group gets the sum).
__device__ __forceinline__ float sum8(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    return v;
}

// Exchange halves of the wave (lanes 32-63 of a with lanes 0-31 of b) and add:
// lanes 0-31 get a[l] + a[l+32], lanes 32-63 get b[l-32] + b[l].
__device__ __forceinline__ float fold32(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
    return as_f(r[0]) + as_f(r[1]);
}
// The same between 16-lane rows: rows 0/2 keep a (plus a's rows 1/3), rows 1/3 keep b
// (plus b's rows 0/2).
__device__ __forceinline__ float fold16(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(as_u(a), as_u(b), false, false);
    return as_f(r[0]) + as_f(r[1]);
}

// Transposed reduction of R per-lane partial sums over the 64 lanes.  Afterwards
// every lane holds the total of row (lane / (64 / R)).
template <int R>
__device__ __forceinline__ float reduce_rows(const float (&a)[R], int lane) {
    if constexpr (R == 1) {
        float v = fold32(a[0], a[0]);
        v = fold16(v, v);
        v = sum8(v);
        return v + dpp<0x128>(v);
    } else if constexpr (R == 2) {
        float v = fold32(a[0], a[1]);          // lanes 0-31: row 0, 32-63: row 1
        v = fold16(v, v);
        v = sum8(v);
        return v + dpp<0x128>(v);
    } else if constexpr (R == 4) {
        const float b0 = fold32(a[0], a[2]);   // lanes 0-31: row 0, 32-63: row 2
        const float b1 = fold32(a[1], a[3]);   // lanes 0-31: row 1, 32-63: row 3
        float v = fold16(b0, b1);              // 16-lane rows: rows 0, 1, 2, 3
        v = sum8(v);
        return v + dpp<0x128>(v);
    } else {
        static_assert(R == 8, "R must be 1, 2, 4 or 8");
        const float b0 = fold32(a[0], a[4]), b1 = fold32(a[1], a[5]);
        const float b2 = fold32(a[2], a[6]), b3 = fold32(a[3], a[7]);
        const float c0 = fold16(b0, b2);       // 16-lane rows: rows 0, 2, 4, 6
        const float c1 = fold16(b1, b3);       // 16-lane rows: rows 1, 3, 5, 7
        const bool lo = (lane & 15) < 8;
        const float t = lo ? c1 : c0;
        const float d = (lo ? c0 : c1) + dpp<0x128>(t);   // 8-lane groups: rows 0..7 in order
        return sum8(d);
    }
}

// Fold the waves' row sums (LDS, fixed wave order) and store y.
template <int R>
__device__ __forceinline__ void finish_rows(const float (&acc)[R], float (*red)[R], int lane, int wave, int waves,
                                            int64_t row0, int64_t n_out, float *__restrict__ y) {
    const float v = reduce_rows<R>(acc, lane);
    constexpr int span = 64 / R;
    if ((lane % span) == 0) red[wave][lane / span] = v;
    __syncthreads();
    if (threadIdx.x < R) {
        float s = red[0][threadIdx.x];
        for (int w = 1; w < waves; ++w) s += red[w][threadIdx.x];
        if (row0 + threadIdx.x < n_out) y[row0 + threadIdx.x] = s;
    }
}

// ---------------------------------------------------------------- bf16
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// c + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4 &w, const uint4 &x, float a) {
    a = dot2(w.x, x.x, a);
    a = dot2(w.y, x.y, a);
    a = dot2(w.z, x.z, a);
    return dot2(w.w, x.w, a);
}

// Lane slice: 8 consecutive bf16 (16 B); a wave step covers 512 k.  R rows per
// workgroup; its waves split the k steps.
template <int R>
__global__ __launch_bounds__(512) void gemv_bf16_kernel(const uint16_t *__restrict__ w, int64_t n_out, int64_t k,
                                                        const uint16_t *__restrict__ x, float *__restrict__ y) {
    __shared__ float red[kMaxWaves][R];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;

    const uint16_t *rowp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rowp[r] = w + ((row0 + r < n_out) ? row0 + r : n_out - 1) * k;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    const int64_t step = static_cast<int64_t>(512) * waves;
    int64_t kk = static_cast<int64_t>(wave) * 512 + lane * 8;
    for (; kk + step < k; kk += 2 * step) {          // two steps in flight
        uint4 q0[R], q1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) q0[r] = load_stream16(rowp[r] + kk);
#pragma unroll
        for (int r = 0; r < R; ++r) q1[r] = load_stream16(rowp[r] + kk + step);
        const uint4 x0 = *reinterpret_cast<const uint4 *>(x + kk);
        const uint4 x1 = *reinterpret_cast<const uint4 *>(x + kk + step);
        __builtin_amdgcn_sched_barrier(0);           // keep every load of the step ahead of the math
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = dot8(q1[r], x1, dot8(q0[r], x0, acc[r]));
    }
    if (kk < k) {
        uint4 q0[R];
#pragma unroll
        for (int r = 0; r < R; ++r) q0[r] = load_stream16(rowp[r] + kk);
        const uint4 x0 = *reinterpret_cast<const uint4 *>(x + kk);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = dot8(q0[r], x0, acc[r]);
    }
    finish_rows<R>(acc, red, lane, wave, waves, row0, n_out, y);
}

// ---------------------------------------------------------------- NF4
// Scales of R consecutive rows (row0 .. row0+R-1, inside one 16-row block) for group g.
template <int R>
__device__ __forceinline__ void load_scales(const uint16_t *__restrict__ scales, bool vec, const int64_t (&rows)[R],
                                            int64_t row0, int64_t g, int64_t groups, int64_t n_out, float (&s)[R]) {
    if (vec) {
        const uint16_t *p = scales + scale_index(row0, g, groups, n_out);
        if constexpr (R == 8) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s[2 * i] = f16_to_f32(u[i] & 0xffffu);
                s[2 * i + 1] = f16_to_f32(u[i] >> 16);
            }
        } else if constexpr (R == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            s[0] = f16_to_f32(v.x & 0xffffu);
            s[1] = f16_to_f32(v.x >> 16);
            s[2] = f16_to_f32(v.y & 0xffffu);
            s[3] = f16_to_f32(v.y >> 16);
        } else if constexpr (R == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
            s[0] = f16_to_f32(v & 0xffffu);
            s[1] = f16_to_f32(v >> 16);
        } else {
            s[0] = f16_to_f32(*p);
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = f16_to_f32(scales[scale_index(rows[r], g, groups, n_out)]);
    }
}

// Byte B of a device-layout word, ANDed with 0x3C: the byte address code*4 of the
// table entry of the code sitting at bits 2..5 of that byte (one SDWA AND).
template <int B>
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, uint32_t m60) {
    uint32_t r;
    if constexpr (B == 0)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    else if constexpr (B == 1)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    else if constexpr (B == 2)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    else
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    return r;
}

template <int B>
__device__ __forceinline__ void nf4_byte(uint32_t we, uint32_t wo, uint32_t m60, const char *lut, const float *xf,
                                         float &p0, float &p1) {
    const float le = *reinterpret_cast<const float *>(lut + lut_addr<B>(we, m60));
    const float lo = *reinterpret_cast<const float *>(lut + lut_addr<B>(wo, m60));
    p0 = __builtin_fmaf(le, xf[2 * B], p0);
    p1 = __builtin_fmaf(lo, xf[2 * B + 1], p1);
}

// Dot product of 32 codes (one 16-byte device-layout load) with 32 fp32 x: per 8
// codes one rotate and eight SDWA ANDs give the table addresses.
__device__ __forceinline__ float nf4_dot32(const uint4 q, const float (&xf)[32], const char *lut, uint32_t m60) {
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t we = wd[i];
        const uint32_t wo = rotr32(we, 4);
        nf4_byte<0>(we, wo, m60, lut, &xf[8 * i], p0, p1);
        nf4_byte<1>(we, wo, m60, lut, &xf[8 * i], p0, p1);
        nf4_byte<2>(we, wo, m60, lut, &xf[8 * i], p0, p1);
        nf4_byte<3>(we, wo, m60, lut, &xf[8 * i], p0, p1);
    }
    return p0 + p1;
}

__device__ __forceinline__ void load_x32(const uint16_t *__restrict__ x, int64_t kk, bool active, float (&xf)[32]) {
    uint4 xv[4];
    const uint4 *xp = reinterpret_cast<const uint4 *>(x + kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = active ? xp[i] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xf[8 * i + 0] = bf16_lo(xv[i].x);
        xf[8 * i + 1] = bf16_hi(xv[i].x);
        xf[8 * i + 2] = bf16_lo(xv[i].y);
        xf[8 * i + 3] = bf16_hi(xv[i].y);
        xf[8 * i + 4] = bf16_lo(xv[i].z);
        xf[8 * i + 5] = bf16_hi(xv[i].z);
        xf[8 * i + 6] = bf16_lo(xv[i].w);
        xf[8 * i + 7] = bf16_hi(xv[i].w);
    }
}

// NF4 GEMV.  Lane slice: 32 consecutive codes (16 B, half a group); a k-slice of
// a row is 2048 codes (1 KB, one wave-wide load).  The workgroup has W waves and
// wave w owns k-slices w, w+W, ...; when there are at most W slices (ONE = true)
// each wave keeps its 32 x values in registers for the whole kernel.
// Workgroups are persistent over row groups of R rows (row group rg = blockIdx.x,
// blockIdx.x + gridDim.x, ...), and the next row group's codes and scales are
// loaded before the current one is multiplied, so every wave keeps two groups
// of loads in flight.  Per row group the W per-wave row sums meet in LDS
// (double-buffered by iteration parity, one barrier per row group).
template <int R, bool ONE>
__global__ __launch_bounds__(1024) void gemv_nf4_kernel(const uint8_t *__restrict__ packed, int64_t n_out, int64_t k,
                                                        const uint16_t *__restrict__ x, float *__restrict__ y) {
    __shared__ float lut[16];
    __shared__ float red[2][16][R];
    if (threadIdx.x < 16) lut[threadIdx.x] = level(threadIdx.x);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int64_t groups = k >> 6;
    const int64_t rowbytes = k >> 1;
    const int64_t row_groups = (n_out + R - 1) / R;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
    const char *lutp = reinterpret_cast<const char *>(lut);
    const uint32_t m60 = 0x3c;
    constexpr int span = 64 / R;

    const int64_t kk0 = static_cast<int64_t>(wave) * 2048 + lane * 32;   // this lane's codes in slice `wave`
    const int64_t kstep = static_cast<int64_t>(2048) * waves;
    float xf[32];
    if constexpr (ONE) load_x32(x, kk0, kk0 < k, xf);

    auto fetch = [&](int64_t rg, int64_t kk, uint4 (&q)[R], float (&s)[R]) {
        const int64_t row0 = rg * R;
        const int64_t rem = n_out - ((row0 >> 4) << 4);
        const int64_t rb = rem < 16 ? rem : 16;
        const bool vec = (row0 + R <= n_out) && (rb % R == 0);
        int64_t rows[R];
#pragma unroll
        for (int r = 0; r < R; ++r) rows[r] = (row0 + r < n_out) ? row0 + r : n_out - 1;
        if (kk < k) {
#pragma unroll
            for (int r = 0; r < R; ++r) q[r] = load_stream16(packed + rows[r] * rowbytes + (kk >> 1));
            load_scales<R>(scales, vec, rows, row0, kk >> 6, groups, n_out, s);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                q[r] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);   // never used
                s[r] = 0.f;
            }
        }
    };

    int64_t rg = blockIdx.x;
    uint4 q[R];
    float s[R];
    if (ONE && rg < row_groups) fetch(rg, kk0, q, s);
    for (int it = 0; rg < row_groups; ++it, rg += gridDim.x) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        if constexpr (ONE) {
            uint4 qn[R];
            float sn[R];
            const int64_t rgn = rg + gridDim.x;
            if (rgn < row_groups) fetch(rgn, kk0, qn, sn);
            if (kk0 < k) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = s[r] * nf4_dot32(q[r], xf, lutp, m60);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                q[r] = qn[r];
                s[r] = sn[r];
            }
        } else {
            for (int64_t kk = kk0; kk < k; kk += kstep) {
                uint4 qc[R];
                float sc[R];
                fetch(rg, kk, qc, sc);
                float xc[32];
                load_x32(x, kk, true, xc);
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(sc[r], nf4_dot32(qc[r], xc, lutp, m60), acc[r]);
            }
        }
        const float v = reduce_rows<R>(acc, lane);
        if ((lane % span) == 0) red[it & 1][wave][lane / span] = v;
        __syncthreads();
        if (threadIdx.x < R) {
            float t = red[it & 1][0][threadIdx.x];
            for (int w = 1; w < waves; ++w) t += red[it & 1][w][threadIdx.x];
            const int64_t row = rg * R + threadIdx.x;
            if (row < n_out) y[row] = t;
        }
    }
}

// ---------------------------------------------------------------- launch plans
// bf16 plan.  Waves per workgroup: the largest divisor of the k-step count that
// is <= 8, so every wave of a workgroup gets the same number of steps.  Rows per
// workgroup: the largest R in {8, 4, 2, 1} that still gives at least `target`
// waves in the grid (about 8 per SIMD on 256 CUs x 4 SIMDs).
static int waves_for(int64_t steps) {
    for (int w = 8; w > 1; --w)
        if (steps % w == 0) return w;
    return steps > 1 ? 2 : 1;
}

static int rows_for(int64_t n_out, int waves, int64_t target) {
    for (int r = 8; r > 1; r >>= 1)
        if (((n_out + r - 1) / r) * waves >= target) return r;
    return 1;
}

#define WSL_GEMV_LAUNCH(KERNEL, R, grid, waves, s, ...) \
    hipLaunchKernelGGL((KERNEL<R>), dim3(static_cast<unsigned>(grid)), dim3(64 * (waves)), 0, s, __VA_ARGS__)

int launch_gemv_bf16(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s) {
    const int waves = waves_for((k + 511) / 512);
    const int r = rows_for(n_out, waves, 8192);
    const int64_t grid = (n_out + r - 1) / r;
    if (grid > 0x7fffffff) return WSL_E_SHAPE;
    const auto *wp = static_cast<const uint16_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    switch (r) {
        case 8: WSL_GEMV_LAUNCH(gemv_bf16_kernel, 8, grid, waves, s, wp, n_out, k, xp, y); break;
        case 4: WSL_GEMV_LAUNCH(gemv_bf16_kernel, 4, grid, waves, s, wp, n_out, k, xp, y); break;
        case 2: WSL_GEMV_LAUNCH(gemv_bf16_kernel, 2, grid, waves, s, wp, n_out, k, xp, y); break;
        default: WSL_GEMV_LAUNCH(gemv_bf16_kernel, 1, grid, waves, s, wp, n_out, k, xp, y); break;
    }
    return WSL_OK;
}

// NF4 plan: W = number of 2048-code k-slices (at most 16), R rows per row group,
// and a persistent grid of about `per_cu` resident waves per CU.
struct Nf4Plan {
    int rows, waves;
    int64_t grid;
    bool one;
};

static Nf4Plan plan_nf4(int64_t n_out, int64_t k) {
    const int64_t slices = (k + 2047) / 2048;
    Nf4Plan p;
    p.waves = static_cast<int>(slices < 16 ? slices : 16);
    p.one = slices <= 16;
    p.rows = (n_out >= 16384) ? 4 : 2;
    const int64_t row_groups = (n_out + p.rows - 1) / p.rows;
    const int64_t per_cu = 24;
    int64_t wgs = 256 * ((per_cu + p.waves - 1) / p.waves);
    if (wgs > row_groups) wgs = row_groups;
    p.grid = wgs;
    return p;
}

int launch_gemv_nf4(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s) {
    const Nf4Plan p = plan_nf4(n_out, k);
    if (p.grid > 0x7fffffff) return WSL_E_SHAPE;
    const auto *wp = static_cast<const uint8_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    const dim3 g(static_cast<unsigned>(p.grid)), b(64 * p.waves);
    if (p.one) {
        if (p.rows == 4) hipLaunchKernelGGL((gemv_nf4_kernel<4, true>), g, b, 0, s, wp, n_out, k, xp, y);
        else hipLaunchKernelGGL((gemv_nf4_kernel<2, true>), g, b, 0, s, wp, n_out, k, xp, y);
    } else {
        if (p.rows == 4) hipLaunchKernelGGL((gemv_nf4_kernel<4, false>), g, b, 0, s, wp, n_out, k, xp, y);
        else hipLaunchKernelGGL((gemv_nf4_kernel<2, false>), g, b, 0, s, wp, n_out, k, xp, y);
    }
    return WSL_OK;
}

}  // namespace wsl
