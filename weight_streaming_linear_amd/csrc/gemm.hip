// Prefill / batch-verification GEMM Y = X T^T for gfx950 on the matrix cores.
//
// deep-fold README, "Метод" table: prefill is an NF4 GEMM that restores
// weights into BF16 register fragments (batches of up to 32 positions).  TCPP
// README, "Quickstart"/"Performance": batch verification runs the bf16
// weights, as stored, over every position of a long context (here M = 8192).
//
// Both operands are k-contiguous (X is [m][k], W is [n][k]), which is exactly
// what v_mfma_f32_32x32x16_bf16 wants: each lane supplies 8 consecutive k of
// one row of A (= X) and 8 consecutive k of one column of B (= W^T).  Because
// the product sums over k, any fixed assignment of k values to (lane half,
// element) works as long as A and B use the same one; the NF4 kernel uses
// that freedom so a lane's four MFMA k-steps read one contiguous 16-byte run
// of codes.
#include "device_common.h"

namespace wsl {

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- bf16, LDS-tiled
// Workgroup tile 128 (m) x 128 (n) x 64 (k); 4 waves in 2 x 2, each 64 x 64 as
// 2 x 2 blocks of 32 x 32.  LDS rows of 64 bf16 (128 B) hold 8 chunks of 16 B;
// chunk c of row r is stored at c ^ (r & 7) so that the 32 lanes reading one
// chunk column from 32 consecutive rows hit distinct banks.
constexpr int kBM = 128, kBN = 128, kBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                        int64_t m, int64_t n_out, int64_t k, int64_t ldx,
                                                        void *__restrict__ y, int ofmt, int64_t ldy) {
    __shared__ __attribute__((aligned(16))) char sa[kBM * 128];
    __shared__ __attribute__((aligned(16))) char sb[kBN * 128];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;

    // global -> register staging: 4 chunks of A and 4 of B per thread
    uint4 ra[4], rb[4];
    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i;
            const int row = id >> 3, c = id & 7;
            const int64_t gm = m0 + row, gn = n0 + row;
            ra[i] = (gm < m) ? *reinterpret_cast<const uint4 *>(x + gm * ldx + k0 + c * 8) : make_uint4(0, 0, 0, 0);
            rb[i] = (gn < n_out) ? *reinterpret_cast<const uint4 *>(w + gn * k + k0 + c * 8) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = tid + 256 * i;
            const int row = id >> 3, c = id & 7;
            *reinterpret_cast<uint4 *>(sa + swz(row, c)) = ra[i];
            *reinterpret_cast<uint4 *>(sb + swz(row, c)) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int half = lane >> 5, l32 = lane & 31;
    const int64_t ktiles = k / kBK;
    load_tile(0);
    store_tile();
    __syncthreads();
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        if (kt + 1 < ktiles) load_tile((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int chunk = ks * 2 + half;
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra_row = wm * 64 + i * 32 + l32;
                a[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(sa + swz(ra_row, chunk)));
                const int rb_row = wn * 64 + i * 32 + l32;
                b[i] = as_bf16x8(*reinterpret_cast<const uint4 *>(sb + swz(rb_row, chunk)));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
        if (kt + 1 < ktiles) {
            store_tile();
            __syncthreads();
        }
    }

    // 32x32 accumulator layout: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + l32;
            if (col >= n_out) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                if (row >= m) continue;
                if (ofmt == WSL_OUT_F32) {
                    static_cast<float *>(y)[row * ldy + col] = acc[i][j][e];
                } else {
                    static_cast<uint16_t *>(y)[row * ldy + col] =
                        static_cast<uint16_t>(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
                }
            }
        }
}

// ---------------------------------------------------------------- NF4, weight-stationary
// Each wave owns 32 weight rows (n) and a k range; it restores 8 codes at a
// time into one bf16 B fragment (t = bf16(fp32(level * s))) and multiplies it
// against MB blocks of 32 positions.  Lane l serves row n0 + l%32 and k half
// h = l/32: per 64-k step it loads the 16-byte run of codes for k in
// [kc + 32h, kc + 32h + 32) -- four MFMA k-steps of 8 -- all inside group kc/64.
// The matching A fragments are X[row][kc + 32h + 8t .. +8].
template <int MB>
__global__ __launch_bounds__(256) void gemm_nf4_kernel(const uint8_t *__restrict__ packed, int64_t n_out,
                                                       int64_t k, const uint16_t *__restrict__ x, int64_t m,
                                                       int64_t ldx, void *__restrict__ y, int ofmt, int64_t ldy,
                                                       float *__restrict__ ws, int64_t k_per_split) {
    __shared__ float lut[16];
    if (threadIdx.x < 16) lut[threadIdx.x] = level(threadIdx.x);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 32;
    const int64_t n = (n0 + l32 < n_out) ? n0 + l32 : n_out - 1;
    const int64_t mbase = static_cast<int64_t>(blockIdx.z) * 32 * MB;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * k_per_split;
    const int64_t kend = (kbeg + k_per_split < k) ? kbeg + k_per_split : k;
    const int64_t groups = k >> 6;
    const int64_t rowbytes = k >> 1;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
    const char *lutp = reinterpret_cast<const char *>(lut);

    const uint16_t *xrow[MB];
    bool xok[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t r = mbase + mb * 32 + l32;
        xok[mb] = r < m;
        xrow[mb] = x + (xok[mb] ? r : 0) * ldx;
    }
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;

    if (n0 < n_out) {
        for (int64_t kc = kbeg; kc < kend; kc += 64) {
            const uint4 q = load_stream16(packed + n * rowbytes + ((kc + 32 * half) >> 1));
            const float s = f16_to_f32(scales[scale_index(n, kc >> 6, groups, n_out)]);
            const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t we = wd[t], wo = rotr32(wd[t], 4);
                uint4 bv;
                uint32_t *bp = reinterpret_cast<uint32_t *>(&bv);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float le = *reinterpret_cast<const float *>(lutp + ((we >> (8 * b)) & 0x3cu));
                    const float lo = *reinterpret_cast<const float *>(lutp + ((wo >> (8 * b)) & 0x3cu));
                    bp[b] = pack_bf16x2(le * s, lo * s);
                }
                const bf16x8 bf = as_bf16x8(bv);
                const int64_t kk = kc + 32 * half + 8 * t;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint4 av = xok[mb] ? *reinterpret_cast<const uint4 *>(xrow[mb] + kk) : make_uint4(0, 0, 0, 0);
                    acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), bf, acc[mb], 0, 0, 0);
                }
            }
        }
    }

    // Output element e of lane l: position row mbase + mb*32 + 8*(e/4) + 4*h + e%4, column n0 + l%32.
    const int64_t col = n0 + l32;
    if (col >= n_out) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = mbase + mb * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
            if (row >= m) continue;
            const float v = acc[mb][e];
            if (ws != nullptr) {
                ws[(static_cast<int64_t>(blockIdx.y) * m + row) * n_out + col] = v;
            } else if (ofmt == WSL_OUT_F32) {
                static_cast<float *>(y)[row * ldy + col] = v;
            } else {
                static_cast<uint16_t *>(y)[row * ldy + col] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
            }
        }
}

// Sum split partials in split order (fixed, so the result is deterministic).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ ws, int splits, int64_t m,
                                                           int64_t n_out, void *__restrict__ y, int ofmt, int64_t ldy) {
    const int64_t total = m * n_out;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float v = ws[i];
        for (int sidx = 1; sidx < splits; ++sidx) v += ws[static_cast<int64_t>(sidx) * total + i];
        const int64_t row = i / n_out, col = i - row * n_out;
        if (ofmt == WSL_OUT_F32) static_cast<float *>(y)[row * ldy + col] = v;
        else static_cast<uint16_t *>(y)[row * ldy + col] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
    }
}

// ---------------------------------------------------------------- planning / launch
static int nf4_splits(int64_t n_out, int64_t k, int64_t m) {
    const int64_t wgs = (n_out + 127) / 128;
    const int64_t mchunks = (m + 127) / 128;
    int64_t splits = 1;
    const int64_t kgroups = k / 64;
    while (wgs * mchunks * splits < 512 && splits * 2 <= kgroups && splits < 16) splits *= 2;
    return static_cast<int>(splits);
}

size_t gemm_ws_bytes(int wfmt, int64_t n_out, int64_t k, int64_t m) {
    if (wfmt != WSL_W_NF4) return 0;
    const int splits = nf4_splits(n_out, k, m);
    if (splits <= 1) return 0;
    return static_cast<size_t>(splits) * static_cast<size_t>(m) * static_cast<size_t>(n_out) * sizeof(float);
}

int launch_gemm_bf16(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                     int ofmt, int64_t ldy, hipStream_t s) {
    const int64_t gx = (n_out + kBN - 1) / kBN, gy = (m + kBM - 1) / kBM;
    if (gx > 0x7fffffff || gy > 65535) return WSL_E_SHAPE;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w), m, n_out, k, ldx, y, ofmt,
                       ldy);
    return WSL_OK;
}

int launch_gemm_nf4(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                    int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s) {
    int splits = nf4_splits(n_out, k, m);
    if (splits > 1 && (ws == nullptr || ws_bytes < gemm_ws_bytes(WSL_W_NF4, n_out, k, m))) splits = 1;
    const int64_t kgroups = k / 64;
    const int64_t kps = ((kgroups + splits - 1) / splits) * 64;
    const int64_t gx = (n_out + 127) / 128;
    const int mb = (m >= 128) ? 4 : static_cast<int>((m + 31) / 32);
    const int64_t gz = (m + 32 * mb - 1) / (32 * mb);
    if (gx > 0x7fffffff || gz > 65535) return WSL_E_SHAPE;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(splits), static_cast<unsigned>(gz));
    float *wsp = splits > 1 ? static_cast<float *>(ws) : nullptr;
    const auto *wp = static_cast<const uint8_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    switch (mb) {
        case 1: hipLaunchKernelGGL((gemm_nf4_kernel<1>), grid, dim3(256), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy, wsp, kps); break;
        case 2: hipLaunchKernelGGL((gemm_nf4_kernel<2>), grid, dim3(256), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy, wsp, kps); break;
        case 3: hipLaunchKernelGGL((gemm_nf4_kernel<3>), grid, dim3(256), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy, wsp, kps); break;
        default: hipLaunchKernelGGL((gemm_nf4_kernel<4>), grid, dim3(256), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy, wsp, kps); break;
    }
    if (splits > 1) {
        const int64_t total = m * n_out;
        int64_t blocks = (total + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, wsp, splits, m,
                           n_out, y, ofmt, ldy);
    }
    return WSL_OK;
}

}  // namespace wsl
