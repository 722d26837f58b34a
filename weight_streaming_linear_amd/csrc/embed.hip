// Packed embedding rows (nf4_embed_rows) for gfx950.
//
// deep-fold README, introduction and Figure 1: the embedding matrix stays
// packed, and only the rows a step asks for are restored, by a path of their
// own next to the linear kernels.  The row indices are read on the device, so a
// decode step never copies token ids to the host.
#include "device_common.h"

namespace wsl {

// One thread per 8 codes (one device word) of one requested row: a uint4 of
// bf16 or two float4 of fp32 per thread; consecutive threads cover consecutive
// words of a row, so loads and stores are contiguous.
__global__ __launch_bounds__(256) void nf4_embed_rows_kernel(const uint8_t *__restrict__ packed, int64_t n_rows,
                                                             int64_t k, const int64_t *__restrict__ ids,
                                                             int64_t count, void *__restrict__ out, int ofmt,
                                                             int64_t ld_out, uint32_t *__restrict__ status) {
    __shared__ float lut[16];
    write_levels(lut);
    __syncthreads();
    const int64_t wpr = k >> 3;                    // device words per row
    const int64_t groups = k >> 6;
    const uint32_t *words = reinterpret_cast<const uint32_t *>(packed);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_rows * (k >> 1));
    const int64_t total = count * wpr;
    for (int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; item < total;
         item += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t i = item / wpr, j = item - i * wpr;
        const int64_t id = ids[i];
        float v[8];
        if (id < 0 || id >= n_rows) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
            if (status != nullptr && j == 0) atomicOr(status, WSL_STATUS_INDEX);
        } else {
            const uint32_t w = rotr32(words[id * wpr + j], 2);   // canonical: code of k = 8j + e at bits 4e
            const float s = f16_to_f32(scales[scale_index(id, j >> 3, groups, n_rows)]);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = lut[(w >> (4 * e)) & 15u] * s;
        }
        if (ofmt == WSL_OUT_BF16) {
            uint16_t *o = static_cast<uint16_t *>(out) + i * ld_out + 8 * j;
            *reinterpret_cast<uint4 *>(o) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        } else {
            float *o = static_cast<float *>(out) + i * ld_out + 8 * j;
            *reinterpret_cast<float4 *>(o) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4 *>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

int launch_embed_rows(const void *packed, int64_t n_rows, int64_t k, const int64_t *ids, int64_t count, void *out,
                      int ofmt, int64_t ld_out, uint32_t *status, hipStream_t s) {
    if (count == 0) return WSL_OK;
    const int64_t total = count * (k >> 3);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(nf4_embed_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint8_t *>(packed), n_rows, k, ids, count, out, ofmt, ld_out, status);
    return WSL_OK;
}

}  // namespace wsl
