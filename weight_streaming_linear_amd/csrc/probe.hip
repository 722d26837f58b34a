// Streaming-read probe: a read-only kernel whose rate is the streaming-read ceiling
// the GEMV figures are compared with.  Not part of the linear path.
#include "device_common.h"

namespace wsl {

constexpr uint32_t kStreamReadMagic = 0x9e3779b9u;

// Each wave reads 4 KB of consecutive bytes per iteration (four 1 KB wave
// instructions of 16-byte loads that bypass the caches, as the GEMV's weight loads
// do), waves striding over the buffer by the number of waves; a tail shorter than
// 4 KB is read word by word.  The words a lane reads are XOR-combined; the lane
// writes the result to sink[0] only if it equals kStreamReadMagic, so the kernel's
// traffic is the read.  (Measured on MI355X against lane-strided forms and 8 or
// 16 KB per wave: this form reached 6.9-7.0 TB/s at every launch shape tried.)
__global__ __launch_bounds__(512) void stream_read_kernel(const uint8_t *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    constexpr int D = 4;   // 1 KB wave loads per iteration
    const int lane = threadIdx.x & 63;
    const int64_t wv = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nw = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    const int64_t blocks = n16 / (64 * D);
    uint32_t acc = 0;
    for (int64_t bk = wv; bk < blocks; bk += nw) {
        const uint8_t *q = p + (bk * 64 * D + lane) * 16;
        uint4 v[D];
#pragma unroll
        for (int j = 0; j < D; ++j) v[j] = load_stream16(q + j * 1024);
#pragma unroll
        for (int j = 0; j < D; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (int64_t i = blocks * 64 * D + wv * 64 + lane; i < n16; i += nw * 64) {
        const uint4 v = load_stream16(p + i * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kStreamReadMagic) sink[0] = acc;
}

int launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    if (n16 == 0) return WSL_OK;
    // 4 workgroups of 8 waves per CU, fewer for small buffers
    int64_t blocks = (n16 + 2047) / 2048;
    if (blocks > 256 * 4) blocks = 256 * 4;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s,
                       static_cast<const uint8_t *>(buf), n16, sink);
    return WSL_OK;
}

}  // namespace wsl
