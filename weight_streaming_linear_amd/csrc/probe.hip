// Streaming-read probe: a read-only kernel whose rate is the streaming-read ceiling
// the GEMV figures are compared with.  Not part of the linear path.
#include "device_common.h"

namespace wsl {

constexpr uint32_t kStreamReadMagic = 0x9e3779b9u;

// The buffer is read as 1 KB units (one wave instruction of 16-byte loads that bypass
// the caches, as the GEMV's weight loads do): wave w of the grid's nw waves takes units
// w, w + nw, w + 2 nw, ... for `per` = units / nw rounds, three units in flight (each
// refilled as soon as it has been consumed); the units past per * nw and a tail shorter
// than 1 KB are then read word by word, so every 16-byte word is read exactly once.  The
// words a lane reads are XOR-combined; the lane writes the result to sink[0] only if it
// equals kStreamReadMagic, so the kernel's traffic is the read.  One 8-wave workgroup
// per CU: measured on MI355X over 2 GiB, 8-16 waves per CU with 16-36 KB in flight per CU
// read at 7.0-7.4 TB/s, and 48-128 KB in flight (more waves or deeper) at 6.6-6.9.
__global__ __launch_bounds__(512) void stream_read_kernel(const uint8_t *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    constexpr int D = 3;   // 1 KB wave loads in flight
    const int lane = threadIdx.x & 63;
    const int64_t wv = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nw = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    const int64_t per = (n16 >> 6) / nw;   // unit wv + i * nw < per * nw <= units for i < per
    auto unit = [&](int64_t i) { return p + ((wv + i * nw) * 64 + lane) * 16; };
    uint32_t acc = 0;
    int64_t i = 0;
    if (per >= D) {
        uint4 v[D];
#pragma unroll
        for (int d = 0; d < D; ++d) v[d] = load_stream16(unit(d));
        for (i = D; i + D <= per; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
                v[d] = load_stream16(unit(i + d));
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
    }
    for (; i < per; ++i) {
        const uint4 v = load_stream16(unit(i));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int64_t e = per * nw * 64 + wv * 64 + lane; e < n16; e += nw * 64) {
        const uint4 v = load_stream16(p + e * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kStreamReadMagic) sink[0] = acc;
}

int launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    const int64_t n16 = static_cast<int64_t>(bytes / 16);
    if (n16 == 0) return WSL_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return WSL_E_DEVICE;
    // one 8-wave workgroup per CU, fewer for small buffers (one per 8 KB)
    int64_t blocks = (n16 + 511) / 512;
    if (blocks > cus) blocks = cus;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s,
                       static_cast<const uint8_t *>(buf), n16, sink);
    return WSL_OK;
}

}  // namespace wsl
