// C ABI entry points (include/wsl.h): validate on the host, check the device,
// enqueue on the caller's stream, report launch errors without synchronizing.
#include <atomic>
#include <cstring>

#include "device_common.h"
#include "validate.h"

namespace wsl {
int launch_pack(const void *w, int64_t n_out, int64_t k, void *packed, uint32_t *status, hipStream_t s);
int launch_dequant_tile(const void *packed, int64_t n_out, int64_t k, int64_t row0, int64_t k0, int64_t rows,
                        int64_t cols, void *tile, int64_t ld, hipStream_t s);
int launch_gemv_bf16(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s);
int launch_gemv_bf16_multi(const wsl_gemv_stage *st, int64_t count, hipStream_t s);
int launch_gemv_nf4(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s);
size_t sweep_ws_bytes();
int launch_gemv_nf4_sweep(const wsl_gemv_stage *d_stages, int64_t count, int64_t max_k, void *ws, hipStream_t s);
int launch_gemm_bf16(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                     int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s);
int launch_gemm_nf4(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                    int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s);
size_t gemm_ws_bytes(int wfmt, int64_t n_out, int64_t k, int64_t m);
int launch_gemm_noalloc(int wfmt, const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx,
                        void *y, int ofmt, int64_t ldy, hipStream_t s);
int check_pinned(int64_t count, const void *const *h_w);
int ring_gemv(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
              const void *const *x, float *const *y, void *const *slot, hipStream_t copy, hipStream_t compute,
              void *const *events, int flags);
int ring_gemm(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
              const void *const *x, int64_t m, int64_t ldx, void *const *y, int ofmt, int64_t ldy, void *ws,
              size_t ws_bytes, void *const *slot, hipStream_t copy, hipStream_t compute, void *const *events,
              int flags);
int launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);
int launch_embed_rows(const void *packed, int64_t n_rows, int64_t k, const int64_t *ids, int64_t count, void *out,
                      int ofmt, int64_t ld_out, uint32_t *status, hipStream_t s);

namespace {

constexpr int kMaxDevices = 64;
// 0 = not yet checked, 1 = gfx950, 2 = something else.
std::atomic<int> g_arch[kMaxDevices];

int device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return WSL_E_DEVICE;
    if (dev >= kMaxDevices) return WSL_E_DEVICE;
    int st = g_arch[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return WSL_E_DEVICE;
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? WSL_OK : WSL_E_DEVICE;
}

int after_launch(int rc) {
    if (rc != WSL_OK) return rc;
    return hipGetLastError() == hipSuccess ? WSL_OK : WSL_E_LAUNCH;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace
}  // namespace wsl

extern "C" {

size_t nf4_packed_bytes(int64_t n_out, int64_t k) { return wsl::nf4_bytes(n_out, k); }

int nf4_codebook(float *out_host) {
    if (!out_host) return WSL_E_NULL;
    for (int i = 0; i < 16; ++i) std::memcpy(&out_host[i], &wsl::kLevelBits[i], sizeof(float));
    return WSL_OK;
}

int nf4_pack(const void *d_w, int64_t n_out, int64_t k, void *d_packed, uint32_t *d_status, void *stream) {
    int rc = wsl::check_pack(d_w, n_out, k, d_packed);
    if (rc != WSL_OK) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    return wsl::after_launch(wsl::launch_pack(d_w, n_out, k, d_packed, d_status, wsl::as_stream(stream)));
}

int nf4_dequant_tile(const void *d_packed, int64_t n_out, int64_t k, int64_t row0, int64_t k0, int64_t rows,
                     int64_t cols, void *d_tile, int64_t ld_tile, void *stream) {
    int rc = wsl::check_dequant_tile(d_packed, n_out, k, row0, k0, rows, cols, d_tile, ld_tile);
    if (rc != WSL_OK) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    return wsl::after_launch(
        wsl::launch_dequant_tile(d_packed, n_out, k, row0, k0, rows, cols, d_tile, ld_tile, wsl::as_stream(stream)));
}

int linear_gemv(int wfmt, const void *d_w, int64_t n_out, int64_t k, const void *d_x, float *d_y, void *stream) {
    int rc = wsl::check_gemv(wfmt, d_w, n_out, k, d_x, d_y);
    if (rc != WSL_OK) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    if (wfmt == WSL_W_NF4) return wsl::after_launch(wsl::launch_gemv_nf4(d_w, n_out, k, d_x, d_y, wsl::as_stream(stream)));
    return wsl::after_launch(wsl::launch_gemv_bf16(d_w, n_out, k, d_x, d_y, wsl::as_stream(stream)));
}

size_t linear_gemv_sweep_workspace_bytes(void) { return wsl::sweep_ws_bytes(); }

int linear_gemv_sweep(int wfmt, int64_t count, const wsl_gemv_stage *h_stages, const wsl_gemv_stage *d_stages,
                      void *d_ws, size_t ws_bytes, void *stream) {
    int rc = wsl::check_sweep(wfmt, count, h_stages, d_stages, d_ws, ws_bytes, wsl::sweep_ws_bytes());
    if (rc != WSL_OK || count == 0) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    int64_t max_k = 0;
    for (int64_t i = 0; i < count; ++i) max_k = h_stages[i].k > max_k ? h_stages[i].k : max_k;
    return wsl::after_launch(wsl::launch_gemv_nf4_sweep(d_stages, count, max_k, d_ws, wsl::as_stream(stream)));
}

int linear_gemv_multi(int wfmt, int64_t count, const wsl_gemv_stage *h_stages, void *stream) {
    int rc = wsl::check_multi(wfmt, count, h_stages);
    if (rc != WSL_OK || count == 0) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    return wsl::after_launch(wsl::launch_gemv_bf16_multi(h_stages, count, wsl::as_stream(stream)));
}

size_t linear_gemm_workspace_bytes(int wfmt, int64_t n_out, int64_t k, int64_t m) {
    if (wfmt != WSL_W_BF16 && wfmt != WSL_W_NF4) return 0;
    if (n_out <= 0 || k <= 0 || m <= 0 || (k % 64) != 0) return 0;
    if (n_out > wsl::kMaxDim || k > wsl::kMaxDim || m > wsl::kMaxDim) return 0;
    return wsl::gemm_ws_bytes(wfmt, n_out, k, m);
}

int linear_gemm(int wfmt, const void *d_w, int64_t n_out, int64_t k, const void *d_x, int64_t m, int64_t ldx,
                void *d_y, int ofmt, int64_t ldy, void *d_ws, size_t ws_bytes, void *stream) {
    int rc = wsl::check_gemm(wfmt, d_w, n_out, k, d_x, m, ldx, d_y, ofmt, ldy, d_ws, ws_bytes);
    if (rc != WSL_OK) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    if (wfmt == WSL_W_NF4)
        return wsl::after_launch(
            wsl::launch_gemm_nf4(d_w, n_out, k, d_x, m, ldx, d_y, ofmt, ldy, d_ws, ws_bytes, wsl::as_stream(stream)));
    return wsl::after_launch(
        wsl::launch_gemm_bf16(d_w, n_out, k, d_x, m, ldx, d_y, ofmt, ldy, d_ws, ws_bytes, wsl::as_stream(stream)));
}

int linear_gemm_noalloc(int wfmt, const void *d_w, int64_t n_out, int64_t k, const void *d_x, int64_t m,
                        int64_t ldx, void *d_y, int ofmt, int64_t ldy, void *stream) {
    int rc = wsl::check_gemm(wfmt, d_w, n_out, k, d_x, m, ldx, d_y, ofmt, ldy, nullptr, 0);
    if (rc != WSL_OK) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    return wsl::after_launch(
        wsl::launch_gemm_noalloc(wfmt, d_w, n_out, k, d_x, m, ldx, d_y, ofmt, ldy, wsl::as_stream(stream)));
}

int nf4_embed_rows(const void *d_packed, int64_t n_rows, int64_t k, const int64_t *d_ids, int64_t count,
                   void *d_out, int ofmt, int64_t ld_out, uint32_t *d_status, void *stream) {
    int rc = wsl::check_embed(d_packed, n_rows, k, d_ids, count, d_out, ofmt, ld_out);
    if (rc != WSL_OK) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    return wsl::after_launch(wsl::launch_embed_rows(d_packed, n_rows, k, d_ids, count, d_out, ofmt, ld_out, d_status,
                                                    wsl::as_stream(stream)));
}

int linear_gemv_streamed(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
                         const void *const *d_x, float *const *d_y, void *const *d_slot, size_t slot_bytes,
                         void *copy_stream, void *compute_stream, void *const *events, int flags) {
    int rc = wsl::check_ring(wfmt, count, h_w, n_out, k, d_x, -1, 0, reinterpret_cast<const void *const *>(d_y), 0,
                             0, nullptr, 0, d_slot, slot_bytes, events, flags);
    if (rc != WSL_OK || count == 0) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    if ((rc = wsl::check_pinned(count, h_w)) != WSL_OK) return rc;
    return wsl::ring_gemv(wfmt, count, h_w, n_out, k, d_x, d_y, d_slot, wsl::as_stream(copy_stream),
                          wsl::as_stream(compute_stream), events, flags);
}

int linear_gemm_streamed(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
                         const void *const *d_x, int64_t m, int64_t ldx, void *const *d_y, int ofmt, int64_t ldy,
                         void *d_ws, size_t ws_bytes, void *const *d_slot, size_t slot_bytes,
                         void *copy_stream, void *compute_stream, void *const *events, int flags) {
    int rc = wsl::check_ring(wfmt, count, h_w, n_out, k, d_x, m < 0 ? 0 : m, ldx,
                             reinterpret_cast<const void *const *>(d_y), ofmt, ldy, d_ws, ws_bytes, d_slot,
                             slot_bytes, events, flags);
    if (rc != WSL_OK || count == 0) return rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    if ((rc = wsl::check_pinned(count, h_w)) != WSL_OK) return rc;
    return wsl::ring_gemm(wfmt, count, h_w, n_out, k, d_x, m, ldx, d_y, ofmt, ldy, d_ws, ws_bytes, d_slot,
                          wsl::as_stream(copy_stream), wsl::as_stream(compute_stream), events, flags);
}

int wsl_stream_read(const void *d_buf, size_t bytes, uint32_t *d_sink, void *stream) {
    if (bytes == 0) return WSL_OK;
    if (!d_buf || !d_sink) return WSL_E_NULL;
    if ((bytes % 16) != 0) return WSL_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(d_buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(d_sink) % 4) != 0)
        return WSL_E_ALIGN;
    int rc;
    if ((rc = wsl::device_ok()) != WSL_OK) return rc;
    return wsl::after_launch(wsl::launch_stream_read(d_buf, bytes, d_sink, wsl::as_stream(stream)));
}

const char *wsl_strerror(int code) {
    switch (code) {
        case WSL_OK: return "ok";
        case WSL_E_NULL: return "a required pointer is NULL";
        case WSL_E_SHAPE: return "invalid shape (non-positive size, k not a multiple of 64, or size overflow)";
        case WSL_E_ALIGN: return "misaligned pointer or leading dimension";
        case WSL_E_FORMAT: return "unknown weight or output format";
        case WSL_E_DEVICE: return "current device is not gfx950 (MI355X) or could not be queried";
        case WSL_E_LAUNCH: return "kernel launch failed";
        case WSL_E_RANGE: return "tile or workspace outside its matrix or buffer";
        case WSL_E_MEMORY: return "host buffer is not pinned (page-locked) host memory";
        case WSL_E_SCRATCH:
            return "linear_gemm_noalloc: the shape's split workspace exceeds WSL_NOALLOC_SCRATCH_BYTES "
                   "(use linear_gemm with a caller workspace)";
        case WSL_E_FLAGS: return "a flags argument holds a bit the call does not define";
        default: return "unknown status code";
    }
}

}  // extern "C"
