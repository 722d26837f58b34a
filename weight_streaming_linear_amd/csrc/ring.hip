// Copy ring: linear kernels over matrices kept in pinned host memory.
//
// deep-fold README, "Метод" table and Figure 1: a model that exceeds the GPU
// budget keeps selected packed matrices in pinned host memory; they pass
// through two reusable device slots to the same kernels that serve resident
// matrices.  Host code only: asynchronous copies on one stream, the kernels on
// another, and four caller-owned events that hand each slot back and forth.
// Nothing is allocated; the host waits only when the caller asks for pacing.
#include "device_common.h"

namespace wsl {

int launch_gemv_bf16(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s);
int launch_gemv_nf4(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s);
int launch_gemm_bf16(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                     int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s);
int launch_gemm_nf4(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                    int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s);

// Every host buffer must be page-locked, or the copies would not overlap the
// kernels (and could stage through pageable memory synchronously).
int check_pinned(int64_t count, const void *const *h_w) {
    for (int64_t i = 0; i < count; ++i) {
        hipPointerAttribute_t attr;
        const hipError_t e = hipPointerGetAttributes(&attr, h_w[i]);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // an unknown pointer is an answer here, not a pending error
            return WSL_E_MEMORY;
        }
        if (attr.type != hipMemoryTypeHost) return WSL_E_MEMORY;
    }
    return WSL_OK;
}

// Enqueue the ring for count matrices; launch(i, slot, stream) enqueues the kernel of matrix i.
// pace: before enqueueing the copy of matrix i >= 2, wait on the host for the kernel of
// matrix i - 2 (the event that copy waits for on the device anyway).  Enqueued far ahead,
// copies that wait on another stream's kernels can be held up inside the runtime for
// milliseconds at a time, while the copy engine runs out of queued work.
template <typename Launch>
int run_ring(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
             void *const *slot, hipStream_t copy, hipStream_t compute, void *const *events, bool pace,
             Launch launch) {
    hipEvent_t filled[2] = {static_cast<hipEvent_t>(events[0]), static_cast<hipEvent_t>(events[1])};
    hipEvent_t freed[2] = {static_cast<hipEvent_t>(events[2]), static_cast<hipEvent_t>(events[3])};
    for (int64_t i = 0; i < count; ++i) {
        const int s = static_cast<int>(i & 1);
        const size_t bytes = wfmt == WSL_W_NF4 ? nf4_packed_bytes(n_out[i], k[i])
                                               : static_cast<size_t>(n_out[i]) * static_cast<size_t>(k[i]) * 2;
        if (pace && i >= 2 && hipEventSynchronize(freed[s]) != hipSuccess) return WSL_E_LAUNCH;
        if (hipStreamWaitEvent(copy, freed[s], 0) != hipSuccess) return WSL_E_LAUNCH;
        if (hipMemcpyAsync(slot[s], h_w[i], bytes, hipMemcpyHostToDevice, copy) != hipSuccess) return WSL_E_LAUNCH;
        if (hipEventRecord(filled[s], copy) != hipSuccess) return WSL_E_LAUNCH;
        if (hipStreamWaitEvent(compute, filled[s], 0) != hipSuccess) return WSL_E_LAUNCH;
        const int rc = launch(i, slot[s], compute);
        if (rc != WSL_OK) return rc;
        if (hipGetLastError() != hipSuccess) return WSL_E_LAUNCH;
        if (hipEventRecord(freed[s], compute) != hipSuccess) return WSL_E_LAUNCH;
    }
    return WSL_OK;
}

int ring_gemv(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
              const void *const *x, float *const *y, void *const *slot, hipStream_t copy, hipStream_t compute,
              void *const *events, int flags) {
    return run_ring(wfmt, count, h_w, n_out, k, slot, copy, compute, events, (flags & WSL_RING_PACE) != 0,
                    [&](int64_t i, void *w, hipStream_t s) {
                        return wfmt == WSL_W_NF4 ? launch_gemv_nf4(w, n_out[i], k[i], x[i], y[i], s)
                                                 : launch_gemv_bf16(w, n_out[i], k[i], x[i], y[i], s);
                    });
}

int ring_gemm(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
              const void *const *x, int64_t m, int64_t ldx, void *const *y, int ofmt, int64_t ldy, void *ws,
              size_t ws_bytes, void *const *slot, hipStream_t copy, hipStream_t compute, void *const *events,
              int flags) {
    return run_ring(wfmt, count, h_w, n_out, k, slot, copy, compute, events, (flags & WSL_RING_PACE) != 0,
                    [&](int64_t i, void *w, hipStream_t s) {
                        return wfmt == WSL_W_NF4
                                   ? launch_gemm_nf4(w, n_out[i], k[i], x[i], m, ldx, y[i], ofmt, ldy, ws, ws_bytes, s)
                                   : launch_gemm_bf16(w, n_out[i], k[i], x[i], m, ldx, y[i], ofmt, ldy, ws, ws_bytes, s);
                    });
}

}  // namespace wsl
