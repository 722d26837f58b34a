// Host-side argument validation of the C ABI (no HIP dependency).
//
// Every entry point validates its arguments here before it enqueues anything,
// so a caller error returns a status code and launches nothing.  This unit is
// plain C++ so it can be built with g++ and exercised under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace wsl {

constexpr int64_t kGroup = 64;          // NF4 group size along k
constexpr int64_t kScaleRowBlock = 16;  // rows per scale block in the device layout

// Size of a packed NF4 matrix, or 0 if the shape is invalid or the size overflows.
size_t nf4_bytes(int64_t n_out, int64_t k);

int check_pack(const void *w, int64_t n_out, int64_t k, const void *packed);
int check_dequant_tile(const void *packed, int64_t n_out, int64_t k, int64_t row0, int64_t k0,
                       int64_t rows, int64_t cols, const void *tile, int64_t ld_tile);
int check_gemv(int wfmt, const void *w, int64_t n_out, int64_t k, const void *x, const void *y);
int check_gemm(int wfmt, const void *w, int64_t n_out, int64_t k, const void *x, int64_t m,
               int64_t ldx, const void *y, int ofmt, int64_t ldy, const void *ws, size_t ws_bytes);
// Copy-ring arguments: the flags, the arrays, the slots, the events, and for each matrix
// check_gemv / check_gemm with the slot as the weight pointer plus the slot size.
// m < 0 selects the GEMV checks.
int check_ring(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
               const void *const *x, int64_t m, int64_t ldx, const void *const *y, int ofmt, int64_t ldy,
               const void *ws, size_t ws_bytes, const void *const *slot, size_t slot_bytes, const void *const *events,
               int flags);
// Decode sweep: count in [0, 2^24], the host descriptors (each as check_gemv for NF4,
// plus k <= 32768), the device descriptor array and the workspace.
int check_sweep(int wfmt, int64_t count, const void *h_stages, const void *d_stages, const void *ws,
                size_t ws_bytes, size_t ws_need);
// Several GEMVs in one launch: bf16 only, count in [0, WSL_GEMV_MULTI_MAX], each descriptor
// as check_gemv, every k equal.
int check_multi(int wfmt, int64_t count, const void *h_stages);
int check_embed(const void *packed, int64_t n_rows, int64_t k, const void *ids, int64_t count, const void *out,
                int ofmt, int64_t ld_out);

// Upper bound on any single dimension accepted by the library (keeps every
// derived index within int64 and every per-row byte offset within int32).
constexpr int64_t kMaxDim = int64_t(1) << 30;

}  // namespace wsl
