// Host-side argument validation of the C ABI (no HIP dependency).
#include "validate.h"

#include "../../include/wsl.h"

namespace wsl {
namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

}  // namespace

size_t nf4_bytes(int64_t n_out, int64_t k) {
    if (n_out <= 0 || k <= 0 || (k % kGroup) != 0) return 0;
    if (n_out > kMaxDim || k > kMaxDim) return 0;
    int64_t codes = 0, scales = 0;
    if (!mul_ok(n_out, k / 2, &codes)) return 0;
    if (!mul_ok(n_out, (k / kGroup) * 2, &scales)) return 0;
    if (codes > INT64_MAX - scales) return 0;
    return static_cast<size_t>(codes + scales);
}

int check_pack(const void *w, int64_t n_out, int64_t k, const void *packed) {
    if (!w || !packed) return WSL_E_NULL;
    if (nf4_bytes(n_out, k) == 0) return WSL_E_SHAPE;
    int64_t elems = 0;
    if (!mul_ok(n_out, k, &elems)) return WSL_E_SHAPE;
    if (!aligned(w, 16) || !aligned(packed, 16)) return WSL_E_ALIGN;
    return WSL_OK;
}

int check_dequant_tile(const void *packed, int64_t n_out, int64_t k, int64_t row0, int64_t k0,
                       int64_t rows, int64_t cols, const void *tile, int64_t ld_tile) {
    if (!packed || !tile) return WSL_E_NULL;
    if (nf4_bytes(n_out, k) == 0) return WSL_E_SHAPE;
    if (rows <= 0 || cols <= 0 || ld_tile <= 0) return WSL_E_SHAPE;
    if (rows > kMaxDim || cols > kMaxDim || ld_tile > kMaxDim) return WSL_E_SHAPE;
    if (ld_tile < cols) return WSL_E_SHAPE;
    if (row0 < 0 || k0 < 0 || row0 > n_out - rows || k0 > k - cols) return WSL_E_RANGE;
    int64_t t = 0;
    if (!mul_ok(rows, ld_tile, &t)) return WSL_E_SHAPE;
    if (!aligned(packed, 16) || !aligned(tile, 2)) return WSL_E_ALIGN;
    return WSL_OK;
}

int check_gemv(int wfmt, const void *w, int64_t n_out, int64_t k, const void *x, const void *y) {
    if (wfmt != WSL_W_BF16 && wfmt != WSL_W_NF4) return WSL_E_FORMAT;
    if (!w || !x || !y) return WSL_E_NULL;
    if (n_out <= 0 || k <= 0 || n_out > kMaxDim || k > kMaxDim) return WSL_E_SHAPE;
    if (wfmt == WSL_W_NF4) {
        if (nf4_bytes(n_out, k) == 0) return WSL_E_SHAPE;
    } else {
        int64_t e = 0;
        if ((k % 8) != 0 || !mul_ok(n_out, k, &e) || e > INT64_MAX / 2) return WSL_E_SHAPE;
    }
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return WSL_E_ALIGN;
    return WSL_OK;
}

int check_gemm(int wfmt, const void *w, int64_t n_out, int64_t k, const void *x, int64_t m,
               int64_t ldx, const void *y, int ofmt, int64_t ldy, const void *ws, size_t ws_bytes) {
    if (wfmt != WSL_W_BF16 && wfmt != WSL_W_NF4) return WSL_E_FORMAT;
    if (ofmt != WSL_OUT_F32 && ofmt != WSL_OUT_BF16) return WSL_E_FORMAT;
    if (!w || !x || !y) return WSL_E_NULL;
    if (n_out <= 0 || k <= 0 || m <= 0) return WSL_E_SHAPE;
    if (n_out > kMaxDim || k > kMaxDim || m > kMaxDim || ldx > kMaxDim || ldy > kMaxDim) return WSL_E_SHAPE;
    if ((k % kGroup) != 0) return WSL_E_SHAPE;
    if (ldx < k || ldy < n_out) return WSL_E_SHAPE;
    int64_t e = 0;
    if (!mul_ok(m, ldx, &e) || !mul_ok(m, ldy, &e) || !mul_ok(n_out, k, &e)) return WSL_E_SHAPE;
    if ((ldx % 8) != 0) return WSL_E_ALIGN;
    if (!aligned(w, 16) || !aligned(x, 16)) return WSL_E_ALIGN;
    if (!aligned(y, ofmt == WSL_OUT_F32 ? 4 : 2)) return WSL_E_ALIGN;
    if (ws && ws_bytes && !aligned(ws, 16)) return WSL_E_ALIGN;
    return WSL_OK;
}

int check_ring(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
               const void *const *x, int64_t m, int64_t ldx, const void *const *y, int ofmt, int64_t ldy,
               const void *ws, size_t ws_bytes, const void *const *slot, size_t slot_bytes, const void *const *events,
               int flags) {
    if (wfmt != WSL_W_BF16 && wfmt != WSL_W_NF4) return WSL_E_FORMAT;
    if (flags & ~WSL_RING_PACE) return WSL_E_FLAGS;
    if (count < 0 || count > kMaxDim) return WSL_E_SHAPE;
    if (count == 0) return WSL_OK;
    if (!h_w || !n_out || !k || !x || !y || !slot || !events) return WSL_E_NULL;
    if (!slot[0] || !slot[1]) return WSL_E_NULL;
    if (!events[0] || !events[1] || !events[2] || !events[3]) return WSL_E_NULL;
    if (!aligned(slot[0], 16) || !aligned(slot[1], 16)) return WSL_E_ALIGN;
    for (int64_t i = 0; i < count; ++i) {
        if (!h_w[i]) return WSL_E_NULL;
        int rc = (m < 0) ? check_gemv(wfmt, slot[0], n_out[i], k[i], x[i], y[i])
                         : check_gemm(wfmt, slot[0], n_out[i], k[i], x[i], m, ldx, y[i], ofmt, ldy, ws, ws_bytes);
        if (rc != WSL_OK) return rc;
        size_t bytes = 0;
        if (wfmt == WSL_W_NF4) {
            bytes = nf4_bytes(n_out[i], k[i]);
        } else {
            int64_t e = 0;
            if (!mul_ok(n_out[i], k[i], &e) || e > INT64_MAX / 2) return WSL_E_SHAPE;
            bytes = static_cast<size_t>(e) * 2;
        }
        if (bytes == 0) return WSL_E_SHAPE;
        if (bytes > slot_bytes) return WSL_E_RANGE;
    }
    return WSL_OK;
}

int check_embed(const void *packed, int64_t n_rows, int64_t k, const void *ids, int64_t count, const void *out,
                int ofmt, int64_t ld_out) {
    if (ofmt != WSL_OUT_F32 && ofmt != WSL_OUT_BF16) return WSL_E_FORMAT;
    if (!packed || (count != 0 && (!ids || !out))) return WSL_E_NULL;   // ids and out may be NULL when count == 0
    if (nf4_bytes(n_rows, k) == 0) return WSL_E_SHAPE;
    if (count < 0 || count > kMaxDim || ld_out < k || ld_out > kMaxDim) return WSL_E_SHAPE;
    int64_t e = 0;
    if (!mul_ok(count, ld_out, &e)) return WSL_E_SHAPE;
    if ((ld_out % (ofmt == WSL_OUT_F32 ? 4 : 8)) != 0) return WSL_E_ALIGN;
    if (!aligned(packed, 16) || !aligned(ids, 8) || !aligned(out, 16)) return WSL_E_ALIGN;
    return WSL_OK;
}

int check_multi(int wfmt, int64_t count, const void *h_stages) {
    if (wfmt != WSL_W_BF16) return WSL_E_FORMAT;
    if (count < 0 || count > WSL_GEMV_MULTI_MAX) return WSL_E_SHAPE;
    if (count == 0) return WSL_OK;
    if (!h_stages) return WSL_E_NULL;
    const wsl_gemv_stage *st = static_cast<const wsl_gemv_stage *>(h_stages);
    for (int64_t i = 0; i < count; ++i) {
        const int rc = check_gemv(WSL_W_BF16, st[i].w, st[i].n_out, st[i].k, st[i].x, st[i].y);
        if (rc != WSL_OK) return rc;
        if (st[i].k != st[0].k) return WSL_E_SHAPE;
    }
    return WSL_OK;
}

int check_sweep(int wfmt, int64_t count, const void *h_stages, const void *d_stages, const void *ws,
                size_t ws_bytes, size_t ws_need) {
    if (wfmt != WSL_W_NF4) return WSL_E_FORMAT;
    if (count < 0 || count > (int64_t(1) << 24)) return WSL_E_SHAPE;
    if (count == 0) return WSL_OK;
    if (!h_stages || !d_stages || !ws) return WSL_E_NULL;
    if (!aligned(d_stages, 8) || !aligned(ws, 128)) return WSL_E_ALIGN;
    if (ws_bytes < ws_need) return WSL_E_RANGE;
    const wsl_gemv_stage *st = static_cast<const wsl_gemv_stage *>(h_stages);
    for (int64_t i = 0; i < count; ++i) {
        const int rc = check_gemv(WSL_W_NF4, st[i].w, st[i].n_out, st[i].k, st[i].x, st[i].y);
        if (rc != WSL_OK) return rc;
        if (st[i].k > 32768) return WSL_E_SHAPE;
    }
    return WSL_OK;
}

}  // namespace wsl
