// Host-only driver for the argument-validation unit, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_abi.py.
#include <cstdint>
#include <cstdio>

#include "../../include/wsl.h"
#include "../../weight_streaming_linear_amd/csrc/validate.h"

static int fails = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL line %d: %s\n", __LINE__, #cond);       \
            ++fails;                                                  \
        }                                                             \
    } while (0)

int main() {
    alignas(256) static char buf[256];   // the strictest alignment any check asks for (the sweep workspace: 128)
    void *p = buf;
    void *odd = buf + 2;
    EXPECT(wsl::nf4_bytes(4096, 4096) == 8912896u);
    EXPECT(wsl::nf4_bytes(1, 64) == 34u);
    EXPECT(wsl::nf4_bytes(0, 64) == 0u);
    EXPECT(wsl::nf4_bytes(4, 63) == 0u);
    EXPECT(wsl::nf4_bytes(-1, 64) == 0u);
    EXPECT(wsl::nf4_bytes(INT64_MAX, 64) == 0u);
    EXPECT(wsl::nf4_bytes(int64_t(1) << 30, int64_t(1) << 30) != 0u);
    EXPECT(wsl::check_pack(nullptr, 4, 64, p) == WSL_E_NULL);
    EXPECT(wsl::check_pack(p, 4, 100, p) == WSL_E_SHAPE);
    EXPECT(wsl::check_pack(odd, 4, 64, p) == WSL_E_ALIGN);
    EXPECT(wsl::check_pack(p, 4, 64, p) == WSL_OK);
    EXPECT(wsl::check_dequant_tile(p, 4, 64, 3, 0, 2, 8, p, 8) == WSL_E_RANGE);
    EXPECT(wsl::check_dequant_tile(p, 4, 64, 0, 60, 1, 8, p, 8) == WSL_E_RANGE);
    EXPECT(wsl::check_dequant_tile(p, 4, 64, 0, 0, 1, 8, p, 4) == WSL_E_SHAPE);
    EXPECT(wsl::check_dequant_tile(p, 4, 64, 0, 0, 4, 64, p, 64) == WSL_OK);
    EXPECT(wsl::check_dequant_tile(p, 4, 64, INT64_MAX, 0, 1, 1, p, 1) == WSL_E_RANGE);
    EXPECT(wsl::check_gemv(7, p, 4, 64, p, p) == WSL_E_FORMAT);
    EXPECT(wsl::check_gemv(WSL_W_NF4, p, 4, 96, p, p) == WSL_E_SHAPE);
    EXPECT(wsl::check_gemv(WSL_W_BF16, p, 4, 12, p, p) == WSL_E_SHAPE);
    EXPECT(wsl::check_gemv(WSL_W_BF16, p, 4, 16, p, p) == WSL_OK);
    EXPECT(wsl::check_gemv(WSL_W_BF16, p, 4, 16, odd, p) == WSL_E_ALIGN);
    EXPECT(wsl::check_gemv(WSL_W_BF16, p, INT64_MAX, INT64_MAX, p, p) == WSL_E_SHAPE);
    EXPECT(wsl::check_gemm(WSL_W_BF16, p, 4, 64, p, 3, 64, p, 9, 8, nullptr, 0) == WSL_E_FORMAT);
    EXPECT(wsl::check_gemm(WSL_W_BF16, p, 4, 64, p, 3, 60, p, WSL_OUT_F32, 8, nullptr, 0) == WSL_E_SHAPE);
    EXPECT(wsl::check_gemm(WSL_W_BF16, p, 4, 64, p, 3, 68, p, WSL_OUT_F32, 8, nullptr, 0) == WSL_E_ALIGN);
    EXPECT(wsl::check_gemm(WSL_W_BF16, p, 4, 64, p, 3, 64, p, WSL_OUT_F32, 8, nullptr, 0) == WSL_OK);
    EXPECT(wsl::check_gemm(WSL_W_NF4, p, 4, 64, p, 0, 64, p, WSL_OUT_F32, 8, nullptr, 0) == WSL_E_SHAPE);
    EXPECT(wsl::check_gemm(WSL_W_NF4, p, 4, 64, p, 3, 64, p, WSL_OUT_F32, 8, odd, 64) == WSL_E_ALIGN);
    EXPECT(wsl::check_gemm(WSL_W_NF4, p, 4, 64, p, INT64_MAX / 2, 64, p, WSL_OUT_F32, 8, nullptr, 0) == WSL_E_SHAPE);
    EXPECT(wsl::check_embed(p, 4, 64, p, 2, p, 9, 64) == WSL_E_FORMAT);
    EXPECT(wsl::check_embed(p, 4, 64, nullptr, 2, p, WSL_OUT_BF16, 64) == WSL_E_NULL);
    EXPECT(wsl::check_embed(p, 4, 60, p, 2, p, WSL_OUT_BF16, 64) == WSL_E_SHAPE);
    EXPECT(wsl::check_embed(p, 4, 64, p, -1, p, WSL_OUT_BF16, 64) == WSL_E_SHAPE);
    EXPECT(wsl::check_embed(p, 4, 64, p, 2, p, WSL_OUT_BF16, 32) == WSL_E_SHAPE);
    EXPECT(wsl::check_embed(p, 4, 64, p, 2, p, WSL_OUT_BF16, 68) == WSL_E_ALIGN);
    EXPECT(wsl::check_embed(p, 4, 64, p, 2, p, WSL_OUT_F32, 68) == WSL_OK);
    EXPECT(wsl::check_embed(p, 4, 64, odd, 2, p, WSL_OUT_F32, 64) == WSL_E_ALIGN);
    EXPECT(wsl::check_embed(p, 4, 64, p, 2, odd, WSL_OUT_F32, 64) == WSL_E_ALIGN);
    EXPECT(wsl::check_embed(p, 4, 64, p, 0, p, WSL_OUT_BF16, 64) == WSL_OK);
    EXPECT(wsl::check_embed(p, 4, 64, nullptr, 0, nullptr, WSL_OUT_BF16, 64) == WSL_OK);
    EXPECT(wsl::check_embed(nullptr, 4, 64, p, 1, p, WSL_OUT_BF16, 64) == WSL_E_NULL);
    EXPECT(wsl::check_embed(p, 4, 64, p, INT64_MAX, p, WSL_OUT_BF16, 64) == WSL_E_SHAPE);
    {
        const void *hw[2] = {p, p};
        const void *xs[2] = {p, p};
        const void *ys[2] = {p, p};
        const void *slots[2] = {p, p};
        const void *evs[4] = {p, p, p, p};
        const int64_t ns[2] = {4, 8}, ks[2] = {64, 128};
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 1024, evs, 0) == WSL_OK);
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 543, evs, 0) == WSL_E_RANGE);
        EXPECT(wsl::check_ring(WSL_W_BF16, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 1024, evs, 0) == WSL_E_RANGE);
        EXPECT(wsl::check_ring(WSL_W_BF16, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 2048, evs, 0) == WSL_OK);
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, 3, 128, ys, WSL_OUT_F32, 8, nullptr, 0, slots, 1024, evs, 0) == WSL_OK);
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, 3, 64, ys, WSL_OUT_F32, 8, nullptr, 0, slots, 1024, evs, 0) == WSL_E_SHAPE);
        const void *badslots[2] = {p, odd};
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, badslots, 1024, evs, 0) == WSL_E_ALIGN);
        const void *hw0[2] = {p, nullptr};
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw0, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 1024, evs, 0) == WSL_E_NULL);
        EXPECT(wsl::check_ring(WSL_W_NF4, 0, nullptr, nullptr, nullptr, nullptr, -1, 0, nullptr, 0, 0, nullptr, 0,
                               nullptr, 0, nullptr, 0) == WSL_OK);
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 1024, evs,
                               WSL_RING_PACE) == WSL_OK);
        EXPECT(wsl::check_ring(WSL_W_NF4, 2, hw, ns, ks, xs, -1, 0, ys, 0, 0, nullptr, 0, slots, 1024, evs, 2) ==
               WSL_E_FLAGS);
        EXPECT(wsl::check_ring(WSL_W_NF4, 0, nullptr, nullptr, nullptr, nullptr, -1, 0, nullptr, 0, 0, nullptr, 0,
                               nullptr, 0, nullptr, -1) == WSL_E_FLAGS);
    }
    {
        // several bf16 GEMVs in one launch: one k, at most WSL_GEMV_MULTI_MAX
        wsl_gemv_stage st[WSL_GEMV_MULTI_MAX + 1];
        for (auto &e : st) e = wsl_gemv_stage{p, p, reinterpret_cast<float *>(const_cast<void *>(p)), 16, 512};
        EXPECT(wsl::check_multi(WSL_W_BF16, 3, st) == WSL_OK);
        EXPECT(wsl::check_multi(WSL_W_BF16, WSL_GEMV_MULTI_MAX, st) == WSL_OK);
        EXPECT(wsl::check_multi(WSL_W_BF16, WSL_GEMV_MULTI_MAX + 1, st) == WSL_E_SHAPE);
        EXPECT(wsl::check_multi(WSL_W_BF16, 0, nullptr) == WSL_OK);
        EXPECT(wsl::check_multi(WSL_W_BF16, 2, nullptr) == WSL_E_NULL);
        EXPECT(wsl::check_multi(WSL_W_NF4, 2, st) == WSL_E_FORMAT);
        st[1].k = 1024;
        EXPECT(wsl::check_multi(WSL_W_BF16, 2, st) == WSL_E_SHAPE);
        st[1].k = 516;
        EXPECT(wsl::check_multi(WSL_W_BF16, 2, st) == WSL_E_SHAPE);
        st[1].k = 512;
        st[1].w = odd;
        EXPECT(wsl::check_multi(WSL_W_BF16, 2, st) == WSL_E_ALIGN);
    }
    {
        // decode sweep: host descriptors, device descriptor array and workspace
        wsl_gemv_stage st[3];
        for (auto &e : st) e = wsl_gemv_stage{p, p, reinterpret_cast<float *>(const_cast<void *>(p)), 4, 64};
        const size_t need = 2048;
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, p, p, need, need) == WSL_OK);
        EXPECT(wsl::check_sweep(WSL_W_NF4, 0, nullptr, nullptr, nullptr, 0, need) == WSL_OK);
        EXPECT(wsl::check_sweep(WSL_W_BF16, 3, st, p, p, need, need) == WSL_E_FORMAT);
        EXPECT(wsl::check_sweep(WSL_W_NF4, -1, st, p, p, need, need) == WSL_E_SHAPE);
        EXPECT(wsl::check_sweep(WSL_W_NF4, (int64_t(1) << 24) + 1, st, p, p, need, need) == WSL_E_SHAPE);
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, nullptr, p, p, need, need) == WSL_E_NULL);
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, odd, p, need, need) == WSL_E_ALIGN);
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, p, p, need - 1, need) == WSL_E_RANGE);
        st[2].k = 32768 + 64;
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, p, p, need, need) == WSL_E_SHAPE);
        st[2].k = 96;
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, p, p, need, need) == WSL_E_SHAPE);
        st[2].k = 64;
        st[1].x = odd;
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, p, p, need, need) == WSL_E_ALIGN);
        st[1].x = p;
        st[0].w = nullptr;
        EXPECT(wsl::check_sweep(WSL_W_NF4, 3, st, p, p, need, need) == WSL_E_NULL);
    }
    std::printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
