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
#include <atomic>
#include <mutex>

#include "device_common.h"

namespace wsl {

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- bf16, LDS-tiled
// Workgroup tile 256 (m) x 256 (n), 8 waves in 2 (m) x 4 (n), each owning a
// 128 x 64 block as 4 x 2 v_mfma_f32_32x32x16_bf16 tiles (128 fp32
// accumulators per lane; two waves per SIMD).
// The k loop runs over 32-k stages held in a 4-deep LDS ring (4 x 32 KB).
// Operands go global -> LDS directly (global_load_lds_dwordx4: a wave-wide
// load writes 1 KB of LDS, lane L at byte 16L), so no registers are spent on
// staging and two to three stages (64-96 KB per CU) stay in flight: enough
// bytes in flight to cover the L2/MALL latency at the operand rate a 256 x 256
// tile needs.  The two waves of a SIMD alternate between multiplying a stage and
// reading the fragments of their next one (see bf16_tile).
// LDS rows are 32 bf16 = 64 B = 4 chunks of 16 B; chunk c of row r sits at
// c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1): the fragment reads (32 rows, one chunk
// column) are free of bank conflicts for 32 and for 64 banks.  Because a
// lane's LDS slot is fixed by its lane index, the swizzle is applied by
// choosing which global chunk each lane copies.
// Workgroups map to tiles XCD-aware: each of the 8 XCDs takes a contiguous
// range of tiles, ordered in bands of 8 m-tiles, so tiles sharing rows of X or
// of W run on the same XCD (one L2) at about the same time.
constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;   // 32 KB

__device__ __forceinline__ int chunk_swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + (chunk_swz(row, chunk) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane direct global -> LDS copy (lane L writes lds_dst + 16 L).  A plain
// function: called straight from a kernel template, the builtin left that template's
// host-side launch stub unemitted.
__device__ __forceinline__ void lds_copy16(const void *src, char *lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_dst, 16, 0, 0);
}

// s_waitcnt with vmcnt <= N and the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One workgroup tile: TM = 256 rows of X (each wave 128 x 64 of the output, 4 x 2
// MFMA tiles) or TM = 128 (each wave 64 x 64, 2 x 2 tiles: the half tiles that
// shorten the last, partly filled round of a launch), over the k range [kb, kb + kl)
// (kb and kl multiples of 64; the whole k unless the launch splits k).
// The four ring stages are separate LDS objects and the k loop is unrolled by
// four, so every copy and every fragment read names its stage at compile time;
// the compiler can then tell that reading stage s does not alias the copies
// still in flight into the other stages, and does not drain them.
template <int TM>
__device__ __forceinline__ void bf16_tile(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t m,
                                          int64_t n_out, int64_t k, int64_t kb, int64_t kl, int64_t ldx,
                                          void *__restrict__ y, int ofmt,
                                          int64_t ldy, int64_t m0, int64_t n0, char *st0, char *st1, char *st2,
                                          char *st3) {
    constexpr int MI = TM / 64;         // 32-row MFMA tiles per wave along m
    constexpr int NA = TM / 128;        // A wave-loads per wave per stage
    constexpr int NV = NA + 2;          // copies per wave per stage
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;

    // Copies: A wave-load g (g = NA*wave + i) and B wave-loads g = 2*wave + i each
    // cover 16 tile rows, lane L row 16g + L/4, LDS slot L % 4.  Rows outside the
    // matrix are clamped (they only feed discarded outputs).
    const uint16_t *asrc[NA];
    const uint16_t *bsrc[2];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int row = 16 * (NA * wave + i) + (lane >> 2);
        const int c = chunk_swz(row, lane & 3);                 // global chunk landing in slot lane % 4
        const int64_t gm = (m0 + row < m) ? m0 + row : m - 1;
        asrc[i] = x + gm * ldx + kb + c * 8;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * (2 * wave + i) + (lane >> 2);
        const int c = chunk_swz(row, lane & 3);
        const int64_t gn = (n0 + row < n_out) ? n0 + row : n_out - 1;
        bsrc[i] = w + gn * k + kb + c * 8;
    }
    auto copy_stage = [&](int64_t kt, char *sa) {
        char *sb = sa + kBM * kBK * 2;
        const int64_t k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < NA; ++i)
            lds_copy16(asrc[i] + k0, sa + (NA * wave + i) * 1024);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            lds_copy16(bsrc[i] + k0, sb + (2 * wave + i) * 1024);
    };

    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int half = lane >> 5, l32 = lane & 31;
    const int64_t ktiles = kl / kBK;   // even: kl % 64 == 0
    // Fragment reads: the lane's MI A rows (and 2 B rows) are 32 rows apart and
    // share their swizzled chunk, so one base address plus immediate offsets
    // (2048 B apart) covers the reads of a 16-k step.  They are issued from
    // inline asm with their own lgkmcnt wait: the compiler then has no LDS read
    // of its own there to order against the copies still in flight into the
    // other stages (it cannot prove those disjoint across the loop back-edge and
    // would drain every copy).
    uint32_t offa[2], offb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        offa[ks] = static_cast<uint32_t>(swz(wm * (TM / 2) + l32, ks * 2 + half));
        offb[ks] = static_cast<uint32_t>(kBM * kBK * 2 + swz(wn * 64 + l32, ks * 2 + half));
    }
    using frags = u32x4[MI + 2];
    auto issue = [&](uint32_t a_addr, uint32_t b_addr, frags &f) {
        if constexpr (MI == 4) {
            asm volatile(
                "ds_read_b128 %0, %6\n\t"
                "ds_read_b128 %1, %6 offset:2048\n\t"
                "ds_read_b128 %2, %6 offset:4096\n\t"
                "ds_read_b128 %3, %6 offset:6144\n\t"
                "ds_read_b128 %4, %7\n\t"
                "ds_read_b128 %5, %7 offset:2048"
                : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5])
                : "v"(a_addr), "v"(b_addr));
        } else {
            asm volatile(
                "ds_read_b128 %0, %4\n\t"
                "ds_read_b128 %1, %4 offset:2048\n\t"
                "ds_read_b128 %2, %5\n\t"
                "ds_read_b128 %3, %5 offset:2048"
                : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
                : "v"(a_addr), "v"(b_addr));
        }
    };
    // The wait is a separate asm statement that takes every fragment as an in/out
    // operand (each named once), so no MFMA can use one before it.
    auto landed = [&](frags &f0, frags &f1) {
        if constexpr (MI == 4) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f0[0]), "+v"(f0[1]), "+v"(f0[2]), "+v"(f0[3]), "+v"(f0[4]), "+v"(f0[5]),
                           "+v"(f1[0]), "+v"(f1[1]), "+v"(f1[2]), "+v"(f1[3]), "+v"(f1[4]), "+v"(f1[5]));
        } else {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f0[0]), "+v"(f0[1]), "+v"(f0[2]), "+v"(f0[3]), "+v"(f1[0]), "+v"(f1[1]),
                           "+v"(f1[2]), "+v"(f1[3]));
        }
    };
    // Two groups of four waves, one wave of each on every SIMD (waves are placed on
    // the SIMDs in turn), take turns: while one group multiplies a k-stage (2 x MI x 2
    // MFMAs that keep the SIMD's matrix pipe busy), the other reads its fragments of
    // the next stage from LDS.  Every wave runs the same sequence -- memory phase,
    // barrier, MFMA phase, barrier -- and the second group starts one barrier later,
    // so the phases of the two groups alternate between consecutive barriers without
    // any branch on the group inside the loop.  In the memory phase the fragment reads
    // go first and the wait for this wave's copies comes after them, so the reads do
    // not queue behind copies still arriving from L2.
    // Ring of four stages.  A wave's copies of k-tile kt + 3 are issued one by one
    // among the MFMAs of its stage kt, into the slot stage kt - 1 used (both groups
    // finished reading it before the barrier that began this phase).  Its memory phase
    // of stage kt then waits until only its copies of kt + 2 are in flight: its share
    // of stage kt + 1 is in LDS, and the barrier that ends the phase publishes it
    // before either group reads stage kt + 1.
    auto bar = []() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lds_addr = [](char *p) { return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p)); };
    const uint32_t a0 = lds_addr(st0), a1 = lds_addr(st1), a2 = lds_addr(st2), a3 = lds_addr(st3);
    auto copy_piece = [&](int q, int64_t kt, char *sa) {
        const int64_t k0 = kt * kBK;
        if (q < NA)
            lds_copy16(asrc[q] + k0, sa + (NA * wave + q) * 1024);
        else
            lds_copy16(bsrc[q - NA] + k0, sa + kBM * kBK * 2 + (2 * wave + q - NA) * 1024);
    };
    frags f0, f1;
    auto stage = [&](int64_t kt, uint32_t cur, char *refill) {
        issue(cur + offa[0], cur + offb[0], f0);
        issue(cur + offa[1], cur + offb[1], f1);
        landed(f0, f1);
        if (kt + 2 < ktiles) {
            wait_vmcnt<NV>();
        } else {
            wait_vmcnt<0>();
        }
        bar();
        const bool rf = kt + 3 < ktiles;
        int q = 0;
        constexpr int MF = 2 * MI;   // MFMAs per 16-k step
#pragma unroll
        for (int t = 0; t < 2 * MF; ++t) {
            const int i = (t % MF) >> 1, j = t & 1;
            const frags &f = t < MF ? f0 : f1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f[i]),
                                                                __builtin_bit_cast(bf16x8, f[MI + j]), acc[i][j], 0, 0, 0);
            if ((t + 1) == (q + 1) * 2 * MF / (NV + 1) && q < NV) {
                __builtin_amdgcn_sched_barrier(0);
                if (rf) copy_piece(q, kt + 3, refill);
                __builtin_amdgcn_sched_barrier(0);
                ++q;
            }
        }
        bar();
    };
    const int group = static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(wave))) >> 2;
    copy_stage(0, st0);
    copy_stage(1, st1);
    if (2 < ktiles) {
        copy_stage(2, st2);
        wait_vmcnt<2 * NV>();
    } else {
        wait_vmcnt<NV>();
    }
    bar();                   // stage 0 in LDS
    if (group != 0) bar();   // the second group runs one phase behind
    int64_t kt = 0;
    for (; kt + 4 <= ktiles; kt += 4) {
        stage(kt + 0, a0, st3);
        stage(kt + 1, a1, st0);
        stage(kt + 2, a2, st1);
        stage(kt + 3, a3, st2);
    }
    if (kt + 0 < ktiles) stage(kt + 0, a0, st3);
    if (kt + 1 < ktiles) stage(kt + 1, a1, st0);
    if (kt + 2 < ktiles) stage(kt + 2, a2, st1);
    if (group == 0) bar();   // both groups pass the same number of barriers

    // 32x32 accumulator layout: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + l32;
            if (col >= n_out) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * (TM / 2) + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
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

// Work item -> tile, XCD-aware: XCD x = blockIdx % nx takes the contiguous tile
// range [start(x), start(x) + count(x)) in its dispatch order blockIdx / nx.  When
// the XCD's last round (count mod its CU count, one workgroup per CU) would
// leave at least half of its CUs idle, those tiles run as two 128-row halves
// each, so that round takes about half as long.  Tiles are ordered in bands of 8
// m-tiles, so tiles sharing rows of X or of W run on the same XCD (one L2) at
// about the same time.  With k split s ways a tile is s work items (its k ranges),
// consecutive in that order: column tn of s * tiles_n is tile column tn / s, split
// tn % s.  tail_halves = false: no tail split (a launch of half tiles only, M <= 128).
// Returns false for a work item past the XCD's end.
struct TileItem {
    int64_t m0, n0;
    int half;    // -1: the whole 256-row tile; 0 / 1: its first / second 128 rows
    int split;   // k range of the item
};
__device__ __forceinline__ bool tile_item(int tiles_m, int tiles_n_splits, int splits, int nx, int xcd_cus,
                                          bool tail_halves, TileItem &it) {
    const int tiles_n = tiles_n_splits;
    const int ntiles = tiles_m * tiles_n;
    const int per_xcd = ntiles / nx, rem = ntiles - per_xcd * nx;
    const int xcd = static_cast<int>(blockIdx.x) % nx, slot = static_cast<int>(blockIdx.x) / nx;
    const int count = per_xcd + (xcd < rem ? 1 : 0);
    const int start = xcd * per_xcd + (xcd < rem ? xcd : rem);
    const int r = count % xcd_cus;
    const int split = (tail_halves && r > 0 && 2 * r <= xcd_cus) ? r : 0;
    const int full = count - split;
    int t;
    it.half = -1;
    if (slot < full) {
        t = start + slot;
    } else {
        const int h = slot - full;
        if (h >= 2 * split) return false;
        t = start + full + (h >> 1);
        it.half = h & 1;
    }
    const int band = 8;
    const int band_tiles = band * tiles_n;
    const int b_idx = t / band_tiles, in_band = t - b_idx * band_tiles;
    const int band_rows = (tiles_m - b_idx * band) < band ? (tiles_m - b_idx * band) : band;
    const int tm = b_idx * band + in_band % band_rows;
    const int tn = in_band / band_rows;
    it.m0 = static_cast<int64_t>(tm) * kBM + (it.half > 0 ? kBM / 2 : 0);
    it.n0 = static_cast<int64_t>(tn / splits) * kBN;
    it.split = tn % splits;
    return true;
}

// A work item's k range and destination: with ws (k split) the item writes its fp32
// partial sums to ws[(split * m + row) * n_out + col], summed by split_reduce_kernel.
struct SplitOut {
    int64_t kb, kl;
    void *y;
    int ofmt;
    int64_t ldy;
};
__device__ __forceinline__ SplitOut split_out(int split, int64_t kps, int64_t k, int64_t m, int64_t n_out, void *y,
                                              int ofmt, int64_t ldy, float *ws) {
    SplitOut o;
    o.kb = static_cast<int64_t>(split) * kps;
    o.kl = (o.kb + kps < k) ? kps : k - o.kb;
    if (ws != nullptr) {
        o.y = ws + static_cast<int64_t>(split) * m * n_out;
        o.ofmt = WSL_OUT_F32;
        o.ldy = n_out;
    } else {
        o.y = y;
        o.ofmt = ofmt;
        o.ldy = ldy;
    }
    return o;
}

__global__ __launch_bounds__(512) void gemm_bf16_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                        int64_t m, int64_t n_out, int64_t k, int64_t ldx,
                                                        void *__restrict__ y, int ofmt, int64_t ldy,
                                                        int tiles_m, int tiles_n, int nx, int xcd_cus, int splits,
                                                        int64_t kps, float *__restrict__ ws, int half_only) {
    __shared__ __attribute__((aligned(1024))) char st0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st2[kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st3[kStageBytes];
    TileItem it;
    if (!tile_item(tiles_m, tiles_n * splits, splits, nx, xcd_cus, half_only == 0, it) || it.m0 >= m) return;
    if (half_only) it.half = 0;
    const SplitOut o = split_out(it.split, kps, k, m, n_out, y, ofmt, ldy, ws);
    if (it.half < 0)
        bf16_tile<256>(x, w, m, n_out, k, o.kb, o.kl, ldx, o.y, o.ofmt, o.ldy, it.m0, it.n0, st0, st1, st2, st3);
    else
        bf16_tile<128>(x, w, m, n_out, k, o.kb, o.kl, ldx, o.y, o.ofmt, o.ldy, it.m0, it.n0, st0, st1, st2, st3);
}

// ---------------------------------------------------------------- NF4, weight-stationary
// Each wave owns NB blocks of 32 weight rows (n) and a k range of its split.
// Lane l serves rows n0 + 32j + l%32 (j < NB) and k half h = l/32.  Per 256-k
// step the lane reads, for each of its rows, one contiguous 64-byte run of codes
// (k in [kc + 128h, kc + 128h + 128): 128 codes, two groups), restores 8 codes
// at a time into a bf16 B fragment t = bf16(fp32(level * s)) and issues one
// v_mfma_f32_32x32x16_bf16 per fragment and block; the A fragment (8 positions'
// worth of X for the same 8 k) is loaded once and shared by the NB blocks.
// A k tail shorter than 256 is done in 64-k steps (lane: 32 codes at
// kc + 32h), with the same rule that A and B use one k assignment per MFMA.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float s, const char *lut) {
    const uint32_t wo = rotr32(w, 4);
    uint4 r;
    r.x = pack_bf16x2(*reinterpret_cast<const float *>(lut + (w & 0x3cu)) * s,
                      *reinterpret_cast<const float *>(lut + (wo & 0x3cu)) * s);
    r.y = pack_bf16x2(*reinterpret_cast<const float *>(lut + ((w >> 8) & 0x3cu)) * s,
                      *reinterpret_cast<const float *>(lut + ((wo >> 8) & 0x3cu)) * s);
    r.z = pack_bf16x2(*reinterpret_cast<const float *>(lut + ((w >> 16) & 0x3cu)) * s,
                      *reinterpret_cast<const float *>(lut + ((wo >> 16) & 0x3cu)) * s);
    r.w = pack_bf16x2(*reinterpret_cast<const float *>(lut + (w >> 24 & 0x3cu)) * s,
                      *reinterpret_cast<const float *>(lut + ((wo >> 24) & 0x3cu)) * s);
    return r;
}

// NF4 GEMM kernel (32 positions per z block).  Every wave is independent: it
// owns NB blocks of 32 weight rows and the k range of its split (blockIdx.y).
// Per 128-k chunk a wave
//   1. copies X[32 positions][128 k] into its private 8 KB LDS buffer with fully
//      coalesced loads (one wave-wide load = 4 rows x 256 B), 16-byte chunks of
//      each row stored at chunk ^ (row & 15) so the fragment reads below hit
//      distinct banks;
//   2. for its NB row blocks reads the codes (lane (n, h): 64 codes of row n at
//      k in [kc + 64h, kc + 64h + 64)), restores 8 at a time into a bf16 B
//      fragment t = bf16(fp32(level * s)), and issues one MFMA per fragment and
//      block, the A fragment X[m][kc + 64h + 8t .. +8] (read once from LDS) being
//      shared by the NB blocks.
// The wave writes its 32 x 32NB result to Y, or to the split workspace.
template <int NB>
__global__ __launch_bounds__(256) void gemm_nf4_kernel(const uint8_t *__restrict__ packed, int64_t n_out,
                                                       int64_t k, const uint16_t *__restrict__ x, int64_t m,
                                                       int64_t ldx, void *__restrict__ y, int ofmt, int64_t ldy,
                                                       float *__restrict__ ws, int64_t k_per_split) {
    __shared__ float lut[16];
    __shared__ __attribute__((aligned(16))) char xs_all[4][32 * 256];
    write_levels(lut);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    char *xs = xs_all[wave];
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 32 * NB;
    if (n0 >= n_out) return;                               // no barrier follows
    const int64_t mbase = static_cast<int64_t>(blockIdx.z) * 32;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * k_per_split;
    const int64_t kend = (kbeg + k_per_split < k) ? kbeg + k_per_split : k;
    const int64_t groups = k >> 6;
    const int64_t rowbytes = k >> 1;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
    const char *lutp = reinterpret_cast<const char *>(lut);

    int64_t rows[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t n = n0 + 32 * j + l32;
        rows[j] = n < n_out ? n : n_out - 1;
    }
    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    // staging: load i (0..7) covers X rows 4i + lane/16, 16-byte chunk lane%16
    const int srow = lane >> 4, schunk = lane & 15;
    for (int64_t kc = kbeg; kc < kend; kc += 128) {
        const int64_t kw = (kend - kc < 128) ? (kend - kc) : 128;   // 64 or 128
        uint4 xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = mbase + 4 * i + srow;
            const bool ok = (r < m) && (schunk * 8 < kw);
            xv[i] = ok ? *reinterpret_cast<const uint4 *>(x + r * ldx + kc + schunk * 8) : make_uint4(0, 0, 0, 0);
        }
        uint4 q[NB][2];
        float s[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t kl = kc + 64 * half;
            if (kl < kend) {
                const uint8_t *src = packed + rows[j] * rowbytes + (kl >> 1);
                q[j][0] = *reinterpret_cast<const uint4 *>(src);
                q[j][1] = *reinterpret_cast<const uint4 *>(src + 16);
                s[j] = f16_to_f32(scales[scale_index(rows[j], kl >> 6, groups, n_out)]);
            } else {
                q[j][0] = q[j][1] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);
                s[j] = 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + srow;
            *reinterpret_cast<uint4 *>(xs + r * 256 + ((schunk ^ (r & 15)) << 4)) = xv[i];
        }
        // the wave reads back what its own lanes wrote: LDS ops of one wave are
        // ordered, so no barrier is needed
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = 8 * half + t;                      // 16-byte chunk of k = kc + 64h + 8t
            const uint4 av = *reinterpret_cast<const uint4 *>(xs + l32 * 256 + ((c ^ (l32 & 15)) << 4));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const uint4 qq = q[j][t >> 2];
                const uint32_t wd = (t & 3) == 0 ? qq.x : (t & 3) == 1 ? qq.y : (t & 3) == 2 ? qq.z : qq.w;
                const uint4 bv = dequant8(wd, s[j], lutp);
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv), acc[j], 0, 0, 0);
            }
        }
    }

    // Output element e of lane l: position mbase + 8*(e/4) + 4*h + e%4, column n0 + 32j + l%32.
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int64_t col = n0 + 32 * j + l32;
        if (col >= n_out) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = mbase + 8 * (e >> 2) + 4 * half + (e & 3);
            if (row >= m) continue;
            const float v = acc[j][e];
            if (ws != nullptr) {
                ws[(static_cast<int64_t>(blockIdx.y) * m + row) * n_out + col] = v;
            } else if (ofmt == WSL_OUT_F32) {
                static_cast<float *>(y)[row * ldy + col] = v;
            } else {
                static_cast<uint16_t *>(y)[row * ldy + col] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
            }
        }
    }
}

// ---------------------------------------------------------------- NF4, shared X, M <= 32
// The prefill kernel for up to 32 positions and k a multiple of 256.  A
// workgroup of 8 waves owns 256 / KH weight rows: waves w and w + 8 / KH share
// rows 32 (w % (8 / KH)) .. + 31 (lane l row l % 32), and with KH = 2 each of the
// two takes half of every chunk's k-steps.  It covers the k range of its split.
// Per 256-k chunk:
//   * the workgroup stages X[32 positions][256 k] (16 KB) once in LDS (two
//     buffers; row i at i * 512, 16-byte chunk c at c ^ (i % 32) so that the
//     fragment reads of a 32-lane half are free of bank conflicts), instead of
//     every wave reading its own copy;
//   * lane (n, h) owns the codes of row n for k in [kc + 128h, kc + 128h + 128)
//     -- 16 MFMA k-steps of 8 codes, 64 bytes -- of which its wave takes steps
//     [16 kh / KH, 16 (kh + 1) / KH), loaded one chunk ahead with the scales of
//     those groups.  When the workgroup is the matrix's only position block (CS),
//     the chunk's codes are instead copied with whole-line streaming loads into an
//     LDS stage and each lane reads its pieces from there: on 27648x5120 at M = 32
//     this runs 28.5 us against 32.7 us for per-lane cached loads, whose lines are
//     split over four instructions.  With several position blocks the per-lane
//     cached loads stay (the blocks share the lines through the caches);
//   * each k-step restores 8 codes through the replicated pair table into a
//     bf16 B fragment t = bf16(fp32(level * s)) and issues one
//     v_mfma_f32_32x32x16_bf16 against the A fragment X[i][same 8 k] from LDS;
//     the table and X reads of step t + 1 are issued before step t's math.
// The barrier that publishes a staged chunk is an asm statement with a memory
// clobber and no vmcnt wait, so the next chunk's loads stay in flight across it
// and the compiler cannot move LDS accesses over it.  With KH = 2 the second
// half's accumulators meet the first's in LDS (a fixed order), then the 32 x 32
// result goes to Y, or to the split workspace.
// The library launches KH = 2 (128 rows per workgroup): tall matrices then fill the
// CUs without splitting k (no workspace, no reduction pass), and short ones need
// half the k splits of the 256-row form.
constexpr int kX32Chunk = 256;
constexpr int kX32Stage = 32 * kX32Chunk * 2;

template <int KH, int MB, int CS>
__global__ __launch_bounds__(512) void gemm_nf4_x32_kernel(const uint8_t *__restrict__ packed, int64_t n_out,
                                                           int64_t k, const uint16_t *__restrict__ x, int64_t m,
                                                           int64_t ldx, void *__restrict__ y, int ofmt, int64_t ldy,
                                                           float *__restrict__ ws, int64_t k_per_split) {
    constexpr int RG = 8 / KH;        // row groups of 32 per workgroup
    constexpr int NQ = 4 / KH;        // 16-byte code loads per lane per chunk
    constexpr int NS = 16 / KH;       // k-steps per wave per chunk
    constexpr int NG = 2 / KH;        // scales per lane per chunk
    // X goes global -> LDS directly for two position groups (M 33..64: 57.5 -> 38.4 us on
    // 27648x5120, where the register staging's loads were moved by the compiler to just
    // before their use); with one group the register staging, whose loads are issued
    // before the barrier, is faster (29.4 against 31.7 us at M = 32).
    constexpr bool XD = MB == 2;
    __shared__ __align__(16) char tab[kPairTableBytes];
    // X stages (position group g at g * kX32Stage), two separate objects so that the
    // compiler can tell reads of one from direct copies still in flight into the other
    __shared__ __attribute__((aligned(1024))) char xs0[MB * kX32Stage];
    __shared__ __attribute__((aligned(1024))) char xs1[MB * kX32Stage];
    __shared__ __align__(16) char cst[CS ? 2 : 1][CS ? 32 * RG * (kX32Chunk / 2) : 16];   // CS: the chunk's codes
    fill_pair_table(tab);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rg = wave % RG, kh = wave / RG;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t groups = k >> 6;
    const int64_t rowbytes = k >> 1;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
    const int64_t rowt = static_cast<int64_t>(blockIdx.x) * (32 * RG) + rg * 32 + l32;
    const int64_t row = rowt < n_out ? rowt : n_out - 1;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * k_per_split;
    const int64_t kend = (kbeg + k_per_split < k) ? kbeg + k_per_split : k;
    const int nch = kend > kbeg ? static_cast<int>((kend - kbeg) / kX32Chunk) : 0;
    uint32_t ad[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = static_cast<uint32_t>(lane & 31) << 3;
    // Codes.  CS = 0: lane (n, h) loads its own 16-byte pieces of row n (ordinary
    // loads: 4 lanes share each 128-byte line, and the line serves the other
    // position blocks of the matrix too).  CS = 1 (the only position block): copy j
    // of thread t moves 16-byte segment t % 8 of row 64 j + t / 8 of the chunk -- 8
    // threads per 128-byte row, whole lines per wave instruction -- with loads that
    // bypass the caches, into LDS at row * 128 + 16 (segment ^ (row % 8)); the lane
    // reads its pieces back from there (conflict-free: 8 consecutive rows of one
    // segment fall in distinct bank groups).
    const uint8_t *crow = packed + row * rowbytes + 64 * half + (64 / KH) * kh;
    const uint8_t *ccp[NQ];
    int coff[NQ], lcoff[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int r = 64 * j + (tid >> 3), sg = tid & 7;
        const int64_t rt = static_cast<int64_t>(blockIdx.x) * (32 * RG) + r;
        ccp[j] = packed + (rt < n_out ? rt : n_out - 1) * rowbytes + 16 * sg;
        coff[j] = r * 128 + ((sg ^ (r & 7)) << 4);
        const int lr = rg * 32 + l32, lsg = 4 * half + NQ * kh + j;
        lcoff[j] = lr * 128 + ((lsg ^ (lr & 7)) << 4);
    }
    const int64_t srem = n_out - ((row >> 4) << 4);
    const int64_t srb = srem < 16 ? srem : 16;
    const uint16_t *srow = scales + (row >> 4) * 16 * groups + (row & 15);   // scale (row, g) at srow[g * srb]
    // Positions of this workgroup: p0 .. p0 + 32 MB - 1 (blockIdx.z), in MB groups of 32.
    // X staging: for each group g, thread t moves the 16-byte chunks (row t / 32, chunk
    // t % 32) and (row t / 32 + 16, same chunk); rows past m repeat row m - 1.
    const int64_t p0 = static_cast<int64_t>(blockIdx.z) * 32 * MB;
    const int xi0 = tid >> 5, xi1 = xi0 + 16, xcc = tid & 31;
    const uint16_t *xrow0[MB], *xrow1[MB];
#pragma unroll
    for (int g = 0; g < MB; ++g) {
        const int64_t r0 = p0 + 32 * g + xi0, r1 = p0 + 32 * g + xi1;
        xrow0[g] = x + (r0 < m ? r0 : m - 1) * ldx + xcc * 8;
        xrow1[g] = x + (r1 < m ? r1 : m - 1) * ldx + xcc * 8;
    }
    const int xoff0 = xi0 * 512 + ((xcc ^ xi0) << 4);
    const int xoff1 = xi1 * 512 + ((xcc ^ xi1) << 4);
    // XD: X goes global -> LDS directly.  Copy i of wave w (i < 2) fills 1 KB of a
    // group's stage: rows r = 2 (2w + i) + (lane / 32), slot lane % 32; since a lane's LDS
    // slot is fixed, the swizzle is applied by copying chunk slot ^ (r % 32) of row r.
    const uint16_t *xdsrc[MB][2];
#pragma unroll
    for (int g = 0; g < MB; ++g)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 2 * (2 * wave + i) + (lane >> 5);
            const int64_t pr = p0 + 32 * g + r;
            xdsrc[g][i] = x + (pr < m ? pr : m - 1) * ldx + ((l32 ^ r) << 3);
        }

    auto fetch = [&](int c, uint4 (&q)[NQ], uint32_t (&sr)[NG], uint4 (&xv0)[MB], uint4 (&xv1)[MB], char *xdst) {
        const int64_t kc = kbeg + static_cast<int64_t>(c) * kX32Chunk;
        if constexpr (XD) {
            // first, so that the wait for this chunk's code loads covers the X copies too
#pragma unroll
            for (int g = 0; g < MB; ++g)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    lds_copy16(xdsrc[g][i] + kc, xdst + g * kX32Stage + (2 * wave + i) * 1024);
        } else {
#pragma unroll
            for (int g = 0; g < MB; ++g) {
                xv0[g] = *reinterpret_cast<const uint4 *>(xrow0[g] + kc);
                xv1[g] = *reinterpret_cast<const uint4 *>(xrow1[g] + kc);
            }
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if constexpr (CS) q[j] = load_stream16(ccp[j] + (kc >> 1));
            else q[j] = *reinterpret_cast<const uint4 *>(crow + (kc >> 1) + 16 * j);
        }
        const int64_t g0 = (kc >> 6) + 2 * half + (KH == 2 ? kh : 0);
#pragma unroll
        for (int j = 0; j < NG; ++j) sr[j] = srow[(g0 + j) * srb];
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage_x = [&](char *st, char *cs, const uint4 (&q)[NQ], const uint4 (&xv0)[MB], const uint4 (&xv1)[MB]) {
        if constexpr (!XD) {
#pragma unroll
            for (int g = 0; g < MB; ++g) {
                *reinterpret_cast<uint4 *>(st + g * kX32Stage + xoff0) = xv0[g];
                *reinterpret_cast<uint4 *>(st + g * kX32Stage + xoff1) = xv1[g];
            }
        }
        if constexpr (CS) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) *reinterpret_cast<uint4 *>(cs + coff[j]) = q[j];
        }
    };
    f32x16 acc[MB];
#pragma unroll
    for (int g = 0; g < MB; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
    // Each k-step: the four pair-table reads of its code word and the X fragment
    // read are issued one step ahead (two register sets), so the LDS latency of a
    // step is covered by the previous step's multiplies and MFMA.
    uint32_t adb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) adb[i] = ad[i];
    auto compute = [&](const char *st, const char *cs, const uint4 (&qr)[NQ], const uint32_t (&sr)[NG]) {
        uint4 q[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if constexpr (CS) q[j] = *reinterpret_cast<const uint4 *>(cs + lcoff[j]);
            else q[j] = qr[j];
        }
        float sv[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) sv[j] = f16_to_f32(sr[j]);
        float2 la[4], lb[4];
        uint4 ava[MB], avb[MB];
        auto issue = [&](int t, uint32_t (&a4)[4], float2 (&l)[4], uint4 (&av)[MB]) {
            const uint4 qq = q[t >> 2];
            const uint32_t wn = rotr32((t & 3) == 0 ? qq.x : (t & 3) == 1 ? qq.y : (t & 3) == 2 ? qq.z : qq.w, 2);
            pair_addr<0>(a4[0], wn);
            pair_addr<1>(a4[1], wn);
            pair_addr<2>(a4[2], wn);
            pair_addr<3>(a4[3], wn);
#pragma unroll
            for (int i = 0; i < 4; ++i) l[i] = *reinterpret_cast<const float2 *>(tab + a4[i]);
            const int c = 16 * half + NS * kh + t;   // 16-byte chunk of k = kc + 128h + 8 (NS kh + t)
#pragma unroll
            for (int g = 0; g < MB; ++g)
                av[g] = *reinterpret_cast<const uint4 *>(st + g * kX32Stage + l32 * 512 + ((c ^ l32) << 4));
        };
        // One restored B fragment feeds the MFMAs of all MB position groups.
        auto finish = [&](int t, const float2 (&l)[4], const uint4 (&av)[MB]) {
            const float sc = sv[t >> 3];
            const uint4 bv = make_uint4(pack_bf16x2(l[0].x * sc, l[0].y * sc), pack_bf16x2(l[1].x * sc, l[1].y * sc),
                                        pack_bf16x2(l[2].x * sc, l[2].y * sc), pack_bf16x2(l[3].x * sc, l[3].y * sc));
#pragma unroll
            for (int g = 0; g < MB; ++g)
                acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[g]), as_bf16x8(bv), acc[g], 0, 0, 0);
        };
        issue(0, ad, la, ava);
#pragma unroll
        for (int t = 0; t < NS; t += 2) {
            issue(t + 1, adb, lb, avb);
            __builtin_amdgcn_sched_barrier(0);
            finish(t, la, ava);
            __builtin_amdgcn_sched_barrier(0);
            if (t + 2 < NS) issue(t + 2, ad, la, ava);
            __builtin_amdgcn_sched_barrier(0);
            finish(t + 1, lb, avb);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto sync = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    // XD without code staging: before the barrier that publishes a chunk, this wave's X
    // copies of it must be complete; they were issued first in the chunk's fetch, so
    // waiting until only its code and scale loads remain is enough.
    auto xd_ready = [&]() {
        if constexpr (XD && !CS) wait_vmcnt<NQ + NG>();
    };

    uint4 qa[NQ], qb[NQ], xa0[MB], xa1[MB], xb0[MB], xb1[MB];
    uint32_t sa[NG], sb[NG];
    __syncthreads();   // pair table complete
    // Chunk c lives in buffer A and LDS stage 0 when c is even, in B and stage 1 when odd.
    // Inside the loop the prefetch of the next chunk is unconditional (the last chunk is
    // peeled), so the compiler waits for exactly the loads of the chunk being used.  A
    // stage is rewritten only after the barrier that follows every wave's use of it.
    // With XD the next chunk's X copies go straight into the stage the previous chunk
    // used, so they are issued only after the barrier at which every wave is done with
    // that chunk; otherwise the next chunk is loaded into registers before the barrier.
    if (nch > 0) {
        fetch(0, qa, sa, xa0, xa1, xs0);
        for (int c = 0;; c += 2) {
            stage_x(xs0, cst[0], qa, xa0, xa1);
            xd_ready();
            if (c + 1 >= nch) {
                sync();
                compute(xs0, cst[0], qa, sa);
                break;
            }
            if constexpr (XD) {
                sync();
                fetch(c + 1, qb, sb, xb0, xb1, xs1);
            } else {
                fetch(c + 1, qb, sb, xb0, xb1, xs1);
                sync();
            }
            compute(xs0, cst[0], qa, sa);
            stage_x(xs1, cst[CS ? 1 : 0], qb, xb0, xb1);
            xd_ready();
            if (c + 2 >= nch) {
                sync();
                compute(xs1, cst[CS ? 1 : 0], qb, sb);
                break;
            }
            if constexpr (XD) {
                sync();
                fetch(c + 2, qa, sa, xa0, xa1, xs0);
            } else {
                fetch(c + 2, qa, sa, xa0, xa1, xs0);
                sync();
            }
            compute(xs1, cst[CS ? 1 : 0], qb, sb);
        }
    }
    if constexpr (KH == 2) {
        // The second half parks its accumulators in the X stages (4 row groups x MB
        // groups x 64 lanes x 16 floats = 16 KB per group); the first half adds them.
        __syncthreads();
        float *park = reinterpret_cast<float *>(xs0);
        if (kh == 1) {
#pragma unroll
            for (int g = 0; g < MB; ++g)
#pragma unroll
                for (int e = 0; e < 16; ++e) park[((rg * MB + g) * 16 + e) * 64 + lane] = acc[g][e];
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int g = 0; g < MB; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[g][e] += park[((rg * MB + g) * 16 + e) * 64 + lane];
    }
    // Output element e of lane l, group g: position p0 + 32 g + 8*(e/4) + 4*h + e%4, column rowt.
    if (rowt < n_out) {
#pragma unroll
        for (int g = 0; g < MB; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t p = p0 + 32 * g + 8 * (e >> 2) + 4 * half + (e & 3);
            if (p >= m) continue;
            const float v = acc[g][e];
            if (ws != nullptr) {
                ws[(static_cast<int64_t>(blockIdx.y) * m + p) * n_out + rowt] = v;
            } else if (ofmt == WSL_OUT_F32) {
                static_cast<float *>(y)[p * ldy + rowt] = v;
            } else {
                static_cast<uint16_t *>(y)[p * ldy + rowt] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
            }
        }
    }
}

// ---------------------------------------------------------------- bf16, shared X, M <= 64
// The bf16 counterpart of the shared-X kernel for up to 64 positions and k a multiple
// of 256: the weights need no restoring, so a lane's 16-byte weight load is an MFMA B
// fragment as it stands.  Same organization: 8 waves, 4 groups of 32 rows x 2 halves of
// each chunk's k-steps (128 rows per workgroup), MB groups of 32 positions sharing each
// B fragment, X staged per 256-k chunk in LDS (XOR-swizzled rows, two buffers), the
// lane's 128 bytes of weights per chunk loaded one chunk ahead, the two halves'
// accumulators summed in LDS at the end.
template <int MB>
__global__ __launch_bounds__(512) void gemm_bf16_x32_kernel(const uint16_t *__restrict__ w, int64_t n_out, int64_t k,
                                                            const uint16_t *__restrict__ x, int64_t m, int64_t ldx,
                                                            void *__restrict__ y, int ofmt, int64_t ldy,
                                                            float *__restrict__ ws, int64_t k_per_split) {
    constexpr int NQ = 8;   // 16-byte weight loads per lane per chunk (8 k-steps of 8 k)
    // Two position groups: X goes global -> LDS directly (as in the NF4 kernel), into two
    // separate stage objects; one group keeps the register staging.
    constexpr bool XD = MB == 2;
    __shared__ __attribute__((aligned(1024))) char xs0[MB * kX32Stage];
    __shared__ __attribute__((aligned(1024))) char xs1[MB * kX32Stage];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rg = wave & 3, kh = wave >> 2;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t rowt = static_cast<int64_t>(blockIdx.x) * 128 + rg * 32 + l32;
    const int64_t row = rowt < n_out ? rowt : n_out - 1;
    const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * k_per_split;
    const int64_t kend = (kbeg + k_per_split < k) ? kbeg + k_per_split : k;
    const int nch = kend > kbeg ? static_cast<int>((kend - kbeg) / kX32Chunk) : 0;
    // Lane (n, h) of wave half kh: k [kc + 128 h + 64 kh, + 64) of row n, 8 k per step.
    const uint16_t *wrow = w + row * k + 128 * half + 64 * kh;
    const int64_t p0 = static_cast<int64_t>(blockIdx.z) * 32 * MB;
    const int xi0 = tid >> 5, xi1 = xi0 + 16, xcc = tid & 31;
    const uint16_t *xrow0[MB], *xrow1[MB];
#pragma unroll
    for (int g = 0; g < MB; ++g) {
        const int64_t r0 = p0 + 32 * g + xi0, r1 = p0 + 32 * g + xi1;
        xrow0[g] = x + (r0 < m ? r0 : m - 1) * ldx + xcc * 8;
        xrow1[g] = x + (r1 < m ? r1 : m - 1) * ldx + xcc * 8;
    }
    const int xoff0 = xi0 * 512 + ((xcc ^ xi0) << 4);
    const int xoff1 = xi1 * 512 + ((xcc ^ xi1) << 4);
    // XD copies: copy i of wave w fills rows 2 (2w + i) + lane / 32 of a group's stage,
    // slot lane % 32 holding chunk slot ^ row.
    const uint16_t *xdsrc[MB][2];
#pragma unroll
    for (int g = 0; g < MB; ++g)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 2 * (2 * wave + i) + (lane >> 5);
            const int64_t pr = p0 + 32 * g + r;
            xdsrc[g][i] = x + (pr < m ? pr : m - 1) * ldx + ((l32 ^ r) << 3);
        }

    auto fetch = [&](int c, uint4 (&q)[NQ], uint4 (&xv0)[MB], uint4 (&xv1)[MB], char *xdst) {
        const int64_t kc = kbeg + static_cast<int64_t>(c) * kX32Chunk;
        if constexpr (XD) {
#pragma unroll
            for (int g = 0; g < MB; ++g)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    lds_copy16(xdsrc[g][i] + kc, xdst + g * kX32Stage + (2 * wave + i) * 1024);
        } else {
#pragma unroll
            for (int g = 0; g < MB; ++g) {
                xv0[g] = *reinterpret_cast<const uint4 *>(xrow0[g] + kc);
                xv1[g] = *reinterpret_cast<const uint4 *>(xrow1[g] + kc);
            }
        }
        // Ordinary (L1-allocating) loads: each load instruction touches 32 rows, and the
        // instructions that share a 128-byte line of a row are served by one fetch.
#pragma unroll
        for (int j = 0; j < NQ; ++j) q[j] = *reinterpret_cast<const uint4 *>(wrow + kc + 8 * j);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage_x = [&](char *st, const uint4 (&xv0)[MB], const uint4 (&xv1)[MB]) {
        if constexpr (XD) {
            // this wave's copies of the chunk were issued before its NQ weight loads:
            // once at most NQ loads are outstanding they are complete
            wait_vmcnt<NQ>();
        } else {
#pragma unroll
            for (int g = 0; g < MB; ++g) {
                *reinterpret_cast<uint4 *>(st + g * kX32Stage + xoff0) = xv0[g];
                *reinterpret_cast<uint4 *>(st + g * kX32Stage + xoff1) = xv1[g];
            }
        }
    };
    f32x16 acc[MB];
#pragma unroll
    for (int g = 0; g < MB; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
    // Step t: X chunk c = 16 h + 8 kh + t (k = kc + 128 h + 64 kh + 8 t) against weight load t;
    // the X reads of step t + 1 are issued before step t's MFMAs.
    auto compute = [&](const char *st, const uint4 (&q)[NQ]) {
        uint4 ava[MB], avb[MB];
        auto issue = [&](int t, uint4 (&av)[MB]) {
            const int c = 16 * half + 8 * kh + t;
#pragma unroll
            for (int g = 0; g < MB; ++g)
                av[g] = *reinterpret_cast<const uint4 *>(st + g * kX32Stage + l32 * 512 + ((c ^ l32) << 4));
        };
        auto finish = [&](int t, const uint4 (&av)[MB]) {
#pragma unroll
            for (int g = 0; g < MB; ++g)
                acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[g]), as_bf16x8(q[t]), acc[g], 0, 0, 0);
        };
        issue(0, ava);
#pragma unroll
        for (int t = 0; t < NQ; t += 2) {
            issue(t + 1, avb);
            __builtin_amdgcn_sched_barrier(0);
            finish(t, ava);
            __builtin_amdgcn_sched_barrier(0);
            if (t + 2 < NQ) issue(t + 2, ava);
            __builtin_amdgcn_sched_barrier(0);
            finish(t + 1, avb);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto sync = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // With XD the next chunk's copies go into the stage of the previous chunk, so they are
    // issued after the barrier at which every wave is done with it.
    uint4 qa[NQ], qb[NQ], xa0[MB], xa1[MB], xb0[MB], xb1[MB];
    if (nch > 0) {
        fetch(0, qa, xa0, xa1, xs0);
        for (int c = 0;; c += 2) {
            stage_x(xs0, xa0, xa1);
            if (c + 1 >= nch) {
                sync();
                compute(xs0, qa);
                break;
            }
            if constexpr (XD) {
                sync();
                fetch(c + 1, qb, xb0, xb1, xs1);
            } else {
                fetch(c + 1, qb, xb0, xb1, xs1);
                sync();
            }
            compute(xs0, qa);
            stage_x(xs1, xb0, xb1);
            if (c + 2 >= nch) {
                sync();
                compute(xs1, qb);
                break;
            }
            if constexpr (XD) {
                sync();
                fetch(c + 2, qa, xa0, xa1, xs0);
            } else {
                fetch(c + 2, qa, xa0, xa1, xs0);
                sync();
            }
            compute(xs1, qb);
        }
    }
    __syncthreads();
    float *park = reinterpret_cast<float *>(xs0);
    if (kh == 1) {
#pragma unroll
        for (int g = 0; g < MB; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) park[((rg * MB + g) * 16 + e) * 64 + lane] = acc[g][e];
    }
    __syncthreads();
    if (kh == 1) return;
    if (rowt < n_out) {
#pragma unroll
        for (int g = 0; g < MB; ++g)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t p = p0 + 32 * g + 8 * (e >> 2) + 4 * half + (e & 3);
                if (p >= m) continue;
                const float v = acc[g][e] + park[((rg * MB + g) * 16 + e) * 64 + lane];
                if (ws != nullptr) {
                    ws[(static_cast<int64_t>(blockIdx.y) * m + p) * n_out + rowt] = v;
                } else if (ofmt == WSL_OUT_F32) {
                    static_cast<float *>(y)[p * ldy + rowt] = v;
                } else {
                    static_cast<uint16_t *>(y)[p * ldy + rowt] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
                }
            }
    }
}

// ---------------------------------------------------------------- NF4, tiled, M > 32
// NF4 GEMM over many positions (batch verification, long prefill): the bf16
// kernel's 256 x 256 tiles, 8 waves of 128 x 64, 4-stage X ring and ping-pong
// schedule, but the weight half of each 32-k stage is restored on the way in.
// X tiles still arrive by direct global -> LDS copies three stages ahead.
// Thread t restores row t/2, k [16 (t % 2), +16) of the weight stage: its 8 code
// bytes and the group's scale are loaded three stages ahead into registers, and in
// the memory phase of stage kt the codes of stage kt + 1 are turned into
// t = bf16(fp32(level * s)) through the replicated pair table (64 KB, one ds_read_b64
// per two codes, no bank conflicts; with it the kernel's LDS is exactly 160 KB) and
// written into one of two weight slots.  Weight slots live in LDS arrays of their own, separate from the
// arrays the copies fill, so the compiler sees that these writes cannot alias
// copies in flight.  Each weight tile is restored once per 256 positions.
// Pair-table reads of the eight codes of one stored code word (rotated left by 2 in
// the device layout), issued from inline asm and not waited for.  a[i] holds the
// table's 64 KB-aligned LDS address plus this lane's copy offset; the SDWA move writes
// code byte i into its bits 8..15.  l[i] = (level(even code), level(odd code)) of
// byte i once the wait that follows (pair_landed) has passed.
__device__ __forceinline__ void pair_issue4(uint32_t wmem, uint32_t (&a)[4], f32x2 (&l)[4]) {
    const uint32_t w = rotr32(wmem, 2);
    pair_addr<0>(a[0], w);
    pair_addr<1>(a[1], w);
    pair_addr<2>(a[2], w);
    pair_addr<3>(a[3], w);
    asm volatile(
        "ds_read_b64 %0, %4\n\t"
        "ds_read_b64 %1, %5\n\t"
        "ds_read_b64 %2, %6\n\t"
        "ds_read_b64 %3, %7"
        : "=&v"(l[0]), "=&v"(l[1]), "=&v"(l[2]), "=&v"(l[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

// Wait until at most N LDS operations are outstanding (those issued after the pair
// reads of a and b), marking the eight entries as written.
template <int N>
__device__ __forceinline__ void pair_landed(f32x2 (&a)[4], f32x2 (&b)[4]) {
    static_assert(N == 0 || N == 8 || N == 12, "LDS operations issued after the pair reads");
    if constexpr (N == 0)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
    else if constexpr (N == 12)
        asm volatile("s_waitcnt lgkmcnt(12)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
    else
        asm volatile("s_waitcnt lgkmcnt(8)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]));
}

// bf16(fp32(level * s)) of the eight codes of a word, even k in the low half of each pair.
__device__ __forceinline__ uint4 scale_pairs(const f32x2 (&l)[4], float s) {
    uint4 r;
    r.x = pack_bf16x2(l[0].x * s, l[0].y * s);
    r.y = pack_bf16x2(l[1].x * s, l[1].y * s);
    r.z = pack_bf16x2(l[2].x * s, l[2].y * s);
    r.w = pack_bf16x2(l[3].x * s, l[3].y * s);
    return r;
}

// 16-byte LDS store from inline asm (the compiler then has no LDS access of its own to
// order against direct global -> LDS copies in flight, which it would drain first).
__device__ __forceinline__ void lds_store16(uint32_t addr, uint4 v) {
    const u32x4 vv = __builtin_bit_cast(u32x4, v);
    asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(vv));
}

// One workgroup tile of the NF4 GEMM: TM = 256 rows of X (each wave 128 x 64 of
// the output) or TM = 128 (each wave 64 x 64: the half tiles of a short last
// round); the restored weight tile is 256 rows either way.
template <int TM>
__device__ __forceinline__ void nf4_tile(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed, int64_t m,
                                         int64_t n_out, int64_t k, int64_t kb, int64_t kl, int64_t ldx,
                                         void *__restrict__ y, int ofmt,
                                         int64_t ldy, int64_t m0, int64_t n0, char *sa0, char *sa1, char *sa2,
                                         char *sa3, char *sb0, char *sb1, char *tab) {
    constexpr int MI = TM / 64;         // 32-row MFMA tiles per wave along m
    constexpr int NA = TM / 128;        // A wave-loads per wave per stage
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;

    const uint16_t *asrc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int row = 16 * (NA * wave + i) + (lane >> 2);
        const int c = chunk_swz(row, lane & 3);
        const int64_t gm = (m0 + row < m) ? m0 + row : m - 1;
        asrc[i] = x + gm * ldx + c * 8;
    }
    // B producer: thread t restores row t/2, k [16*(t%2), +16) of the 32-k stage.
    const int brow = tid >> 1, bhp = tid & 1;
    const int64_t gn = (n0 + brow < n_out) ? n0 + brow : n_out - 1;
    const int64_t groups = k >> 6;
    const uint8_t *crow = packed + gn * (k >> 1) + 8 * bhp;          // + k0/2
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * (k >> 1));
    const int64_t srem = n_out - ((gn >> 4) << 4);
    const int64_t srb = srem < 16 ? srem : 16;
    const uint16_t *srow = scales + (gn >> 4) * 16 * groups + (gn & 15);
    const uint32_t boff0 = static_cast<uint32_t>(swz(brow, 2 * bhp));
    const uint32_t boff1 = static_cast<uint32_t>(swz(brow, 2 * bhp + 1));
    // pair-table addresses: the table's base (64 KB-aligned) plus this lane's copy offset
    uint32_t pa[4], pb[4];
    {
        const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)tab)) +
                              (static_cast<uint32_t>(lane & 31) << 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) pa[i] = pb[i] = base;
    }

    const int64_t ktiles = kl / kBK;   // even: kl % 64 == 0
    // Loads for k-tiles past the end are clamped to the last one: they land in a
    // slot or register set nobody reads again, and keep the loop free of branches
    // around loads (with them the compiler's own waits turn conservative).
    auto tile_k0 = [&](int64_t kt) { return kb + (kt < ktiles ? kt : ktiles - 1) * kBK; };
    // The code and scale loads are issued from inline asm: the compiler does not
    // track them, so it adds no waits of its own (around the loop's back edge it
    // waited for every load in flight).  The explicit vmcnt wait of the memory phase
    // covers them; put_b then marks the registers as written.
    auto load_codes = [&](int64_t kt, u32x2 &q, uint32_t &sraw) {
        const int64_t k0 = tile_k0(kt);
        const uint8_t *cp = crow + (k0 >> 1);
        const uint16_t *sp = srow + (k0 >> 6) * srb;
        asm volatile("global_load_dwordx2 %0, %2, off\n\tglobal_load_ushort %1, %3, off"
                     : "=&v"(q), "=&v"(sraw)
                     : "v"(cp), "v"(sp));
    };
    auto copy_a = [&](int64_t kt, char *sa) {
        const int64_t k0 = tile_k0(kt);
#pragma unroll
        for (int i = 0; i < NA; ++i)
            lds_copy16(asrc[i] + k0, sa + (NA * wave + i) * 1024);
    };
    auto put_b = [&](char *sb, u32x2 &q, uint32_t &sraw) {
        asm volatile("" : "+v"(q), "+v"(sraw));   // loaded: the caller waited for them
        f32x2 la[4], lb[4];
        pair_issue4(q.x, pa, la);
        pair_issue4(q.y, pb, lb);
        pair_landed<0>(la, lb);
        const float s = f16_to_f32(sraw);
        const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)sb));
        lds_store16(base + boff0, scale_pairs(la, s));
        lds_store16(base + boff1, scale_pairs(lb, s));
    };

    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int half = lane >> 5, l32 = lane & 31;
    uint32_t offa[2], offb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        offa[ks] = static_cast<uint32_t>(swz(wm * (TM / 2) + l32, ks * 2 + half));
        offb[ks] = static_cast<uint32_t>(swz(wn * 64 + l32, ks * 2 + half));
    }
    using frags = u32x4[MI + 2];
    auto issue = [&](uint32_t a_addr, uint32_t b_addr, frags &f) {
        if constexpr (MI == 4) {
            asm volatile(
                "ds_read_b128 %0, %6\n\t"
                "ds_read_b128 %1, %6 offset:2048\n\t"
                "ds_read_b128 %2, %6 offset:4096\n\t"
                "ds_read_b128 %3, %6 offset:6144\n\t"
                "ds_read_b128 %4, %7\n\t"
                "ds_read_b128 %5, %7 offset:2048"
                : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5])
                : "v"(a_addr), "v"(b_addr));
        } else {
            asm volatile(
                "ds_read_b128 %0, %4\n\t"
                "ds_read_b128 %1, %4 offset:2048\n\t"
                "ds_read_b128 %2, %5\n\t"
                "ds_read_b128 %3, %5 offset:2048"
                : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
                : "v"(a_addr), "v"(b_addr));
        }
    };
    auto landed = [&](frags &f0, frags &f1) {
        if constexpr (MI == 4) {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f0[0]), "+v"(f0[1]), "+v"(f0[2]), "+v"(f0[3]), "+v"(f0[4]), "+v"(f0[5]),
                           "+v"(f1[0]), "+v"(f1[1]), "+v"(f1[2]), "+v"(f1[3]), "+v"(f1[4]), "+v"(f1[5]));
        } else {
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f0[0]), "+v"(f0[1]), "+v"(f0[2]), "+v"(f0[3]), "+v"(f1[0]), "+v"(f1[1]),
                           "+v"(f1[2]), "+v"(f1[3]));
        }
    };
    // The bf16 kernel's ping-pong: two groups of four waves (one of each per SIMD)
    // alternate between an MFMA phase and a memory phase, the second group one
    // barrier behind.  The memory phase of stage kt reads the stage's fragments, then
    // restores this thread's share of weight stage kt + 1 (table reads, multiplies,
    // conversions: VALU work that runs beside the other group's MFMAs) and waits for
    // its LDS writes; the barrier that ends the phase publishes that share and this
    // wave's X copy of stage kt + 1.  Weight stages need only two slots: stage kt + 1
    // goes into the slot of stage kt - 1, which both groups finished reading before
    // this phase began.  The MFMA phase of stage kt issues, among its MFMAs, the code
    // and scale loads and the X copies of k-tile kt + 3 (NV = 2 + NA vector memory
    // operations per stage); at the memory phase of stage kt only those of kt + 2 may
    // still be in flight.
    constexpr int NV = NA + 2;
    auto bar = []() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lds_addr = [](char *p) { return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p)); };
    const uint32_t A0 = lds_addr(sa0), A1 = lds_addr(sa1), A2 = lds_addr(sa2), A3 = lds_addr(sa3);
    const uint32_t B0 = lds_addr(sb0), B1 = lds_addr(sb1);
    u32x2 q0, q1, q2, q3;
    uint32_t r0, r1, r2, r3;
    frags f0, f1;
    auto stage = [&](int64_t kt, uint32_t acur, uint32_t bcur, char *bnext, u32x2 &qnext, uint32_t &rnext,
                     char *arefill, u32x2 &qload, uint32_t &rload) {
        // codes of stage kt + 1 landed; their pair-table reads go ahead of the fragment
        // reads, and the multiplies and conversions run while those are in flight
        wait_vmcnt<NV>();
        asm volatile("" : "+v"(qnext), "+v"(rnext));
        f32x2 la[4], lb[4];
        pair_issue4(qnext.x, pa, la);
        pair_issue4(qnext.y, pb, lb);
        issue(acur + offa[0], bcur + offb[0], f0);
        issue(acur + offa[1], bcur + offb[1], f1);
        pair_landed<2 * (MI + 2)>(la, lb);
        {
            const float sc = f16_to_f32(rnext);
            const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)bnext));
            lds_store16(base + boff0, scale_pairs(la, sc));
            lds_store16(base + boff1, scale_pairs(lb, sc));
        }
        landed(f0, f1);
        bar();
        constexpr int MF = 2 * MI;   // MFMAs per 16-k step
        constexpr int NP = NA + 1;   // load pieces: the codes and scale, then the X copies
        int q = 0;
#pragma unroll
        for (int t = 0; t < 2 * MF; ++t) {
            const int i = (t % MF) >> 1, j = t & 1;
            const frags &f = t < MF ? f0 : f1;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f[i]),
                                                                __builtin_bit_cast(bf16x8, f[MI + j]), acc[i][j], 0, 0, 0);
            if (q < NP && t + 1 == (q + 1) * 2 * MF / (NP + 1)) {
                __builtin_amdgcn_sched_barrier(0);
                if (q == 0) load_codes(kt + 3, qload, rload);
                else lds_copy16(asrc[q - 1] + tile_k0(kt + 3), arefill + (NA * wave + q - 1) * 1024);
                __builtin_amdgcn_sched_barrier(0);
                ++q;
            }
        }
        bar();
    };
    const int group = static_cast<int>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(wave))) >> 2;
    __syncthreads();   // pair table
    load_codes(0, q0, r0);
    copy_a(0, sa0);
    load_codes(1, q1, r1);
    copy_a(1, sa1);
    load_codes(2, q2, r2);
    copy_a(2, sa2);
    wait_vmcnt<2 * NV>();
    put_b(sb0, q0, r0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bar();                   // weight stage 0 and X stage 0 in LDS
    if (group != 0) bar();   // the second group runs one phase behind
    int64_t kt = 0;
    for (; kt + 4 <= ktiles; kt += 4) {
        stage(kt + 0, A0, B0, sb1, q1, r1, sa3, q3, r3);
        stage(kt + 1, A1, B1, sb0, q2, r2, sa0, q0, r0);
        stage(kt + 2, A2, B0, sb1, q3, r3, sa1, q1, r1);
        stage(kt + 3, A3, B1, sb0, q0, r0, sa2, q2, r2);
    }
    if (kt + 0 < ktiles) stage(kt + 0, A0, B0, sb1, q1, r1, sa3, q3, r3);
    if (kt + 1 < ktiles) stage(kt + 1, A1, B1, sb0, q2, r2, sa0, q0, r0);
    if (kt + 2 < ktiles) stage(kt + 2, A2, B0, sb1, q3, r3, sa1, q1, r1);
    if (group == 0) bar();   // both groups pass the same number of barriers
    // The last stages' code loads (clamped, never used) may still be in flight: keep
    // their registers allocated until they have landed.
    wait_vmcnt<0>();
    asm volatile("" : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3), "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3));
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + l32;
            if (col >= n_out) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * (TM / 2) + i * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
                if (row >= m) continue;
                if (ofmt == WSL_OUT_F32) static_cast<float *>(y)[row * ldy + col] = acc[i][j][e];
                else static_cast<uint16_t *>(y)[row * ldy + col] = static_cast<uint16_t>(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
            }
        }
}

__global__ __launch_bounds__(512) void gemm_nf4_tiled_kernel(const uint16_t *__restrict__ x, const uint8_t *__restrict__ packed,
                                                      int64_t m, int64_t n_out, int64_t k, int64_t ldx,
                                                      void *__restrict__ y, int ofmt, int64_t ldy, int tiles_m, int tiles_n,
                                                      int nx, int xcd_cus, int splits, int64_t kps,
                                                      float *__restrict__ ws, int half_only) {
    constexpr int kHalf = kBM * kBK * 2;   // 16 KB per operand per stage
    __shared__ __attribute__((aligned(1024))) char sa0[kHalf];
    __shared__ __attribute__((aligned(1024))) char sa1[kHalf];
    __shared__ __attribute__((aligned(1024))) char sa2[kHalf];
    __shared__ __attribute__((aligned(1024))) char sa3[kHalf];
    __shared__ __attribute__((aligned(1024))) char sb0[kHalf];
    __shared__ __attribute__((aligned(1024))) char sb1[kHalf];
    __shared__ __attribute__((aligned(65536))) char tab[kPairTableBytes];   // bits 8..15 of its address are 0
    TileItem it;
    if (!tile_item(tiles_m, tiles_n * splits, splits, nx, xcd_cus, half_only == 0, it) || it.m0 >= m) return;
    if (half_only) it.half = 0;
    fill_pair_table(tab);
    const SplitOut o = split_out(it.split, kps, k, m, n_out, y, ofmt, ldy, ws);
    if (it.half < 0)
        nf4_tile<256>(x, packed, m, n_out, k, o.kb, o.kl, ldx, o.y, o.ofmt, o.ldy, it.m0, it.n0, sa0, sa1, sa2, sa3,
                      sb0, sb1, tab);
    else
        nf4_tile<128>(x, packed, m, n_out, k, o.kb, o.kl, ldx, o.y, o.ofmt, o.ldy, it.m0, it.n0, sa0, sa1, sa2, sa3,
                      sb0, sb1, tab);
}

// Sum split partials in split order (fixed, so the result is deterministic).  A
// thread takes 4 consecutive outputs of one row (n_out % 4 == 0; one output
// otherwise) and issues the loads of up to 8 splits before adding them, so their
// latencies overlap instead of adding up.
__device__ __forceinline__ void store_out(void *y, int ofmt, int64_t idx, float v) {
    if (ofmt == WSL_OUT_F32) static_cast<float *>(y)[idx] = v;
    else static_cast<uint16_t *>(y)[idx] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
}

__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ ws, int splits, int64_t m,
                                                           int64_t n_out, void *__restrict__ y, int ofmt, int64_t ldy) {
    const int64_t total = m * n_out;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    if ((n_out & 3) == 0) {
        const float4 *w4 = reinterpret_cast<const float4 *>(ws);
        const int64_t t4 = total >> 2;
        for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < t4; i += stride) {
            float4 v = w4[i];
            for (int s0 = 1; s0 < splits; s0 += 8) {
                float4 t[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < splits) t[j] = w4[static_cast<int64_t>(s0 + j) * t4 + i];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (s0 + j < splits) {
                        v.x += t[j].x;
                        v.y += t[j].y;
                        v.z += t[j].z;
                        v.w += t[j].w;
                    }
            }
            const int64_t e = i << 2, row = e / n_out, col = e - row * n_out;
            const int64_t o = row * ldy + col;
            store_out(y, ofmt, o, v.x);
            store_out(y, ofmt, o + 1, v.y);
            store_out(y, ofmt, o + 2, v.z);
            store_out(y, ofmt, o + 3, v.w);
        }
        return;
    }
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
        float v = ws[i];
        for (int s0 = 1; s0 < splits; s0 += 8) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < splits) t[j] = ws[static_cast<int64_t>(s0 + j) * total + i];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < splits) v += t[j];
        }
        const int64_t row = i / n_out, col = i - row * n_out;
        store_out(y, ofmt, row * ldy + col, v);
    }
}

// ---------------------------------------------------------------- planning / launch
// NF4 GEMM plans.  M > 32: the tiled kernel (no workspace).  M <= 32 with
// k % 256 == 0: the shared-X kernel, 256 rows per workgroup (one workgroup per
// CU: 96 KB of LDS), k split into as many ranges of whole 256-k chunks as keep
// the grid within one pass over the 256 CUs.  Otherwise the general kernel:
// NB = 1 (32 rows per wave), 4 waves per workgroup, 32 positions per grid z, k
// split (multiples of 128) as far as needed for about 2 waves per SIMD.  Splits
// need the caller's workspace.
constexpr int kNf4Nb = 1;
constexpr int64_t kNf4RowsPerWg = 4 * 32 * kNf4Nb;

// k split of the tiled kernels.  When the 256 x 256 tiles of a launch would leave more
// than half of the 256 CUs idle, k (a multiple of 256) is split into s ranges, one work
// item per (tile, range), up to one round over the CUs: each item reads, or restores, only
// its own k range of the weights, so no weight is read twice, and the fp32 partials
// (s * M * N * 4 bytes of workspace) are summed in split order by split_reduce_kernel.
// s minimises a time model: t_full per unit of k for a round of full tiles, t_half for a
// last round of at most 128 tiles run as halves (unsplit launches only), and for a split
// the partials written and read back and the output written, at 5 TB/s, plus 3 us for the
// reduction's launch and the shorter k loops' pipeline ramp; every range is at least 512
// long.  With M <= 128 the split items may also be half tiles (128 rows: no MFMA work on
// rows past M), a round of which takes t_half per unit of k.
struct TiledPlan {
    int splits;
    int64_t kps;   // k per split (k when unsplit)
    double t;      // modelled seconds
    bool half;     // every item a 128-row half tile
};
static TiledPlan tiled_plan(int64_t n_out, int64_t k, int64_t m, double t_full, double t_half) {
    const int64_t tiles = ((m + kBM - 1) / kBM) * ((n_out + kBN - 1) / kBN);
    const int64_t full = tiles / 256, tail = tiles % 256;
    double per_k = static_cast<double>(full) * t_full;
    if (tail > 0) per_k += tail <= 128 ? t_half : t_full;
    TiledPlan best{1, k, per_k * static_cast<double>(k), false};
    if (k % 256 != 0 || 2 * tiles > 256) return best;
    const int64_t units = k / 256;
    const double out = static_cast<double>(m) * static_cast<double>(n_out) * 4.0;
    for (int64_t sp = 2; sp <= 64 && sp * tiles <= 256 && 2 * sp <= units; ++sp) {
        const int64_t kps = ((units + sp - 1) / sp) * 256;
        const int64_t used = (k + kps - 1) / kps;   // no empty trailing range
        const double extra = static_cast<double>(2 * used + 1) * out / 5e12 + 3e-6;
        const double t = t_full * static_cast<double>(kps) + extra;
        if (t < best.t) best = TiledPlan{static_cast<int>(used), kps, t, false};
        const double th = t_half * static_cast<double>(kps) + extra;
        if (m <= kBM / 2 && th < best.t) best = TiledPlan{static_cast<int>(used), kps, th, true};
    }
    return best;
}
static TiledPlan nf4_tiled_plan(int64_t n_out, int64_t k, int64_t m) { return tiled_plan(n_out, k, m, 33e-9, 23.5e-9); }
static TiledPlan bf16_tiled_plan(int64_t n_out, int64_t k, int64_t m) { return tiled_plan(n_out, k, m, 30e-9, 21e-9); }

// k a multiple of 256: the shared-X kernel for M <= 32; above that, the shared-X or the
// tiled kernel, whichever a time model fitted to MI355X measurements puts first.  The
// shared-X kernel streams the packed weights once per 64 positions at about 1.7 TB/s; a
// round of 256 x 256 tiles (one workgroup per CU) takes about 33 ns per unit of k, and a
// last round of at most 128 tiles, which runs as half tiles, about 23.5 ns; a k split
// (tiled_plan) shortens a sparse round.  Measured (us): 27648x5120 M = 64 127 tiled / 42
// shared-X; M = 128 84 shared-X, 74 as half tiles with 2 k ranges (5120x27648: 77 / 65
// with 12); M = 256 121 tiled, 112 as halves, 101.5 with 2 k ranges, 158 shared-X;
// 5120x27648 M = 256 608 tiled, 197 shared-X, 94.5 with 12 k ranges; M = 512 381
// shared-X, 158.5 with 6; M = 1024 565 / 293 with 3; 5120x17408, 17408x5120 and
// 6144x16384 at M = 256 127 / 119 / 121 shared-X or halves, 70 / 75 / 76 split.  Other k:
// the tiled kernel for M > 32, the general kernel for M <= 32.
static bool x32_faster(int64_t n_out, int64_t k, int64_t m) {
    const double packed = static_cast<double>(n_out) * static_cast<double>(k / 2 + (k / 64) * 2);
    const double t_x32 = static_cast<double>((m + 63) / 64) * packed / 1.7e12;
    return t_x32 <= nf4_tiled_plan(n_out, k, m).t;
}
static bool use_x32(int64_t n_out, int64_t k, int64_t m) {
    return (k % kX32Chunk) == 0 && (m <= 32 || x32_faster(n_out, k, m));
}
static bool use_tiled(int64_t n_out, int64_t k, int64_t m) { return m > 32 && !use_x32(n_out, k, m); }
// The shared-X kernel always runs its 128-row form (KH = 2), with MB = 2 groups of 32
// positions per workgroup when M > 32 (one restored weight fragment feeds both groups'
// MFMAs) and further position blocks on grid z; k is split into as many ranges as keep
// the grid within one pass over the 256 CUs.  Measured at M = 32: 27648x5120 32.6 us
// unsplit against 38.7 us for the 256-row form with 2 splits; 5120x27648 32.9 us with
// 6 splits against 38.2 us for the 256-row form with 12.
constexpr int kX32Kh = 2;
constexpr int64_t kX32BlockRows = 256 / kX32Kh;
static int x32_mb(int64_t m) { return m > 32 ? 2 : 1; }
static int64_t x32_zblocks(int64_t m) { return (m + 32 * x32_mb(m) - 1) / (32 * x32_mb(m)); }

// k split of the shared-X kernels (NF4 and bf16): as many ranges of whole 256-k chunks as
// keep the grid within one pass over the 256 CUs.
static int x32_splits(int64_t n_out, int64_t k, int64_t m) {
    const int64_t blocks = (n_out + kX32BlockRows - 1) / kX32BlockRows * x32_zblocks(m);
    const int64_t chunks = k / kX32Chunk;
    int64_t splits = 256 / blocks;
    if (splits < 1) splits = 1;
    if (splits > chunks) splits = chunks;
    if (splits > 64) splits = 64;
    return static_cast<int>(splits);
}

static int nf4_splits(int64_t n_out, int64_t k, int64_t m) {
    if (use_tiled(n_out, k, m)) return nf4_tiled_plan(n_out, k, m).splits;
    if (use_x32(n_out, k, m)) return x32_splits(n_out, k, m);
    const int64_t waves = ((n_out + 32 * kNf4Nb - 1) / (32 * kNf4Nb)) * ((m + 31) / 32);
    const int64_t chunks = (k + 127) / 128;
    int64_t splits = 1;
    while (waves * splits < 2048 && splits * 2 * 4 <= chunks && splits < 16) splits *= 2;
    return static_cast<int>(splits);
}

static int64_t nf4_k_per_split(int64_t n_out, int64_t k, int64_t m, int splits) {
    const int64_t unit = use_x32(n_out, k, m) ? kX32Chunk : 128;
    const int64_t chunks = (k + unit - 1) / unit;
    return ((chunks + splits - 1) / splits) * unit;
}

// bf16, k a multiple of 256: the shared-X kernel for M <= 32; above that, the same kind of
// time model as for NF4, fitted to bf16 measurements: every 64 positions re-stream the
// 2-byte weights at about 3.6 TB/s; a round of 256 x 256 tiles takes about 30 ns per unit
// of k, a last round of at most 128 (half) tiles about 21 ns, and a k split shortens a
// sparse round.  Measured (us): 27648x5120 M = 64 106 tiled, 85 with 2 k ranges, 78
// shared-X, 75 as half tiles with 2; M = 128 117 shared-X, 95 split, 89.5 as halves;
// 5120x27648 M = 128 474 tiled, 115 shared-X, 88 with 12 ranges, 78 as halves; M = 256 443 / 291 / 103; M = 512 446 tiled, 491 shared-X, 159 with 6;
// 5120x17408 M = 256 187 shared-X, 76 split; 1000x16384 M = 1000 91 / 59.  Other k: tiled.
static bool bf16_x32_faster(int64_t n_out, int64_t k, int64_t m) {
    const double bytes = 2.0 * static_cast<double>(n_out) * static_cast<double>(k);
    const double t_x32 = static_cast<double>((m + 63) / 64) * bytes / 3.6e12;
    return t_x32 <= bf16_tiled_plan(n_out, k, m).t;
}
static bool use_bf16_x32(int64_t n_out, int64_t k, int64_t m) {
    return (k % kX32Chunk) == 0 && (m <= 32 || bf16_x32_faster(n_out, k, m));
}
static int bf16_splits(int64_t n_out, int64_t k, int64_t m) {
    return use_bf16_x32(n_out, k, m) ? x32_splits(n_out, k, m) : bf16_tiled_plan(n_out, k, m).splits;
}

size_t gemm_ws_bytes(int wfmt, int64_t n_out, int64_t k, int64_t m) {
    const int splits = wfmt == WSL_W_NF4 ? nf4_splits(n_out, k, m) : bf16_splits(n_out, k, m);
    if (splits <= 1) return 0;
    return static_cast<size_t>(splits) * static_cast<size_t>(m) * static_cast<size_t>(n_out) * sizeof(float);
}

// CUs per XCD of the current device (one workgroup of the tiled kernels per CU),
// cached per device; 32 on MI355X (256 CUs in 8 XCDs).
// The device's XCDs and compute units per XCD (queried once per device): workgroup b
// is dispatched to XCD b % nx.
struct XcdShape {
    int nx, cus;   // XCDs; compute units per XCD
};
static XcdShape xcd_shape() {
    constexpr int kDevs = 64;
    static std::atomic<int> cache[kDevs];   // nx << 16 | cus, 0 until queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return XcdShape{8, 32};
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, nx = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
        if (hipDeviceGetAttribute(&nx, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || nx < 1) nx = 1;
        if (nx > 64) nx = 64;
        const int per = cus / nx > 0 ? cus / nx : 1;
        v = (nx << 16) | per;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return XcdShape{v >> 16, v & 0xffff};
}

// Grid of the tiled kernels: 8 XCDs times the largest per-XCD item count (whole
// tiles plus the half tiles of a short last round), as tile_item() assigns them.
static unsigned tile_grid(int64_t ntiles, const XcdShape &xs) {
    int64_t most = 0;
    for (int x = 0; x < xs.nx; ++x) {
        const int64_t count = ntiles / xs.nx + (x < ntiles % xs.nx ? 1 : 0);
        const int64_t r = count % xs.cus;
        const int64_t items = count + ((r > 0 && 2 * r <= xs.cus) ? r : 0);
        if (items > most) most = items;
    }
    return static_cast<unsigned>(xs.nx * most);
}

static void launch_split_reduce(const float *wsp, int splits, int64_t m, int64_t n_out, void *y, int ofmt,
                                int64_t ldy, hipStream_t s) {
    const int64_t items = (n_out % 4 == 0) ? m * n_out / 4 : m * n_out;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, wsp, splits, m,
                       n_out, y, ofmt, ldy);
}

// The tiled kernels' plan for a launch: the modelled split, or none when the caller's
// workspace cannot hold its partials.
static TiledPlan tiled_launch_plan(int wfmt, int64_t n_out, int64_t k, int64_t m, const void *ws, size_t ws_bytes) {
    TiledPlan pl = wfmt == WSL_W_NF4 ? nf4_tiled_plan(n_out, k, m) : bf16_tiled_plan(n_out, k, m);
    const size_t need = static_cast<size_t>(pl.splits) * static_cast<size_t>(m) * static_cast<size_t>(n_out) * 4;
    if (pl.splits > 1 && (ws == nullptr || ws_bytes < need)) pl = TiledPlan{1, k, pl.t, false};
    return pl;
}

int launch_gemm_bf16(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                     int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s) {
    const auto *wp = static_cast<const uint16_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    if (!use_bf16_x32(n_out, k, m)) {
        const int64_t tn = (n_out + kBN - 1) / kBN, tm = (m + kBM - 1) / kBM;
        const TiledPlan pl = tiled_launch_plan(WSL_W_BF16, n_out, k, m, ws, ws_bytes);
        if (tn * tm * pl.splits > 0x7fffffff / 4) return WSL_E_SHAPE;
        float *wsp = pl.splits > 1 ? static_cast<float *>(ws) : nullptr;
        const XcdShape xs = xcd_shape();
        hipLaunchKernelGGL(gemm_bf16_kernel, dim3(tile_grid(tm * tn * pl.splits, xs)), dim3(512), 0, s, xp, wp, m,
                           n_out, k, ldx, y, ofmt, ldy, static_cast<int>(tm), static_cast<int>(tn), xs.nx, xs.cus,
                           pl.splits, pl.kps, wsp, pl.half ? 1 : 0);
        if (pl.splits > 1) launch_split_reduce(wsp, pl.splits, m, n_out, y, ofmt, ldy, s);
        return WSL_OK;
    }
    int splits = bf16_splits(n_out, k, m);
    if (splits > 1 && (ws == nullptr || ws_bytes < gemm_ws_bytes(WSL_W_BF16, n_out, k, m))) splits = 1;
    const int64_t chunks = k / kX32Chunk;
    const int64_t kps = ((chunks + splits - 1) / splits) * kX32Chunk;
    splits = static_cast<int>((k + kps - 1) / kps);   // no empty trailing split
    float *wsp = splits > 1 ? static_cast<float *>(ws) : nullptr;
    const int64_t gx = (n_out + kX32BlockRows - 1) / kX32BlockRows;
    if (gx > 0x7fffffff) return WSL_E_SHAPE;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(splits), static_cast<unsigned>(x32_zblocks(m)));
    if (x32_mb(m) == 2)
        hipLaunchKernelGGL((gemm_bf16_x32_kernel<2>), grid, dim3(512), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy,
                           wsp, kps);
    else
        hipLaunchKernelGGL((gemm_bf16_x32_kernel<1>), grid, dim3(512), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy,
                           wsp, kps);
    if (splits > 1) launch_split_reduce(wsp, splits, m, n_out, y, ofmt, ldy, s);
    return WSL_OK;
}

int launch_gemm_nf4(const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx, void *y,
                    int ofmt, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t s) {
    if (use_tiled(n_out, k, m)) {
        const int64_t tn = (n_out + kBN - 1) / kBN, tm = (m + kBM - 1) / kBM;
        const TiledPlan pl = tiled_launch_plan(WSL_W_NF4, n_out, k, m, ws, ws_bytes);
        if (tn * tm * pl.splits > 0x7fffffff / 4) return WSL_E_SHAPE;
        float *wsp = pl.splits > 1 ? static_cast<float *>(ws) : nullptr;
        const XcdShape xs = xcd_shape();
        hipLaunchKernelGGL(gemm_nf4_tiled_kernel, dim3(tile_grid(tm * tn * pl.splits, xs)), dim3(512), 0, s,
                           static_cast<const uint16_t *>(x), static_cast<const uint8_t *>(w), m, n_out, k, ldx, y,
                           ofmt, ldy, static_cast<int>(tm), static_cast<int>(tn), xs.nx, xs.cus, pl.splits, pl.kps,
                           wsp, pl.half ? 1 : 0);
        if (pl.splits > 1) launch_split_reduce(wsp, pl.splits, m, n_out, y, ofmt, ldy, s);
        return WSL_OK;
    }
    int splits = nf4_splits(n_out, k, m);
    if (splits > 1 && (ws == nullptr || ws_bytes < gemm_ws_bytes(WSL_W_NF4, n_out, k, m))) splits = 1;
    int64_t kps = nf4_k_per_split(n_out, k, m, splits);
    splits = static_cast<int>((k + kps - 1) / kps);   // no empty trailing split
    float *wsp = splits > 1 ? static_cast<float *>(ws) : nullptr;
    const auto *wp = static_cast<const uint8_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    if (use_x32(n_out, k, m)) {
        const int64_t gx = (n_out + kX32BlockRows - 1) / kX32BlockRows;
        if (gx > 0x7fffffff) return WSL_E_SHAPE;
        const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(splits), static_cast<unsigned>(x32_zblocks(m)));
        // one position block: codes staged through LDS from streaming loads
        if (x32_zblocks(m) == 1) {
            if (x32_mb(m) == 2)
                hipLaunchKernelGGL((gemm_nf4_x32_kernel<kX32Kh, 2, 1>), grid, dim3(512), 0, s, wp, n_out, k, xp, m, ldx,
                                   y, ofmt, ldy, wsp, kps);
            else
                hipLaunchKernelGGL((gemm_nf4_x32_kernel<kX32Kh, 1, 1>), grid, dim3(512), 0, s, wp, n_out, k, xp, m, ldx,
                                   y, ofmt, ldy, wsp, kps);
        } else {
            hipLaunchKernelGGL((gemm_nf4_x32_kernel<kX32Kh, 2, 0>), grid, dim3(512), 0, s, wp, n_out, k, xp, m, ldx, y,
                               ofmt, ldy, wsp, kps);
        }
    } else {
        const int64_t gx = (n_out + kNf4RowsPerWg - 1) / kNf4RowsPerWg;
        const int64_t gz = (m + 31) / 32;
        if (gx > 0x7fffffff || gz > 65535) return WSL_E_SHAPE;
        const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(splits), static_cast<unsigned>(gz));
        hipLaunchKernelGGL((gemm_nf4_kernel<kNf4Nb>), grid, dim3(256), 0, s, wp, n_out, k, xp, m, ldx, y, ofmt, ldy,
                           wsp, kps);
    }
    if (splits > 1) launch_split_reduce(wsp, splits, m, n_out, y, ofmt, ldy, s);
    return WSL_OK;
}

// ---------------------------------------------------------------- no-allocation variant
// Split partials of linear_gemm_noalloc live in this array: one copy per device, created
// with the code object when the library is first used on that device.  In host code its
// name stands for a host-side shadow, not a device address, so kernels only ever receive
// the address hipGetSymbolAddress returns for the current device.
namespace {
constexpr size_t kScratchBytes = WSL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kScratchDevs = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevs];
}  // namespace

// Device address of this device's scratch, looked up once per device (with that device
// current) and kept.
static int scratch_ptr(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevs) return WSL_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return WSL_E_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return WSL_OK;
}

// linear_gemm with the split partials in the scratch array.  The split kernels write
// every partial before split_reduce_kernel reads it, so nothing needs clearing.
int launch_gemm_noalloc(int wfmt, const void *w, int64_t n_out, int64_t k, const void *x, int64_t m, int64_t ldx,
                        void *y, int ofmt, int64_t ldy, hipStream_t s) {
    size_t need = gemm_ws_bytes(wfmt, n_out, k, m);
    if (need > kScratchBytes) {
        // a k split of the tiled kernels only saves time: without room they run unsplit
        const bool tiled = wfmt == WSL_W_NF4 ? use_tiled(n_out, k, m) : !use_bf16_x32(n_out, k, m);
        if (!tiled) return WSL_E_SCRATCH;
        need = 0;
    }
    void *ws = nullptr;
    if (need > 0) {
        const int rc = scratch_ptr(&ws);
        if (rc != WSL_OK) return rc;
    }
    if (wfmt == WSL_W_NF4) return launch_gemm_nf4(w, n_out, k, x, m, ldx, y, ofmt, ldy, ws, need, s);
    return launch_gemm_bf16(w, n_out, k, x, m, ldx, y, ofmt, ldy, ws, need, s);
}

}  // namespace wsl
