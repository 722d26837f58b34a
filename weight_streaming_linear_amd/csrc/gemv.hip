// Decode GEMV y = W x for gfx950: bf16 weights or packed NF4 weights.
//
// deep-fold README, "Метод" table: decode runs an N=1 NF4 GEMV, with codes and
// scales resident in video memory and restored in registers only for the
// fragment being multiplied.  TCPP README, "What exact means here": bf16 weights
// are used as stored.  The work is a pure weight stream (each weight byte is
// read once and feeds one multiply-add), so both kernels are built around HBM:
//   * a wavefront reads 1 KB of one row per step (64 lanes x 16-byte
//     non-temporal loads) and keeps several rows in flight;
//   * the waves of a workgroup split the k range of the same rows; each wave
//     folds its per-row sums across lanes with a transposed reduction
//     (v_permlane32_swap, v_permlane16_swap, then DPP inside 16 or 8 lanes),
//     and the per-wave partials meet in LDS in a fixed order -- deterministic,
//     no atomics;
//   * x (<= 64 KB) is read through the cache hierarchy;
//   * NF4 codes become fp32 levels through a table in LDS.  Small matrices use
//     a 16-entry table (one read per code; the device layout's 2-bit word
//     rotation makes the byte address a single SDWA AND); large ones a 64 KB
//     table of level pairs indexed by a whole code byte and replicated per
//     lane so that no read ever meets a bank conflict (one 8-byte read per
//     two codes, about half the VALU work per code).  With the loads
//     prefetched one row group ahead, the lookups and multiply-adds are what
//     bounds the NF4 kernel, not HBM.
#include <atomic>
#include <type_traits>

#include "device_common.h"

namespace wsl {

// Global-address-space qualifier for pointers the kernels read back from memory.
#define WSL_GLOBAL __attribute__((address_space(1)))

constexpr int kMaxWaves = 8;

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float as_f(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ uint32_t as_u(float v) { return __builtin_bit_cast(uint32_t, v); }

// DPP controls (gfx9): quad_perm(1,0,3,2) = 0xB1, quad_perm(2,3,0,1) = 0x4E,
// row_half_mirror = 0x141, row_ror:8 = 0x128.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f(__builtin_amdgcn_update_dpp(0u, as_u(v), CTRL, 0xF, 0xF, false));
}

// Sum inside groups of 8 consecutive lanes (every lane of the group gets the sum).
__device__ __forceinline__ float sum8(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    return v;
}

// Exchange halves of the wave (lanes 32-63 of a with lanes 0-31 of b) and add:
// lanes 0-31 get a[l] + a[l+32], lanes 32-63 get b[l-32] + b[l].
__device__ __forceinline__ float fold32(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
    return as_f(r[0]) + as_f(r[1]);
}
// The same between 16-lane rows: rows 0/2 keep a (plus a's rows 1/3), rows 1/3 keep b
// (plus b's rows 0/2).
__device__ __forceinline__ float fold16(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(as_u(a), as_u(b), false, false);
    return as_f(r[0]) + as_f(r[1]);
}

// Transposed reduction of R per-lane partial sums over the 64 lanes.  Afterwards
// every lane holds the total of row (lane / (64 / R)).
template <int R>
__device__ __forceinline__ float reduce_rows(const float (&a)[R], int lane) {
    if constexpr (R == 1) {
        float v = fold32(a[0], a[0]);
        v = fold16(v, v);
        v = sum8(v);
        return v + dpp<0x128>(v);
    } else if constexpr (R == 2) {
        float v = fold32(a[0], a[1]);          // lanes 0-31: row 0, 32-63: row 1
        v = fold16(v, v);
        v = sum8(v);
        return v + dpp<0x128>(v);
    } else if constexpr (R == 4) {
        const float b0 = fold32(a[0], a[2]);   // lanes 0-31: row 0, 32-63: row 2
        const float b1 = fold32(a[1], a[3]);   // lanes 0-31: row 1, 32-63: row 3
        float v = fold16(b0, b1);              // 16-lane rows: rows 0, 1, 2, 3
        v = sum8(v);
        return v + dpp<0x128>(v);
    } else {
        static_assert(R == 8, "R must be 1, 2, 4 or 8");
        const float b0 = fold32(a[0], a[4]), b1 = fold32(a[1], a[5]);
        const float b2 = fold32(a[2], a[6]), b3 = fold32(a[3], a[7]);
        const float c0 = fold16(b0, b2);       // 16-lane rows: rows 0, 2, 4, 6
        const float c1 = fold16(b1, b3);       // 16-lane rows: rows 1, 3, 5, 7
        const bool lo = (lane & 15) < 8;
        const float t = lo ? c1 : c0;
        const float d = (lo ? c0 : c1) + dpp<0x128>(t);   // 8-lane groups: rows 0..7 in order
        return sum8(d);
    }
}

// The team GEMV's reduction of two rows (fewer instructions than reduce_rows<2>): the
// halves are exchanged and added (lanes 0-31 row 0, 32-63 row 1), summed in groups of 8
// and then of 16 lanes (DPP), and the last lane of each 16-lane row adds the last lane of
// the row before it (DPP row broadcast into rows 1 and 3).  Only lanes 31 and 63 end
// with their row's total (rows 0 and 1).
constexpr int kTwoRowsLastLane = 31;
__device__ __forceinline__ float reduce_two_rows_last(float a0, float a1) {
    float v = fold32(a0, a1);
    v = sum8(v);
    v += as_f(__builtin_amdgcn_update_dpp(0u, as_u(v), 0x128, 0xF, 0xF, true));   // row_ror:8
    v += as_f(__builtin_amdgcn_update_dpp(0u, as_u(v), 0x142, 0xA, 0xF, true));   // row_bcast:15, rows 1 and 3
    return v;
}

// Per-lane partial sums of a team step -> this wave's row totals, and whether this lane
// holds one (row lane / (64 / R)).
template <int R>
__device__ __forceinline__ float team_reduce(const float (&acc)[R], int lane, bool &holder) {
    constexpr int span = 64 / R;
    if constexpr (R == 2) {
        holder = (lane % span) == kTwoRowsLastLane;
        return reduce_two_rows_last(acc[0], acc[1]);
    } else {
        holder = (lane % span) == 0;
        return reduce_rows<R>(acc, lane);
    }
}

// Fold the waves' row sums (LDS, fixed wave order) and store y.
template <int R>
__device__ __forceinline__ void finish_rows(const float (&acc)[R], float (*red)[R], int lane, int wave, int waves,
                                            int64_t row0, int64_t n_out, float *__restrict__ y) {
    const float v = reduce_rows<R>(acc, lane);
    constexpr int span = 64 / R;
    if ((lane % span) == 0) red[wave][lane / span] = v;
    __syncthreads();
    if (threadIdx.x < R) {
        float s = red[0][threadIdx.x];
        for (int w = 1; w < waves; ++w) s += red[w][threadIdx.x];
        if (row0 + threadIdx.x < n_out) y[row0 + threadIdx.x] = s;
    }
}

// ---------------------------------------------------------------- bf16
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// c + a.lo*b.lo + a.hi*b.hi with fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot8(const uint4 &w, const uint4 &x, float a) {
    a = dot2(w.x, x.x, a);
    a = dot2(w.y, x.y, a);
    a = dot2(w.z, x.z, a);
    return dot2(w.w, x.w, a);
}

// Lane slice: 8 consecutive bf16 (16 B); a wave step covers 512 k.  R rows per
// workgroup (rows row0 .. row0 + R - 1 of one matrix); its waves split the k steps.
template <int R>
__device__ __forceinline__ void bf16_rows(const uint16_t *__restrict__ w, int64_t n_out, int64_t k,
                                          const uint16_t *__restrict__ x, float *__restrict__ y, int64_t row0,
                                          float (*red)[R]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;

    const uint16_t *rowp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rowp[r] = w + ((row0 + r < n_out) ? row0 + r : n_out - 1) * k;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    const int64_t step = static_cast<int64_t>(512) * waves;
    int64_t kk = static_cast<int64_t>(wave) * 512 + lane * 8;
    for (; kk + step < k; kk += 2 * step) {          // two steps in flight
        uint4 q0[R], q1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) q0[r] = load_stream16(rowp[r] + kk);
#pragma unroll
        for (int r = 0; r < R; ++r) q1[r] = load_stream16(rowp[r] + kk + step);
        const uint4 x0 = *reinterpret_cast<const uint4 *>(x + kk);
        const uint4 x1 = *reinterpret_cast<const uint4 *>(x + kk + step);
        __builtin_amdgcn_sched_barrier(0);           // keep every load of the step ahead of the math
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = dot8(q1[r], x1, dot8(q0[r], x0, acc[r]));
    }
    if (kk < k) {
        uint4 q0[R];
#pragma unroll
        for (int r = 0; r < R; ++r) q0[r] = load_stream16(rowp[r] + kk);
        const uint4 x0 = *reinterpret_cast<const uint4 *>(x + kk);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = dot8(q0[r], x0, acc[r]);
    }
    finish_rows<R>(acc, red, lane, wave, waves, row0, n_out, y);
}

template <int R>
__global__ __launch_bounds__(512) void gemv_bf16_kernel(const uint16_t *__restrict__ w, int64_t n_out, int64_t k,
                                                        const uint16_t *__restrict__ x, float *__restrict__ y) {
    __shared__ float red[kMaxWaves][R];
    bf16_rows<R>(w, n_out, k, x, y, static_cast<int64_t>(blockIdx.x) * R, red);
}

// Several independent bf16 GEMVs of one k in one launch (a layer's q, k and v, or its gate
// and up projections, kept as separate matrices): workgroup b serves matrix i for b in
// [first[i], first[i + 1]), rows (b - first[i]) * R .., with the same row body as a single
// launch, so every output is bit for bit what linear_gemv gives.  The descriptors are
// kernel arguments; the matrix is picked with compile-time indices (the index is the same
// for the whole workgroup), which keeps the argument arrays out of scratch memory.
constexpr int kGemvMultiMax = 8;
struct GemvMulti {
    const uint16_t *w[kGemvMultiMax];
    const uint16_t *x[kGemvMultiMax];
    float *y[kGemvMultiMax];
    int64_t n_out[kGemvMultiMax];
    uint32_t first[kGemvMultiMax + 1];
    int count;
};

template <int R>
__global__ __launch_bounds__(512) void gemv_bf16_multi_kernel(const GemvMulti a, int64_t k) {
    __shared__ float red[kMaxWaves][R];
    const uint32_t b = blockIdx.x;
    const uint16_t *w = a.w[0], *x = a.x[0];
    float *y = a.y[0];
    int64_t n_out = a.n_out[0];
    uint32_t first = 0;
#pragma unroll
    for (int i = 1; i < kGemvMultiMax; ++i) {
        if (i < a.count && b >= a.first[i]) {
            w = a.w[i];
            x = a.x[i];
            y = a.y[i];
            n_out = a.n_out[i];
            first = a.first[i];
        }
    }
    bf16_rows<R>(w, n_out, k, x, y, static_cast<int64_t>(b - first) * R, red);
}

// ---------------------------------------------------------------- NF4
// Scales of R consecutive rows (row0 .. row0+R-1, inside one 16-row block) for group g.
template <int R>
__device__ __forceinline__ void load_scales(const uint16_t *__restrict__ scales, bool vec, const int64_t (&rows)[R],
                                            int64_t row0, int64_t g, int64_t groups, int64_t n_out, float (&s)[R]) {
    if (vec) {
        const uint16_t *p = scales + scale_index(row0, g, groups, n_out);
        if constexpr (R == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            s[0] = f16_to_f32(v.x & 0xffffu);
            s[1] = f16_to_f32(v.x >> 16);
            s[2] = f16_to_f32(v.y & 0xffffu);
            s[3] = f16_to_f32(v.y >> 16);
        } else {
            static_assert(R == 2, "R must be 2 or 4");
            const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
            s[0] = f16_to_f32(v & 0xffffu);
            s[1] = f16_to_f32(v >> 16);
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = f16_to_f32(scales[scale_index(rows[r], g, groups, n_out)]);
    }
}

// Raw fp16 scale bits of R consecutive rows of one group, kept packed until the
// multiply so that a prefetch of the next row group is never waited on early.
template <int R> struct ScaleBits;
template <> struct ScaleBits<2> { typedef uint32_t T; };
template <> struct ScaleBits<4> { typedef uint2 T; };

template <int R>
__device__ __forceinline__ float scale_at(const typename ScaleBits<R>::T &v, int r) {
    if constexpr (R == 2) {
        return f16_to_f32(r == 0 ? (v & 0xffffu) : (v >> 16));
    } else {
        const uint32_t w = (r < 2) ? v.x : v.y;
        return f16_to_f32((r & 1) ? (w >> 16) : (w & 0xffffu));
    }
}

// --- table lookups
// 16-entry table (64 B, one ds_read_b32 per code).  Byte B of a device-layout word,
// ANDed with 0x3C, is the byte address code*4 of the entry of the code at bits 2..5
// of that byte (one SDWA AND); the odd codes come from the word rotated right by 4.
template <int B>
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, uint32_t m60) {
    uint32_t r;
    if constexpr (B == 0)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    else if constexpr (B == 1)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    else if constexpr (B == 2)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    else
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(m60));
    return r;
}

template <int B>
__device__ __forceinline__ void nf4_byte(uint32_t we, uint32_t wo, uint32_t m60, const char *lut, const float *xf,
                                         float &p0, float &p1) {
    const float le = *reinterpret_cast<const float *>(lut + lut_addr<B>(we, m60));
    const float lo = *reinterpret_cast<const float *>(lut + lut_addr<B>(wo, m60));
    p0 = __builtin_fmaf(le, xf[2 * B], p0);
    p1 = __builtin_fmaf(lo, xf[2 * B + 1], p1);
}

// Dot product of 32 codes (one 16-byte device-layout load) with 32 fp32 x through
// the 16-entry table.  Even codes accumulate in p0, odd codes in p1.
__device__ __forceinline__ float nf4_dot32(const uint4 q, const float (&xf)[32], const char *lut, uint32_t m60) {
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t we = wd[i];
        const uint32_t wo = rotr32(we, 4);
        nf4_byte<0>(we, wo, m60, lut, &xf[8 * i], p0, p1);
        nf4_byte<1>(we, wo, m60, lut, &xf[8 * i], p0, p1);
        nf4_byte<2>(we, wo, m60, lut, &xf[8 * i], p0, p1);
        nf4_byte<3>(we, wo, m60, lut, &xf[8 * i], p0, p1);
    }
    return p0 + p1;
}

__device__ __forceinline__ float nf4_dot32_pair(const uint4 q, const float (&xf)[32], const char *tab,
                                                uint32_t (&ad)[4]) {
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = rotr32(wd[i], 2);   // undo the layout's rotation: byte B = codes 2B, 2B+1
        pair_addr<0>(ad[0], w);
        pair_addr<1>(ad[1], w);
        pair_addr<2>(ad[2], w);
        pair_addr<3>(ad[3], w);
        float2 l[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) l[b] = *reinterpret_cast<const float2 *>(tab + ad[b]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            p0 = __builtin_fmaf(l[b].x, xf[8 * i + 2 * b], p0);
            p1 = __builtin_fmaf(l[b].y, xf[8 * i + 2 * b + 1], p1);
        }
    }
    return p0 + p1;
}

// 32 bf16 x values from x + kk (zeros when !active), raw and then widened to fp32:
// issue_x32 lets a prologue start the load before work that does not need x.
__device__ __forceinline__ void issue_x32(const uint16_t *__restrict__ x, int64_t kk, bool active, uint4 (&xv)[4]) {
    const uint4 *xp = reinterpret_cast<const uint4 *>(x + kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = active ? xp[i] : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void widen_x32(const uint4 (&xv)[4], float (&xf)[32]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xf[8 * i + 0] = bf16_lo(xv[i].x);
        xf[8 * i + 1] = bf16_hi(xv[i].x);
        xf[8 * i + 2] = bf16_lo(xv[i].y);
        xf[8 * i + 3] = bf16_hi(xv[i].y);
        xf[8 * i + 4] = bf16_lo(xv[i].z);
        xf[8 * i + 5] = bf16_hi(xv[i].z);
        xf[8 * i + 6] = bf16_lo(xv[i].w);
        xf[8 * i + 7] = bf16_hi(xv[i].w);
    }
}

__device__ __forceinline__ void load_x32(const uint16_t *__restrict__ x, int64_t kk, bool active, float (&xf)[32]) {
    uint4 xv[4];
    issue_x32(x, kk, active, xv);
    widen_x32(xv, xf);
}

// Contiguous chunk of `total` work items owned by workgroup group `xcd` (of nx: one group
// per XCD, workgroup b dispatched to XCD b % nx).
__device__ __forceinline__ void xcd_chunk(int64_t total, int xcd, int nx, int64_t &first, int64_t &count) {
    const int64_t per = total / nx, rem = total - per * nx;
    first = xcd * per + (xcd < rem ? xcd : rem);
    count = per + (xcd < rem ? 1 : 0);
}

// NF4 GEMV for k <= 32768.  A lane owns 32 consecutive codes (16 B, half a group) of
// a row; a wave covers a 2048-code k-slice.  A workgroup holds T teams of S waves,
// S = ceil(k / 2048): the S waves of a team split the row into slices and keep their
// 32 x values in registers for the whole matrix; team t works on row group
// sg * T + t of super-group sg (R rows per row group).
// Super-groups of rows in whole 16-row scale blocks are split into 8 contiguous
// chunks, one per XCD (workgroup b runs on XCD b % 8), so the rows that share a scale
// block are read through one L2 and each XCD streams a contiguous range.  The wave
// index is made wave-uniform, so a super-group's row index and its code and scale
// addresses are scalar, plus a per-lane offset fixed for the whole matrix.  Workgroups are persistent over their
// chunk, and the codes and scales of the next super-group are loaded before the
// current one is multiplied; the scales stay raw fp16 until they are used.  The
// last super-group of a round is peeled, so no load is issued past it.
// Row sums: transposed wave reduction, then the S per-wave partials of each row meet
// in LDS in a fixed order (one LDS-only barrier per super-group, double-buffered) --
// the result is deterministic.  A workgroup with four or more super-groups parks the
// finished sums of a round in LDS and writes them to y after the round, so no global
// store sits between the loads of its loop.  The rows of a last partial 16-row block and
// of super-groups left incomplete are done at the end with per-row loads.  TAB selects the 16-entry table (0) or the replicated pair table (1).
// Waves of the workgroup beyond the T teams (the decode sweep runs every matrix in
// 16-wave workgroups) take part in the barriers only.
constexpr int kRowSumCap = 2048;   // finished row sums parked per round

// The workgroup-independent geometry of one matrix for the team GEMV, in 32-bit
// arithmetic (n_out <= 2^30, so every count fits): computed on the host for a single
// launch and passed by value, and on the device per decode-sweep stage.  (The 64-bit
// divisions this replaces took about a microsecond per wave in every kernel prologue,
// ahead of the first weight load.)
struct TeamGeom {
    int32_t S, T;          // waves per team, teams per workgroup
    int32_t row_groups;    // ceil(n_out / R)
    int32_t supers;        // super-groups: full row groups / T
    int32_t cap;           // super-groups whose row sums a round parks in LDS
    int32_t nloc;          // workgroups per XCD share (grid / nx)
    int32_t per, rem;      // super-groups per XCD share: per, one more for the first rem
};

template <int R>
__host__ __device__ __forceinline__ TeamGeom team_geom(int64_t n_out, int S, int T, uint32_t grid, uint32_t nx) {
    TeamGeom g;
    const uint32_t n = static_cast<uint32_t>(n_out);
    g.S = S;
    g.T = T;
    g.row_groups = static_cast<int32_t>((n + R - 1) / R);
    const uint32_t full = ((n >> 4) << 4) / R;   // rows of whole 16-row scale blocks
    g.supers = static_cast<int32_t>(full / static_cast<uint32_t>(T));
    g.cap = kRowSumCap / (T * R);
    g.nloc = static_cast<int32_t>(grid / nx);
    g.per = static_cast<int32_t>(static_cast<uint32_t>(g.supers) / nx);
    g.rem = g.supers - g.per * static_cast<int32_t>(nx);
    return g;
}

// LDS of the team GEMV: the level table, the cross-wave row sums (double-buffered)
// and the parked row sums of a round.
template <int R, int TAB>
struct TeamLds {
    __align__(16) char tab[TAB == 0 ? 64 : kPairTableBytes];
    float red[2][16][R];
    float yl[kRowSumCap];
};

// One matrix as seen by one workgroup: geometry, this wave's slice and this
// workgroup's super-groups first + i0 + j * nloc, j = 0 .. n - 1.  WIDE: the workgroup
// may hold more waves than the T teams need (idle waves: they run the barrier-only form
// of team_run).
template <int R, bool WIDE>
struct TeamStage {
    typedef typename ScaleBits<R>::T SB;
    const uint8_t *packed;
    const uint16_t *scales;
    const uint16_t *x;
    float *y;
    int64_t n_out, groups, rowbytes, row_groups, supers, first, i0, nloc, n, cap;
    int S, T, team, fteam;
    bool idle, active, park;
    int64_t kkl;
    uint32_t coff, gl, soff;   // this lane's byte offsets: codes in a row, scale in a full block

    __device__ __forceinline__ void init(const uint8_t *p, int64_t n_out_, int64_t k, const uint16_t *x_, float *y_,
                                         const TeamGeom &g, int wave, int lane, int nx) {
        packed = p;
        x = x_;
        y = y_;
        n_out = n_out_;
        S = g.S;
        T = g.T;
        groups = k >> 6;
        rowbytes = k >> 1;
        row_groups = g.row_groups;
        supers = g.supers;
        cap = g.cap;
        nloc = g.nloc;
        scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
        // The wave index is made wave-uniform, so that rows, row addresses and the idle
        // test are scalar: per-lane 64-bit address arithmetic costs about 30 vector
        // instructions per super-group and the registers the prefetch needs.
        const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
        team = static_cast<int>(wv / static_cast<uint32_t>(S));
        idle = WIDE && team >= T;
        fteam = idle ? T - 1 : team;
        const int slice = static_cast<int>(wv) - team * S;
        // Lanes past k read valid codes of the row's last group and multiply them by x = 0.
        const int32_t kk0 = slice * 2048 + lane * 32;
        active = kk0 < k;
        kkl = active ? kk0 : k - 32;
        coff = static_cast<uint32_t>(kkl >> 1);
        gl = static_cast<uint32_t>(kkl >> 6);
        soff = gl * 32u;
        const uint32_t b = blockIdx.x, ux = static_cast<uint32_t>(nx);
        const uint32_t i0u = b / ux, xcd = b - i0u * ux;
        const int32_t count = g.per + (static_cast<int32_t>(xcd) < g.rem ? 1 : 0);
        first = static_cast<int64_t>(xcd) * g.per + (static_cast<int32_t>(xcd) < g.rem ? xcd : g.rem);
        i0 = i0u;
        n = static_cast<int32_t>(i0u) < count
                ? static_cast<int64_t>(static_cast<uint32_t>(count - static_cast<int32_t>(i0u) + g.nloc - 1) /
                                       static_cast<uint32_t>(g.nloc))
                : 0;
        // Parking pays off once a workgroup owns several super-groups; with one or two
        // the two extra barriers of the flush cost more than the stores they move.
        park = n >= 4;
    }

    // The same from a workgroup plan of a decode-sweep stage (SweepPlan, below): only the
    // per-wave part is computed here.
    // The plan is read from LDS into vector registers; every field is wave-uniform, and
    // taking it into a scalar register keeps the address arithmetic of the loop scalar.
    template <typename Plan>
    __device__ __forceinline__ void init_plan(const Plan &p, int wave, int lane, int64_t i0_, int64_t nloc_) {
        auto u32 = [](int32_t v) { return __builtin_amdgcn_readfirstlane(v); };
        auto uptr = [](uint64_t v) {
            const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(v)));
            const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(v >> 32)));
            return lo | (hi << 32);
        };
        // back to global-space pointers before they become the generic fields, so that the
        // compiler still knows where they point
        packed = (const uint8_t *)reinterpret_cast<const WSL_GLOBAL uint8_t *>(uptr((uint64_t)p.w));
        x = (const uint16_t *)reinterpret_cast<const WSL_GLOBAL uint16_t *>(uptr((uint64_t)p.x));
        y = (float *)reinterpret_cast<WSL_GLOBAL float *>(uptr((uint64_t)p.y));
        const int32_t k = u32(p.k);
        n_out = u32(p.n_out);
        S = u32(p.S);
        T = u32(p.T);
        groups = k >> 6;
        rowbytes = k >> 1;
        row_groups = u32(p.row_groups);
        supers = u32(p.supers);
        cap = u32(p.cap);
        nloc = nloc_;
        first = u32(p.first);
        i0 = i0_;
        n = u32(p.n);
        park = n >= 4;
        scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
        const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
        team = static_cast<int>((wv * static_cast<uint32_t>(u32(p.inv_s))) >> 16);   // wv / S for wv < 16
        idle = WIDE && team >= T;
        fteam = idle ? T - 1 : team;
        const int slice = static_cast<int>(wv) - team * S;
        const int32_t kk0 = slice * 2048 + lane * 32;
        active = kk0 < k;
        kkl = active ? kk0 : k - 32;
        coff = static_cast<uint32_t>(kkl >> 1);
        gl = static_cast<uint32_t>(kkl >> 6);
        soff = gl * 32u;
    }

    // Loads of super-group j of this wave's team.  An idle wave loads what the last team
    // loads (in bounds, and never used): with no branch around the loads, every path has
    // the same loads in flight, and the compiler's waits before the first multiply stay
    // exact (a branch that issues no loads makes it wait for every load in flight).
    // The row index is wave-uniform (scalar) and a super-group lies in whole 16-row scale
    // blocks, so both addresses are a scalar base plus this lane's constant offset.
    __device__ __forceinline__ void fetch(int64_t j, uint4 (&q)[R], SB &sb) const {
        const uint32_t sg = static_cast<uint32_t>(first + i0) + static_cast<uint32_t>(j) * static_cast<uint32_t>(nloc);
        const uint32_t row0 = (sg * static_cast<uint32_t>(T) + static_cast<uint32_t>(fteam)) * R;
        const uint8_t *rowp = packed + static_cast<int64_t>(row0) * rowbytes;
#pragma unroll
        for (int r = 0; r < R; ++r) q[r] = load_stream16(rowp + r * rowbytes + coff);
        const char *sp = reinterpret_cast<const char *>(scales + static_cast<int64_t>(row0 >> 4) * 16 * groups + (row0 & 15));
        sb = *reinterpret_cast<const SB *>(sp + soff);
        __builtin_amdgcn_sched_barrier(0);   // the whole prefetch is issued before the math below
    }

    __device__ __forceinline__ void issue_x(uint4 (&xv)[4]) const { issue_x32(x, kkl, active, xv); }
};

// The loads of one super-group in a compact form (what fetch() computes for it): kept
// across the tail of the previous stage by the decode sweep instead of a whole geometry.
struct FirstLoads {
    const uint8_t *rowp;   // first row of this wave's team, at the wave's slice
    const char *sp;        // scale block of those rows, at this lane's group
    int64_t rowbytes;
    bool has;
};

// `dummy`: 16-byte aligned device memory of at least 16 bytes, read instead when the
// workgroup has no super-group in the stage (the loads are then issued all the same, so
// that no branch decides whether they are); the sweep passes a stage's x, read-only and
// cached (not the barrier counters, which every workgroup would then load).
template <int R, bool WIDE>
__device__ __forceinline__ FirstLoads first_loads(const TeamStage<R, WIDE> &st, const void *dummy) {
    FirstLoads f;
    f.has = st.n > 0;
    if (!f.has) {
        f.rowp = static_cast<const uint8_t *>(dummy);
        f.sp = static_cast<const char *>(dummy);
        f.rowbytes = 0;
        return f;
    }
    const int64_t row0 = ((st.first + st.i0) * st.T + st.fteam) * R;
    f.rowp = st.packed + row0 * st.rowbytes + st.coff;
    f.sp = reinterpret_cast<const char *>(st.scales + (row0 >> 4) * 16 * st.groups + (row0 & 15)) + st.soff;
    f.rowbytes = st.rowbytes;
    return f;
}

template <int R>
__device__ __forceinline__ void issue_first(const FirstLoads &f, uint4 (&q)[R], typename ScaleBits<R>::T &sb) {
#pragma unroll
    for (int r = 0; r < R; ++r) q[r] = load_stream16(f.rowp + r * f.rowbytes);
    sb = *reinterpret_cast<const typename ScaleBits<R>::T *>(f.sp);
    __builtin_amdgcn_sched_barrier(0);
}

template <int TAB>
__device__ __forceinline__ float team_dot(const uint4 &q, const float (&xf)[32], const char *tab, uint32_t (&ad)[4]) {
    if constexpr (TAB == 0) return nf4_dot32(q, xf, tab, 0x3cu);
    else return nf4_dot32_pair(q, xf, tab, ad);
}

// Multiply this workgroup's share of the matrix: the pipelined super-groups, the
// parked-sum flushes and the leftover row groups.  On entry qa/sa hold the loads of
// super-group 0 (when st.n > 0), xf this wave's x slice and the table is built.
// SKIP: the form an idle wave runs -- no loads and no math, the same barriers and the
// same share of the parked-sum stores as the other waves.  `next` (decode sweep) issues
// the loads of whatever comes after this matrix into the buffer it is given; it is
// called once, before the last super-group is multiplied, so that those loads are in
// flight meanwhile.  Returns true if it was given qb/sb, false if qa/sa or not called.
// EARLY: refill each buffer between the multiply and the reduction of the super-group it
// held, so that its loads are in flight through the workgroup barrier (faster for the
// single-matrix launch); otherwise after the reduction (faster in the decode sweep).
struct NoNext {
    template <typename Q, typename S_>
    __device__ __forceinline__ void operator()(Q &, S_ &) const {}
};

template <int R, int TAB, bool SKIP, bool WIDE, bool EARLY = false, typename Next = NoNext>
__device__ __forceinline__ bool team_run(const TeamStage<R, WIDE> &st, TeamLds<R, TAB> &lds, const float (&xf)[32],
                                         uint32_t (&ad)[4], uint4 (&qa)[R], typename ScaleBits<R>::T &sa,
                                         uint4 (&qb)[R], typename ScaleBits<R>::T &sb, Next next = Next()) {
    typedef typename ScaleBits<R>::T SB;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    constexpr int span = 64 / R;
    const int T = st.T, S = st.S;
    int ph = 0;
    int64_t jbeg = 0;
    bool in_b = false;
    // A super-group is multiplied (mul: this wave's partial sums into the reduction
    // buffer) and then reduced (reduce: the workgroup barrier, the sum over the team's
    // waves and its store); the prefetch of a later super-group goes between the two,
    // once the registers it overwrites have been read, so that its loads are in flight
    // while the waves meet at the barrier.
    auto mul = [&](const uint4 (&q)[R], const SB &sb_) {
        if constexpr (!SKIP) {
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = scale_at<R>(sb_, r) * team_dot<TAB>(q[r], xf, lds.tab, ad);
            bool holder;
            const float v = team_reduce<R>(acc, lane, holder);
            if (holder) lds.red[ph][wave][lane / span] = v;
        }
    };
    auto reduce = [&](int64_t j) {
        lds_barrier();
        if (threadIdx.x < T * R) {
            const int tm = threadIdx.x / R, r = threadIdx.x - tm * R;
            float t = lds.red[ph][tm * S][r];
            for (int s = 1; s < S; ++s) t += lds.red[ph][tm * S + s][r];
            if (st.park) lds.yl[(j - jbeg) * T * R + threadIdx.x] = t;
            else st.y[(st.first + st.i0 + j * st.nloc) * T * R + threadIdx.x] = t;
        }
        ph ^= 1;
    };

    auto fetch = [&](int64_t j, uint4 (&q)[R], SB &s_) {
        if constexpr (!SKIP) st.fetch(j, q, s_);
    };
    const int64_t n = st.n;
    // One round of up to cap super-groups.  LAST: the matrix's last round, whose tail
    // calls next() -- a separate copy of the body, so that no runtime branch decides
    // whether loads are issued (with one, the compiler waits for every load in flight,
    // the next matrix's included, before the last multiply).
    auto round = [&](auto last_tag) {
        constexpr bool LAST = decltype(last_tag)::value;
        const int64_t jend = (jbeg + st.cap < n) ? jbeg + st.cap : n;
        if (jbeg > 0) fetch(jbeg, qa, sa);
        int64_t j = jbeg;
        if constexpr (EARLY) {
            // Unrolled by two so that the two buffers swap without copies, with the last one,
            // two or three super-groups written out: every path between branches is straight
            // code, each buffer is refilled right after it was multiplied, and at the loop
            // head the two buffers are pending in the same order on every path, so the waits
            // before each multiply leave the other buffer's loads in flight.
            if (j + 1 < jend) {
                fetch(j + 1, qb, sb);
                for (; j + 3 < jend; j += 2) {   // qa: j, qb: j + 1; four or more remain
                    mul(qa, sa);
                    fetch(j + 2, qa, sa);
                    reduce(j);
                    mul(qb, sb);
                    fetch(j + 3, qb, sb);
                    reduce(j + 1);
                }
                if (j + 2 < jend) {              // three remain
                    mul(qa, sa);
                    fetch(j + 2, qa, sa);
                    reduce(j);
                    mul(qb, sb);
                    if constexpr (LAST) {
                        next(qb, sb);
                        in_b = true;
                    }
                    reduce(j + 1);
                    mul(qa, sa);
                    reduce(j + 2);
                } else {                         // two remain
                    mul(qa, sa);
                    if constexpr (LAST) next(qa, sa);
                    reduce(j);
                    mul(qb, sb);
                    reduce(j + 1);
                }
            } else {                             // one remains
                if constexpr (LAST) {
                    next(qb, sb);
                    in_b = true;
                }
                mul(qa, sa);
                reduce(j);
            }
        } else {
            // Each buffer is refilled after the reduction of the super-group it held
            // (the order the decode sweep measures fastest in); otherwise as above, with
            // the last one or two super-groups written out.
            for (; j + 2 < jend; j += 2) {
                fetch(j + 1, qb, sb);
                mul(qa, sa);
                reduce(j);
                fetch(j + 2, qa, sa);
                mul(qb, sb);
                reduce(j + 1);
            }
            if (j + 1 < jend) {
                fetch(j + 1, qb, sb);
                mul(qa, sa);
                reduce(j);
                if constexpr (LAST) next(qa, sa);
                mul(qb, sb);
                reduce(j + 1);
            } else {
                if constexpr (LAST) {
                    next(qb, sb);
                    in_b = true;
                }
                mul(qa, sa);
                reduce(j);
            }
        }
        if (st.park) {
            lds_barrier();
            // at most cap * T * R <= kRowSumCap sums: 32-bit index arithmetic
            const uint32_t tr = static_cast<uint32_t>(T * R), cnt = static_cast<uint32_t>(jend - jbeg) * tr;
            for (uint32_t e = threadIdx.x; e < cnt; e += blockDim.x) {
                const uint32_t q = e / tr, rest = e - q * tr;
                st.y[(st.first + st.i0 + (jbeg + q) * st.nloc) * T * R + rest] = lds.yl[e];
            }
            lds_barrier();
        }
    };
    if (n > 0) {
        for (jbeg = 0; jbeg + st.cap < n; jbeg += st.cap) round(std::false_type());
        round(std::true_type());
    }
    // Leftover row groups [supers * T, row_groups): T per workgroup, one per team,
    // rows clamped to the matrix and scales read one row at a time.  They go to the
    // last workgroups, which own one super-group fewer than the first ones when the
    // super-groups do not divide evenly, so the leftovers do not lengthen the kernel.
    // The first leftover round uses the reduction buffer the last reduce() did not:
    // without the flush's barriers (n < 4) a team of this round may write its partials
    // while wave 0 still reads that reduce()'s partials from the other buffer.
    const int64_t left0 = st.supers * T;
    const int64_t nleft = st.row_groups - left0;
    int it = ph;
    for (int64_t b = gridDim.x - 1 - blockIdx.x; b * T < nleft; b += gridDim.x) {
        const int64_t rg = left0 + b * T + st.team;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        if (!SKIP && rg < st.row_groups) {
            const int64_t row0 = rg * R;
            uint4 q[R];
            float s[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = (row0 + r < st.n_out) ? row0 + r : st.n_out - 1;
                q[r] = load_stream16(st.packed + row * st.rowbytes + st.coff);
                s[r] = f16_to_f32(st.scales[scale_index(row, st.gl, st.groups, st.n_out)]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = s[r] * team_dot<TAB>(q[r], xf, lds.tab, ad);
        }
        bool holder;
        const float v = team_reduce<R>(acc, lane, holder);
        if (holder) lds.red[it & 1][wave][lane / span] = v;
        lds_barrier();
        if (threadIdx.x < T * R) {
            const int tm = threadIdx.x / R, r = threadIdx.x - tm * R;
            float t = lds.red[it & 1][tm * S][r];
            for (int s = 1; s < S; ++s) t += lds.red[it & 1][tm * S + s][r];
            const int64_t row = (left0 + b * T) * R + tm * R + r;
            if (row < st.n_out) st.y[row] = t;
        }
        ++it;
    }
    return in_b;
}

template <int R, int TAB, bool EARLY>
__global__ __launch_bounds__(1024) void gemv_nf4_team_kernel(const uint8_t *__restrict__ packed, int64_t n_out,
                                                             int64_t k, const uint16_t *__restrict__ x,
                                                             float *__restrict__ y, TeamGeom g, int nx) {
    __shared__ TeamLds<R, TAB> lds;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    TeamStage<R, false> st;
    st.init(packed, n_out, k, x, y, g, wave, lane, nx);
    uint32_t ad[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = static_cast<uint32_t>(lane & 31) << 3;
    uint4 qa[R];
    typename ScaleBits<R>::T sa;
    // The first super-group's loads and the x loads are in flight while the table is
    // built (x last: the first multiply needs both, so one wait for all is no loss).
    if (st.n > 0) st.fetch(0, qa, sa);
    uint4 xv[4];
    st.issue_x(xv);
    if constexpr (TAB == 0) {
        write_levels(reinterpret_cast<float *>(lds.tab));
    } else {
        fill_pair_table(lds.tab);
    }
    __syncthreads();
    float xf[32];
    widen_x32(xv, xf);
    uint4 qb[R];
    typename ScaleBits<R>::T sb;
    team_run<R, TAB, false, false, EARLY>(st, lds, xf, ad, qa, sa, qb, sb);
}

// ---------------------------------------------------------------- decode sweep
// Teams per workgroup for a k of S slices in a 16-wave workgroup: 16 / S, one team fewer
// when that makes the busy waves a multiple of 4 (equal waves per SIMD; k = 6144: 4
// teams of 3 waves rather than 5).
__host__ __device__ __forceinline__ int sweep_teams(int S, int waves = 16) {
    int T = waves / S;
    if ((S * T) % 4 != 0 && T > 1 && (S * (T - 1)) % 4 == 0) --T;
    return T;
}

// Words of the sweep's synchronization workspace (each counter in its own 128-byte line).
constexpr int kSyncGroupWord = 0;      // + 32 * g, g = 0..7: arrivals of workgroup group g
constexpr int kSyncExitWord = 9 * 32;  // workgroups finished
constexpr int kSyncStatusWord = 10 * 32;

// A stage descriptor as the kernel reads it: wsl_gemv_stage with its pointers typed in the
// global address space.  A pointer read from memory as a plain pointer is generic to the
// compiler, which then emits flat loads and stores -- counted by lgkmcnt as well, so
// every LDS-only wait would also wait for the weight loads in flight.
struct SweepStage {
    const WSL_GLOBAL uint8_t *w;
    const WSL_GLOBAL uint16_t *x;
    WSL_GLOBAL float *y;
    int64_t n_out, k;
};
static_assert(sizeof(SweepStage) == sizeof(wsl_gemv_stage), "descriptor layouts differ");

__device__ __forceinline__ bool sweep_stage_ok(const SweepStage &d) {
    const uintptr_t a = (uintptr_t)d.w | (uintptr_t)d.x;
    return d.w != nullptr && d.x != nullptr && d.y != nullptr && (a & 15) == 0 && ((uintptr_t)d.y & 3) == 0 && d.n_out >= 1 && d.k >= 64 && d.k <= 32768 &&
           (d.k & 63) == 0;
}

// Device-wide barrier between two stages, the b-th of the call.  Each workgroup adds one
// to its group's counter (workgroup % 8, one group per XCD, each counter in its own cache
// line), without waiting for the add to return; a waiter reads the 8 counters with one
// 8-lane load per poll and goes on once every group has all its arrivals for this
// barrier.  It orders execution only: no stage reads another stage's output, so no cache
// write-back or invalidation is made here (device-scope release/acquire fences cost about
// 6 us per barrier on this GPU); every output is visible when the kernel ends, as for
// any launch.  The wait is bounded: past `spin_limit` polls it sets
// WSL_STATUS_SWEEP_TIMEOUT and goes on, so the kernel always ends; a workgroup that has
// given up once waits at no later barrier.
__device__ __forceinline__ void sweep_arrive(uint32_t *sync, int nx) {
    __hip_atomic_fetch_add(sync + kSyncGroupWord + 32 * (blockIdx.x % nx), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Called by all 64 lanes of one wave.
__device__ __forceinline__ void sweep_wait(uint32_t *sync, uint32_t b, uint32_t spin_limit, int nx, bool &gave_up) {
    const uint32_t target = (b + 1) * (gridDim.x / nx);
    const int lane = threadIdx.x & 63;
    uint32_t polls = 0;
    while (!gave_up) {
        uint32_t v = target;
        if (lane < nx) v = __hip_atomic_load(sync + kSyncGroupWord + 32 * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__all(v >= target)) break;
        __builtin_amdgcn_s_sleep(1);
        if (++polls > spin_limit) {
            if (lane == 0)
                __hip_atomic_fetch_or(sync + kSyncStatusWord, WSL_STATUS_SWEEP_TIMEOUT, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            gave_up = true;
        }
    }
}

// The wave-independent geometry of a decode-sweep stage for one workgroup: what every
// wave of the workgroup would otherwise derive for itself from the stage's descriptor
// at every stage boundary (the descriptor load and about a dozen divisions, scalar work
// that the CU's waves share one scalar unit for).  One lane per stage computes it; the
// waves read it from LDS.  An invalid descriptor gives ok = 0 and no rows.
struct SweepPlan {
    const WSL_GLOBAL uint8_t *w;   // global address space: a generic pointer read back from
    const WSL_GLOBAL uint16_t *x;  // memory would make the weight loads flat loads, which
    WSL_GLOBAL float *y;           // every LDS wait would also wait for
    int32_t n_out, k, S, T, inv_s, row_groups, supers, cap, first, n, ok, pad;
};

template <int R>
__device__ __forceinline__ void sweep_plan(const wsl_gemv_stage *stages, int s, int waves, int nx, SweepPlan &p) {
    const SweepStage d = reinterpret_cast<const SweepStage *>(stages)[s];
    const bool ok = sweep_stage_ok(d);
    const int S = ok ? static_cast<int>((d.k + 2047) / 2048) : 1;
    const int64_t n_out = ok ? d.n_out : 0;
    const int T = sweep_teams(S, waves);
    const TeamGeom g = team_geom<R>(n_out, S, T, gridDim.x, static_cast<uint32_t>(nx));
    const uint32_t b = blockIdx.x, ux = static_cast<uint32_t>(nx);
    const uint32_t i0 = b / ux, xcd = b - i0 * ux;
    const int32_t cnt = g.per + (static_cast<int32_t>(xcd) < g.rem ? 1 : 0);
    p.w = d.w;
    p.x = d.x;
    p.y = d.y;
    p.n_out = static_cast<int32_t>(n_out);
    p.k = ok ? static_cast<int32_t>(d.k) : 64;
    p.S = S;
    p.T = T;
    p.inv_s = (65536 + S - 1) / S;
    p.row_groups = ok ? g.row_groups : 0;
    p.supers = ok ? g.supers : 0;
    p.cap = g.cap;
    p.first = static_cast<int32_t>(xcd) * g.per + (static_cast<int32_t>(xcd) < g.rem ? static_cast<int32_t>(xcd) : g.rem);
    p.n = (ok && static_cast<int32_t>(i0) < cnt)
              ? static_cast<int32_t>(static_cast<uint32_t>(cnt - static_cast<int32_t>(i0) + g.nloc - 1) /
                                     static_cast<uint32_t>(g.nloc))
              : 0;
    p.ok = ok ? 1 : 0;
    p.pad = 0;
}

// The decode sweep: `count` NF4 GEMVs (stages) in order in one launch, one 16-wave
// workgroup per CU for the whole call.  Each stage runs as the team kernel with the pair
// table (R = 2, T = sweep_teams(S)); waves beyond a stage's teams run its barrier-only
// form.  Between stages every workgroup meets a device-wide barrier, so no workgroup
// starts a stage (nor reads its x) before every workgroup has finished the previous one,
// as in a decode step where each stage's input depends on the stage before.  The weight
// stream does not wait for the barrier: a stage's descriptor is read a stage ahead, and
// the loads of this workgroup's first super-group of the next stage are issued before
// the last super-group of the current one is multiplied, so they are in flight through
// the stage's tail, the barrier and the next x load.  The 64 KB pair table is built once
// per call.  On exit the last workgroup to finish returns the counters to zero.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_nf4_sweep_kernel(const wsl_gemv_stage *__restrict__ stages,
                                                                   int count, uint32_t *__restrict__ sync,
                                                                   uint32_t spin_limit, int nx) {
    constexpr int R = 2;
    typedef ScaleBits<R>::T SB;
    __shared__ TeamLds<R, 1> lds;
    // Plans of the first 64 * WAVES stages (one per thread); later stages are set up from
    // their descriptors at the stage boundary as the plans are.
    constexpr int kPlans = 64 * WAVES;
    __shared__ SweepPlan plans[kPlans];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t i0 = blockIdx.x / nx, nloc = gridDim.x / nx;
    uint32_t ad[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ad[i] = static_cast<uint32_t>(lane & 31) << 3;
    auto setup = [&](int s, TeamStage<R, true> &st) -> bool {
        const SweepStage d = reinterpret_cast<const SweepStage *>(stages)[s];
        const bool ok = sweep_stage_ok(d);
        const int S = ok ? static_cast<int>((d.k + 2047) / 2048) : 1;
        const int64_t n_out = ok ? d.n_out : 0;
        st.init((const uint8_t *)d.w, n_out, ok ? d.k : 64, (const uint16_t *)d.x, (float *)d.y,
                team_geom<R>(n_out, S, sweep_teams(S, WAVES), gridDim.x, static_cast<uint32_t>(nx)), wave, lane, nx);
        if (!ok) {
            st.n = 0;
            st.row_groups = 0;
            st.supers = 0;
        }
        return ok;
    };
    // The first loads of stage t, whose geometry is needed a stage early; past the last
    // stage they read the dummy (a stage's x).
    auto first_of = [&](int t, const void *dummy) -> FirstLoads {
        TeamStage<R, true> ns;
        if (t < count) setup(t, ns);
        else ns.n = 0;
        return first_loads(ns, dummy);
    };
    TeamStage<R, true> cs;   // the stage being multiplied
    FirstLoads nf;           // this workgroup's first loads of the next stage
    uint4 qa[R], qb[R];
    SB sa, sb;
    bool ok = setup(0, cs), gave_up = false;
    if (cs.n > 0) cs.fetch(0, qa, sa);
    uint4 xv[4];
    cs.issue_x(xv);
    nf = first_of(1, cs.x);
    fill_pair_table(lds.tab);   // while the first loads are in flight
    // The plans, one thread per stage (their descriptor loads queue behind the first loads,
    // which the first multiply waits for anyway).  Every thread loads a descriptor (threads
    // past the last stage load the last one again), so no branch decides whether these
    // loads are issued -- with one, the compiler's waits for the weight loads of the stage
    // loop below turn conservative and drain the prefetch.
    {
        const int t = static_cast<int>(threadIdx.x);
        SweepPlan p;
        sweep_plan<R>(stages, t < count ? t : count - 1, WAVES, nx, p);
        if (t < count) plans[t] = p;
    }
    __syncthreads();
    for (int s = 0; s < count; ++s) {
        float xf[32];
        widen_x32(xv, xf);
        bool hooked = false;
        auto next = [&](uint4 (&q)[R], SB &sq) {
            issue_first<R>(nf, q, sq);
            hooked = true;
        };
        bool in_b = false;
        if (ok) {
            if (cs.idle) in_b = team_run<R, 1, true, true>(cs, lds, xf, ad, qa, sa, qb, sb, next);   // wave-uniform
            else in_b = team_run<R, 1, false, true>(cs, lds, xf, ad, qa, sa, qb, sb, next);
        } else if (threadIdx.x == 0 && blockIdx.x == 0) {
            __hip_atomic_fetch_or(sync + kSyncStatusWord, WSL_STATUS_DESCRIPTOR, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
        if (s + 1 == count) break;
        if (!hooked) {   // this workgroup had no super-group of stage s
            issue_first<R>(nf, qa, sa);
            in_b = false;
        }
        lds_barrier();   // this stage's LDS reads are done (its y stores may still drain)
        if (threadIdx.x == 0) sweep_arrive(sync, nx);
        // The next stage's geometry and the first loads of the one after are set up here,
        // where the wait hides them: from the workgroup's plans, or from the descriptor for
        // stages past them.
        if (s + 1 < kPlans) {
            cs.init_plan(plans[s + 1], wave, lane, i0, nloc);
            ok = __builtin_amdgcn_readfirstlane(plans[s + 1].ok) != 0;
        } else {
            ok = setup(s + 1, cs);
        }
        {
            TeamStage<R, true> ns;
            if (s + 2 >= count) ns.n = 0;
            else if (s + 2 < kPlans) ns.init_plan(plans[s + 2], wave, lane, i0, nloc);
            else setup(s + 2, ns);
            nf = first_loads(ns, cs.x);
        }
        if (wave == 0) sweep_wait(sync, static_cast<uint32_t>(s), spin_limit, nx, gave_up);
        lds_barrier();   // every wave waits for the wait (not for its own loads)
        cs.issue_x(xv);
        if (in_b) {      // the next stage's first super-group landed in the second buffer
#pragma unroll
            for (int r = 0; r < R; ++r) qa[r] = qb[r];
            sa = sb;
        }
    }
    lds_barrier();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(sync + kSyncExitWord, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done + 1 == gridDim.x) {   // every workgroup is past its last wait
            for (int g = 0; g < nx; ++g)
                __hip_atomic_store(sync + kSyncGroupWord + 32 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + kSyncExitWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// NF4 GEMV for k > 32768: a workgroup of 16 waves per row group of R rows; wave w
// takes the 2048-code slices w, w + 16, ... and reloads its x slice each time.
template <int R>
__global__ __launch_bounds__(1024) void gemv_nf4_wide_kernel(const uint8_t *__restrict__ packed, int64_t n_out,
                                                             int64_t k, const uint16_t *__restrict__ x,
                                                             float *__restrict__ y) {
    __shared__ float lut[16];
    __shared__ float red[2][16][R];
    write_levels(lut);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
    const int64_t groups = k >> 6;
    const int64_t rowbytes = k >> 1;
    const int64_t row_groups = (n_out + R - 1) / R;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(packed + n_out * rowbytes);
    const char *lutp = reinterpret_cast<const char *>(lut);
    const uint32_t m60 = 0x3c;
    constexpr int span = 64 / R;
    const int64_t kstep = static_cast<int64_t>(2048) * waves;

    int it = 0;
    for (int64_t rg = blockIdx.x; rg < row_groups; rg += gridDim.x, ++it) {
        const int64_t row0 = rg * R;
        const int64_t rem = n_out - ((row0 >> 4) << 4);
        const int64_t rb = rem < 16 ? rem : 16;
        const bool vec = (row0 + R <= n_out) && (rb % R == 0);
        int64_t rows[R];
#pragma unroll
        for (int r = 0; r < R; ++r) rows[r] = (row0 + r < n_out) ? row0 + r : n_out - 1;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        for (int64_t kk = static_cast<int64_t>(wave) * 2048 + lane * 32; kk < k; kk += kstep) {
            uint4 q[R];
            float s[R];
#pragma unroll
            for (int r = 0; r < R; ++r) q[r] = load_stream16(packed + rows[r] * rowbytes + (kk >> 1));
            load_scales<R>(scales, vec, rows, row0, kk >> 6, groups, n_out, s);
            float xf[32];
            load_x32(x, kk, true, xf);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(s[r], nf4_dot32(q[r], xf, lutp, m60), acc[r]);
        }
        const float v = reduce_rows<R>(acc, lane);
        if ((lane % span) == 0) red[it & 1][wave][lane / span] = v;
        __syncthreads();
        if (threadIdx.x < R) {
            float t = red[it & 1][0][threadIdx.x];
            for (int w = 1; w < waves; ++w) t += red[it & 1][w][threadIdx.x];
            if (row0 + threadIdx.x < n_out) y[row0 + threadIdx.x] = t;
        }
    }
}

// ---------------------------------------------------------------- launch plans
// bf16 plan: 8 waves per workgroup (fewer when k has fewer 512-k steps; waves may
// get one step more than others), 2 rows per workgroup.  Measured on the dense
// decoder layer shapes (k = 5120 and 17408) this beats equal-step splits with more
// rows: the 17408-deep down projection runs 15% faster than with 2 waves and one
// row, and no shape is more than 0.5% off the best (waves, rows) pair.
static void plan_gemv_bf16(int64_t k, int &waves, int &rows) {
    const int64_t steps = (k + 511) / 512;
    waves = steps < kMaxWaves ? static_cast<int>(steps) : kMaxWaves;
    rows = 2;
}

#define WSL_GEMV_LAUNCH(KERNEL, R, grid, waves, s, ...) \
    hipLaunchKernelGGL((KERNEL<R>), dim3(static_cast<unsigned>(grid)), dim3(64 * (waves)), 0, s, __VA_ARGS__)

int launch_gemv_bf16(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s) {
    int waves, r;
    plan_gemv_bf16(k, waves, r);
    const int64_t grid = (n_out + r - 1) / r;
    if (grid > 0x7fffffff) return WSL_E_SHAPE;
    const auto *wp = static_cast<const uint16_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    WSL_GEMV_LAUNCH(gemv_bf16_kernel, 2, grid, waves, s, wp, n_out, k, xp, y);
    return WSL_OK;
}

// count (1 .. kGemvMultiMax) independent bf16 GEMVs of one k, validated by the caller.
int launch_gemv_bf16_multi(const wsl_gemv_stage *st, int64_t count, hipStream_t s) {
    int waves, r;
    const int64_t k = st[0].k;
    plan_gemv_bf16(k, waves, r);
    GemvMulti a{};
    int64_t grid = 0;
    for (int64_t i = 0; i < count; ++i) {
        a.w[i] = static_cast<const uint16_t *>(st[i].w);
        a.x[i] = static_cast<const uint16_t *>(st[i].x);
        a.y[i] = st[i].y;
        a.n_out[i] = st[i].n_out;
        a.first[i] = static_cast<uint32_t>(grid);
        grid += (st[i].n_out + r - 1) / r;
        if (grid > 0x7fffffff) return WSL_E_SHAPE;
    }
    a.first[count] = static_cast<uint32_t>(grid);
    a.count = static_cast<int>(count);
    WSL_GEMV_LAUNCH(gemv_bf16_multi_kernel, 2, grid, waves, s, a, k);
    return WSL_OK;
}

// Compute units and XCDs of the current device, queried once per device.  Workgroups
// are grouped by XCD (workgroup b on XCD b % xccs) for L2 locality; the grouping is at
// most 8-way (the sweep's barrier has 8 counters) and any grouping gives the same results.
struct DeviceShape {
    int cus, xccs;
};

static int device_shape(DeviceShape &out) {
    constexpr int kDevs = 64;
    static std::atomic<int> cus_cache[kDevs], xcc_cache[kDevs];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return WSL_E_DEVICE;
    int cus = cus_cache[dev].load(std::memory_order_relaxed);
    int xccs = xcc_cache[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return WSL_E_DEVICE;
        if (hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xccs < 1) xccs = 1;
        if (xccs > 8) xccs = 8;
        xcc_cache[dev].store(xccs, std::memory_order_relaxed);
        cus_cache[dev].store(cus, std::memory_order_relaxed);
    }
    out.cus = cus;
    out.xccs = xccs;
    return WSL_OK;
}

// NF4 plan.  k <= 32768: the team kernel with S = ceil(k / 2048) waves per team.
// Large matrices (>= 32 Mi weights; >= 96 Mi when k <= 4096, where the 64 KB table
// is built for few steps) take the pair table, 2 rows per row group and up to 16 / S
// teams in one workgroup per CU, one team fewer when that makes the waves a multiple
// of 4 (k = 6144: 4 teams of 3 waves, 3 per SIMD, instead of 5 teams); the others
// the 16-entry table, 4 rows (2 up to 4096 rows), at most 2 teams, and two
// workgroups per CU -- three below 32 Mi weights when that stays within 16 waves per
// CU.  The grid is a multiple of 8 (one share per XCD) and never larger than
// needed.  k > 32768: the wide kernel.
// (Measured per launch on the decode shapes: 8192x6144 8.8 us with the pair table
// and 4 teams, 9.9 us with the 16-entry table; 32768x6144 21.7 us with 4 teams,
// 22.4 us with 5; 4096x4096 5.3 us with the 16-entry table, 2 rows and three
// workgroups per CU, 5.6-5.8 us with the pair table.)
struct Nf4GemvPlan {
    bool wide, pair;
    int rows, S, T;
    int64_t grid;
};

static Nf4GemvPlan plan_gemv_nf4(int64_t n_out, int64_t k, const DeviceShape &ds) {
    Nf4GemvPlan p{};
    const int64_t slices = (k + 2047) / 2048;
    if (slices > 16) {
        p.wide = true;
        p.rows = n_out >= 16384 ? 4 : 2;
        p.S = 16;
        p.T = 1;
        const int64_t rg = (n_out + p.rows - 1) / p.rows;
        p.grid = rg < 512 ? rg : 512;
        return p;
    }
    p.wide = false;
    p.S = static_cast<int>(slices);
    int64_t per_cu;
    const int64_t weights = n_out * k;
    if (weights >= (static_cast<int64_t>(p.S <= 2 ? 96 : 32) << 20)) {
        p.pair = true;
        p.rows = 2;
        p.T = 16 / p.S;
        // a multiple of 4 waves when one team fewer gives it: equal waves per SIMD
        if ((p.S * p.T) % 4 != 0 && p.T > 1 && (p.S * (p.T - 1)) % 4 == 0) --p.T;
        per_cu = 1;
    } else {
        p.pair = false;
        p.rows = n_out > 4096 ? 4 : 2;
        p.T = 16 / p.S < 2 ? 1 : 2;
        per_cu = (weights < (static_cast<int64_t>(32) << 20) && 3 * p.S * p.T <= 16) ? 3 : 2;
    }
    const int64_t rg = (n_out + p.rows - 1) / p.rows;
    const int64_t full = (n_out % p.rows == 0) ? rg : ((n_out >> 4) << 4) / p.rows;
    const int64_t supers = full / p.T;
    const int64_t nx = ds.xccs;
    const int64_t need = ((supers > 0 ? supers : 1) + nx - 1) / nx * nx;
    const int64_t most = static_cast<int64_t>(ds.cus) * per_cu / nx * nx;   // one pass over the CUs
    p.grid = most < need ? (most > 0 ? most : nx) : need;
    return p;
}

int launch_gemv_nf4(const void *w, int64_t n_out, int64_t k, const void *x, float *y, hipStream_t s) {
    DeviceShape ds;
    if (device_shape(ds) != WSL_OK) return WSL_E_DEVICE;
    const Nf4GemvPlan p = plan_gemv_nf4(n_out, k, ds);
    const auto *wp = static_cast<const uint8_t *>(w);
    const auto *xp = static_cast<const uint16_t *>(x);
    const dim3 g(static_cast<unsigned>(p.grid)), b(64 * p.S * p.T);
    if (p.wide) {
        if (p.rows == 4) hipLaunchKernelGGL((gemv_nf4_wide_kernel<4>), g, b, 0, s, wp, n_out, k, xp, y);
        else hipLaunchKernelGGL((gemv_nf4_wide_kernel<2>), g, b, 0, s, wp, n_out, k, xp, y);
    } else {
        const uint32_t grid = static_cast<uint32_t>(p.grid), nx = static_cast<uint32_t>(ds.xccs);
        // The early refill (team_run) where it measured faster: rows of up to three
        // 2048-code slices (k <= 6144: 3-4 % on 6144x6144 and 32768x6144); at k = 16384
        // (eight slices) it was 2 % slower.
        if (p.pair && p.S <= 3) {
            hipLaunchKernelGGL((gemv_nf4_team_kernel<2, 1, true>), g, b, 0, s, wp, n_out, k, xp, y,
                               team_geom<2>(n_out, p.S, p.T, grid, nx), ds.xccs);
        } else if (p.pair) {
            hipLaunchKernelGGL((gemv_nf4_team_kernel<2, 1, false>), g, b, 0, s, wp, n_out, k, xp, y,
                               team_geom<2>(n_out, p.S, p.T, grid, nx), ds.xccs);
        } else if (p.rows == 4) {
            hipLaunchKernelGGL((gemv_nf4_team_kernel<4, 0, false>), g, b, 0, s, wp, n_out, k, xp, y,
                               team_geom<4>(n_out, p.S, p.T, grid, nx), ds.xccs);
        } else {
            hipLaunchKernelGGL((gemv_nf4_team_kernel<2, 0, false>), g, b, 0, s, wp, n_out, k, xp, y,
                               team_geom<2>(n_out, p.S, p.T, grid, nx), ds.xccs);
        }
    }
    return WSL_OK;
}

// Decode sweep: one 16-wave workgroup per compute unit (a multiple of 8, one share per
// XCD), all resident at once for the device-wide stage barriers.
constexpr size_t kSweepWsBytes = 2048;
constexpr uint32_t kSweepSpinLimit = 1u << 20;   // polls of a stage barrier (about a second)

size_t sweep_ws_bytes() { return kSweepWsBytes; }

// 12-wave workgroups when every stage's k fits 12 slices of 2048 (k <= 24576): a limit
// of 170 registers per lane instead of 128, and the k = 6144 stages of a decoder (3
// slices) use all 12 waves in 4 teams; otherwise 16 waves.
int launch_gemv_nf4_sweep(const wsl_gemv_stage *d_stages, int64_t count, int64_t max_k, void *ws, hipStream_t s) {
    DeviceShape ds;
    int per_cu = 0;
    if (device_shape(ds) != WSL_OK) return WSL_E_DEVICE;
    const bool narrow = max_k <= 12 * 2048;
    const void *kern = narrow ? reinterpret_cast<const void *>(gemv_nf4_sweep_kernel<12>)
                              : reinterpret_cast<const void *>(gemv_nf4_sweep_kernel<16>);
    const int threads = narrow ? 768 : 1024;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess || per_cu < 1)
        return WSL_E_LAUNCH;
    const int nx = ds.xccs;
    const unsigned grid = static_cast<unsigned>(ds.cus / nx * nx);   // one workgroup per CU, all resident
    if (grid == 0) return WSL_E_DEVICE;
    if (narrow)
        hipLaunchKernelGGL((gemv_nf4_sweep_kernel<12>), dim3(grid), dim3(threads), 0, s, d_stages,
                           static_cast<int>(count), static_cast<uint32_t *>(ws), kSweepSpinLimit, nx);
    else
        hipLaunchKernelGGL((gemv_nf4_sweep_kernel<16>), dim3(grid), dim3(threads), 0, s, d_stages,
                           static_cast<int>(count), static_cast<uint32_t *>(ws), kSweepSpinLimit, nx);
    return WSL_OK;
}

}  // namespace wsl
