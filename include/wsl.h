/*
 * wsl.h -- C ABI of the weight-streaming linear library for AMD Instinct MI355X (gfx950).
 *
 * The library computes the linear layers y = W x of a decoder whose weights W
 * are held either as plain bf16 or as packed NF4 (4-bit codes in groups of 64
 * along K plus one fp16 scale per group).  NF4 weights stay packed in device
 * memory and are dequantized in registers inside the linear kernels; no dense
 * copy of W is ever written back.  Sources:
 *   - deep-fold README, "Метод" section: codes and scales live in video
 *     memory; linear kernels restore only the fragment of the current tile
 *     and never write a dense weight matrix back; a group of 64 weights holds
 *     4-bit NF4 codes and one FP16 scale; prefill is a GEMM that restores
 *     into BF16 register fragments for batches of up to 32 positions, decode
 *     an N=1 GEMV; both paths share one compressed representation (Figure 1).
 *   - TCPP README, "What exact means here": bf16 weights used as stored, no
 *     dequantization; "Quickstart"/"Performance": batch verification scores
 *     every position of a K-token context in one sweep (a wide GEMM).
 *   - IPE page, "What is built": a decode step indexes preallocated buffers
 *     with host integers and never reads device values back; "How it is
 *     checked": zero host-device synchronizations and zero allocator growth.
 *
 * Conventions for every entry point:
 *   - Shapes are int64_t.  W is [n_out][k] row-major (k contiguous), like a
 *     torch Linear weight; y = W x has n_out entries; the GEMM computes
 *     Y[m][n_out] = X[m][k] * W^T for m token positions.
 *   - Pointers named d_* or documented "device" are caller-owned device
 *     memory; "host" pointers are ordinary host memory.  The library never
 *     allocates, frees, copies or synchronizes: every call only validates its
 *     arguments on the host and enqueues kernels on `stream` (a hipStream_t;
 *     NULL means the default stream), so calls are legal inside HIP stream or
 *     graph capture.
 *   - Argument errors are returned synchronously, before anything is
 *     enqueued (nothing is launched).  Launch failures are reported as
 *     WSL_E_LAUNCH (from hipGetLastError, which does not synchronize).
 *     Errors in the *data* (non-finite weights) are reported through an
 *     optional device status word (nf4_pack only).
 *   - The library refuses any device other than gfx950 (WSL_E_DEVICE).
 *   - Results are deterministic: no floating-point atomics; the same inputs
 *     give the same bits on every run.
 *   - Calls that share output buffers and overlap on one device race; calls
 *     on the same stream are ordered.
 */
#ifndef WSL_H
#define WSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
    WSL_OK = 0,
    WSL_E_NULL = 1,    /* a required pointer is NULL */
    WSL_E_SHAPE = 2,   /* a size <= 0 (or < 0 where 0 is allowed), k % 64 != 0, or a size overflow */
    WSL_E_ALIGN = 3,   /* a pointer or leading dimension breaks the documented alignment */
    WSL_E_FORMAT = 4,  /* unknown weight or output format */
    WSL_E_DEVICE = 5,  /* current device is not gfx950, or the device query failed */
    WSL_E_LAUNCH = 6,  /* a kernel launch failed */
    WSL_E_RANGE = 7,   /* a tile or workspace lies outside its matrix or buffer */
    WSL_E_MEMORY = 8,  /* a host buffer of a streamed call is not pinned (page-locked) host memory */
    WSL_E_SCRATCH = 9, /* linear_gemm_noalloc: the shape needs more split workspace than its scratch holds */
    WSL_E_FLAGS = 10   /* a flags argument holds a bit the call does not define */
};

/* Weight formats. */
enum { WSL_W_BF16 = 0, WSL_W_NF4 = 1 };
/* Output formats. */
enum { WSL_OUT_F32 = 0, WSL_OUT_BF16 = 1 };

/* Bits OR-ed into nf4_pack's optional device status word. */
#define WSL_STATUS_NONFINITE 1u   /* a group held a NaN or an infinity */
#define WSL_STATUS_OVERFLOW  2u   /* a group's absmax rounds to +inf in fp16 (>= 65520) */
#define WSL_STATUS_INDEX     4u   /* nf4_embed_rows: a requested row index was outside the matrix */
#define WSL_STATUS_SWEEP_TIMEOUT 8u   /* linear_gemv_sweep: a stage barrier waited past its bound */
#define WSL_STATUS_DESCRIPTOR    16u  /* linear_gemv_sweep: a device stage descriptor was invalid (skipped) */

/* Flags of linear_gemv_streamed / linear_gemm_streamed. */
#define WSL_RING_PACE 1   /* the host keeps the copies at most two matrices ahead of the kernels */

/*
 * nf4_packed_bytes -- size in bytes of one packed NF4 matrix.
 *   = n_out*k/2 (codes, 4 bits each) + n_out*(k/64)*2 (fp16 scales),
 *   i.e. 17/32 byte per weight (deep-fold README, "Метод": the payload is
 *   about 3.76x smaller than BF16 for aligned matrices).
 *   Returns 0 if n_out <= 0, k <= 0, k % 64 != 0 or the size overflows.
 */
size_t nf4_packed_bytes(int64_t n_out, int64_t k);

/*
 * nf4_codebook -- copies the 16 binary32 NF4 levels (ascending; c[0] = -1,
 * c[7] = +0, c[15] = +1) into host memory out_host[0..15].  The levels are
 * normal quantiles with an exact zero, scaled to [-1, 1] (NF4 as introduced
 * in QLoRA, credited in deep-fold README, "Метод").  Returns WSL_E_NULL if
 * out_host is NULL.
 */
int nf4_codebook(float *out_host);

/*
 * nf4_pack -- encode a bf16 weight matrix into the packed NF4 device layout.
 *   (deep-fold README, "Метод": per group of 64 weights, 4-bit NF4 codes and
 *   one FP16 scale; the compressor there runs offline on the CPU.)
 * d_w       device, bf16 [n_out][k], 16-byte aligned (read only).
 * n_out, k  n_out >= 1, k >= 64, k % 64 == 0.
 * d_packed  device, nf4_packed_bytes(n_out, k) bytes, 16-byte aligned (written).
 * d_status  device uint32 or NULL.  If non-NULL, the kernel ORs
 *           WSL_STATUS_* bits into it for groups it cannot encode (the
 *           caller zeroes it first).  Such a group is written as s = +0 with
 *           every code 7, i.e. as zeros.
 * Encoding per row and group of 64 consecutive k: s = fp16_RNE(max|w|);
 * code = nearest level to w/s with ties to the lower index, decided
 * exactly as #{i : w > m_i * s} in fp64, m_i = (c_i + c_{i+1}) / 2; an
 * all-zero or fp16-underflowing group stores s = +0 and codes 7.
 * Layout written:
 *   codes  bytes [0, n_out*k/2): row-major, two codes per byte (even k in the
 *          low nibble), and every aligned little-endian 32-bit word (codes
 *          k = 8j..8j+7 of a row) rotated left by 2 bits;
 *   scales fp16 following the codes; rows in blocks of 16 (the last block
 *          may have rb < 16 rows), ordered [group][row] inside a block:
 *          scale(n, g) at index (n/16)*16*(k/64) + g*rb + n%16.
 * Bit-exact and deterministic.
 */
int nf4_pack(const void *d_w, int64_t n_out, int64_t k, void *d_packed,
             uint32_t *d_status, void *stream);

/*
 * nf4_dequant_tile -- restore a rectangular tile of a packed NF4 matrix to bf16.
 *   (deep-fold README, "Метод": kernels restore only the current tile's
 *   fragment into BF16.)  A test and diagnostic export: the linear kernels
 *   restore tiles in registers and never call it.
 * Value written for (r, c): bf16_RNE(fp32_RN(level[code] * s)) of weight
 * (row0 + r, k0 + c).  Tile: rows x cols at d_tile[r*ld_tile + c] (bf16).
 * Requires 0 <= row0, rows >= 1, row0 + rows <= n_out, 0 <= k0, cols >= 1,
 * k0 + cols <= k (else WSL_E_RANGE), ld_tile >= cols, d_tile 2-byte aligned.
 */
int nf4_dequant_tile(const void *d_packed, int64_t n_out, int64_t k,
                     int64_t row0, int64_t k0, int64_t rows, int64_t cols,
                     void *d_tile, int64_t ld_tile, void *stream);

/*
 * linear_gemv -- decode (one position): y[n] = sum_k W[n][k] * x[k], fp32 result.
 *   (deep-fold README, "Метод" table: decode is an N=1 NF4 GEMV; TCPP
 *   README: bf16 weights used as stored.)
 * wfmt      WSL_W_BF16: d_w is bf16 [n_out][k], 16-byte aligned;
 *           WSL_W_NF4 : d_w is a packed NF4 matrix (nf4_pack layout).
 * d_x       device bf16 [k], 16-byte aligned.   d_y device fp32 [n_out], 4-byte aligned.
 * n_out >= 1; k >= 64 and k % 64 == 0 for NF4; k >= 8 and k % 8 == 0 for bf16.
 * Accumulation is fp32.  NF4 multiplies the binary32 level by x and applies
 * the fp32 scale once per group partial sum; each row satisfies
 * |y - y_exact| <= 1e-4 * sum_k |w_hat x| with w_hat = level * s exactly.
 */
int linear_gemv(int wfmt, const void *d_w, int64_t n_out, int64_t k,
                const void *d_x, float *d_y, void *stream);

/* One stage of linear_gemv_sweep: y = W x with W a packed NF4 [n_out][k] matrix. */
typedef struct wsl_gemv_stage {
    const void *w;   /* device, packed NF4 (nf4_pack layout), 16-byte aligned */
    const void *x;   /* device, bf16 [k], 16-byte aligned */
    float *y;        /* device, fp32 [n_out], 4-byte aligned */
    int64_t n_out;   /* >= 1 */
    int64_t k;       /* 64 <= k <= 32768, k % 64 == 0 */
} wsl_gemv_stage;

/*
 * linear_gemv_sweep_workspace_bytes -- size of the synchronization workspace that
 * linear_gemv_sweep needs (a few KB of counters).
 */
size_t linear_gemv_sweep_workspace_bytes(void);

/*
 * linear_gemv_sweep -- a decode sweep: `count` NF4 GEMVs (the linear stages of every
 * layer of a decoder, in decoder order) in one launch.
 *   (deep-fold README, "Метод" table: decode runs N=1 NF4 GEMVs inside one graph of
 *   the whole greedy step; a token's step sweeps every layer's weights once.)
 * Computes, for i = 0 .. count-1, what linear_gemv(WSL_W_NF4, ...) of stage i computes
 * (same per-row tolerance: |y - y_exact| <= 1e-4 * sum_k |w_hat x|).  The stages run in
 * order: no part of stage i + 1 starts (nor reads its x) before every part of stage i
 * has finished (a device-wide barrier between stages); the loads of its weights may
 * begin earlier.  No stage may read another stage's output: every y must be disjoint
 * from every w and x of the call.  Every y is written when the call completes.
 * wfmt       WSL_W_NF4 (bf16 weights return WSL_E_FORMAT).
 * count      number of stages, 0 <= count <= 2^24 (0 enqueues nothing).
 * h_stages   host array of count descriptors: every argument is validated from it
 *            before anything is enqueued (as linear_gemv validates; k <= 32768).
 * d_stages   device array holding the same count descriptors (8-byte aligned), which
 *            the kernel reads.  If the two differ the results are undefined; a device
 *            descriptor that is invalid is skipped and WSL_STATUS_DESCRIPTOR is ORed
 *            into the status word.
 * d_ws       device workspace of at least linear_gemv_sweep_workspace_bytes() bytes,
 *            128-byte aligned, all zero before the first call; every call leaves it
 *            zero again except the status word, its uint32 at byte offset 1280, into
 *            which WSL_STATUS_SWEEP_TIMEOUT / WSL_STATUS_DESCRIPTOR bits are ORed (a
 *            caller that sees a nonzero status zeroes the workspace before reuse).
 *            Calls that share a workspace must not overlap.
 * The call launches one workgroup per compute unit and needs all of them resident at
 * once (nothing else occupying the GPU's compute units); a barrier that is not reached
 * within about a second is abandoned with WSL_STATUS_SWEEP_TIMEOUT so the kernel always
 * ends.  Deterministic: the same inputs give the same bits.
 */
int linear_gemv_sweep(int wfmt, int64_t count, const wsl_gemv_stage *h_stages,
                      const wsl_gemv_stage *d_stages, void *d_ws, size_t ws_bytes, void *stream);

/*
 * linear_gemv_multi -- several independent bf16 GEMVs in one launch: y_i = W_i x_i for
 * i < count, bit for bit what count linear_gemv calls give.  For matrices that read the
 * same k and none of whose outputs another reads -- a layer's q, k and v projections, or
 * its gate and up projections, kept as separate tensors (TCPP README, "What 'exact' means
 * here": weights used as stored) -- so that they share one launch instead of paying one
 * launch each (IPE page, "How it is benchmarked": a decode step's linear layers).
 * wfmt      WSL_W_BF16 (WSL_W_NF4: WSL_E_FORMAT; linear_gemv_sweep serves NF4 layers).
 * count     0 <= count <= WSL_GEMV_MULTI_MAX; 0 enqueues nothing.
 * h_stages  host array of count descriptors (read before the call returns), each with
 *           linear_gemv's bf16 arguments: w bf16 [n_out][k] 16-byte aligned, x bf16 [k]
 *           16-byte aligned, y fp32 [n_out] 4-byte aligned, n_out >= 1, k >= 8,
 *           k % 8 == 0; every descriptor has the same k (else WSL_E_SHAPE).
 * Returns linear_gemv's errors for a bad descriptor; asynchronous on stream.
 */
#define WSL_GEMV_MULTI_MAX 8
int linear_gemv_multi(int wfmt, int64_t count, const wsl_gemv_stage *h_stages, void *stream);

/*
 * linear_gemm_workspace_bytes -- workspace linear_gemm can use for a shape
 * (0 if it would not split the reduction): splits * m * n_out * 4 bytes of fp32
 * partials, for a k split of the shared-X kernels or of the 256 x 256 tiles
 * (a launch whose tiles would leave most compute units idle).  Passing a smaller
 * (or NULL) workspace is legal and only selects a path with less parallelism.
 */
size_t linear_gemm_workspace_bytes(int wfmt, int64_t n_out, int64_t k, int64_t m);

/*
 * linear_gemm -- prefill / batch verification: Y[i][n] = sum_k X[i][k] * T[n][k].
 *   (deep-fold README, "Метод" table: prefill is an NF4 GEMM that restores
 *   weights into BF16 register fragments; TCPP README, "Quickstart" and
 *   "Performance": batch verification over thousands of positions.)
 * T is the bf16 weight (WSL_W_BF16) or the restored bf16 tile value
 * bf16_RNE(fp32_RN(level * s)) (WSL_W_NF4).  Products are accumulated in fp32
 * on the matrix cores (MFMA); Y is written as fp32 (WSL_OUT_F32) or rounded
 * once to bf16 (WSL_OUT_BF16, round to nearest even).
 * d_x       device bf16 [m][ldx], ldx >= k, ldx % 8 == 0, 16-byte aligned.
 * d_y       device [m][ldy] of the output type, ldy >= n_out, aligned to its element size.
 * m >= 1.   n_out, k as for linear_gemv (k % 64 == 0 for both formats).
 * d_ws      optional device workspace (16-byte aligned) of ws_bytes bytes.
 *           It holds split-reduction partials; its contents on entry do not
 *           matter.  Calls that share a workspace and overlap race.
 */
int linear_gemm(int wfmt, const void *d_w, int64_t n_out, int64_t k,
                const void *d_x, int64_t m, int64_t ldx,
                void *d_y, int ofmt, int64_t ldy,
                void *d_ws, size_t ws_bytes, void *stream);

/*
 * linear_gemm_noalloc -- linear_gemm for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and kernels as linear_gemm; instead of a caller workspace, the
 * split-reduction partials go to a scratch array of WSL_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory of every GPU it runs on, from the first call on that GPU
 * until the process ends.  The call itself allocates nothing: on its first call on a device
 * it looks up that device's copy of the array (hipGetSymbolAddress), afterwards it only
 * enqueues kernels.  When the shape's split workspace (linear_gemm_workspace_bytes) fits in
 * the scratch, the results are bit for bit those of linear_gemm given that workspace.
 * Beyond it, a shape that runs on the 256 x 256 tiles runs them without a k split (bit for
 * bit linear_gemm without a workspace), and any other shape returns WSL_E_SCRATCH,
 * launching nothing (4 MiB is enough for every shape at up to 32 positions with
 * k % 256 == 0, the prefill width); linear_gemm with a caller workspace serves those.
 * Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one device (different streams, or different host threads without
 * ordering) race and may return wrong results; calls ordered on one stream do not.
 */
#define WSL_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int linear_gemm_noalloc(int wfmt, const void *d_w, int64_t n_out, int64_t k,
                        const void *d_x, int64_t m, int64_t ldx,
                        void *d_y, int ofmt, int64_t ldy, void *stream);

/*
 * nf4_embed_rows -- restore only the requested rows of a packed NF4 matrix (a
 * packed embedding table [n_rows][k]).
 *   (deep-fold README, introduction and Figure 1: embeddings stay packed and
 *   only the rows that are asked for are restored, separately from the linear
 *   kernels.)
 * d_packed  device, nf4_pack layout of an [n_rows][k] matrix, 16-byte aligned.
 * d_ids     device int64 [count], the rows to restore (any order, repeats allowed),
 *           8-byte aligned.  Read by the kernel only: indices are never copied
 *           to the host.
 * count     >= 0 (0 launches nothing; d_ids and d_out may then be NULL).
 * d_out     device [count][ld_out], 16-byte aligned; row i receives row d_ids[i]:
 *           WSL_OUT_BF16: bf16_RNE(fp32_RN(level * s)) (the restored tile value,
 *                         bit-identical to nf4_dequant_tile), ld_out % 8 == 0;
 *           WSL_OUT_F32 : fp32_RN(level * s), ld_out % 4 == 0.
 *           ld_out >= k; entries past k are not written.
 * d_status  device uint32 or NULL.  An index outside [0, n_rows) gives an
 *           all-zero output row and ORs WSL_STATUS_INDEX into *d_status.
 * Bit-exact and deterministic.
 */
int nf4_embed_rows(const void *d_packed, int64_t n_rows, int64_t k, const int64_t *d_ids, int64_t count,
                   void *d_out, int ofmt, int64_t ld_out, uint32_t *d_status, void *stream);

/*
 * linear_gemv_streamed / linear_gemm_streamed -- the linear kernels over matrices
 * that live in pinned host memory, brought to the device through two reusable
 * caller-owned device slots (a copy ring).
 *   (deep-fold README, "Метод" table and Figure 1: a model larger than the GPU
 *   budget keeps selected packed matrices in pinned host memory and passes them
 *   through two reusable device slots to the same kernels; the 32B model of the
 *   results keeps 9.5 GiB resident and 6.7 GiB in pinned host memory.)
 * For matrix i (slot s = i % 2) the call enqueues:
 *   copy_stream:    wait events[2 + s]; copy h_w[i] -> d_slot[s]; record events[s];
 *   compute_stream: wait events[s]; linear_gemv / linear_gemm on d_slot[s];
 *                   record events[2 + s].
 * So the copy of matrix i + 1 runs while matrix i is multiplied, and a slot is
 * overwritten only after the kernel that read it finished (also across calls,
 * since the events carry over).  Without WSL_RING_PACE the call enqueues everything
 * without waiting (it may be captured in a graph).  With it, before enqueueing the copy
 * of matrix i >= 2 the host waits for events[2 + s] -- the kernel of matrix i - 2, which
 * that copy waits for on the device anyway -- so the call returns once the kernel of
 * matrix count - 3 has finished.  The pacing is for long streams: when hundreds of copies
 * that each wait on a kernel of another stream are enqueued ahead, the HIP runtime can
 * hold the host inside a copy's enqueue for milliseconds, long enough for the copy engine
 * to run out of queued copies; kept two matrices ahead, the ring stays within a few
 * percent of the rate of plain back-to-back copies.
 * wfmt          WSL_W_NF4 or WSL_W_BF16, the format of every h_w[i].
 * count         number of matrices (>= 0; 0 enqueues nothing).
 * h_w           host array of count pointers to page-locked host buffers (allocated
 *               with hipHostMalloc; any other host memory gives WSL_E_MEMORY), each
 *               holding a matrix in its device format (nf4_pack layout, or bf16
 *               [n_out][k]).  They must stay allocated until the copies complete.
 * n_out, k      host arrays of count shapes (as for linear_gemv / linear_gemm).
 * d_x, d_y      host arrays of count device pointers: GEMV x bf16 [k] and y fp32
 *               [n_out]; GEMM X bf16 [m][ldx] and Y [m][ldy] of type ofmt.
 * m, ldx, ldy, ofmt, d_ws, ws_bytes   GEMM only, shared by every matrix (the
 *               workspace is used by one kernel at a time: all run on compute_stream).
 * d_slot        host array of 2 device pointers, 16-byte aligned, slot_bytes each;
 *               every matrix must fit (else WSL_E_RANGE).
 * copy_stream, compute_stream   hipStream_t (NULL = default stream); inputs and
 *               outputs are ordered on compute_stream.
 * events        host array of 4 hipEvent_t created by the caller.
 * flags         0 or WSL_RING_PACE (other bits: WSL_E_FLAGS).
 * Every argument is validated before anything is enqueued; a HIP error while
 * enqueuing (or waiting, with WSL_RING_PACE) returns WSL_E_LAUNCH (earlier matrices
 * may already be enqueued).
 */
int linear_gemv_streamed(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
                         const void *const *d_x, float *const *d_y, void *const *d_slot, size_t slot_bytes,
                         void *copy_stream, void *compute_stream, void *const *events, int flags);
int linear_gemm_streamed(int wfmt, int64_t count, const void *const *h_w, const int64_t *n_out, const int64_t *k,
                         const void *const *d_x, int64_t m, int64_t ldx, void *const *d_y, int ofmt, int64_t ldy,
                         void *d_ws, size_t ws_bytes, void *const *d_slot, size_t slot_bytes,
                         void *copy_stream, void *compute_stream, void *const *events, int flags);

/*
 * wsl_stream_read -- measurement aid, not part of the linear path: a read-only
 * kernel that reads bytes bytes at d_buf once, with the access form of the GEMV
 * weight stream (16-byte loads that bypass the caches, 1 KB of consecutive bytes
 * per wave instruction; one 8-wave workgroup per compute unit, three such
 * loads in flight per wave), so that its rate over a buffer much larger than
 * the caches is the streaming-read ceiling the GB/s
 * figures are compared with (a figure the pages do not give: measured on the GPU at hand).
 * d_buf    device, 16-byte aligned; bytes a multiple of 16.  bytes == 0 enqueues
 *          nothing and returns 0.
 * d_sink   device uint32 [1], 4-byte aligned: each lane XOR-combines the words it
 *          reads and writes the result to d_sink[0] only if it equals 0x9e3779b9,
 *          so the kernel writes nothing in practice (a test plants that value to
 *          check that every word is read).
 * Returns WSL_E_NULL, WSL_E_SHAPE (bytes % 16 != 0), WSL_E_ALIGN, WSL_E_DEVICE or
 * WSL_E_LAUNCH as the other entry points do; asynchronous on stream.
 */
int wsl_stream_read(const void *d_buf, size_t bytes, uint32_t *d_sink, void *stream);

/* wsl_strerror -- static description of a status code (never NULL). */
const char *wsl_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* WSL_H */
