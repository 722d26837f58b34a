"""NF4 group-64 encoding, byte packing, device layout and dequantization (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: deep-fold README, "Метод" section -- a group of 64 weights carries
4-bit NF4 codes and one FP16 scale; the codes-plus-scales payload is about
3.76x smaller than BF16 for aligned matrices (17/32 byte per weight: 4 bits
of code plus 16 bits of scale per 64 weights); the kernels restore only the
current tile's fragment; prefill restores into BF16 fragments.  deep-fold's
"Контрибьюторы" table: compression is checked by a CPU round trip.

Readings where the pages are silent:
* weights are y = W x with W stored [n_out][k], k contiguous; a group is 64
  consecutive k of one row, so k must be a multiple of 64;
* scale s = fp16_RNE(max |w|) over the group; codes are chosen against the
  stored s (the dequantizer only ever sees s);
* code = nearest level to w / s, ties to the lower index, evaluated exactly
  as code(w) = #{i : w > m_i * s} with midpoints m_i = (c_i + c_{i+1}) / 2
  (exact in float64, as is m_i * s);
* an all-zero (or fp16-underflowing) group stores s = +0 and every code 7
  (the exact-zero level); a non-finite weight or s = inf is an error;
* two codes per byte, the even k in the low nibble;
* dequantized value for the GEMV: c * s (exact); restored tile value for the
  GEMM: bf16_RNE(fp32_RN(c * s)).

Device layout (a fixed bijection of the canonical bytes, built for gfx950):
* codes: row-major [n_out][k/2] bytes; every aligned little-endian 32-bit
  word (codes k = 8j .. 8j+7 of one row) is rotated LEFT by 2 bits;
* scales: follow the codes; rows are taken in blocks of 16 (the last block
  may be shorter, rb rows); inside a block the order is [group][row], i.e.
  scale (n, g) sits at index (n // 16) * 16 * G + g * rb + n % 16.
"""

import numpy as np

from .numfmt import fp16_from_real, f64_from_fp16, bf16_bits_from_f32
from .codebook import nf4_levels_f32

GROUP = 64
SCALE_ROW_BLOCK = 16


class PackError(ValueError):
    """Raised for inputs the encoding does not define (non-finite, fp16 overflow)."""


def nf4_midpoints(levels=None):
    """m_i = (c_i + c_{i+1}) / 2, i = 0..14, in float64 (exact for binary32 levels)."""
    c = (nf4_levels_f32() if levels is None else np.asarray(levels, np.float32)).astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def pack_codes(w, levels=None, rows_per_chunk=256):
    """Encode w [n_out][k] (any real dtype, exact values) into codes and scales.

    Returns (codes uint8 [n_out][k] in 0..15, scales float16 [n_out][k/64]).
    """
    w = np.asarray(w)
    if w.ndim != 2 or w.shape[1] % GROUP != 0:
        raise PackError("w must be [n_out][k] with k a multiple of 64")
    n_out, k = w.shape
    g = k // GROUP
    mids = nf4_midpoints(levels)
    codes = np.empty((n_out, k), dtype=np.uint8)
    scales = np.empty((n_out, g), dtype=np.float16)
    for r0 in range(0, n_out, rows_per_chunk):
        wc = w[r0:r0 + rows_per_chunk].astype(np.float64)
        if not np.all(np.isfinite(wc)):
            raise PackError("non-finite weight")
        wg = wc.reshape(wc.shape[0], g, GROUP)
        a = np.max(np.abs(wg), axis=2)                 # exact absmax per group
        with np.errstate(over="ignore"):
            s = fp16_from_real(a)                      # stored scale
        if np.any(np.isinf(s)):
            raise PackError("group absmax overflows fp16")
        s64 = f64_from_fp16(s)
        thr = mids[None, None, :] * s64[:, :, None]    # exact products m_i * s
        cnt = np.zeros(wg.shape, dtype=np.uint8)
        for i in range(mids.size):
            cnt += (wg > thr[:, :, i:i + 1]).astype(np.uint8)
        zero = (s64 == 0.0)
        if zero.any():
            cnt[zero] = 7
            s = np.where(zero, np.float16(0.0), s)     # +0, never -0
        codes[r0:r0 + rows_per_chunk] = cnt.reshape(wc.shape[0], k)
        scales[r0:r0 + rows_per_chunk] = s
    return codes, scales


def codes_to_bytes(codes):
    """Two codes per byte: byte j = code[2j] | code[2j+1] << 4 (low nibble = even k)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def bytes_to_codes(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def packed_bytes(n_out, k):
    """Size of a packed matrix: n_out*k/2 code bytes + n_out*(k/64) fp16 scales."""
    return n_out * k // 2 + n_out * (k // GROUP) * 2


def _scale_perm(n_out, g):
    """Index map: device scale position -> canonical flat index n*g_count + grp."""
    idx = np.empty(n_out * g, dtype=np.int64)
    pos = 0
    for b0 in range(0, n_out, SCALE_ROW_BLOCK):
        rb = min(SCALE_ROW_BLOCK, n_out - b0)
        rows = np.arange(b0, b0 + rb)
        blk = rows[None, :] * g + np.arange(g)[:, None]   # [grp][row]
        idx[pos:pos + rb * g] = blk.reshape(-1)
        pos += rb * g
    return idx


def device_from_canonical(code_bytes, scales):
    """Canonical (bytes [n_out][k/2], scales fp16 [n_out][G]) -> device buffer (uint8 1-D)."""
    cb = np.ascontiguousarray(code_bytes, dtype=np.uint8)
    n_out, half_k = cb.shape
    words = cb.view("<u4").astype(np.uint64)
    rot = (((words << np.uint64(2)) | (words >> np.uint64(30))) & np.uint64(0xFFFFFFFF)).astype("<u4")
    sc = np.ascontiguousarray(scales, dtype=np.float16).reshape(-1)
    g = scales.shape[1]
    dev_sc = sc[_scale_perm(n_out, g)]
    return np.concatenate([rot.view(np.uint8).reshape(-1), dev_sc.view(np.uint8)])


def canonical_from_device(buf, n_out, k):
    """Inverse of ``device_from_canonical``."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    half_k = k // 2
    g = k // GROUP
    nb = n_out * half_k
    words = buf[:nb].view("<u4").astype(np.uint64)
    orig = (((words >> np.uint64(2)) | (words << np.uint64(30))) & np.uint64(0xFFFFFFFF)).astype("<u4")
    cb = orig.view(np.uint8).reshape(n_out, half_k)
    dev_sc = buf[nb:nb + n_out * g * 2].view(np.float16)
    sc = np.empty(n_out * g, dtype=np.float16)
    sc[_scale_perm(n_out, g)] = dev_sc
    return cb, sc.reshape(n_out, g)


def pack_device(w, levels=None):
    """Encode and lay out: w [n_out][k] -> device buffer (uint8 1-D)."""
    codes, scales = pack_codes(w, levels)
    return device_from_canonical(codes_to_bytes(codes), scales)


def dequant_exact(codes, scales, levels=None):
    """w_hat = c[code] * s, in float64 (exact)."""
    c = (nf4_levels_f32() if levels is None else np.asarray(levels, np.float32)).astype(np.float64)
    codes = np.asarray(codes)
    n_out, k = codes.shape
    s = np.repeat(f64_from_fp16(scales), GROUP, axis=1)
    return c[codes] * s


def dequant_tile_bits(codes, scales, levels=None):
    """Restored GEMM tile values t = bf16_RNE(fp32_RN(c * s)); returns uint16 bf16 bits."""
    c = (nf4_levels_f32() if levels is None else np.asarray(levels, np.float32))
    codes = np.asarray(codes)
    s32 = np.repeat(np.asarray(scales, np.float16).astype(np.float32), GROUP, axis=1)
    prod = (c[codes].astype(np.float32) * s32).astype(np.float32)   # one binary32 rounding
    return bf16_bits_from_f32(prod)
