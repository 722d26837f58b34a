"""Number-format helpers of the oracle (bf16 and IEEE binary16).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The deep-fold README ("Метод" section) stores one FP16 scale per group of 64
weights and restores weights into BF16 register fragments for the prefill
GEMM.  These helpers define the roundings used for both:

* bf16 is the upper 16 bits of an IEEE binary32 value; rounding from binary32
  is round-to-nearest, ties to even, on the bit pattern.  NaN stays NaN
  (quiet), infinities stay infinities, overflow rounds to infinity.
* binary16 rounding is IEEE round-to-nearest-even with subnormals, done by
  numpy's direct float64 -> float16 conversion (a single rounding).
"""

import numpy as np


def bf16_bits_from_f32(a):
    """Round binary32 values to bf16 (RNE on the bit pattern); returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        # keep sign and payload top bits, force the quiet bit
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b):
    """Widen bf16 bit patterns to binary32 values (exact)."""
    u = np.ascontiguousarray(np.asarray(b, dtype=np.uint16)).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def bf16_bits_from_f64_via_f32(a):
    """bf16 bits of ``bf16_RNE(fp32_RN(a))`` for float64 input (two roundings by definition)."""
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float64).astype(np.float32))


def fp16_from_real(a):
    """IEEE binary16 round-to-nearest-even of float64 values (subnormals kept, overflow -> inf)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def f64_from_fp16(h):
    """Widen binary16 values to float64 (exact)."""
    return np.asarray(h, dtype=np.float16).astype(np.float64)
