"""Plain CPU oracle for weight-streaming linear layers (NF4 group-64 and bf16).

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct CPU
reference that the HIP library is checked against.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``weight_streaming_linear_amd``) never imports
it, and this package never imports the product: the two share no code.  The
only module both sides use is ``synth`` (seeded input generation), which
holds none of the method's arithmetic.

Sources (the pages describing the method):
  * deep-fold README ("Метод" section): a group of 64 weights holds 4-bit NF4
    codes and one FP16 scale; kernels restore only the current tile's
    fragment; prefill restores into BF16 register fragments; NF4 was
    introduced in QLoRA; the payload is about 3.76x smaller than BF16.
  * deep-fold README ("Контрибьюторы" table): compression is checked by a
    round trip on the CPU.
  * IPE page ("What is built", "How it is checked"): an fp64 mode serves as
    the numerical oracle; bitwise parity where the order of operations is the
    same, residuals against fp64 where it differs.
  * Tarfa 2 blog ("Speculative decoding" section): batched and unbatched
    evaluation round differently, so GEMV and GEMM are each checked against
    their own reference.

Every function computes in float64 (or exact integer/rational arithmetic)
unless a rounding step is part of the definition.

Parity status: the NF4 level *values* are parity-unpinned by the pages (no
codebook table is printed); they follow the QLoRA normal-quantile
construction as read in ``oracle.codebook``.  Everything else is pinned by
exhaustive, brute-force or closed-form checks in ``tests/``.
"""

from .numfmt import (bf16_bits_from_f32, f32_from_bf16_bits, fp16_from_real,
                     f64_from_fp16, bf16_bits_from_f64_via_f32)
from .codebook import nf4_levels_f64, nf4_levels_f32, NF4_DELTA
from .nf4 import (GROUP, SCALE_ROW_BLOCK, PackError, nf4_midpoints, pack_codes,
                  codes_to_bytes, bytes_to_codes, device_from_canonical,
                  canonical_from_device, packed_bytes, dequant_exact,
                  dequant_tile_bits, pack_device)
from .linear import (gemv_ref, gemm_ref, check_rows_f32, check_bf16,
                     ulp_bf16)

__all__ = [
    "bf16_bits_from_f32", "f32_from_bf16_bits", "fp16_from_real",
    "f64_from_fp16", "bf16_bits_from_f64_via_f32",
    "nf4_levels_f64", "nf4_levels_f32", "NF4_DELTA",
    "GROUP", "SCALE_ROW_BLOCK", "PackError", "nf4_midpoints", "pack_codes",
    "codes_to_bytes", "bytes_to_codes", "device_from_canonical",
    "canonical_from_device", "packed_bytes", "dequant_exact",
    "dequant_tile_bits", "pack_device",
    "gemv_ref", "gemm_ref", "check_rows_f32", "check_bf16", "ulp_bf16",
]
