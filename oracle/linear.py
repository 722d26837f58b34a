"""fp64 references for y = W x (GEMV) and Y = X W^T (GEMM), and the tolerance checks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

IPE page, "What is built" / "How it is checked": an fp64 mode is the
numerical oracle; where reduction orders differ, results are judged by their
residual against fp64.  The residual bound used here: for an fp32 output,
|y - y_ref| <= 1e-4 * sum_j |w_j x_j| per output element; for a bf16 output
one extra bf16 ulp of |y_ref| is allowed for the final rounding.

Which weights each reference multiplies (Tarfa 2 blog, "Speculative
decoding": batched and unbatched evaluation round differently, so each kernel
is judged against what it is defined to compute):
* GEMV: the exact dequantized weight c * s (NF4) or the bf16 weight;
* GEMM: the restored bf16 tile bf16(fp32(c * s)) (NF4) or the bf16 weight.
The matmul is numpy's float64 BLAS product (a library primitive).
"""

import numpy as np

REL_TOL = 1e-4


def gemv_ref(w, x):
    """y = W x and S = |W| |x| in float64; w [n_out][k], x [k]."""
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return w @ x, np.abs(w) @ np.abs(x)


def gemm_ref(x, t):
    """Y = X T^T and S = |X| |T|^T in float64; x [m][k], t [n_out][k]."""
    x = np.asarray(x, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    return x @ t.T, np.abs(x) @ np.abs(t).T


def check_rows_f32(y, y_ref, s, rel=REL_TOL):
    """Elementwise |y - y_ref| <= rel * S; where S == 0, y must be exactly 0.

    Returns (ok: bool, worst ratio |y - y_ref| / (rel * S) over S > 0, index of the worst).
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return False, np.inf, int(np.argmax(~np.isfinite(y).ravel()))
    err = np.abs(y - y_ref)
    zero = (s == 0)
    if np.any(zero & (y != 0)):
        return False, np.inf, int(np.argmax((zero & (y != 0)).ravel()))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(zero, 0.0, err / (rel * s))
    i = int(np.argmax(ratio.ravel())) if ratio.size else 0
    worst = float(ratio.ravel()[i]) if ratio.size else 0.0
    return bool(worst <= 1.0), worst, i


def ulp_bf16(v):
    """Spacing of bf16 values in the binade that holds |v|: 2^(e-7) for |v| in [2^e, 2^(e+1)),
    and the subnormal spacing 2^-133 for |v| < 2^-126 (0 included).

    The binade e is read exactly from the binary exponent (frexp gives |v| = f * 2^x with
    f in [0.5, 1), so e = x - 1); a logarithm would round values just below a power of two
    up into the next binade."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, x = np.frexp(v)
    e = np.maximum(x.astype(np.int64) - 1, -126)
    return np.where(v > 0, np.ldexp(1.0, e - 7), np.ldexp(1.0, -133))


def check_bf16(y_bits, y_ref, s, rel=REL_TOL):
    """bf16 outputs: |y - y_ref| <= rel * S + ulp_bf16(|y_ref|)."""
    from .numfmt import f32_from_bf16_bits
    y = f32_from_bf16_bits(y_bits).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return False, np.inf, int(np.argmax(~np.isfinite(y).ravel()))
    bound = rel * s + ulp_bf16(y_ref)
    err = np.abs(y - y_ref)
    ratio = err / bound
    i = int(np.argmax(ratio.ravel())) if ratio.size else 0
    worst = float(ratio.ravel()[i]) if ratio.size else 0.0
    return bool(worst <= 1.0), worst, i
