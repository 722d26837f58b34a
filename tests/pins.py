"""Independent checks that pin the CPU oracle to the mathematics (no GPU).

Each ``pin_*`` function returns True when the oracle agrees with something
other than itself: an exact rational re-derivation of an IEEE rounding, a
bisection inverse of the normal CDF built on ``math.erfc``, brute-force
argmin over the 16 levels, hand-written byte fixtures, closed forms or pure
Python loops over Fractions.  The mutation tests plant defects in the oracle
and require that some pin returns False.

Oracle functions are looked up through their modules at call time
(``oracle.nf4.pack_codes`` rather than a name imported once) so that a
planted defect is seen.
"""

import math
import os
from fractions import Fraction

import numpy as np

import oracle.numfmt as onum
import oracle.codebook as ocb
import oracle.nf4 as onf4
import oracle.linear as olin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact rounding
def _floor_log2(q):
    """Exact floor(log2(q)) for a positive Fraction."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_binary(q, p, emin, emax):
    """IEEE round-to-nearest-even of a rational to a binary format with p significant
    bits, minimum normal exponent emin and maximum exponent emax.  Returns a Fraction,
    or +-inf (float) on overflow."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def fp16_exact(q):
    return round_binary(q, 11, -14, 15)


def bf16_exact(q):
    return round_binary(q, 8, -126, 127)


def all_positive_finite_bf16_bits():
    b = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    return b


# ---------------------------------------------------------------- number formats
def pin_fp16_rounding_exhaustive():
    """Every positive finite bf16 value: oracle fp16 RNE == exact rational RNE."""
    bits = all_positive_finite_bf16_bits()
    vals = onum.f32_from_bf16_bits(bits).astype(np.float64)
    with np.errstate(over="ignore"):
        got = onum.fp16_from_real(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        want = fp16_exact(Fraction(v))
        if isinstance(want, float):
            if not math.isinf(g):
                return False
        elif Fraction(g) != want:
            return False
    return True


def pin_fp16_rounding_f32_sample(n=20000, seed=7):
    """A sample of binary32 values incl. fp16 subnormal range and ties."""
    rng = np.random.default_rng(seed)
    e = rng.integers(-30, 17, size=n)
    m = rng.integers(0, 1 << 23, size=n)
    v = np.ldexp(1.0 + m / float(1 << 23), e).astype(np.float32).astype(np.float64)
    # exact ties of the fp16 grid: (2j+1) * 2^-25 (subnormal) and 1 + (2j+1) * 2^-11
    ties = np.concatenate([(2 * np.arange(50) + 1) * 2.0 ** -25, 1.0 + (2 * np.arange(50) + 1) * 2.0 ** -11,
                           [65504.0, 65519.0, 65520.0, 2.0 ** -25, 2.0 ** -26 * 3]])
    v = np.concatenate([v, ties])
    with np.errstate(over="ignore"):
        got = onum.fp16_from_real(v)
    for x, g in zip(v.tolist(), got.tolist()):
        want = fp16_exact(Fraction(x))
        if isinstance(want, float):
            if not math.isinf(g):
                return False
        elif Fraction(g) != want:
            return False
    return True


def pin_bf16_rounding(n=200000, seed=11):
    """bf16 RNE of binary32: oracle bit formula == torch's cast on a large sample, and
    == exact rational rounding on a smaller sample that includes exact ties."""
    import torch
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    # force a share of exact ties (low 16 bits = 0x8000) and near-ties
    u[: n // 8] = (u[: n // 8] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[n // 8: n // 4] = (u[n // 8: n // 4] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    f = u.view(np.float32)
    fin = np.isfinite(f)
    f = f[fin]
    got = onum.bf16_bits_from_f32(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(got, want):
        return False
    for x, g in zip(f[:3000].astype(np.float64).tolist(), got[:3000].tolist()):
        w = bf16_exact(Fraction(x))
        gv = float(onum.f32_from_bf16_bits(np.array([g], np.uint16))[0])
        if isinstance(w, float):
            if not (math.isinf(gv) and np.sign(gv) == np.sign(w)):
                return False
        elif Fraction(gv) != w:
            return False
    return True


# ---------------------------------------------------------------- codebook
def inv_norm_cdf_bisect(p):
    """Phi^-1(p) by bisection on Phi(x) = erfc(-x / sqrt 2) / 2 (math.erfc), to fp64 resolution."""
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = (lo + hi) / 2.0
        if mid == lo or mid == hi:
            break
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return (lo + hi) / 2.0


def pin_codebook_invariants():
    c = ocb.nf4_levels_f32()
    if c.dtype != np.float32 or c.shape != (16,):
        return False
    if not np.all(np.diff(c.astype(np.float64)) > 0):
        return False
    if c[0] != -1.0 or c[15] != 1.0:
        return False
    if not (c[7] == 0.0 and not np.signbit(c[7])):
        return False
    return int(np.sum(c < 0)) == 7 and int(np.sum(c > 0)) == 8


def pin_codebook_recomputed():
    """Rebuild the levels with an independent inverse CDF; the binary32 bits must match."""
    d = 1.0 - (1.0 / 32.0 + 1.0 / 30.0) / 2.0
    top = inv_norm_cdf_bisect(d)
    pos = [inv_norm_cdf_bisect(d + (0.5 - d) * i / 8.0) / top for i in range(8)]
    neg = [-inv_norm_cdf_bisect(d + (0.5 - d) * i / 7.0) / top for i in range(7)]
    ref = np.sort(np.array(pos + neg + [0.0])).astype(np.float32)
    got = ocb.nf4_levels_f32()
    return np.array_equal(ref.view(np.uint32), got.view(np.uint32))


# ---------------------------------------------------------------- code rule
def brute_code(w, s, levels):
    """argmin_i |w/s - c_i| with ties to the lower index, in exact rationals (s > 0)."""
    wf = Fraction(w) / Fraction(s)
    best, bi = None, None
    for i, c in enumerate(levels):
        d = abs(wf - Fraction(float(c)))
        if best is None or d < best:
            best, bi = d, i
    return bi


_FIX = 200   # every bf16, fp16 and binary32 value and every product c*s is an integer multiple of 2^-200


def _fixed(v):
    """v * 2^_FIX as an exact Python integer (v a float whose lowest bit is >= 2^-200)."""
    n, d = float(v).as_integer_ratio()
    q, r = divmod(n << _FIX, d)
    assert r == 0
    return q


def brute_codes_exact(ws, s, levels):
    """Exact nearest-level codes for many w at one scale s > 0: argmin_i |w - c_i s| (the
    same order as |w/s - c_i|, s being positive) over all 16 levels, ties to the lower index,
    in integer arithmetic on multiples of 2^-200.  Plain brute force, no midpoints."""
    ts = [_fixed(float(c)) * _fixed(s) >> _FIX for c in levels]
    assert all(_fixed(float(c)) * _fixed(s) % (1 << _FIX) == 0 for c in levels)
    out = []
    for w in ws:
        wi = _fixed(w)
        best, bi = None, 0
        for i, t in enumerate(ts):
            d = abs(wi - t)
            if best is None or d < best:
                best, bi = d, i
        out.append(bi)
    return out


def _groups_for(anchor, ws):
    """One 64-wide group per candidate w: [anchor, w, 0, ...]; anchor fixes the absmax."""
    m = np.zeros((len(ws), 64), dtype=np.float64)
    m[:, 0] = anchor
    m[:, 1] = ws
    return m


# Group absmax values a (the anchor of every test group) and the stored scale s = fp16(a)
# they give: s == a (1.0, 0.0234375), s < a by fp16 rounding (1 + 2^-12 and 3 - 2^-12 round
# down), fp16-subnormal scales where s < a by up to half a subnormal step (1.46875 * 2^-24
# stores s = 2^-24, so |w| / s reaches 1.47 and the grid covers [-1.1 s, 1.1 s] and beyond),
# and s > a (3 * 2^-25 rounds up to 2^-23; 2^-20 * 1.0078125 is exact).
CODE_RULE_ANCHORS = [1.0, 0.0234375, 2.0 ** -20 * 1.0078125, 1.0 + 2.0 ** -12, 3.0 - 2.0 ** -12, 6e-8,
                     1.46875 * 2.0 ** -24, 3.0 * 2.0 ** -25]


def pin_code_rule_bruteforce(anchors=None):
    """For each anchor absmax a: EVERY bf16 value w with |w| <= a (both signs, +-0, the
    subnormals) and every midpoint * s (+- one binary32 ulp) in that range: oracle code ==
    exact argmin over the 16 levels with ties to the lower index (integer arithmetic)."""
    levels = ocb.nf4_levels_f32()
    mids = (levels[:-1].astype(np.float64) + levels[1:].astype(np.float64)) / 2.0
    all_bits = np.arange(0, 0x7F80, dtype=np.uint16)
    all_vals = onum.f32_from_bf16_bits(all_bits).astype(np.float64)
    for a in (CODE_RULE_ANCHORS if anchors is None else anchors):
        s = float(np.float64(a).astype(np.float16))
        if s == 0.0:
            continue
        vals = all_vals[all_vals <= a]
        cand = np.concatenate([vals, -vals])
        ex = mids * s
        near = np.concatenate([ex, np.nextafter(ex.astype(np.float32), np.float32(np.inf)).astype(np.float64),
                               np.nextafter(ex.astype(np.float32), np.float32(-np.inf)).astype(np.float64)])
        near = near[np.abs(near) <= a]
        cand = np.concatenate([cand, near, [0.0, -0.0, a, -a]])
        codes, scales = onf4.pack_codes(_groups_for(a, cand))
        if np.any(scales[:, 0].astype(np.float64) != s):
            return False
        if codes[:, 1].tolist() != brute_codes_exact(cand.tolist(), s, levels):
            return False
        if np.any(codes[:, 2:] != 7):
            return False
    return True


def pin_code_rule_fraction_spotcheck():
    """The integer brute force itself against Fraction argmin on a few hundred values."""
    levels = ocb.nf4_levels_f32()
    rng = np.random.default_rng(41)
    for a in (1.0, 6e-8, 3.0 - 2.0 ** -12):
        s = float(np.float64(a).astype(np.float16))
        ws = (rng.uniform(-1.0, 1.0, 300) * a).astype(np.float32).astype(np.float64).tolist()
        if brute_codes_exact(ws, s, levels) != [brute_code(w, s, levels) for w in ws]:
            return False
    return True


def pin_pack_invariants(seed=3):
    """Exact zero -> code 7 and value +0; the absmax element -> +-s exactly (and bf16(+-s) in
    the tile); all-zero and fp16-underflowing groups -> s = +0, codes 7; codes in 0..15;
    size = n_out*k*17/32."""
    levels = ocb.nf4_levels_f32()
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32).astype(np.float64)
    w[0, 5] = 0.0
    w[1, 64:128] = 0.0                       # an all-zero group
    w[2, 128:192] = 1e-9                     # underflows fp16 -> s = 0
    codes, scales = onf4.pack_codes(w)
    if codes.max() > 15:
        return False
    if codes[0, 5] != 7 or codes[1, 64:128].tolist() != [7] * 64 or codes[2, 128:192].tolist() != [7] * 64:
        return False
    if scales[1, 1] != 0 or np.signbit(scales[1, 1]) or scales[2, 2] != 0:
        return False
    deq = onf4.dequant_exact(codes, scales)
    if deq[0, 5] != 0.0 or np.signbit(deq[0, 5]):
        return False
    tile = onf4.dequant_tile_bits(codes, scales)
    g = w.reshape(8, 4, 64)
    for r in range(8):
        for gi in range(4):
            s = float(scales[r, gi])
            if s == 0.0:
                continue
            j = int(np.argmax(np.abs(g[r, gi])))
            sign = 1.0 if g[r, gi, j] > 0 else -1.0
            if codes[r, gi * 64 + j] != (15 if sign > 0 else 0):
                return False
            if deq[r, gi * 64 + j] != sign * s:
                return False
            want_bits = int(bf16_bits_scalar(sign * s))
            if int(tile[r, gi * 64 + j]) != want_bits:
                return False
    return onf4.packed_bytes(8, 256) * 32 == 8 * 256 * 17 and \
        onf4.pack_device(w).size == onf4.packed_bytes(8, 256)


def bf16_bits_scalar(v):
    """bf16 bits of a binary32-representable value via exact rational rounding."""
    r = bf16_exact(Fraction(float(v)))
    f = np.array([float(r)], dtype=np.float32)
    return int(f.view(np.uint32)[0] >> 16)


def pin_tile_rounding_exhaustive():
    """All 16 codes x every non-negative finite fp16 scale: the tile value equals the exact
    rational bf16(binary32(c * s)) (one binary32 rounding of the product, then bf16 RNE)."""
    levels = ocb.nf4_levels_f32()
    sbits = np.arange(0, 0x7C00, dtype=np.uint16)
    svals = sbits.view(np.float16)
    ok = True
    # oracle over [scales][16 codes]: build a matrix with one group per scale
    codes = np.tile(np.repeat(np.arange(16, dtype=np.uint8), 4), (svals.size, 1))
    scales = svals.reshape(-1, 1)
    tile = onf4.dequant_tile_bits(codes, scales)[:, ::4]          # [n_scales][16]
    # exact check on a deterministic subsample (all scales would take minutes in Fractions)
    rng = np.random.default_rng(5)
    pick = np.unique(np.concatenate([np.arange(0, 1024), rng.integers(0, svals.size, 3000),
                                     np.arange(svals.size - 64, svals.size)]))
    for i in pick.tolist():
        s = Fraction(float(svals[i]))
        for cidx in range(16):
            p = Fraction(float(levels[cidx])) * s
            p32 = round_binary(p, 24, -126, 127)
            want = bf16_exact(p32)
            got = float(onum.f32_from_bf16_bits(np.array([tile[i, cidx]], np.uint16))[0])
            if Fraction(got) != want:
                return False
    # full sweep against an independent float64 formulation: binary32 product via float64
    # (exact: 24x11 bits) then round to binary32 and to bf16 via exact integer arithmetic.
    prod = (levels.astype(np.float64)[None, :] * svals.astype(np.float64)[:, None])
    p32 = prod.astype(np.float32)
    u = p32.view(np.uint32).astype(np.int64)
    hi = u >> 16
    lo = u & 0xFFFF
    rnd = hi + ((lo > 0x8000) | ((lo == 0x8000) & (hi & 1 == 1))).astype(np.int64)
    ok = ok and np.array_equal(rnd.astype(np.uint16), tile)
    return bool(ok)


# ---------------------------------------------------------------- layout fixtures
def read_fixture(name):
    """Parse a golden text fixture: 'key: hex hex ...' lines, '#' comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def pin_byte_fixtures():
    fx = read_fixture("nf4_layout_fixtures.txt")
    # case A: one 64-wide row whose codes are 0..15 repeated four times
    codes = np.tile(np.arange(16, dtype=np.uint8), 4).reshape(1, 64)
    cb = onf4.codes_to_bytes(codes)
    if cb.reshape(-1).tolist() != [int(h, 16) for h in fx["A_canonical_bytes"]]:
        return False
    if not np.array_equal(onf4.bytes_to_codes(cb), codes):
        return False
    scales = np.array([[2.0]], dtype=np.float16)
    dev = onf4.device_from_canonical(cb, scales)
    if dev.tolist() != [int(h, 16) for h in fx["A_device_bytes"]]:
        return False
    # case A as an encoding: w = c_code * 2 reproduces those codes and s = 2
    levels = ocb.nf4_levels_f32().astype(np.float64)
    w = (levels[codes] * 2.0)
    c2, s2 = onf4.pack_codes(w)
    if not np.array_equal(c2, codes) or s2.view(np.uint16).reshape(-1).tolist() != [int(fx["A_scale_bits"][0], 16)]:
        return False
    # case B: 2 x 128 with four distinct scales -> device scale bytes
    w = np.zeros((2, 128))
    w[0, 3], w[0, 64 + 9], w[1, 10], w[1, 64 + 63] = 1.0, -2.0, 4.0, 0.5
    cB, sB = onf4.pack_codes(w)
    devB = onf4.device_from_canonical(onf4.codes_to_bytes(cB), sB)
    if devB[2 * 64:].tolist() != [int(h, 16) for h in fx["B_device_scale_bytes"]]:
        return False
    # case C: 18 rows x 128 -> device scale position of selected (row, group)
    n_out, g = 18, 2
    sc = (np.arange(n_out * g, dtype=np.float64) + 1.0).reshape(n_out, g).astype(np.float16)
    cb = np.zeros((n_out, 64), dtype=np.uint8)
    devC = onf4.device_from_canonical(cb, sc)[n_out * 64:].view(np.float16)
    for item in fx["C_row_group_devindex"]:
        r, gi, di = (int(t) for t in item.split(","))
        if devC[di] != sc[r, gi]:
            return False
    # round trip of the layout
    cb2, sc2 = onf4.canonical_from_device(onf4.device_from_canonical(cb, sc), n_out, 128)
    return np.array_equal(cb2, cb) and np.array_equal(sc2.view(np.uint16), sc.view(np.uint16))


def pin_layout_roundtrip(seed=9):
    rng = np.random.default_rng(seed)
    for n_out, k in [(1, 64), (16, 128), (17, 192), (33, 512), (5, 64)]:
        cb = rng.integers(0, 256, size=(n_out, k // 2), dtype=np.uint8)
        sc = rng.standard_normal((n_out, k // 64)).astype(np.float16)
        dev = onf4.device_from_canonical(cb, sc)
        if dev.size != onf4.packed_bytes(n_out, k):
            return False
        cb2, sc2 = onf4.canonical_from_device(dev, n_out, k)
        if not (np.array_equal(cb2, cb) and np.array_equal(sc2.view(np.uint16), sc.view(np.uint16))):
            return False
    return True


def pin_roundtrip_idempotent(seed=13):
    """deep-fold's CPU round trip: pack(dequant_exact(pack(W))) == pack(W)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((24, 320)) * 0.02).astype(np.float32)
    w[3, :64] = 0.0
    c1, s1 = onf4.pack_codes(w)
    c2, s2 = onf4.pack_codes(onf4.dequant_exact(c1, s1))
    return np.array_equal(c1, c2) and np.array_equal(s1.view(np.uint16), s2.view(np.uint16))


# ---------------------------------------------------------------- linear references
def _py_dot_rows(w, x):
    """Exact y_i = sum_j w_ij x_j with Fractions (pure Python loops)."""
    return [sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(row, x)), Fraction(0)) for row in w]


def pin_gemv_bruteforce(seed=17):
    rng = np.random.default_rng(seed)
    for n_out, k in [(1, 64), (3, 128), (4, 256)]:
        w = rng.standard_normal((n_out, k)).astype(np.float32)
        x = rng.standard_normal(k).astype(np.float32)
        y, s = olin.gemv_ref(w, x)
        ex = _py_dot_rows(w.tolist(), x.tolist())
        sx = _py_dot_rows(np.abs(w).tolist(), np.abs(x).tolist())
        for a, b, c, d in zip(y.tolist(), ex, s.tolist(), sx):
            if abs(Fraction(a) - b) > Fraction(1, 10 ** 12) * (abs(d) + 1) or abs(Fraction(c) - d) > Fraction(1, 10 ** 12) * (abs(d) + 1):
                return False
    return True


def pin_gemm_bruteforce(seed=19):
    rng = np.random.default_rng(seed)
    for m, n_out, k in [(1, 2, 64), (3, 4, 128), (2, 3, 256)]:
        x = rng.standard_normal((m, k)).astype(np.float32)
        t = rng.standard_normal((n_out, k)).astype(np.float32)
        y, s = olin.gemm_ref(x, t)
        for i in range(m):
            ex = _py_dot_rows(t.tolist(), x[i].tolist())
            for j in range(n_out):
                if abs(Fraction(float(y[i, j])) - ex[j]) > Fraction(1, 10 ** 12) * (1 + abs(ex[j])):
                    return False
    return True


def pin_exact_integer_cases():
    """Small integers give exact results; one-hot x picks a column; W = 0 gives 0."""
    rng = np.random.default_rng(23)
    w = rng.integers(-8, 9, size=(5, 128)).astype(np.float64)
    x = rng.integers(-8, 9, size=128).astype(np.float64)
    y, _ = olin.gemv_ref(w, x)
    if not np.array_equal(y, np.array([sum(int(a) * int(b) for a, b in zip(r, x)) for r in w], dtype=np.float64)):
        return False
    e = np.zeros(128)
    e[77] = 1.0
    y1, _ = olin.gemv_ref(w, e)
    if not np.array_equal(y1, w[:, 77]):
        return False
    y0, s0 = olin.gemv_ref(np.zeros((3, 64)), x[:64])
    if np.any(y0 != 0) or np.any(s0 != 0):
        return False
    Y, _ = olin.gemm_ref(np.stack([x, 2 * x]), w)
    return np.array_equal(Y[0], y) and np.array_equal(Y[1], 2 * y)


def pin_tolerance_checker():
    """The checker accepts errors within 1e-4*S, rejects beyond, and requires exact 0 at S=0."""
    y_ref = np.array([1.0, -2.0, 0.0, 5.0])
    s = np.array([10.0, 10.0, 0.0, 100.0])
    ok1, _, _ = olin.check_rows_f32(y_ref + np.array([9e-4, -9e-4, 0.0, 9e-3]), y_ref, s)
    ok2, _, i2 = olin.check_rows_f32(y_ref + np.array([0.0, 1.1e-3, 0.0, 0.0]), y_ref, s)
    ok3, _, _ = olin.check_rows_f32(y_ref + np.array([0.0, 0.0, 1e-30, 0.0]), y_ref, s)
    ok4, _, _ = olin.check_rows_f32(np.array([1.0, np.nan, 0.0, 5.0]), y_ref, s)
    return ok1 and (not ok2) and i2 == 1 and (not ok3) and (not ok4)


def _exact_bf16_spacing(q):
    """Spacing of the bf16 grid in the binade of a non-negative rational q: 2^(e-7) for q in
    [2^e, 2^(e+1)), e >= -126; 2^-133 below 2^-126 (subnormals) and at 0."""
    if q == 0:
        return Fraction(1, 2 ** 133)
    return Fraction(2) ** (max(_floor_log2(q), -126) - 7)


def pin_ulp_bf16_exact(seed=43):
    """ulp_bf16 against exact rational spacing: at every positive finite bf16 value (where it
    must also equal the gap to the next bf16 value up), the binary64 value just below and just
    above each of them, every power of two from 2^-140 to 2^127 and its neighbours, zero, the
    subnormal range, negative arguments, and a log-uniform binary64 sample."""
    bits = all_positive_finite_bf16_bits()
    vals = onum.f32_from_bf16_bits(bits).astype(np.float64)
    nxt = onum.f32_from_bf16_bits(bits + np.uint16(1)).astype(np.float64)
    gap_ok = bits < 0x7F7F                                   # the next pattern up is finite
    got = olin.ulp_bf16(vals)
    if not np.array_equal(got[gap_ok], (nxt - vals)[gap_ok]):
        return False
    pw = np.ldexp(1.0, np.arange(-140, 128))
    rng = np.random.default_rng(seed)
    sample = np.ldexp(rng.uniform(1.0, 2.0, 4000), rng.integers(-150, 128, 4000))
    probes = np.concatenate([vals, np.nextafter(vals, 0.0), np.nextafter(vals, np.inf), pw,
                             np.nextafter(pw, 0.0), np.nextafter(pw, np.inf), sample, [0.0, 5e-324, 1e-40]])
    probes = probes[np.isfinite(probes)]
    got = olin.ulp_bf16(probes)
    want = [_exact_bf16_spacing(Fraction(float(v))) for v in probes.tolist()]
    if any(Fraction(float(g)) != w for g, w in zip(got.tolist(), want)):
        return False
    neg = olin.ulp_bf16(-probes)
    return bool(np.array_equal(neg, got)) and np.ndim(olin.ulp_bf16(1.0)) == 0


def pin_check_bf16_boundary():
    """check_bf16 accepts an error of exactly 1e-4*S + ulp(|y_ref|) and rejects one bf16 step
    beyond it, and rejects a binary64 hair beyond it.  Built so every quantity is exact in
    binary64: S = 10000 (fl(1e-4) * 10000 rounds to exactly 1), y_ref in [1024, 2048) where the
    bf16 spacing is 8, so the allowed error is 9; the bf16 values are multiples of 8 there."""
    b = lambda v: onum.bf16_bits_from_f32(np.array([v], np.float32))
    S = np.array([10000.0])
    if float(np.float64(olin.REL_TOL) * 10000.0) != 1.0:
        return False
    cases = [  # (bf16 output, y_ref, accepted?)
        (1040.0, 1031.0, True), (1048.0, 1031.0, False), (1040.0, float(np.nextafter(1031.0, 0.0)), False),
        (-1040.0, -1031.0, True), (-1048.0, -1031.0, False), (1024.0, 1033.0, True), (1016.0, 1025.0, True),
        (1016.0, float(np.nextafter(1025.0, 0.0)), True), (1008.0, 1025.0, False),
    ]
    for yv, r, want in cases:
        ok, _, _ = olin.check_bf16(b(yv), np.array([r]), S)
        if ok != want:
            return False
    # S = 0: the bound is one ulp of |y_ref|; just below a power of two the ulp is the lower binade's
    ok_lo, _, _ = olin.check_bf16(b(1.0), np.array([1.0 - 2.0 ** -8]), np.array([0.0]))
    bad_lo, _, _ = olin.check_bf16(b(1.0), np.array([float(np.nextafter(1.0 - 2.0 ** -8, 0.0))]), np.array([0.0]))
    nan_out, _, _ = olin.check_bf16(np.array([0x7FC0], np.uint16), np.array([1.0]), np.array([1.0]))
    return ok_lo and not bad_lo and not nan_out


ALL_PINS = [
    pin_fp16_rounding_exhaustive, pin_fp16_rounding_f32_sample, pin_bf16_rounding,
    pin_codebook_invariants, pin_codebook_recomputed, pin_code_rule_bruteforce,
    pin_code_rule_fraction_spotcheck,
    pin_pack_invariants, pin_tile_rounding_exhaustive, pin_byte_fixtures,
    pin_layout_roundtrip, pin_roundtrip_idempotent, pin_gemv_bruteforce,
    pin_gemm_bruteforce, pin_exact_integer_cases, pin_tolerance_checker,
    pin_ulp_bf16_exact, pin_check_bf16_boundary,
]
