"""Seeded defects planted in the CPU oracle must each be caught by a pin.

The IPE page ("How it is checked") asks that a test suite catch seeded
defects; here each defect is planted in the oracle (on the CPU, through
monkeypatching) and the named pin must then fail.
"""

import numpy as np
import pytest

import oracle.numfmt as onum
import oracle.codebook as ocb
import oracle.nf4 as onf4
import oracle.linear as olin
import pins

_orig_levels = ocb.nf4_levels_f32
_orig_mids = onf4.nf4_midpoints
_orig_pack = onf4.pack_codes
_orig_dev = onf4.device_from_canonical
_orig_perm = onf4._scale_perm
_orig_gemv = olin.gemv_ref
_orig_gemm = olin.gemm_ref


def _swap_nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 1::2] | (c[:, 0::2] << 4)).astype(np.uint8)


def _wrong_group_dequant(codes, scales, levels=None):
    return _orig_dequant(codes, np.roll(np.asarray(scales), 1, axis=1), levels)


_orig_dequant = onf4.dequant_exact


def _bf16_truncate(a):
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _drop_last_group(w, levels=None, rows_per_chunk=256):
    c, s = _orig_pack(w, levels, rows_per_chunk)
    c = c.copy()
    c[:, -64:] = 7
    return c, s


def _perm_off_by_one(n_out, g):
    p = _orig_perm(n_out, g)
    return np.roll(p, 1)


def _fp16_truncate(a):
    a = np.asarray(a, dtype=np.float64)
    r = a.astype(np.float16)
    back = r.astype(np.float64)
    fix = np.abs(back) > np.abs(a)
    r = np.where(fix, np.nextafter(r, np.float16(0)), r)
    return r.astype(np.float16)


def _ties_up(levels=None):
    m = _orig_mids(levels)
    return np.nextafter(m, -np.inf)


def _perturbed_levels():
    c = _orig_levels().copy()
    c[3] = np.nextafter(c[3], np.float32(1.0))
    return c


def _gemv_drop_last(w, x):
    w = np.asarray(w, dtype=np.float64).copy()
    w[:, -1] = 0.0
    return _orig_gemv(w, x)


def _gemm_reversed_k(x, t):
    return _orig_gemm(np.asarray(x)[:, ::-1], t)


def _mids_upper(levels=None):
    c = (_orig_levels() if levels is None else np.asarray(levels, np.float32)).astype(np.float64)
    return c[1:].copy()


def _dev_rot4(code_bytes, scales):
    cb = np.ascontiguousarray(code_bytes, dtype=np.uint8)
    words = cb.view("<u4").astype(np.uint64)
    rot = (((words << np.uint64(4)) | (words >> np.uint64(28))) & np.uint64(0xFFFFFFFF)).astype("<u4")
    base = _orig_dev(code_bytes, scales)
    base[:rot.size * 4] = rot.view(np.uint8).reshape(-1)
    return base


_orig_ulp = olin.ulp_bf16


def _ulp_doubled(v):
    return 2.0 * _orig_ulp(v)


def _ulp_binade_low(v):
    """The binade taken one too low: half the spacing everywhere."""
    return 0.5 * _orig_ulp(v)


def _ulp_binade_high_near_powers(v):
    """The binade read with a rounded logarithm: values just below a power of two land in the
    binade above (the defect an inexact log2 makes)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.maximum(np.floor(np.log2(np.where(v > 0, v, 1.0))), -126.0)
    return np.where(v > 0, np.exp2(e - 7.0), np.exp2(-133.0))


def _check_bf16_no_ulp(y_bits, y_ref, s, rel=olin.REL_TOL):
    y = onum.f32_from_bf16_bits(y_bits).astype(np.float64)
    err = np.abs(y - np.asarray(y_ref, np.float64))
    ratio = err / np.maximum(rel * np.asarray(s, np.float64), 1e-300)
    i = int(np.argmax(ratio))
    return bool(ratio[i] <= 1.0), float(ratio[i]), i


DEFECTS = [
    ("swapped nibble order", onf4, "codes_to_bytes", _swap_nibbles, [pins.pin_byte_fixtures]),
    ("scale of the wrong group", onf4, "dequant_exact", _wrong_group_dequant, [pins.pin_pack_invariants]),
    ("bf16 truncation instead of RNE", onum, "bf16_bits_from_f32", _bf16_truncate, [pins.pin_bf16_rounding]),
    ("last group dropped", onf4, "pack_codes", _drop_last_group, [pins.pin_roundtrip_idempotent]),
    ("scale layout row off by one", onf4, "_scale_perm", _perm_off_by_one, [pins.pin_byte_fixtures]),
    ("fp16 scale truncated", onum, "fp16_from_real", _fp16_truncate, [pins.pin_fp16_rounding_exhaustive]),
    ("tie-break flipped", onf4, "nf4_midpoints", _ties_up, [pins.pin_code_rule_bruteforce]),
    ("level perturbed by one ulp", ocb, "nf4_levels_f32", _perturbed_levels, [pins.pin_codebook_recomputed]),
    ("GEMV drops a term", olin, "gemv_ref", _gemv_drop_last, [pins.pin_gemv_bruteforce]),
    ("GEMM reversed reduction index", olin, "gemm_ref", _gemm_reversed_k, [pins.pin_gemm_bruteforce]),
    ("midpoints replaced by upper levels", onf4, "nf4_midpoints", _mids_upper, [pins.pin_code_rule_bruteforce]),
    ("device word rotated by 4", onf4, "device_from_canonical", _dev_rot4, [pins.pin_byte_fixtures]),
    ("bf16 ulp doubled", olin, "ulp_bf16", _ulp_doubled, [pins.pin_ulp_bf16_exact, pins.pin_check_bf16_boundary]),
    ("bf16 ulp binade one too low", olin, "ulp_bf16", _ulp_binade_low,
     [pins.pin_ulp_bf16_exact, pins.pin_check_bf16_boundary]),
    ("bf16 ulp binade from a rounded log2", olin, "ulp_bf16", _ulp_binade_high_near_powers,
     [pins.pin_ulp_bf16_exact]),
    ("bf16 checker without the rounding ulp", olin, "check_bf16", _check_bf16_no_ulp, [pins.pin_check_bf16_boundary]),
]


@pytest.mark.parametrize("name,mod,attr,bad,catchers", DEFECTS, ids=[d[0] for d in DEFECTS])
def test_defect_is_caught(monkeypatch, name, mod, attr, bad, catchers):
    for pin in catchers:
        assert pin(), f"{pin.__name__} must pass on the intact oracle"
    monkeypatch.setattr(mod, attr, bad)
    assert not all(pin() for pin in catchers), f"defect '{name}' was not caught"
