"""Compiled-code check (CPU, needs hipcc): no kernel touches a register that an LDS read
or load issued from inline asm may still be writing.

The GEMM kernels issue their MFMA fragment reads from inline asm and wait for them in a
separate asm statement.  Whether that is safe depends on the compiler's register
allocation (a copy of a fragment register placed before the wait would read stale
data), so the gfx950 assembly of every HIP source is built with the library's own flags
and scanned (tests/asm_scan.py).  Two small hand-written listings check the scanner
itself: one with a copy before the wait (must be reported), one with the copy after it.
"""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import asm_scan
from weight_streaming_linear_amd import build as wbuild

SOURCES = list(wbuild.HIP_SOURCES)

BAD = """\
	.amdhsa_kernel k_bad
k_bad:
	;;#ASMSTART
	ds_read_b128 v[4:7], v1
	ds_read_b128 v[8:11], v1 offset:2048
	;;#ASMEND
	v_mov_b64_e32 v[20:21], v[8:9]
	;;#ASMSTART
	s_waitcnt lgkmcnt(0)
	;;#ASMEND
	v_mfma_f32_32x32x16_bf16 v[32:47], v[4:7], v[20:23], v[32:47]
	s_endpgm
"""
GOOD = BAD.replace("k_bad", "k_good").replace(
    "\tv_mov_b64_e32 v[20:21], v[8:9]\n\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n",
    "\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n\tv_mov_b64_e32 v[20:21], v[8:9]\n")
# an asm read still in flight behind a partial wait: lgkmcnt(1) releases only the first read
PARTIAL = BAD.replace("k_bad", "k_partial").replace(
    "\tv_mov_b64_e32 v[20:21], v[8:9]\n\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(0)\n\t;;#ASMEND\n",
    "\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(1)\n\t;;#ASMEND\n\tv_mov_b64_e32 v[20:21], v[8:9]\n")


def test_scanner_controls():
    assert asm_scan.kernels(BAD) == ["k_bad"]
    assert asm_scan.scan_kernel(BAD, "k_bad") == ["v_mov_b64_e32 v[20:21], v[8:9]"]
    assert asm_scan.scan_kernel(GOOD, "k_good") == []
    assert asm_scan.scan_kernel(PARTIAL, "k_partial") == ["v_mov_b64_e32 v[20:21], v[8:9]"]


def _device_asm(src, out_dir):
    flags = [f for f in wbuild.HIP_FLAGS if f not in ("-fPIC",)]
    out = os.path.join(out_dir, src + ".s")
    cmd = [wbuild._hipcc(), *flags, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(wbuild.CSRC, src), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(shutil.which(wbuild._hipcc()) is None and not os.path.exists(wbuild._hipcc()),
                    reason="hipcc not available")
def test_no_kernel_reads_an_asm_load_in_flight():
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=4) as ex:
            listings = dict(zip(SOURCES, ex.map(lambda s: _device_asm(s, d), SOURCES)))
    scanned, bad = 0, {}
    for src, text in listings.items():
        for k in asm_scan.kernels(text):
            scanned += 1
            found = asm_scan.scan_kernel(text, k)
            if found:
                bad[f"{src}:{k}"] = found[:3]
    assert scanned >= 15, scanned
    assert not bad, bad
