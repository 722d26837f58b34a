"""The C-ABI library without a GPU: load, exported symbols, constants, argument checks."""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import weight_streaming_linear_amd as wsl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = wsl.lib()
    names = declared_functions()
    assert set(names) == set(wsl.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_codebook_bits_match_oracle():
    lv = np.array(wsl.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), oracle.nf4_levels_f32().view(np.uint32))


@pytest.mark.parametrize("n_out,k", [(4096, 4096), (1, 64), (17, 192), (27648, 5120), (6144, 16384)])
def test_packed_bytes_formula(n_out, k):
    assert wsl.nf4_packed_bytes(n_out, k) == oracle.packed_bytes(n_out, k) == n_out * k * 17 // 32


def test_packed_bytes_invalid():
    assert wsl.nf4_packed_bytes(0, 64) == 0
    assert wsl.nf4_packed_bytes(4, 65) == 0
    assert wsl.nf4_packed_bytes(-3, 64) == 0


# The launch's choice of a k split, read on the host through the workspace it asks for:
# splits * m * n_out * 4 bytes.  The 256 x 256 tiles split k where they are few (mid M on
# matrices with few rows; half tiles at M <= 128), not where they fill the CUs (M = 8192)
# nor where k % 256 != 0; the shared-X kernel (NF4 at M = 64) splits the down projection
# and not the tall up projection.
@pytest.mark.parametrize("wfmt,n_out,k,m,splits", [
    (wsl.WSL_W_BF16, 5120, 27648, 256, 12), (wsl.WSL_W_NF4, 5120, 27648, 256, 12),
    (wsl.WSL_W_NF4, 5120, 27648, 512, 6), (wsl.WSL_W_NF4, 5120, 27648, 1024, 3),
    (wsl.WSL_W_BF16, 27648, 5120, 128, 2), (wsl.WSL_W_NF4, 27648, 5120, 256, 2),
    (wsl.WSL_W_NF4, 27648, 5120, 128, 2), (wsl.WSL_W_NF4, 5120, 27648, 128, 12),
    (wsl.WSL_W_NF4, 27648, 5120, 64, 0), (wsl.WSL_W_NF4, 5120, 27648, 64, 6),
    (wsl.WSL_W_BF16, 27648, 5120, 64, 2), (wsl.WSL_W_BF16, 17408, 5120, 8192, 0),
    (wsl.WSL_W_NF4, 5120, 17408, 8192, 0), (wsl.WSL_W_BF16, 5120, 27584, 256, 0),
    (wsl.WSL_W_NF4, 5120, 27648, 32, 6), (wsl.WSL_W_NF4, 27648, 5120, 32, 0)])
def test_gemm_split_choice(wfmt, n_out, k, m, splits):
    assert wsl.linear_gemm_workspace_bytes(wfmt, n_out, k, m) == splits * m * n_out * 4


def test_argument_errors_return_before_any_launch():
    L = wsl.lib()
    a = ctypes.c_void_p(4096)     # aligned, never dereferenced: validation fails first
    odd = ctypes.c_void_p(4098)
    assert L.linear_gemv(wsl.WSL_W_NF4, None, 4, 64, a, a, None) == 1
    assert L.linear_gemv(wsl.WSL_W_NF4, a, 4, 96, a, a, None) == 2
    assert L.linear_gemv(wsl.WSL_W_NF4, odd, 4, 64, a, a, None) == 3
    assert L.linear_gemv(5, a, 4, 64, a, a, None) == 4
    assert L.linear_gemm(wsl.WSL_W_BF16, a, 4, 64, a, 3, 64, a, 7, 8, None, 0, None) == 4
    assert L.linear_gemm(wsl.WSL_W_BF16, a, 4, 64, a, 3, 32, a, 0, 8, None, 0, None) == 2
    assert L.linear_gemm_noalloc(wsl.WSL_W_BF16, a, 4, 64, a, 3, 64, a, 7, 8, None) == 4
    assert L.linear_gemm_noalloc(wsl.WSL_W_NF4, a, 4, 96, a, 3, 96, a, 0, 8, None) == 2
    assert L.nf4_pack(a, 4, 100, a, None, None) == 2
    st = (wsl.WslGemvStage * 2)(wsl.WslGemvStage(4096, 4096, 4096, 4, 64), wsl.WslGemvStage(4096, 4096, 4096, 4, 64))
    ws = wsl.lib().linear_gemv_sweep_workspace_bytes()
    assert ws >= 1284
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 0, None, None, None, 0, None) == 0          # nothing to do
    assert L.linear_gemv_sweep(wsl.WSL_W_BF16, 2, st, a, a, ws, None) == 4
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 2, None, a, a, ws, None) == 1
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 2, st, a, ctypes.c_void_p(4096 + 64), ws, None) == 3
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 2, st, a, a, ws - 1, None) == 7
    st[1].k = 96
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 2, st, a, a, ws, None) == 2
    st[1].k = 32768 + 64
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 2, st, a, a, ws, None) == 2
    st[1].k = 64
    st[1].w = 4098
    assert L.linear_gemv_sweep(wsl.WSL_W_NF4, 2, st, a, a, ws, None) == 3
    assert L.nf4_dequant_tile(a, 4, 64, 4, 0, 1, 1, a, 1, None) == 7
    assert L.nf4_embed_rows(a, 4, 64, None, 2, a, wsl.WSL_OUT_BF16, 64, None, None) == 1
    assert L.nf4_embed_rows(a, 4, 64, a, 2, a, 9, 64, None, None) == 4
    assert L.nf4_embed_rows(a, 4, 64, a, 2, a, wsl.WSL_OUT_BF16, 68, None, None) == 3
    assert L.nf4_embed_rows(a, 4, 96, a, 2, a, wsl.WSL_OUT_BF16, 96, None, None) == 2
    one = (ctypes.c_void_p * 1)(4096)
    two = (ctypes.c_void_p * 2)(4096, 8192)
    four = (ctypes.c_void_p * 4)(1, 2, 3, 4)
    shp = (ctypes.c_int64 * 1)(64)
    assert L.linear_gemv_streamed(wsl.WSL_W_NF4, 0, None, None, None, None, None, None, 0, None, None, None, 0) == 0
    assert L.linear_gemv_streamed(wsl.WSL_W_NF4, -1, one, shp, shp, one, one, two, 4096, None, None, four, 0) == 2
    assert L.linear_gemv_streamed(9, 1, one, shp, shp, one, one, two, 4096, None, None, four, 0) == 4
    assert L.linear_gemv_streamed(wsl.WSL_W_NF4, 1, one, shp, shp, one, one, two, 4096, None, None, None, 1) == 1
    assert L.linear_gemv_streamed(wsl.WSL_W_NF4, 1, one, shp, shp, one, one, two, 100, None, None, four, 1) == 7
    assert L.linear_gemv_streamed(wsl.WSL_W_NF4, 1, one, shp, shp, one, one, two, 4096, None, None, four, 2) == 10
    assert L.linear_gemv_streamed(wsl.WSL_W_NF4, 0, None, None, None, None, None, None, 0, None, None, None, -1) == 10
    assert L.linear_gemm_streamed(wsl.WSL_W_NF4, 1, one, shp, shp, one, 0, 64, one, 0, 64, None, 0, two, 4096,
                                  None, None, four, 0) == 2
    assert L.linear_gemm_streamed(wsl.WSL_W_NF4, 1, one, shp, shp, one, 1, 64, one, 0, 64, None, 0, two, 4096,
                                  None, None, four, 4) == 10
    assert L.wsl_stream_read(a, 0, None, None) == 0
    assert L.wsl_stream_read(None, 16, a, None) == 1
    assert L.wsl_stream_read(a, 24, a, None) == 2
    assert L.wsl_stream_read(odd, 16, a, None) == 3
    st = (wsl.WslGemvStage * 3)(wsl.WslGemvStage(4096, 4096, 4096, 16, 512), wsl.WslGemvStage(4096, 4096, 4096, 8, 512),
                                wsl.WslGemvStage(4096, 4096, 4096, 4, 512))
    assert L.linear_gemv_multi(wsl.WSL_W_BF16, 0, None, None) == 0
    assert L.linear_gemv_multi(wsl.WSL_W_NF4, 3, st, None) == 4
    assert L.linear_gemv_multi(wsl.WSL_W_BF16, 9, st, None) == 2
    assert L.linear_gemv_multi(wsl.WSL_W_BF16, 3, None, None) == 1
    st[2].k = 1024
    assert L.linear_gemv_multi(wsl.WSL_W_BF16, 3, st, None) == 2
    st[2].k = 512
    st[1].x = 4100
    assert L.linear_gemv_multi(wsl.WSL_W_BF16, 3, st, None) == 3
    st[1].x = 4096
    st[0].y = None
    assert L.linear_gemv_multi(wsl.WSL_W_BF16, 3, st, None) == 1
    assert wsl.wsl_strerror(7).startswith("tile")
    assert "flags" in wsl.wsl_strerror(wsl.WSL_E_FLAGS)
    assert L.nf4_codebook(None) == 1


def test_validation_unit_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "validate_asan")
    srcs = [os.path.join(ROOT, "tests", "cpp", "validate_main.cpp"),
            os.path.join(ROOT, "weight_streaming_linear_amd", "csrc", "validate.cpp")]
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", *srcs, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
