"""Weight-streaming linear layers for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libwsl.so`` (declared in
``include/wsl.h``).  Every step of the computation runs in the library's HIP
kernels; this module only marshals arguments: it takes torch tensors (device
memory) and the current torch stream, passes raw pointers and sizes, and turns
status codes into exceptions.  There is no fallback: if the library is not
built, every call raises.

Entry points (same names as the C ABI):
  nf4_packed_bytes, nf4_codebook, nf4_pack, nf4_dequant_tile,
  linear_gemv, linear_gemm, linear_gemm_workspace_bytes, nf4_embed_rows, wsl_strerror;
  linear_gemm_noalloc; linear_gemv_multi; GemvSweep (linear_gemv_sweep,
  linear_gemv_sweep_workspace_bytes);
  stream_read (wsl_stream_read); CopyRing.gemv / CopyRing.gemm (linear_gemv_streamed /
  linear_gemm_streamed, weights streamed from page-locked host memory, see to_pinned).
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwsl.so")

WSL_OK = 0
WSL_W_BF16 = 0
WSL_W_NF4 = 1
WSL_OUT_F32 = 0
WSL_OUT_BF16 = 1
WSL_STATUS_NONFINITE = 1
WSL_STATUS_OVERFLOW = 2

EXPORTED = [
    "nf4_packed_bytes", "nf4_codebook", "nf4_pack", "nf4_dequant_tile", "linear_gemv",
    "linear_gemm_workspace_bytes", "linear_gemm", "nf4_embed_rows", "linear_gemv_streamed",
    "linear_gemm_streamed", "wsl_stream_read", "wsl_strerror", "linear_gemm_noalloc",
    "linear_gemv_sweep_workspace_bytes", "linear_gemv_sweep", "linear_gemv_multi",
]
WSL_STATUS_SWEEP_TIMEOUT = 8
WSL_STATUS_DESCRIPTOR = 16
SWEEP_STATUS_OFFSET = 1280      # byte offset of the status word in the sweep workspace
WSL_E_SCRATCH = 9
WSL_E_FLAGS = 10
WSL_RING_PACE = 1               # linear_*_streamed: the host keeps the copies two matrices ahead
NOALLOC_SCRATCH_BYTES = 4 << 20


class WSLError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: status {code} ({wsl_strerror(code)})")


_lib = None


def lib():
    """The loaded libwsl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libwsl.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                           "or python -m weight_streaming_linear_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.nf4_packed_bytes.argtypes = [i64, i64]
    L.nf4_packed_bytes.restype = sz
    L.nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.nf4_codebook.restype = ctypes.c_int
    L.nf4_pack.argtypes = [vp, i64, i64, vp, vp, vp]
    L.nf4_pack.restype = ctypes.c_int
    L.nf4_dequant_tile.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, i64, vp]
    L.nf4_dequant_tile.restype = ctypes.c_int
    L.linear_gemv.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp, vp]
    L.linear_gemv.restype = ctypes.c_int
    L.linear_gemm_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64]
    L.linear_gemm_workspace_bytes.restype = sz
    L.linear_gemm.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, i64, vp, ctypes.c_int, i64, vp, sz, vp]
    L.linear_gemm.restype = ctypes.c_int
    L.linear_gemv_sweep_workspace_bytes.argtypes = []
    L.linear_gemv_sweep_workspace_bytes.restype = sz
    L.linear_gemv_sweep.argtypes = [ctypes.c_int, i64, vp, vp, vp, sz, vp]
    L.linear_gemv_sweep.restype = ctypes.c_int
    L.linear_gemv_multi.argtypes = [ctypes.c_int, i64, vp, vp]
    L.linear_gemv_multi.restype = ctypes.c_int
    L.linear_gemm_noalloc.argtypes = [ctypes.c_int, vp, i64, i64, vp, i64, i64, vp, ctypes.c_int, i64, vp]
    L.linear_gemm_noalloc.restype = ctypes.c_int
    L.nf4_embed_rows.argtypes = [vp, i64, i64, vp, i64, vp, ctypes.c_int, i64, vp, vp]
    L.nf4_embed_rows.restype = ctypes.c_int
    L.linear_gemv_streamed.argtypes = [ctypes.c_int, i64, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, ctypes.c_int]
    L.linear_gemv_streamed.restype = ctypes.c_int
    L.linear_gemm_streamed.argtypes = [ctypes.c_int, i64, vp, vp, vp, vp, i64, i64, vp, ctypes.c_int, i64, vp, sz, vp,
                                       sz, vp, vp, vp, ctypes.c_int]
    L.linear_gemm_streamed.restype = ctypes.c_int
    L.wsl_stream_read.argtypes = [vp, sz, vp, vp]
    L.wsl_stream_read.restype = ctypes.c_int
    L.wsl_strerror.argtypes = [ctypes.c_int]
    L.wsl_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def wsl_strerror(code):
    return lib().wsl_strerror(int(code)).decode()


def _check(rc, where):
    if rc != WSL_OK:
        raise WSLError(rc, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtypes, device=None, contiguous=False, ndim=None):
    """Raise ValueError unless t is a device tensor of one of ``dtypes`` whose last
    dimension is unit-stride (whole tensor contiguous if ``contiguous``), on ``device``.
    The C ABI reads raw row-major memory, so a transposed or sliced view, or a tensor of
    another element type, must be refused here rather than misread."""
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {[str(d) for d in dtypes]}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dimensions, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.dim() > 0 and t.numel() > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must have stride 1 (got strides {t.stride()})")


def _weight(w, wfmt, n_out, k, name="w"):
    """Check a weight tensor against its format and shape: bf16 [n_out][k] contiguous, or a
    contiguous uint8 buffer of at least nf4_packed_bytes(n_out, k) bytes."""
    import torch
    if wfmt == WSL_W_NF4:
        _require(w, name, (torch.uint8,), contiguous=True)
        need = nf4_packed_bytes(n_out, k)
        if need and w.numel() < need:
            raise ValueError(f"{name}: {w.numel()} bytes, a packed {n_out}x{k} matrix needs {need}")
    elif wfmt == WSL_W_BF16:
        _require(w, name, (torch.bfloat16,), contiguous=True)
        if w.numel() < n_out * k:
            raise ValueError(f"{name}: {w.numel()} elements, a {n_out}x{k} bf16 matrix needs {n_out * k}")
    else:
        raise ValueError(f"{name}: unknown weight format {wfmt}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- format helpers
def nf4_packed_bytes(n_out, k):
    return int(lib().nf4_packed_bytes(int(n_out), int(k)))


def nf4_codebook():
    """The 16 binary32 levels the kernels use (a Python list of floats)."""
    buf = (ctypes.c_float * 16)()
    _check(lib().nf4_codebook(buf), "nf4_codebook")
    return [float(v) for v in buf]


# ---------------------------------------------------------------- entry points
def nf4_pack(w, packed=None, status=None, stream=None):
    """Encode a bf16 [n_out][k] device tensor into a packed NF4 uint8 device tensor."""
    import torch
    _require(w, "w", (torch.bfloat16,), contiguous=True, ndim=2)
    n_out, k = w.shape
    nbytes = nf4_packed_bytes(n_out, k)
    if packed is not None:
        _require(packed, "packed", (torch.uint8,), device=w.device, contiguous=True)
        if packed.numel() < nbytes:
            raise ValueError(f"packed: {packed.numel()} bytes, {n_out}x{k} needs {nbytes}")
    if status is not None:
        _require(status, "status", (torch.int32, torch.uint32), device=w.device)
    if packed is None:
        packed = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    rc = lib().nf4_pack(_ptr(w), n_out, k, _ptr(packed), _ptr(status), _stream(stream))
    _check(rc, "nf4_pack")
    return packed


def nf4_dequant_tile(packed, n_out, k, row0, k0, rows, cols, tile=None, ld_tile=None, stream=None):
    """Restore the bf16 tile [rows][cols] at (row0, k0) of a packed NF4 matrix."""
    import torch
    _weight(packed, WSL_W_NF4, n_out, k, "packed")
    if tile is None:
        tile = torch.empty((rows, cols), dtype=torch.bfloat16, device=packed.device)
        ld_tile = cols
    _require(tile, "tile", (torch.bfloat16,), device=packed.device)
    if ld_tile is None:
        ld_tile = tile.stride(0)
    rc = lib().nf4_dequant_tile(_ptr(packed), n_out, k, row0, k0, rows, cols, _ptr(tile), ld_tile, _stream(stream))
    _check(rc, "nf4_dequant_tile")
    return tile


def nf4_embed_rows(packed, n_rows, k, ids, out=None, ofmt=WSL_OUT_BF16, status=None, stream=None):
    """Restore rows ids (int64 device tensor) of a packed NF4 [n_rows][k] matrix into out [count][>= k]."""
    import torch
    _weight(packed, WSL_W_NF4, n_rows, k, "packed")
    _require(ids, "ids", (torch.int64,), device=packed.device, contiguous=True)
    count = int(ids.numel())
    dt = torch.bfloat16 if ofmt == WSL_OUT_BF16 else torch.float32
    if out is None:
        out = torch.empty((count, k), dtype=dt, device=packed.device)
    _require(out, "out", (dt,), device=packed.device, ndim=2)
    if status is not None:
        _require(status, "status", (torch.int32, torch.uint32), device=packed.device)
    rc = lib().nf4_embed_rows(_ptr(packed), n_rows, k, _ptr(ids), count, _ptr(out), int(ofmt), out.stride(0),
                              _ptr(status), _stream(stream))
    _check(rc, "nf4_embed_rows")
    return out


def linear_gemv(w, x, y=None, wfmt=None, n_out=None, k=None, stream=None):
    """y = W x (fp32).  w: bf16 [n_out][k] or packed NF4 uint8 (give n_out and k)."""
    import torch
    if wfmt is None:
        wfmt = WSL_W_NF4 if w.dtype == torch.uint8 else WSL_W_BF16
    if n_out is None or k is None:
        n_out, k = w.shape
    _weight(w, wfmt, n_out, k)
    _require(x, "x", (torch.bfloat16,), device=w.device, contiguous=True)
    if x.numel() < k:
        raise ValueError(f"x: {x.numel()} elements, k = {k}")
    if y is None:
        y = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _require(y, "y", (torch.float32,), device=w.device, contiguous=True)
    if y.numel() < n_out:
        raise ValueError(f"y: {y.numel()} elements, n_out = {n_out}")
    rc = lib().linear_gemv(int(wfmt), _ptr(w), n_out, k, _ptr(x), _ptr(y), _stream(stream))
    _check(rc, "linear_gemv")
    return y


def linear_gemm_workspace_bytes(wfmt, n_out, k, m):
    return int(lib().linear_gemm_workspace_bytes(int(wfmt), int(n_out), int(k), int(m)))


def linear_gemm(w, x, y=None, wfmt=None, n_out=None, k=None, ofmt=WSL_OUT_F32, workspace=None, stream=None):
    """Y = X W^T.  x: bf16 [m][k] (row stride = x.stride(0)); y fp32 or bf16 [m][n_out]."""
    import torch
    if wfmt is None:
        wfmt = WSL_W_NF4 if w.dtype == torch.uint8 else WSL_W_BF16
    if n_out is None or k is None:
        n_out, k = w.shape
    _weight(w, wfmt, n_out, k)
    _require(x, "x", (torch.bfloat16,), device=w.device, ndim=2)
    if x.shape[1] < k:
        raise ValueError(f"x: shape {tuple(x.shape)}, k = {k}")
    m = x.shape[0]
    dt = torch.float32 if ofmt == WSL_OUT_F32 else torch.bfloat16
    if y is None:
        y = torch.empty((m, n_out), dtype=dt, device=x.device)
    _require(y, "y", (dt,), device=w.device, ndim=2)
    if y.shape[0] < m or y.shape[1] < n_out:
        raise ValueError(f"y: shape {tuple(y.shape)}, need at least ({m}, {n_out})")
    if workspace is not None:
        _require(workspace, "workspace", (workspace.dtype,), device=w.device, contiguous=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().linear_gemm(int(wfmt), _ptr(w), n_out, k, _ptr(x), m, x.stride(0), _ptr(y), int(ofmt), y.stride(0),
                           _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "linear_gemm")
    return y


def linear_gemm_noalloc(w, x, y, wfmt=None, n_out=None, k=None, ofmt=WSL_OUT_F32, stream=None):
    """linear_gemm without a workspace argument and without allocating: the split partials use
    the library's per-device scratch (linear_gemm_noalloc).  y must be given (nothing is
    allocated here either)."""
    import torch
    if wfmt is None:
        wfmt = WSL_W_NF4 if w.dtype == torch.uint8 else WSL_W_BF16
    if n_out is None or k is None:
        n_out, k = w.shape
    _weight(w, wfmt, n_out, k)
    _require(x, "x", (torch.bfloat16,), device=w.device, ndim=2)
    if x.shape[1] < k:
        raise ValueError(f"x: shape {tuple(x.shape)}, k = {k}")
    m = x.shape[0]
    dt = torch.float32 if ofmt == WSL_OUT_F32 else torch.bfloat16
    _require(y, "y", (dt,), device=w.device, ndim=2)
    if y.shape[0] < m or y.shape[1] < n_out:
        raise ValueError(f"y: shape {tuple(y.shape)}, need at least ({m}, {n_out})")
    rc = lib().linear_gemm_noalloc(int(wfmt), _ptr(w), n_out, k, _ptr(x), m, x.stride(0), _ptr(y), int(ofmt),
                                   y.stride(0), _stream(stream))
    _check(rc, "linear_gemm_noalloc")
    return y


class WslGemvStage(ctypes.Structure):
    """struct wsl_gemv_stage of the C ABI."""
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n_out", ctypes.c_int64), ("k", ctypes.c_int64)]


class GemvSweep:
    """A decode sweep for linear_gemv_sweep: NF4 GEMVs run in order in one launch.

    stages: [(packed NF4 uint8 tensor, x bf16 [k], y fp32 [n_out], n_out, k)].  The host and
    device descriptor arrays and the zeroed synchronization workspace are built once here;
    each call enqueues the one launch on the current (or given) stream."""

    def __init__(self, stages):
        import torch
        if not stages:
            raise ValueError("a sweep needs at least one stage")
        dev = stages[0][0].device
        self.h = (WslGemvStage * len(stages))()
        for i, (w, x, y, n_out, k) in enumerate(stages):
            _weight(w, WSL_W_NF4, n_out, k, f"w[{i}]")
            _require(x, f"x[{i}]", (torch.bfloat16,), device=dev, contiguous=True)
            _require(y, f"y[{i}]", (torch.float32,), device=dev, contiguous=True)
            if x.numel() < k or y.numel() < n_out:
                raise ValueError(f"stage {i}: x has {x.numel()} of {k}, y {y.numel()} of {n_out} elements")
            self.h[i] = WslGemvStage(w.data_ptr(), x.data_ptr(), y.data_ptr(), int(n_out), int(k))
        self.count = len(stages)
        self.tensors = [t for st in stages for t in st[:3]]      # keep the buffers alive
        raw = bytes(self.h)
        self.d = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(dev)
        self.ws_bytes = int(lib().linear_gemv_sweep_workspace_bytes())
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)

    def __call__(self, stream=None):
        rc = lib().linear_gemv_sweep(WSL_W_NF4, self.count, ctypes.byref(self.h), _ptr(self.d), _ptr(self.ws),
                                     self.ws_bytes, _stream(stream))
        _check(rc, "linear_gemv_sweep")

    def status(self):
        """The workspace's status word (reads the device: for tests and diagnostics)."""
        return int(self.ws[SWEEP_STATUS_OFFSET:SWEEP_STATUS_OFFSET + 4].view(__import__("torch").int32).item())


GEMV_MULTI_MAX = 8


def linear_gemv_multi(mats, stream=None):
    """Independent bf16 GEMVs of one k in one launch (linear_gemv_multi): mats is a list of
    (w bf16 [n_out][k], x bf16 [k], y fp32 [n_out] or None); returns the ys."""
    import torch
    if not mats:
        return []
    if len(mats) > GEMV_MULTI_MAX:
        raise ValueError(f"{len(mats)} matrices, at most {GEMV_MULTI_MAX}")
    dev = mats[0][0].device
    h = (WslGemvStage * len(mats))()
    ys = []
    for i, (w, x, y) in enumerate(mats):
        n_out, k = w.shape
        _weight(w, WSL_W_BF16, n_out, k, f"w[{i}]")
        _require(x, f"x[{i}]", (torch.bfloat16,), device=dev, contiguous=True)
        if x.numel() < k:
            raise ValueError(f"x[{i}]: {x.numel()} elements, k = {k}")
        if y is None:
            y = torch.empty(n_out, dtype=torch.float32, device=dev)
        _require(y, f"y[{i}]", (torch.float32,), device=dev, contiguous=True)
        if y.numel() < n_out:
            raise ValueError(f"y[{i}]: {y.numel()} elements, n_out = {n_out}")
        h[i] = WslGemvStage(w.data_ptr(), x.data_ptr(), y.data_ptr(), int(n_out), int(k))
        ys.append(y)
    rc = lib().linear_gemv_multi(WSL_W_BF16, len(mats), ctypes.byref(h), _stream(stream))
    _check(rc, "linear_gemv_multi")
    return ys


def stream_read(buf, sink, stream=None):
    """Read every byte of the device tensor ``buf`` once (wsl_stream_read): the
    streaming-read ceiling probe.  ``sink`` is a device int32/uint32 tensor of one
    element, written only if a lane's words XOR to 0x9e3779b9."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().wsl_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "wsl_stream_read")


# ---------------------------------------------------------------- copy ring
def to_pinned(t):
    """A page-locked host copy (uint8) of a device or host tensor's bytes."""
    import torch
    src = t.contiguous().view(torch.uint8).reshape(-1)
    h = torch.empty(src.numel(), dtype=torch.uint8, pin_memory=True)
    h.copy_(src)
    return h


def _ptr_array(items):
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = t if isinstance(t, int) else t.data_ptr()
    return arr


def _i64_array(vals):
    arr = (ctypes.c_int64 * max(1, len(vals)))()
    for i, v in enumerate(vals):
        arr[i] = int(v)
    return arr


class CopyRing:
    """Two device slots, a copy stream and four events for linear_*_streamed.

    Matrices stay in page-locked host memory (see to_pinned); each call copies them one
    by one into the slots on the ring's copy stream while the kernels run on the compute
    stream (torch's current stream unless given).  pace=True (WSL_RING_PACE) keeps the
    host at most two matrices ahead of the kernels, so a call returns shortly before its
    last kernels finish; pace=False enqueues everything without waiting (capturable)."""

    def __init__(self, slot_bytes, device="cuda"):
        import torch
        self.slot_bytes = int(slot_bytes)
        self.slots = [torch.empty(max(self.slot_bytes, 16), dtype=torch.uint8, device=device) for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(device=device)
        self.events = [torch.cuda.Event() for _ in range(4)]
        for e in self.events:
            e.record()          # creates the events; a recorded, completed event is a no-op to wait on

    def _common(self, mats, xs, ys, x_dtype, y_dtypes):
        import torch
        if not (len(mats) == len(xs) == len(ys)):
            raise ValueError(f"{len(mats)} matrices, {len(xs)} inputs, {len(ys)} outputs")
        dev = self.slots[0].device
        for i, ((h, _, _), x, y) in enumerate(zip(mats, xs, ys)):
            if h.is_cuda or not h.is_contiguous():
                raise ValueError(f"matrix {i}: expected a contiguous host tensor (see to_pinned)")
            _require(x, f"x[{i}]", (x_dtype,), device=dev)
            _require(y, f"y[{i}]", y_dtypes, device=dev)
        hs = _ptr_array([h for h, _, _ in mats])
        ns = _i64_array([n for _, n, _ in mats])
        ks = _i64_array([k for _, _, k in mats])
        slots = _ptr_array(self.slots)
        evs = _ptr_array([e.cuda_event for e in self.events])
        return hs, ns, ks, slots, evs

    def gemv(self, mats, xs, ys, wfmt=WSL_W_NF4, stream=None, pace=True):
        """mats: [(pinned host tensor, n_out, k)]; xs: bf16 [k] device tensors; ys: fp32 [n_out]."""
        import torch
        hs, ns, ks, slots, evs = self._common(mats, xs, ys, torch.bfloat16, (torch.float32,))
        rc = lib().linear_gemv_streamed(int(wfmt), len(mats), hs, ns, ks, _ptr_array(xs), _ptr_array(ys), slots,
                                        self.slot_bytes, ctypes.c_void_p(self.copy_stream.cuda_stream),
                                        _stream(stream), evs, WSL_RING_PACE if pace else 0)
        _check(rc, "linear_gemv_streamed")
        return ys

    def gemm(self, mats, xs, ys, m, ldx, ldy, wfmt=WSL_W_NF4, ofmt=WSL_OUT_F32, workspace=None, stream=None,
             pace=True):
        import torch
        ydt = torch.float32 if ofmt == WSL_OUT_F32 else torch.bfloat16
        hs, ns, ks, slots, evs = self._common(mats, xs, ys, torch.bfloat16, (ydt,))
        nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = lib().linear_gemm_streamed(int(wfmt), len(mats), hs, ns, ks, _ptr_array(xs), int(m), int(ldx),
                                        _ptr_array(ys), int(ofmt), int(ldy), _ptr(workspace), nb, slots,
                                        self.slot_bytes, ctypes.c_void_p(self.copy_stream.cuda_stream),
                                        _stream(stream), evs, WSL_RING_PACE if pace else 0)
        _check(rc, "linear_gemm_streamed")
        return ys

