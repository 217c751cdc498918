"""Python binding of libsgemv.so: argument marshalling only.

Every step of the GEMV runs in the HIP library; this module converts torch
tensors and NumPy arrays to pointers and sizes, passes the current HIP
stream, and turns status codes into exceptions.  PyTorch is used for device
memory and streams only.  The names match the C entry points.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsgemv.so")

SGEMV_OK = 0
SGEMV_EINVAL = -1
SGEMV_ESIZE = -2
SGEMV_EALIGN = -3
SGEMV_EUNSUPPORTED = -4
SGEMV_EHIP = -5
SGEMV_OUT_F32 = 1
SGEMV_GROUP = 128
SGEMV_TILE_N = 512
SGEMV_LAYOUT_PAIRS = 1    # layout version 1: (s, z) fp16 pairs
SGEMV_LAYOUT_Z4 = 2       # layout version 2: fp16 scales, 4-bit zero-points
SGEMV_LAYOUT_NG = 3       # layout version 3: groups along N, (s, z) per column and 128 outputs
SGEMV_MAX_BATCH = 16
SGEMV_MAX_K = 65536
SGEMV_MAX_N = 1 << 20

EXPORTED = ["sgemv_pack_layout", "sgemv_pack_layout_z4", "sgemv_pack_layout_ng", "sgemv_pack_layout_parts",
            "sgemv_desc_from_header",
            "sgemv_gather_indices",
            "sgemv_run", "sgemv_run_batched", "sgemv_run_fused", "sgemv_run_fused_static", "sgemv_workspace_bytes",
            "sgemv_strerror", "sgemv_last_hip_error"]


class SgemvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})")


class Desc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("group", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("w_off", ctypes.c_uint64),
                ("w_bytes", ctypes.c_uint64), ("m_off", ctypes.c_uint64),
                ("m_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("version", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None


def lib():
    """Load libsgemv.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    pd = ctypes.POINTER(Desc)
    L.sgemv_pack_layout.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, sz, pd]
    L.sgemv_pack_layout.restype = ctypes.c_int
    L.sgemv_pack_layout_z4.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, sz, pd]
    L.sgemv_pack_layout_z4.restype = ctypes.c_int
    L.sgemv_pack_layout_ng.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, sz, pd]
    L.sgemv_pack_layout_ng.restype = ctypes.c_int
    L.sgemv_pack_layout_parts.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, u32, vp, sz, pd]
    L.sgemv_pack_layout_parts.restype = ctypes.c_int
    L.sgemv_desc_from_header.argtypes = [vp, sz, pd]
    L.sgemv_desc_from_header.restype = ctypes.c_int
    L.sgemv_gather_indices.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    L.sgemv_gather_indices.restype = ctypes.c_int
    L.sgemv_run.argtypes = [pd, vp, vp, vp, vp, vp, u32, vp, vp]
    L.sgemv_run.restype = ctypes.c_int
    L.sgemv_run_batched.argtypes = [pd, vp, vp, i32, i32, vp, vp, vp, vp, i32, u32, vp, vp]
    L.sgemv_run_batched.restype = ctypes.c_int
    L.sgemv_run_fused.argtypes = [pd, vp, vp, i32, i32, vp, vp, vp, vp, i32, u32, vp, vp]
    L.sgemv_run_fused.restype = ctypes.c_int
    L.sgemv_run_fused_static.argtypes = [pd, vp, vp, i32, i32, vp, vp, vp, vp, i32, u32, vp]
    L.sgemv_run_fused_static.restype = ctypes.c_int
    L.sgemv_workspace_bytes.argtypes = [pd, i32]
    L.sgemv_workspace_bytes.restype = sz
    L.sgemv_strerror.argtypes = [ctypes.c_int]
    L.sgemv_strerror.restype = ctypes.c_char_p
    L.sgemv_last_hip_error.argtypes = []
    L.sgemv_last_hip_error.restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().sgemv_strerror(int(status)).decode()


def _check(status: int, what: str):
    if status != SGEMV_OK:
        raise SgemvError(status, what)


def _ptr(t):
    """Address of a torch tensor, a NumPy array, or None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _require(t, what: str, dtypes, min_numel: int, rows: int | None = None):
    """Check a device buffer before its address crosses the ABI: a torch
    tensor of one of `dtypes` holding at least `min_numel` elements, its last
    dimension contiguous (and, for `rows`, 1-D or 2-D with that many rows),
    (the device is checked by _require_gpu, after every other check of a
    call).  A plain integer is taken as a raw device address and passed
    through unchecked.  Raises ValueError on the first failed check, before
    any library call."""
    if isinstance(t, int):
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        names = ", ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{what}: dtype {str(t.dtype).replace('torch.', '')}, expected {names}")
    if rows is not None:
        if t.dim() not in (1, 2) or (t.dim() == 2 and t.shape[0] != rows) or (t.dim() == 1 and rows != 1):
            raise ValueError(f"{what}: shape {tuple(t.shape)}, expected [{rows}][...] rows")
    if t.dim() >= 1 and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{what}: the last dimension must be contiguous")
    if t.dim() == 2 and t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{what}: rows overlap (stride {t.stride(0)} < {t.shape[1]})")
    if rows is None and t.dim() > 1 and not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{what}: {t.numel()} elements, at least {min_numel} needed")


def _require_gpu(**bufs):
    """Every tensor among `bufs` (name=tensor; None and raw addresses are
    skipped) lives on a GPU."""
    import torch
    for what, t in bufs.items():
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError(f"{what}: must be a GPU tensor")


def _f16():
    import torch
    return (torch.float16,)


def _i32():
    import torch
    return (torch.int32,)


def _u8():
    import torch
    return (torch.uint8,)


def _yt():
    import torch
    return (torch.float16, torch.float32)


def _require_matrix(desc: "Desc", packed, workspace, M: int):
    _require(packed, "packed", _u8(), int(desc.total_bytes))
    if workspace is None:   # the library says whether the call needs one (SGEMV_EINVAL)
        return
    _require(workspace, "workspace", _u8(), sgemv_workspace_bytes(desc, M))


def _thresholds(t, M):
    if t is None:
        return None
    arr = np.ascontiguousarray(np.asarray(t, dtype=np.float32).reshape(-1))
    if arr.size == 1 and M > 1:
        arr = np.repeat(arr, M)
    if arr.size != M:
        raise ValueError("one threshold per row")
    return arr


# ---------------------------------------------------------------------------
# the device and host calls
# ---------------------------------------------------------------------------
def sgemv_pack_layout(q, scales_f16, zeros_f16, tile_n: int = SGEMV_TILE_N, _which: str = "sgemv_pack_layout"):
    """Pack int4 codes q (uint8 [N][K]) and fp16 bit patterns of scales and
    zero-points (uint16 [N][K/128]) into a blob.  Returns (Desc, uint8 blob)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(scales_f16)
    z = np.ascontiguousarray(zeros_f16)
    if s.dtype == np.float16:
        s = s.view(np.uint16)
    if z.dtype == np.float16:
        z = z.view(np.uint16)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    z = np.ascontiguousarray(z, dtype=np.uint16)
    N, K = q.shape
    if _which == "sgemv_pack_layout_ng":
        if s.shape != (N // SGEMV_GROUP, K) or z.shape != (N // SGEMV_GROUP, K) or N % SGEMV_GROUP:
            raise ValueError("scales/zeros must be [N/128][K] (groups along N)")
    elif s.shape != (N, K // SGEMV_GROUP) or z.shape != (N, K // SGEMV_GROUP):
        raise ValueError("scales/zeros must be [N][K/128]")
    d = Desc()
    fn = getattr(lib(), _which)
    _check(fn(None, None, None, N, K, SGEMV_GROUP, tile_n, None, 0, ctypes.byref(d)), f"{_which}(size)")
    blob = np.empty(d.total_bytes, dtype=np.uint8)
    _check(fn(_ptr(q), _ptr(s), _ptr(z), N, K, SGEMV_GROUP, tile_n, _ptr(blob), blob.nbytes, ctypes.byref(d)),
           _which)
    return d, blob


def sgemv_pack_layout_z4(q, scales_f16, zeros_f16, tile_n: int = SGEMV_TILE_N):
    """As sgemv_pack_layout, with the compact metadata of layout version 2
    (fp16 scales, then the integer zero-points in 4 bits)."""
    return sgemv_pack_layout(q, scales_f16, zeros_f16, tile_n, _which="sgemv_pack_layout_z4")


def sgemv_pack_layout_ng(q, scales_f16, zeros_f16, tile_n: int = SGEMV_TILE_N):
    """Layout version 3, for weights quantized with groups along N: scales
    and zero-points are uint16 [N/128][K] (one per input column and 128
    outputs)."""
    return sgemv_pack_layout(q, scales_f16, zeros_f16, tile_n, _which="sgemv_pack_layout_ng")


def sgemv_pack_layout_parts(parts, tile_n: int = SGEMV_TILE_N, version: int = SGEMV_LAYOUT_PAIRS):
    """One blob for several projections sharing their input, rows stacked in
    the order given.  `parts` is a list of (q, scales_f16, zeros_f16), each
    with a row count that is a multiple of tile_n and the same K.  Returns
    (Desc, uint8 blob)."""
    qs, ss, zs, ns = [], [], [], []
    for q, s_, z in parts:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s_ = np.asarray(s_)
        z = np.asarray(z)
        s_ = np.ascontiguousarray(s_.view(np.uint16) if s_.dtype == np.float16 else s_, dtype=np.uint16)
        z = np.ascontiguousarray(z.view(np.uint16) if z.dtype == np.float16 else z, dtype=np.uint16)
        want = ((q.shape[0] // SGEMV_GROUP, q.shape[1]) if version == SGEMV_LAYOUT_NG
                else (q.shape[0], q.shape[1] // SGEMV_GROUP))
        if s_.shape != want or z.shape != s_.shape:
            raise ValueError("scales/zeros of a part must be " +
                             ("[N/128][K]" if version == SGEMV_LAYOUT_NG else "[N][K/128]"))
        qs.append(q); ss.append(s_); zs.append(z); ns.append(q.shape[0])
    Ks = {q.shape[1] for q in qs}
    if len(Ks) != 1:
        raise ValueError("parts must share K")
    K = Ks.pop()
    n = len(qs)
    qa = (ctypes.c_void_p * n)(*[a.ctypes.data for a in qs])
    sa = (ctypes.c_void_p * n)(*[a.ctypes.data for a in ss])
    za = (ctypes.c_void_p * n)(*[a.ctypes.data for a in zs])
    na = np.ascontiguousarray(ns, dtype=np.int32)
    d = Desc()
    L = lib()
    _check(L.sgemv_pack_layout_parts(n, None, None, None, na.ctypes.data, K, SGEMV_GROUP, tile_n, version,
                                     None, 0, ctypes.byref(d)), "sgemv_pack_layout_parts(size)")
    blob = np.empty(d.total_bytes, dtype=np.uint8)
    _check(L.sgemv_pack_layout_parts(n, qa, sa, za, na.ctypes.data, K, SGEMV_GROUP, tile_n, version,
                                     blob.ctypes.data, blob.nbytes, ctypes.byref(d)), "sgemv_pack_layout_parts")
    return d, blob


def sgemv_desc_from_header(blob) -> Desc:
    b = np.ascontiguousarray(np.asarray(blob, dtype=np.uint8)[:64])
    d = Desc()
    _check(lib().sgemv_desc_from_header(_ptr(b), b.nbytes, ctypes.byref(d)),
           "sgemv_desc_from_header")
    return d


def sgemv_gather_indices(x, thresholds, idx, count, K: int | None = None, stream=None):
    """x: fp16 device tensor [K] or [M][ldx]; writes idx (int32 [K]) and
    count (int32 [1]) on the device."""
    M = 1 if x.dim() == 1 else x.shape[0]
    ldx = x.shape[-1] if x.dim() == 1 else x.stride(0)
    K = x.shape[-1] if K is None else K
    _require(x, "x", _f16(), K, rows=M)
    if K > x.shape[-1]:
        raise ValueError(f"x: {x.shape[-1]} columns, K = {K}")
    _require(idx, "idx", _i32(), K)
    _require(count, "count", _i32(), 1)
    _require_gpu(x=x, idx=idx, count=count)
    t = _thresholds(thresholds, M)
    _check(lib().sgemv_gather_indices(_ptr(x), M, K, ldx, _ptr(t), _ptr(idx), _ptr(count),
                                      _stream(stream)), "sgemv_gather_indices")


def _flags(y):
    import torch
    if y.dtype == torch.float32:
        return SGEMV_OUT_F32
    if y.dtype == torch.float16:
        return 0
    raise TypeError("y must be float16 or float32")


def sgemv_run(desc: Desc, packed, x, idx, count, y, workspace, stream=None):
    """y = W . x over idx[:count] (idx None: all columns)."""
    _require_matrix(desc, packed, workspace, 1)
    _require(x, "x", _f16(), desc.K)
    if idx is not None or count is not None:
        _require(idx, "idx", _i32(), desc.K)
        _require(count, "count", _i32(), 1)
    _require(y, "y", _yt(), desc.N)
    _require_gpu(packed=packed, workspace=workspace, x=x, idx=idx, count=count, y=y)
    _check(lib().sgemv_run(ctypes.byref(desc), _ptr(packed), _ptr(x), _ptr(idx), _ptr(count),
                           _ptr(y), _flags(y), _ptr(workspace), _stream(stream)), "sgemv_run")


def sgemv_run_batched(desc: Desc, packed, x, thresholds, idx, count, y, workspace, stream=None):
    """y[m] = W . xe[m] over the union list; x is [M][ldx], y is [M][ldy]."""
    M = x.shape[0]
    _require_matrix(desc, packed, workspace, M)
    _require(x, "x", _f16(), desc.K, rows=M)
    _require(y, "y", _yt(), desc.N, rows=M)
    if x.shape[-1] < desc.K or y.shape[-1] < desc.N:
        raise ValueError(f"x/y: rows of {x.shape[-1]}/{y.shape[-1]}, need K = {desc.K} and N = {desc.N}")
    if idx is not None or count is not None:
        _require(idx, "idx", _i32(), desc.K)
        _require(count, "count", _i32(), 1)
    _require_gpu(packed=packed, workspace=workspace, x=x, idx=idx, count=count, y=y)
    t = _thresholds(thresholds, M)
    _check(lib().sgemv_run_batched(ctypes.byref(desc), _ptr(packed), _ptr(x), M, x.stride(0),
                                   _ptr(t), _ptr(idx), _ptr(count), _ptr(y), y.stride(0),
                                   _flags(y), _ptr(workspace), _stream(stream)),
           "sgemv_run_batched")


def sgemv_run_fused(desc: Desc, packed, x, thresholds, y, workspace, idx=None, count=None,
                    stream=None):
    """Threshold + compact + GEMV in one launch; x is [K] or [M][ldx] with
    M <= 16, y matches; idx/count (optional) receive the active list (the
    union over the rows)."""
    M = 1 if x.dim() == 1 else x.shape[0]
    ldx = desc.K if x.dim() == 1 else x.stride(0)
    ldy = desc.N if y.dim() == 1 else y.stride(0)
    _require_matrix(desc, packed, workspace, M)
    _require(x, "x", _f16(), desc.K, rows=M)
    _require(y, "y", _yt(), desc.N, rows=M)
    if x.shape[-1] < desc.K or y.shape[-1] < desc.N:
        raise ValueError(f"x/y: rows of {x.shape[-1]}/{y.shape[-1]}, need K = {desc.K} and N = {desc.N}")
    if (idx is None) != (count is None):
        raise ValueError("idx and count: both or neither")
    if idx is not None:
        _require(idx, "idx", _i32(), desc.K)
        _require(count, "count", _i32(), 1)
    _require_gpu(packed=packed, workspace=workspace, x=x, idx=idx, count=count, y=y)
    t = _thresholds(thresholds, M)
    _check(lib().sgemv_run_fused(ctypes.byref(desc), _ptr(packed), _ptr(x), M, ldx, _ptr(t),
                                 _ptr(idx), _ptr(count), _ptr(y), ldy, _flags(y),
                                 _ptr(workspace), _stream(stream)), "sgemv_run_fused")


def sgemv_run_fused_static(desc: Desc, packed, x, thresholds, y, idx=None, count=None, stream=None):
    """sgemv_run_fused without a workspace: the library's fixed device array
    holds the scratch (for callers that cannot allocate); no call may overlap
    another such call on the same GPU."""
    M = 1 if x.dim() == 1 else x.shape[0]
    ldx = desc.K if x.dim() == 1 else x.stride(0)
    ldy = desc.N if y.dim() == 1 else y.stride(0)
    _require(packed, "packed", _u8(), int(desc.total_bytes))
    _require(x, "x", _f16(), desc.K, rows=M)
    _require(y, "y", _yt(), desc.N, rows=M)
    if x.shape[-1] < desc.K or y.shape[-1] < desc.N:
        raise ValueError(f"x/y: rows of {x.shape[-1]}/{y.shape[-1]}, need K = {desc.K} and N = {desc.N}")
    if (idx is None) != (count is None):
        raise ValueError("idx and count: both or neither")
    if idx is not None:
        _require(idx, "idx", _i32(), desc.K)
        _require(count, "count", _i32(), 1)
    _require_gpu(packed=packed, x=x, idx=idx, count=count, y=y)
    t = _thresholds(thresholds, M)
    _check(lib().sgemv_run_fused_static(ctypes.byref(desc), _ptr(packed), _ptr(x), M, ldx, _ptr(t),
                                        _ptr(idx), _ptr(count), _ptr(y), ldy, _flags(y), _stream(stream)),
           "sgemv_run_fused_static")


def sgemv_workspace_bytes(desc: Desc, M: int = 1) -> int:
    return int(lib().sgemv_workspace_bytes(ctypes.byref(desc), M))


def sgemv_last_hip_error() -> int:
    return int(lib().sgemv_last_hip_error())


# ---------------------------------------------------------------------------
# convenience: device buffers for one matrix
# ---------------------------------------------------------------------------
class PackedMatrix:
    """A packed matrix on the device with its workspace (torch tensors)."""

    def __init__(self, q, scales_f16, zeros_f16, device="cuda", max_batch: int = SGEMV_MAX_BATCH,
                 z4: bool = False, _packed=None, ng: bool = False):
        import torch
        if _packed is None:
            pack = sgemv_pack_layout_ng if ng else sgemv_pack_layout_z4 if z4 else sgemv_pack_layout
            _packed = pack(q, scales_f16, zeros_f16)
        self.desc, blob = _packed
        self.blob = torch.from_numpy(blob).to(device)
        self.workspace = torch.zeros(max(sgemv_workspace_bytes(self.desc, max_batch), 256),
                                     dtype=torch.uint8, device=device)
        self.N, self.K = self.desc.N, self.desc.K

    @classmethod
    def from_parts(cls, parts, device="cuda", max_batch: int = SGEMV_MAX_BATCH, z4: bool = False,
                   ng: bool = False):
        """Several projections sharing their input as one matrix (rows
        stacked in order), packed by sgemv_pack_layout_parts (ng: parts
        quantized with groups along N, layout version 3)."""
        version = SGEMV_LAYOUT_NG if ng else SGEMV_LAYOUT_Z4 if z4 else SGEMV_LAYOUT_PAIRS
        packed = sgemv_pack_layout_parts(parts, version=version)
        return cls(None, None, None, device=device, max_batch=max_batch, z4=z4, _packed=packed, ng=ng)


class FusedProjections:
    """Projections that read the same activations (q/k/v, gate/up), packed
    as one matrix with their rows concatenated, so that one call of
    sgemv_run_fused thresholds x once and computes all of them.  Each
    projection's N must be a multiple of 512 (the layout tile), so every
    tile belongs to one projection.  `split(y)` returns the per-projection
    views of the concatenated output."""

    def __init__(self, parts, device="cuda", max_batch: int = 2, z4: bool = False, ng: bool = False):
        names = [p[0] for p in parts]
        if len(set(names)) != len(names):
            raise ValueError("projection names must be unique")
        Ks = {np.asarray(p[1]).shape[1] for p in parts}
        if len(Ks) != 1:
            raise ValueError("fused projections must share K")
        self.offsets = {}
        start = 0
        for name, q, _, _ in parts:
            n = np.asarray(q).shape[0]
            if n % SGEMV_TILE_N:
                raise ValueError(f"{name}: N = {n} is not a multiple of {SGEMV_TILE_N}")
            self.offsets[name] = (start, n)
            start += n
        self.matrix = PackedMatrix.from_parts([p[1:] for p in parts], device=device, max_batch=max_batch, z4=z4,
                                              ng=ng)
        self.N, self.K = self.matrix.N, self.matrix.K

    def split(self, y):
        return {name: y[..., a:a + n] for name, (a, n) in self.offsets.items()}
