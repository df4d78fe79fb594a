"""ctypes binding of libq8moe.so: the same names as the C ABI (include/q8moe.h).

Argument marshalling only: every computation happens in the HIP kernels of the
library.  Tensors are torch tensors on the GPU; Q8_0 data is a uint8 tensor
whose last dimension is (k/32)*34 bytes.  Work is enqueued on torch's current
stream of the tensors' device.  A negative status raises Q8Error.

There is no fallback: if libq8moe.so is missing or cannot be loaded, importing
this module raises.
"""
import ctypes
import os

import torch

QK = 32
BLOCK_BYTES = 34

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8moe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                      "python moe_expert_ffn_q8_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t


class Q8MatmulDesc(ctypes.Structure):
    _fields_ = [("w", _vp), ("x", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("m", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_row_stride", _i64), ("x_batch_stride", _i64),
                ("y_row_stride", _i64), ("y_batch_stride", _i64)]


class Q8R8Desc(ctypes.Structure):
    _fields_ = [("w_r8", _vp), ("x", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_batch_stride", _i64), ("y_batch_stride", _i64)]


class Q8R8F32Desc(ctypes.Structure):
    _fields_ = [("w_r8", _vp), ("x", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_batch_stride", _i64), ("y_batch_stride", _i64)]


class Q8R8MmDesc(ctypes.Structure):
    _fields_ = [("w_r8", _vp), ("x", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("m", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_row_stride", _i64), ("x_batch_stride", _i64),
                ("y_row_stride", _i64), ("y_batch_stride", _i64)]


class MoeR8FfnDesc(ctypes.Structure):
    _fields_ = [("w_up_gate_r8", _vp), ("w_down_r8", _vp), ("x", _vp), ("ids", _vp), ("cw", _vp),
                ("h", _vp), ("out", _vp), ("ws", _vp), ("ws_bytes", ctypes.c_size_t)]


class KqMatvecDesc(ctypes.Structure):
    _fields_ = [("w", _vp), ("x", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_batch_stride", _i64), ("y_batch_stride", _i64)]


class Q8UpGateDesc(ctypes.Structure):
    _fields_ = [("w", _vp), ("x", _vp), ("h", _vp),
                ("n_ff", _i64), ("n_embd", _i64), ("m", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_row_stride", _i64), ("x_batch_stride", _i64),
                ("h_row_stride", _i64), ("h_batch_stride", _i64)]


class Q8MatmulF32Desc(ctypes.Structure):
    _fields_ = [("w", _vp), ("x", _vp), ("y", _vp),
                ("n", _i64), ("k", _i64), ("m", _i64), ("batch", _i64),
                ("w_batch_stride", _i64), ("x_row_stride", _i64), ("x_batch_stride", _i64),
                ("y_row_stride", _i64), ("y_batch_stride", _i64)]


class MoeUpGateDesc(ctypes.Structure):
    _fields_ = [("w_up_gate", _vp), ("x", _vp), ("ids", _vp), ("h", _vp), ("ws", _vp),
                ("ws_bytes", _size)]


class MoeDownDesc(ctypes.Structure):
    _fields_ = [("w_down", _vp), ("h", _vp), ("ids", _vp), ("cw", _vp), ("out", _vp),
                ("ws", _vp), ("ws_bytes", _size)]


_SIGS = {
    "q8_status_str": (ctypes.c_char_p, [_int]),
    "q8_version": (ctypes.c_char_p, []),
    "q8_0_quantize_rows": (_int, [_vp, _i64, _vp, _i64, _i64, _vp]),
    "q8_0_matvec": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "q8_0_matmul": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q8_0_matmul_batched": (_int, [ctypes.POINTER(Q8MatmulDesc), _i64, _vp]),
    "q8_0_matmul_f32_batched": (_int, [ctypes.POINTER(Q8MatmulF32Desc), _i64, _vp]),
    "q8_0_up_gate_swiglu_batched": (_int, [ctypes.POINTER(Q8UpGateDesc), _i64, _vp]),
    "q8_0_matmul_f32_step_ws_bytes": (_i64, [ctypes.POINTER(Q8MatmulF32Desc), _i64]),
    "q8_0_matmul_f32_step": (_int, [ctypes.POINTER(Q8MatmulF32Desc), _i64, _vp, _i64, _vp]),
    "moe_workspace_bytes": (_size, [_i64, _i64, _i64, _i64, _i64]),
    "moe_up_gate_swiglu": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp,
                                  _size, _vp]),
    "moe_down_combine": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp,
                                _size, _vp]),
    "moe_up_gate_swiglu_batched": (_int, [ctypes.POINTER(MoeUpGateDesc), _i64, _i64, _i64, _i64,
                                          _i64, _i64, _vp]),
    "moe_down_combine_batched": (_int, [ctypes.POINTER(MoeDownDesc), _i64, _i64, _i64, _i64, _i64,
                                        _i64, _vp]),
    "q8_0_matmul_blocksums": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q8v_matvec_r8_batched_blocksums": (_int, [ctypes.POINTER(Q8R8Desc), _i64,
                                               ctypes.POINTER(_vp), _vp]),
    "q8v_matvec_r8_f32_batched_blocksums": (_int, [ctypes.POINTER(Q8R8F32Desc), _i64,
                                                   ctypes.POINTER(_vp), _vp]),
    "q8v_matmul_r8_batched_blocksums": (_int, [ctypes.POINTER(Q8R8MmDesc), _i64,
                                               ctypes.POINTER(_vp), _vp]),
    "moe_route": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _size, _vp]),
    "q8v_moe_up_gate": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                               _i64, _vp, _size, _vp]),
    "q8v_moe_hq": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp,
                          _size, _vp]),
    "q8v_moe_r8_ffn": (_int, [ctypes.POINTER(MoeR8FfnDesc), _i64, _i64, _i64, _i64, _i64, _vp,
                              _vp, _vp, _vp, _vp, _vp, _vp]),
    "q8_read_probe": (_int, [_vp, _i64, _vp, _i64, _vp]),
    "q8_0_r8_bytes": (_i64, [_i64, _i64]),
    "q8_0_repack_r8": (_int, [_vp, _vp, _i64, _i64, _vp]),
    "q8_0_matvec_r8": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "q8_0_matvec_r8_batched": (_int, [ctypes.POINTER(Q8R8Desc), _i64, _vp]),
    "q8_0_matvec_r8_f32_batched": (_int, [ctypes.POINTER(Q8R8F32Desc), _i64, _vp]),
    "q8_0_matmul_r8_batched": (_int, [ctypes.POINTER(Q8R8MmDesc), _i64, _vp]),
    "q8_1_quantize_rows": (_int, [_vp, _i64, _vp, _i64, _i64, _vp]),
    "moe_r8_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64]),
    "moe_r8_ffn_batched": (_int, [ctypes.POINTER(MoeR8FfnDesc), _i64, _i64, _i64, _i64, _i64,
                                  _i64, _vp]),
    "moe_r8_ffn_batched_noalloc": (_int, [ctypes.POINTER(MoeR8FfnDesc), _i64, _i64, _i64, _i64,
                                          _i64, _i64, _vp]),
    "moe_r8_fused_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64]),
    "moe_r8_ffn_fused": (_int, [ctypes.POINTER(MoeR8FfnDesc), _i64, _i64, _i64, _i64, _vp]),
    "kq_matvec_batched": (_int, [_int, ctypes.POINTER(KqMatvecDesc), _i64, _vp]),
    "q4_k_matvec": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "q5_k_matvec": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
}

EXPORTS = tuple(_SIGS)

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

STATUS = {0: "Q8_OK", -1: "Q8_E_NULL", -2: "Q8_E_SHAPE", -3: "Q8_E_ALIGN",
          -4: "Q8_E_UNSUPPORTED", -5: "Q8_E_WORKSPACE", -6: "Q8_E_HIP"}


class Q8Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib.q8_status_str(status).decode()
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")


def _check(fn, rc):
    if rc != 0:
        raise Q8Error(fn, rc)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    if t is None or not t.is_cuda:
        return None
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, name):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")


def _nbytes(t):
    return t.numel() * t.element_size()


def _fit(t, nbytes, name):
    """A contiguous GPU tensor that holds at least nbytes (the extent the
    kernels touch for the shape arguments of the call)."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if nbytes > _nbytes(t):
        raise ValueError(f"{name}: the shape arguments need {nbytes} bytes, the tensor holds "
                         f"{_nbytes(t)}")


def _one_device(*ts):
    """Every tensor (or (tensor, offset) pair) of a call on one device."""
    devs = {(t[0] if isinstance(t, tuple) else t).device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(map(str, devs))}")


def _addr(t, unit, nbytes, name):
    """Address of a descriptor operand: t is a tensor or a (tensor, offset)
    pair with the offset in `unit` bytes; the tensor must hold nbytes from
    that address on."""
    base, off = (t if isinstance(t, tuple) else (t, 0))
    if not base.is_contiguous() or not base.is_cuda:
        raise ValueError(f"{name}: must be a contiguous GPU tensor")
    if off < 0:
        raise ValueError(f"{name}: negative offset")
    avail = _nbytes(base) - off * unit
    if nbytes > 0 and nbytes > avail:
        raise ValueError(f"{name}: the descriptor needs {nbytes} bytes from its start, the "
                         f"tensor holds {max(avail, 0)}")
    return base.data_ptr() + off * unit


def _span(batch, bstride, rows, rstride, last):
    """Elements from the first to one past the last one touched: `batch`
    entries `bstride` apart, each `rows` rows `rstride` apart of `last`
    elements (0 when nothing is touched)."""
    if batch <= 0 or rows <= 0 or last <= 0:
        return 0
    return (batch - 1) * bstride + (rows - 1) * rstride + last


def _r8_bytes_py(n, k):
    return (n + 7) // 8 * 272 * (k // QK)


def status_str(status):
    return _lib.q8_status_str(int(status)).decode()


def version():
    return _lib.q8_version().decode()


def q8_empty(rows, k, device):
    """Uninitialised Q8_0 storage for [rows][k] values (uint8 [rows][k/32*34])."""
    return torch.empty((rows, k // QK * BLOCK_BYTES), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------

def q8_0_quantize_rows(x, y=None, k=None):
    """x: fp32 [n_rows][stride] (or [k]) -> y: uint8 [n_rows][k/32*34]."""
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x: GPU fp32 with unit column stride")
    n_rows = x.shape[0]
    k = x.shape[1] if k is None else k
    if x.shape[1] < k:
        raise ValueError(f"x: rows of {x.shape[1]} values, k = {k}")
    if y is None:
        y = q8_empty(n_rows, k, x.device)
    _need(y, torch.uint8, "y")
    _one_device(x, y)
    _fit(y, n_rows * (k // QK) * BLOCK_BYTES, "y")
    _check("q8_0_quantize_rows", _lib.q8_0_quantize_rows(
        _ptr(x), x.stride(0) if n_rows > 1 else k, _ptr(y), n_rows, k, _stream(x)))
    return y


def q8_0_matvec(w, x, n, k, y=None):
    _need(w, torch.uint8, "w")
    _need(x, torch.uint8, "x")
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w.device)
    _need(y, torch.float32, "y")
    _one_device(w, x, y)
    nb = k // QK
    _fit(w, n * nb * BLOCK_BYTES, "w")
    _fit(x, nb * BLOCK_BYTES, "x")
    _fit(y, n * 4, "y")
    _check("q8_0_matvec", _lib.q8_0_matvec(_ptr(w), _ptr(x), _ptr(y), n, k, _stream(w)))
    return y


def q8_0_r8_bytes(n, k):
    v = _lib.q8_0_r8_bytes(n, k)
    _check("q8_0_r8_bytes", v if v < 0 else 0)
    return int(v)


def q8_0_repack_r8(w, n, k, out=None):
    """Native Q8_0 rows (uint8 GPU tensor) -> the row-interleaved (R8) layout."""
    _need(w, torch.uint8, "w")
    if out is None:
        out = torch.empty(q8_0_r8_bytes(n, k), dtype=torch.uint8, device=w.device)
    _need(out, torch.uint8, "out")
    _one_device(w, out)
    _fit(w, n * (k // QK) * BLOCK_BYTES, "w")
    _fit(out, q8_0_r8_bytes(n, k), "out")
    _check("q8_0_repack_r8", _lib.q8_0_repack_r8(_ptr(w), _ptr(out), n, k, _stream(w)))
    return out


def q8_0_matvec_r8(w_r8, x, n, k, y=None):
    _need(w_r8, torch.uint8, "w_r8")
    _need(x, torch.uint8, "x")
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w_r8.device)
    _need(y, torch.float32, "y")
    _one_device(w_r8, x, y)
    _fit(w_r8, q8_0_r8_bytes(n, k), "w_r8")
    _fit(x, (k // QK) * BLOCK_BYTES, "x")
    _fit(y, n * 4, "y")
    _check("q8_0_matvec_r8", _lib.q8_0_matvec_r8(_ptr(w_r8), _ptr(x), _ptr(y), n, k,
                                                 _stream(w_r8)))
    return y


def make_r8_desc(w_r8, x, y, n, k, batch=1, w_batch_stride=0, x_batch_stride=0,
                 y_batch_stride=0):
    """One q8_0_r8_desc.  w_r8 (bytes), x (blocks), y (floats) are (tensor,
    element offset) pairs or tensors; w_batch_stride in bytes, x_batch_stride
    in blocks, y_batch_stride in floats."""
    _one_device(w_r8, x, y)
    nb = k // QK
    wb = _span(batch, w_batch_stride, 1, 0, _r8_bytes_py(n, k)) if n > 0 else 0
    return Q8R8Desc(_addr(w_r8, 1, wb, "w_r8"),
                    _addr(x, BLOCK_BYTES, _span(batch, x_batch_stride, 1, 0, nb) * BLOCK_BYTES, "x"),
                    _addr(y, 4, _span(batch, y_batch_stride, 1, 0, n) * 4, "y"), n, k, batch,
                    w_batch_stride, x_batch_stride, y_batch_stride)


def q8_0_matvec_r8_batched(descs, stream_of):
    """descs: list of Q8R8Desc; stream_of: a tensor on the target device."""
    arr = (Q8R8Desc * max(1, len(descs)))(*descs)
    _check("q8_0_matvec_r8_batched",
           _lib.q8_0_matvec_r8_batched(arr, len(descs), _stream(stream_of)))


def make_r8_f32_desc(w_r8, x, y, n, k, batch=1, w_batch_stride=0, x_batch_stride=0,
                     y_batch_stride=0):
    """One q8_0_r8_f32_desc.  w_r8 (bytes), x (floats), y (floats) are (tensor,
    element offset) pairs or tensors; w_batch_stride in bytes, the others in
    floats."""
    _one_device(w_r8, x, y)
    wb = _span(batch, w_batch_stride, 1, 0, _r8_bytes_py(n, k)) if n > 0 else 0
    return Q8R8F32Desc(_addr(w_r8, 1, wb, "w_r8"),
                       _addr(x, 4, _span(batch, x_batch_stride, 1, 0, k) * 4 if n > 0 else 0, "x"),
                       _addr(y, 4, _span(batch, y_batch_stride, 1, 0, n) * 4, "y"), n, k, batch,
                       w_batch_stride, x_batch_stride, y_batch_stride)


def _sum_ptrs(sums):
    for i, t in enumerate(sums):
        _need(t, torch.int32, f"sums[{i}]")
    return (_vp * max(1, len(sums)))(*[t.data_ptr() for t in sums])


def q8v_matvec_r8_batched_blocksums(descs, sums, stream_of):
    """q8_0_matvec_r8_batched plus the int32 block sums of descriptor i in
    sums[i] (a GPU int32 tensor of batch*n*(k/32) elements)."""
    for d, t in zip(descs, sums):
        _fit(t, max(d.batch, 0) * max(d.n, 0) * (d.k // QK) * 4, "sums")
    arr = (Q8R8Desc * max(1, len(descs)))(*descs)
    _check("q8v_matvec_r8_batched_blocksums", _lib.q8v_matvec_r8_batched_blocksums(
        arr, len(descs), _sum_ptrs(sums), _stream(stream_of)))


def q8v_matvec_r8_f32_batched_blocksums(descs, sums, stream_of):
    """q8_0_matvec_r8_f32_batched plus the int32 block sums of descriptor i in
    sums[i] (batch*n*(k/32) elements)."""
    for d, t in zip(descs, sums):
        _fit(t, max(d.batch, 0) * max(d.n, 0) * (d.k // QK) * 4, "sums")
    arr = (Q8R8F32Desc * max(1, len(descs)))(*descs)
    _check("q8v_matvec_r8_f32_batched_blocksums", _lib.q8v_matvec_r8_f32_batched_blocksums(
        arr, len(descs), _sum_ptrs(sums), _stream(stream_of)))


def q8v_matmul_r8_batched_blocksums(descs, sums, stream_of):
    """q8_0_matmul_r8_batched plus the int32 block sums of descriptor i in
    sums[i] (batch*m*n*(k/32) elements)."""
    for d, t in zip(descs, sums):
        _fit(t, max(d.batch, 0) * max(d.m, 0) * max(d.n, 0) * (d.k // QK) * 4, "sums")
    arr = (Q8R8MmDesc * max(1, len(descs)))(*descs)
    _check("q8v_matmul_r8_batched_blocksums", _lib.q8v_matmul_r8_batched_blocksums(
        arr, len(descs), _sum_ptrs(sums), _stream(stream_of)))


def q8_0_matvec_r8_f32_batched(descs, stream_of):
    """descs: list of Q8R8F32Desc; stream_of: a tensor on the target device."""
    arr = (Q8R8F32Desc * max(1, len(descs)))(*descs)
    _check("q8_0_matvec_r8_f32_batched",
           _lib.q8_0_matvec_r8_f32_batched(arr, len(descs), _stream(stream_of)))


def make_r8_mm_desc(w_r8, x, y, n, k, m=1, batch=1, w_batch_stride=0, x_row_stride=None,
                    x_batch_stride=0, y_row_stride=None, y_batch_stride=0):
    """One q8_0_r8_mm_desc.  w_r8 (bytes), x (blocks), y (floats) are (tensor,
    element offset) pairs or tensors; w_batch_stride in bytes, x strides in
    blocks, y strides in floats."""
    nb = k // QK
    xrs = nb if x_row_stride is None else x_row_stride
    yrs = n if y_row_stride is None else y_row_stride
    _one_device(w_r8, x, y)
    live = n > 0 and m > 0
    wb = _span(batch, w_batch_stride, 1, 0, _r8_bytes_py(n, k)) if live else 0
    xb = _span(batch, x_batch_stride, m, xrs, nb) * BLOCK_BYTES if live else 0
    return Q8R8MmDesc(_addr(w_r8, 1, wb, "w_r8"), _addr(x, BLOCK_BYTES, xb, "x"),
                      _addr(y, 4, _span(batch, y_batch_stride, m, yrs, n) * 4, "y"), n, k, m,
                      batch, w_batch_stride, xrs, x_batch_stride, yrs, y_batch_stride)


def q8_0_matmul_r8_batched(descs, stream_of):
    arr = (Q8R8MmDesc * max(1, len(descs)))(*descs)
    _check("q8_0_matmul_r8_batched",
           _lib.q8_0_matmul_r8_batched(arr, len(descs), _stream(stream_of)))


Q8_1_BLOCK_BYTES = 36
KQ_BLOCK_BYTES = {4: 144, 5: 176}


def q8_1_quantize_rows(x, k=None, y=None):
    """x: fp32 [n_rows][stride] (or [k]) -> y: uint8 [n_rows][k/32*36] (Q8_1)."""
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x: GPU fp32 with unit column stride")
    n_rows = x.shape[0]
    k = x.shape[1] if k is None else k
    if x.shape[1] < k:
        raise ValueError(f"x: rows of {x.shape[1]} values, k = {k}")
    if y is None:
        y = torch.empty((n_rows, k // QK * Q8_1_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    _need(y, torch.uint8, "y")
    _one_device(x, y)
    _fit(y, n_rows * (k // QK) * Q8_1_BLOCK_BYTES, "y")
    _check("q8_1_quantize_rows", _lib.q8_1_quantize_rows(
        _ptr(x), x.stride(0) if n_rows > 1 else k, _ptr(y), n_rows, k, _stream(x)))
    return y


def kq_matvec(t, w, x, n, k, y=None):
    """One product over K-quant weights (t = 4: Q4_K, t = 5: Q5_K) and a Q8_1 row."""
    _need(w, torch.uint8, "w")
    _need(x, torch.uint8, "x")
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w.device)
    _need(y, torch.float32, "y")
    fn = {4: _lib.q4_k_matvec, 5: _lib.q5_k_matvec}.get(t)
    if fn is None:
        raise ValueError(f"unknown K-quant type {t}")
    _one_device(w, x, y)
    _fit(w, n * (k // 256) * KQ_BLOCK_BYTES[t], "w")
    _fit(x, (k // QK) * Q8_1_BLOCK_BYTES, "x")
    _fit(y, n * 4, "y")
    _check("q4_k_matvec" if t == 4 else "q5_k_matvec",
           fn(_ptr(w), _ptr(x), _ptr(y), n, k, _stream(w)))
    return y


def make_kq_desc(w, x, y, n, k, batch=1, w_batch_stride=0, x_batch_stride=0, y_batch_stride=0,
                 t=4):
    """One kq_matvec_desc for K-quant type t (4: Q4_K, 5: Q5_K).  w (bytes), x
    (bytes), y (floats) are (tensor, element offset) pairs or tensors; strides
    in super-blocks, Q8_1 blocks, floats."""
    _one_device(w, x, y)
    bb = KQ_BLOCK_BYTES[t]
    live = n > 0
    wb = _span(batch, w_batch_stride, 1, 0, n * (k // 256)) * bb if live else 0
    xb = _span(batch, x_batch_stride, 1, 0, k // QK) * Q8_1_BLOCK_BYTES if live else 0
    return KqMatvecDesc(_addr(w, 1, wb, "w"), _addr(x, 1, xb, "x"),
                        _addr(y, 4, _span(batch, y_batch_stride, 1, 0, n) * 4, "y"), n, k, batch,
                        w_batch_stride, x_batch_stride, y_batch_stride)


def kq_matvec_batched(t, descs, stream_of):
    arr = (KqMatvecDesc * max(1, len(descs)))(*descs)
    _check("kq_matvec_batched", _lib.kq_matvec_batched(t, arr, len(descs), _stream(stream_of)))


def q8_0_matmul(w, x, n, k, m, y=None):
    _need(w, torch.uint8, "w")
    _need(x, torch.uint8, "x")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _need(y, torch.float32, "y")
    _one_device(w, x, y)
    nb = k // QK
    _fit(w, n * nb * BLOCK_BYTES, "w")
    _fit(x, m * nb * BLOCK_BYTES, "x")
    _fit(y, m * n * 4, "y")
    _check("q8_0_matmul", _lib.q8_0_matmul(_ptr(w), _ptr(x), _ptr(y), n, k, m, _stream(w)))
    return y


def make_desc(w, x, y, n, k, m=1, batch=1, w_batch_stride=0, x_row_stride=None,
              x_batch_stride=0, y_row_stride=None, y_batch_stride=0):
    """One q8_0_matmul_desc.  w, x, y are (tensor, element offset) pairs or tensors;
    strides are in blocks (w, x) and floats (y)."""
    nb = k // QK
    xrs = nb if x_row_stride is None else x_row_stride
    yrs = n if y_row_stride is None else y_row_stride
    _one_device(w, x, y)
    live = n > 0 and m > 0
    wb = _span(batch, w_batch_stride, 1, 0, n * nb) * BLOCK_BYTES if live else 0
    xb = _span(batch, x_batch_stride, m, xrs, nb) * BLOCK_BYTES if live else 0
    return Q8MatmulDesc(_addr(w, BLOCK_BYTES, wb, "w"), _addr(x, BLOCK_BYTES, xb, "x"),
                        _addr(y, 4, _span(batch, y_batch_stride, m, yrs, n) * 4, "y"), n, k, m,
                        batch, w_batch_stride, xrs, x_batch_stride, yrs, y_batch_stride)


def make_up_gate_desc(w, x, h, n_ff, n_embd, m=1, batch=1, w_batch_stride=0, x_row_stride=None,
                      x_batch_stride=0, h_row_stride=None, h_batch_stride=0):
    """One q8_0_up_gate_desc.  w (combined [2*n_ff][n_embd/32] blocks, gate rows
    first), x (Q8_0 rows), h are (tensor, element offset) pairs or tensors;
    strides are in blocks (w, x) and floats (h)."""
    nb = n_embd // QK
    xrs = nb if x_row_stride is None else x_row_stride
    hrs = n_ff if h_row_stride is None else h_row_stride
    _one_device(w, x, h)
    live = n_ff > 0 and m > 0
    wb = _span(batch, w_batch_stride, 1, 0, 2 * n_ff * nb) * BLOCK_BYTES if live else 0
    xb = _span(batch, x_batch_stride, m, xrs, nb) * BLOCK_BYTES if live else 0
    return Q8UpGateDesc(_addr(w, BLOCK_BYTES, wb, "w"), _addr(x, BLOCK_BYTES, xb, "x"),
                        _addr(h, 4, _span(batch, h_batch_stride, m, hrs, n_ff) * 4, "h"), n_ff,
                        n_embd, m, batch, w_batch_stride, xrs, x_batch_stride, hrs,
                        h_batch_stride)


def q8_0_up_gate_swiglu_batched(descs, stream_of):
    """descs: list of Q8UpGateDesc; stream_of: a tensor on the target device."""
    arr = (Q8UpGateDesc * max(1, len(descs)))(*descs)
    _check("q8_0_up_gate_swiglu_batched",
           _lib.q8_0_up_gate_swiglu_batched(arr, len(descs), _stream(stream_of)))


def q8_0_matmul_batched(descs, stream_of):
    """descs: list of Q8MatmulDesc; stream_of: a tensor on the target device."""
    arr = (Q8MatmulDesc * len(descs))(*descs)
    _check("q8_0_matmul_batched", _lib.q8_0_matmul_batched(arr, len(descs), _stream(stream_of)))


def make_f32_desc(w, x, y, n, k, m=1, batch=1, w_batch_stride=0, x_row_stride=None,
                  x_batch_stride=0, y_row_stride=None, y_batch_stride=0):
    """One q8_0_matmul_f32_desc (fp32 activations, quantized inside).  w, x, y
    are (tensor, element offset) pairs or tensors; strides are in blocks (w)
    and floats (x, y)."""
    xrs = k if x_row_stride is None else x_row_stride
    yrs = n if y_row_stride is None else y_row_stride
    _one_device(w, x, y)
    live = n > 0 and m > 0
    wb = _span(batch, w_batch_stride, 1, 0, n * (k // QK)) * BLOCK_BYTES if live else 0
    xb = _span(batch, x_batch_stride, m, xrs, k) * 4 if live else 0
    return Q8MatmulF32Desc(_addr(w, BLOCK_BYTES, wb, "w"), _addr(x, 4, xb, "x"),
                           _addr(y, 4, _span(batch, y_batch_stride, m, yrs, n) * 4, "y"), n, k,
                           m, batch, w_batch_stride, xrs, x_batch_stride, yrs, y_batch_stride)


def q8_0_matmul_f32_batched(descs, stream_of):
    """descs: list of Q8MatmulF32Desc; stream_of: a tensor on the target device."""
    arr = (Q8MatmulF32Desc * len(descs))(*descs)
    _check("q8_0_matmul_f32_batched",
           _lib.q8_0_matmul_f32_batched(arr, len(descs), _stream(stream_of)))


def q8_0_matmul_f32_step_ws_bytes(descs):
    """Workspace bytes q8_0_matmul_f32_step needs for these descriptors."""
    arr = (Q8MatmulF32Desc * max(1, len(descs)))(*descs)
    n = int(_lib.q8_0_matmul_f32_step_ws_bytes(arr, len(descs)))
    if n < 0:
        raise Q8Error("q8_0_matmul_f32_step_ws_bytes", n)
    return n


def q8_0_matmul_f32_step_workspace(descs, device):
    """A zero-filled workspace for q8_0_matmul_f32_step (uint8 tensor)."""
    n = q8_0_matmul_f32_step_ws_bytes(descs)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def q8_0_matmul_f32_step(descs, ws, stream_of=None):
    """descs: list of Q8MatmulF32Desc (m <= 2); ws: the zero-filled uint8
    workspace tensor (reused across calls)."""
    _need(ws, torch.uint8, "ws")
    arr = (Q8MatmulF32Desc * max(1, len(descs)))(*descs)
    _check("q8_0_matmul_f32_step", _lib.q8_0_matmul_f32_step(
        arr, len(descs), _ptr(ws), ws.numel(), _stream(ws if stream_of is None else stream_of)))


def q8_0_matmul_blocksums(w, x, n, k, m):
    _need(w, torch.uint8, "w")
    _need(x, torch.uint8, "x")
    _one_device(w, x)
    _fit(w, n * (k // QK) * BLOCK_BYTES, "w")
    _fit(x, m * (k // QK) * BLOCK_BYTES, "x")
    y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    s = torch.empty((m, n, k // QK), dtype=torch.int32, device=w.device)
    _check("q8_0_matmul_blocksums", _lib.q8_0_matmul_blocksums(
        _ptr(w), _ptr(x), _ptr(y), _ptr(s), n, k, m, _stream(w)))
    return y, s


def _ids_shape(ids):
    if ids.dim() != 2:
        raise ValueError(f"ids: expected [n_tok][n_used], got shape {tuple(ids.shape)}")
    return int(ids.shape[0]), int(ids.shape[1])


def _check_up_gate(w, x, ids, h, n_tok, n_used, n_embd, n_ff, n_expert, r8=False):
    """Extents of one expert-FFN up_gate layer (native rows, or R8 with r8=True)."""
    _one_device(w, x, ids, h)
    if tuple(ids.shape) != (n_tok, n_used):
        raise ValueError(f"ids: shape {tuple(ids.shape)}, expected {(n_tok, n_used)}")
    rows = n_expert * 2 * n_ff
    _fit(w, _r8_bytes_py(rows, n_embd) if r8 else rows * (n_embd // QK) * BLOCK_BYTES,
         "w_up_gate_r8" if r8 else "w_up_gate")
    _fit(x, n_tok * n_embd * 4, "x")
    _fit(h, n_tok * n_used * n_ff * 4, "h")


def _check_down(w, h, ids, cw, out, n_tok, n_used, n_ff, n_embd, n_expert, r8=False):
    """Extents of one expert-FFN down + combine layer."""
    _one_device(w, h, ids, cw, out)
    if tuple(ids.shape) != (n_tok, n_used):
        raise ValueError(f"ids: shape {tuple(ids.shape)}, expected {(n_tok, n_used)}")
    rows = n_expert * n_embd
    _fit(w, _r8_bytes_py(rows, n_ff) if r8 else rows * (n_ff // QK) * BLOCK_BYTES,
         "w_down_r8" if r8 else "w_down")
    _fit(h, n_tok * n_used * n_ff * 4, "h")
    _fit(cw, n_tok * n_used * 4, "cw")
    _fit(out, n_tok * n_embd * 4, "out")


def moe_workspace_bytes(n_tok, n_embd, n_ff, n_expert, n_used):
    return int(_lib.moe_workspace_bytes(n_tok, n_embd, n_ff, n_expert, n_used))


def moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, device):
    nbytes = moe_workspace_bytes(n_tok, n_embd, n_ff, n_expert, n_used)
    if nbytes == 0:
        raise Q8Error("moe_workspace_bytes", -4)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def moe_up_gate_swiglu(w_up_gate, x, ids, n_embd, n_ff, n_expert, ws, h=None):
    """h[t][u][j] = silu(gate) * up from fp32 token rows x [n_tok][n_embd]
    (quantized inside); returns h fp32 [n_tok][n_used][n_ff]."""
    _need(w_up_gate, torch.uint8, "w_up_gate")
    _need(x, torch.float32, "x")
    _need(ids, torch.int32, "ids")
    _need(ws, torch.uint8, "ws")
    n_tok, n_used = _ids_shape(ids)
    if h is None:
        h = torch.empty((n_tok, n_used, n_ff), dtype=torch.float32, device=ids.device)
    _need(h, torch.float32, "h")
    _check_up_gate(w_up_gate, x, ids, h, n_tok, n_used, n_embd, n_ff, n_expert)
    _one_device(ids, ws)
    _check("moe_up_gate_swiglu", _lib.moe_up_gate_swiglu(
        _ptr(w_up_gate), _ptr(x), _ptr(ids), _ptr(h), n_tok, n_embd, n_ff, n_expert, n_used,
        _ptr(ws), ws.numel(), _stream(ids)))
    return h


def moe_down_combine(w_down, h, ids, cw, n_ff, n_embd, n_expert, ws, out=None):
    """out[t] = sum_u cw[t][u] * down_e(q(h[t][u])); returns fp32 [n_tok][n_embd]."""
    _need(w_down, torch.uint8, "w_down")
    _need(h, torch.float32, "h")
    _need(ids, torch.int32, "ids")
    _need(cw, torch.float32, "cw")
    _need(ws, torch.uint8, "ws")
    n_tok, n_used = _ids_shape(ids)
    if out is None:
        out = torch.empty((n_tok, n_embd), dtype=torch.float32, device=ids.device)
    _need(out, torch.float32, "out")
    _check_down(w_down, h, ids, cw, out, n_tok, n_used, n_ff, n_embd, n_expert)
    _one_device(ids, ws)
    _check("moe_down_combine", _lib.moe_down_combine(
        _ptr(w_down), _ptr(h), _ptr(ids), _ptr(cw), _ptr(out), n_tok, n_ff, n_embd, n_expert,
        n_used, _ptr(ws), ws.numel(), _stream(ids)))
    return out


def moe_up_gate_swiglu_batched(layers, n_embd, n_ff, n_expert):
    """Grouped up_gate over independent layers of one shape.  layers: list of
    dicts with w_up_gate, x, ids, h (written), ws; returns the list of h."""
    if not layers:
        return []
    for d in layers:
        _need(d["w_up_gate"], torch.uint8, "w_up_gate")
        _need(d["x"], torch.float32, "x")
        _need(d["ids"], torch.int32, "ids")
        _need(d["h"], torch.float32, "h")
        _need(d["ws"], torch.uint8, "ws")
    n_tok, n_used = _ids_shape(layers[0]["ids"])
    for d in layers:
        _check_up_gate(d["w_up_gate"], d["x"], d["ids"], d["h"], n_tok, n_used, n_embd, n_ff,
                       n_expert)
        _one_device(layers[0]["ids"], d["ids"], d["ws"])
    arr = (MoeUpGateDesc * len(layers))(*[
        MoeUpGateDesc(_ptr(d["w_up_gate"]), _ptr(d["x"]), _ptr(d["ids"]), _ptr(d["h"]),
                      _ptr(d["ws"]), d["ws"].numel()) for d in layers])
    _check("moe_up_gate_swiglu_batched", _lib.moe_up_gate_swiglu_batched(
        arr, len(layers), n_tok, n_embd, n_ff, n_expert, n_used, _stream(layers[0]["ids"])))
    return [d["h"] for d in layers]


def moe_down_combine_batched(layers, n_ff, n_embd, n_expert):
    """Grouped down projection + combine over independent layers of one shape.
    layers: list of dicts with w_down, h, ids, cw, out (written), ws."""
    if not layers:
        return []
    for d in layers:
        _need(d["w_down"], torch.uint8, "w_down")
        _need(d["h"], torch.float32, "h")
        _need(d["ids"], torch.int32, "ids")
        _need(d["cw"], torch.float32, "cw")
        _need(d["out"], torch.float32, "out")
        _need(d["ws"], torch.uint8, "ws")
    n_tok, n_used = _ids_shape(layers[0]["ids"])
    for d in layers:
        _check_down(d["w_down"], d["h"], d["ids"], d["cw"], d["out"], n_tok, n_used, n_ff, n_embd,
                    n_expert)
        _one_device(layers[0]["ids"], d["ids"], d["ws"])
    arr = (MoeDownDesc * len(layers))(*[
        MoeDownDesc(_ptr(d["w_down"]), _ptr(d["h"]), _ptr(d["ids"]), _ptr(d["cw"]), _ptr(d["out"]),
                    _ptr(d["ws"]), d["ws"].numel()) for d in layers])
    _check("moe_down_combine_batched", _lib.moe_down_combine_batched(
        arr, len(layers), n_tok, n_ff, n_embd, n_expert, n_used, _stream(layers[0]["ids"])))
    return [d["out"] for d in layers]


def q8v_moe_up_gate(w_up_gate, x, ids, n_embd, n_ff, n_expert, ws, sums=True, route=True):
    """moe_up_gate_swiglu plus its validation outputs: returns (h, sums, counts,
    offsets, pairs) -- sums int32 [n_tok*n_used][2*n_ff][n_embd/32] and the
    expert-major grouping the kernels served (None where not asked for)."""
    _need(w_up_gate, torch.uint8, "w_up_gate")
    _need(x, torch.float32, "x")
    _need(ids, torch.int32, "ids")
    _need(ws, torch.uint8, "ws")
    n_tok, n_used = _ids_shape(ids)
    dev = ids.device
    h = torch.full((n_tok, n_used, n_ff), float("nan"), dtype=torch.float32, device=dev)
    _check_up_gate(w_up_gate, x, ids, h, n_tok, n_used, n_embd, n_ff, n_expert)
    _one_device(ids, ws)
    slots = n_tok * n_used
    s = (torch.full((slots, 2 * n_ff, n_embd // QK), -(1 << 31), dtype=torch.int32, device=dev)
         if sums else None)
    c = torch.full((n_expert,), -1, dtype=torch.int32, device=dev) if route else None
    o = torch.full((n_expert + 1,), -1, dtype=torch.int32, device=dev) if route else None
    p = torch.full((max(slots, 1),), -1, dtype=torch.int32, device=dev) if route else None
    _check("q8v_moe_up_gate", _lib.q8v_moe_up_gate(
        _ptr(w_up_gate), _ptr(x), _ptr(ids), _ptr(h), _ptr(s), _ptr(c), _ptr(o), _ptr(p), n_tok,
        n_embd, n_ff, n_expert, n_used, _ptr(ws), ws.numel(), _stream(ids)))
    return h, s, c, o, (p[:slots] if p is not None else None)


def q8v_moe_hq(w_down, h, ids, cw, n_ff, n_embd, n_expert, ws, sums=True):
    """moe_down_combine plus its validation outputs: returns (out, hq, sums) --
    hq uint8 [n_tok*n_used][n_ff/32*34] (the Q8_0 bytes of h the down products
    used), sums int32 [n_tok*n_used][n_embd][n_ff/32] (None if not asked)."""
    _need(w_down, torch.uint8, "w_down")
    _need(h, torch.float32, "h")
    _need(ids, torch.int32, "ids")
    _need(cw, torch.float32, "cw")
    _need(ws, torch.uint8, "ws")
    n_tok, n_used = _ids_shape(ids)
    dev = ids.device
    out = torch.full((n_tok, n_embd), float("nan"), dtype=torch.float32, device=dev)
    _check_down(w_down, h, ids, cw, out, n_tok, n_used, n_ff, n_embd, n_expert)
    _one_device(ids, ws)
    slots = n_tok * n_used
    hq = torch.zeros((slots, n_ff // QK * BLOCK_BYTES), dtype=torch.uint8, device=dev)
    s = (torch.full((slots, n_embd, n_ff // QK), -(1 << 31), dtype=torch.int32, device=dev)
         if sums else None)
    _check("q8v_moe_hq", _lib.q8v_moe_hq(
        _ptr(w_down), _ptr(h), _ptr(ids), _ptr(cw), _ptr(out), _ptr(hq), _ptr(s), n_tok, n_ff,
        n_embd, n_expert, n_used, _ptr(ws), ws.numel(), _stream(ids)))
    return out, hq, s


def q8v_moe_r8_ffn(layer, n_embd, n_ff, n_expert, route=False):
    """moe_r8_ffn_batched for one layer (a dict as for moe_r8_ffn_batched) plus
    the validation outputs: returns (ug_sums, dn_sums, hq, counts, offsets,
    pairs); the routing only with route=True (grouped path only)."""
    arr, n_tok, n_used = _r8_ffn_descs([layer], n_embd, n_ff, n_expert, True)
    dev = layer["ids"].device
    slots = n_tok * n_used
    ug = torch.full((slots, 2 * n_ff, n_embd // QK), -(1 << 31), dtype=torch.int32, device=dev)
    dn = torch.full((slots, n_embd, n_ff // QK), -(1 << 31), dtype=torch.int32, device=dev)
    hq = torch.zeros((slots, n_ff // QK * BLOCK_BYTES), dtype=torch.uint8, device=dev)
    c = torch.full((n_expert,), -1, dtype=torch.int32, device=dev) if route else None
    o = torch.full((n_expert + 1,), -1, dtype=torch.int32, device=dev) if route else None
    p = torch.full((max(slots, 1),), -1, dtype=torch.int32, device=dev) if route else None
    _check("q8v_moe_r8_ffn", _lib.q8v_moe_r8_ffn(
        arr, n_tok, n_embd, n_ff, n_expert, n_used, _ptr(ug), _ptr(dn), _ptr(hq), _ptr(c), _ptr(o),
        _ptr(p), _stream(layer["ids"])))
    return ug, dn, hq, c, o, (p[:slots] if p is not None else None)


def moe_route(ids, n_expert, ws):
    _need(ids, torch.int32, "ids")
    _need(ws, torch.uint8, "ws")
    _one_device(ids, ws)
    n_tok, n_used = _ids_shape(ids)
    dev = ids.device
    counts = torch.empty(n_expert, dtype=torch.int32, device=dev)
    offsets = torch.empty(n_expert + 1, dtype=torch.int32, device=dev)
    pairs = torch.empty(max(n_tok * n_used, 1), dtype=torch.int32, device=dev)
    _check("moe_route", _lib.moe_route(_ptr(ids), _ptr(counts), _ptr(offsets), _ptr(pairs),
                                       n_tok, n_expert, n_used, _ptr(ws), ws.numel(),
                                       _stream(ids)))
    return counts, offsets, pairs[: n_tok * n_used]


def q8_read_probe(buf, sink):
    """Stream-read the bytes of `buf` (a GPU tensor); sink: int32 GPU tensor."""
    _need(sink, torch.int32, "sink")
    _fit(buf, 0, "buf")
    _one_device(buf, sink)
    _check("q8_read_probe", _lib.q8_read_probe(_ptr(buf), buf.numel() * buf.element_size(),
                                               _ptr(sink), sink.numel(), _stream(buf)))


def moe_r8_workspace(n_tok, n_embd, n_ff, n_expert, n_used, device):
    nbytes = _lib.moe_r8_workspace_bytes(n_tok, n_embd, n_ff, n_expert, n_used)
    if nbytes == 0:
        raise Q8Error("moe_r8_workspace_bytes", -4)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _r8_ffn_descs(layers, n_embd, n_ff, n_expert, with_ws):
    for d in layers:
        _need(d["w_up_gate_r8"], torch.uint8, "w_up_gate_r8")
        _need(d["w_down_r8"], torch.uint8, "w_down_r8")
        _need(d["x"], torch.float32, "x")
        _need(d["ids"], torch.int32, "ids")
        _need(d["cw"], torch.float32, "cw")
        _need(d["h"], torch.float32, "h")
        _need(d["out"], torch.float32, "out")
        if with_ws:
            _need(d["ws"], torch.uint8, "ws")
    n_tok, n_used = _ids_shape(layers[0]["ids"])
    for d in layers:
        _check_up_gate(d["w_up_gate_r8"], d["x"], d["ids"], d["h"], n_tok, n_used, n_embd, n_ff,
                       n_expert, r8=True)
        _check_down(d["w_down_r8"], d["h"], d["ids"], d["cw"], d["out"], n_tok, n_used, n_ff,
                    n_embd, n_expert, r8=True)
        _one_device(layers[0]["ids"], d["ids"], d["ws"] if with_ws else None)
    arr = (MoeR8FfnDesc * len(layers))(*[
        MoeR8FfnDesc(_ptr(d["w_up_gate_r8"]), _ptr(d["w_down_r8"]), _ptr(d["x"]), _ptr(d["ids"]),
                     _ptr(d["cw"]), _ptr(d["h"]), _ptr(d["out"]),
                     _ptr(d["ws"]) if with_ws else None, d["ws"].numel() if with_ws else 0)
        for d in layers])
    return arr, n_tok, n_used


def moe_r8_ffn_batched(layers, n_embd, n_ff, n_expert):
    """The expert FFN over R8 expert weights for independent layers of one
    shape (decode kernels up to 16 tokens, the grouped matrix-core path above).
    layers: list of dicts with w_up_gate_r8, w_down_r8, x, ids, cw, h
    (written), out (written), ws."""
    if not layers:
        return
    arr, n_tok, n_used = _r8_ffn_descs(layers, n_embd, n_ff, n_expert, True)
    _check("moe_r8_ffn_batched", _lib.moe_r8_ffn_batched(
        arr, len(layers), n_tok, n_embd, n_ff, n_expert, n_used, _stream(layers[0]["ids"])))


def moe_r8_ffn_batched_noalloc(layers, n_embd, n_ff, n_expert):
    """moe_r8_ffn_batched without a caller workspace (the library's own
    per-device array; decode shapes, up to 16 tokens).  layers: dicts as for
    moe_r8_ffn_batched; a "ws" entry, if present, is ignored."""
    if not layers:
        return
    arr, n_tok, n_used = _r8_ffn_descs(layers, n_embd, n_ff, n_expert, False)
    _check("moe_r8_ffn_batched_noalloc", _lib.moe_r8_ffn_batched_noalloc(
        arr, len(layers), n_tok, n_embd, n_ff, n_expert, n_used, _stream(layers[0]["ids"])))


def moe_r8_fused_workspace(n_embd, n_ff, n_expert, n_used, device):
    """A workspace for moe_r8_ffn_fused (zeroed: its counters must start at
    zero; every call leaves them zero)."""
    nbytes = _lib.moe_r8_fused_workspace_bytes(n_embd, n_ff, n_expert, n_used)
    if nbytes == 0:
        raise Q8Error("moe_r8_fused_workspace_bytes", -4)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def moe_r8_ffn_fused(layer, n_embd, n_ff, n_expert):
    """One token through one layer of the expert FFN over R8 weights in one
    launch.  layer: a dict as for moe_r8_ffn_batched (one token) whose ws comes
    from moe_r8_fused_workspace."""
    arr, n_tok, n_used = _r8_ffn_descs([layer], n_embd, n_ff, n_expert, True)
    if n_tok != 1:
        raise Q8Error("moe_r8_ffn_fused", -4)
    _check("moe_r8_ffn_fused", _lib.moe_r8_ffn_fused(arr, n_embd, n_ff, n_expert, n_used,
                                                     _stream(layer["ids"])))


def moe_error_word(ws):
    """The int32 error word at the start of a MoE workspace (1 = an id was out of range)."""
    return int(ws[:4].view(torch.int32).item())


# Raw access for tests of the argument checks (no tensors needed).
raw = _lib
