"""CPU oracle for the Q8_0 decode path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  It wraps liboracle.so (q8_oracle.c, plain scalar C) with
numpy marshalling.  It shares no code with the HIP library.

Quantized data is passed as numpy uint8 arrays holding 34-byte Q8_0 blocks back
to back (scale as little-endian binary16, then 32 int8 codes).  Floating point
results of the contractions are fp64.

Parity status of each function (the pins live in tests/test_oracle_*.py):
  f32_to_f16, f16_to_f32 ....... pinned (exhaustive against numpy float16)
  quantize_rows ................ pinned (hand cases, rule invariants)
  block sums / matmul .......... pinned (int64 brute force, closed forms,
                                  dequantize-then-fp64 matmul)
  moe_up_gate_swiglu ........... pinned (split-path identity, dense special
                                  case, dequantized fp64 brute force)
  up_gate_swiglu (dense) ....... pinned (split form, dequantized fp64 brute
                                  force, exact small case)
  moe_route .................... pinned (invariants, brute force)
  moe_down_combine ............. pinned (one-hot / single-expert reductions,
                                  dequantized fp64 brute force)
  repack_r8, matvec_r8 ......... pinned (hand-listed byte positions of a small
                                  case, byte multiset, matvec identity with the
                                  native layout)
  quantize_rows_q8_1 ........... pinned (d and codes equal the pinned Q8_0
                                  quantizer's, hand-computed s values)
  kq_scale_min, kq_dequantize .. pinned (hand-packed 6-bit fields and hand-made
                                  Q4_K / Q5_K super-blocks with values listed
                                  by hand)
  kq_matvec .................... pinned (dequantize-then-fp64 numpy product,
                                  per-sub-block integer-sum identity, exact
                                  small cases)
"""
import ctypes
import os

import numpy as np

QK = 32
BLOCK_BYTES = 34

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "or_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "or_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "or_quantize_rows": (ctypes.c_int, [_f32p, _i64, _u8p, _i64, _i64]),
        "or_block_dot": (ctypes.c_int32, [_u8p, _u8p]),
        "or_matmul": (ctypes.c_int, [_u8p, _u8p, _f64p, _i64, _i64, _i64, _i64, _i64]),
        "or_matmul_select": (ctypes.c_int, [_u8p, _u8p, _i64, _i64, _i64, _i64p, _i64p,
                                            _i64, _f64p]),
        "or_matmul_blocksums": (ctypes.c_int, [_u8p, _u8p, _i32p, _i64, _i64, _i64]),
        "or_mul_mat_id": (ctypes.c_int, [_u8p, _i64, _i64, _i64, _u8p, _i32p, _f64p,
                                         _i64, _i64, _i64, _i64]),
        "or_fused_mul_silu": (None, [_f64p, _f64p, _f64p, _i64]),
        "or_f32_to_f16_array": (None, [_f32p, ctypes.POINTER(ctypes.c_uint16), _i64]),
        "or_f16_to_f32_array": (None, [ctypes.POINTER(ctypes.c_uint16), _f32p, _i64]),
        "or_moe_up_gate_swiglu": (ctypes.c_int, [_u8p, _u8p, _i32p, _f64p, _i64, _i64,
                                                 _i64, _i64, _i64]),
        "or_moe_route": (ctypes.c_int, [_i32p, _i64, _i64, _i64, _i32p, _i32p, _i32p]),
        "or_moe_down_combine": (ctypes.c_int, [_u8p, _f32p, _i32p, _f32p, _f64p, _u8p,
                                               _i64, _i64, _i64, _i64, _i64, _i64p, _i64,
                                               _u8p]),
        "or_r8_bytes": (ctypes.c_int64, [_i64, _i64]),
        "or_repack_r8": (ctypes.c_int, [_u8p, _u8p, _i64, _i64]),
        "or_matvec_r8": (ctypes.c_int, [_u8p, _u8p, _f64p, _i64, _i64]),
        "or_quantize_rows_q8_1": (ctypes.c_int, [_f32p, _i64, _u8p, _i64, _i64]),
        "or_kq_scale_min": (None, [_u8p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                   ctypes.POINTER(ctypes.c_int)]),
        "or_kq_dequantize_rows": (ctypes.c_int, [ctypes.c_int, _u8p, _f64p, _i64, _i64]),
        "or_kq_matvec": (ctypes.c_int, [ctypes.c_int, _u8p, _u8p, _f64p, _i64, _i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a, typ):
    return a.ctypes.data_as(typ)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: status {rc}")


def _blocks(a, nbytes_expected=None):
    a = np.ascontiguousarray(a, dtype=np.uint8)
    if nbytes_expected is not None and a.size != nbytes_expected:
        raise ValueError(f"expected {nbytes_expected} bytes of Q8_0 blocks, got {a.size}")
    return a


# --------------------------------------------------------------------------
# binary16 codec
# --------------------------------------------------------------------------

def f32_to_f16_bits(x):
    """Scalar fp32 -> binary16 bits (round to nearest even)."""
    return int(_load().or_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h):
    return float(_load().or_f16_to_f32(int(h)))


def f32_to_f16_bits_array(x):
    """Vector form of f32_to_f16_bits (same C routine, applied per element)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    h = np.empty(x.size, dtype=np.uint16)
    _load().or_f32_to_f16_array(_p(x, _f32p), h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                x.size)
    return h


def f16_bits_to_f32_array(h):
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    x = np.empty(h.size, dtype=np.float32)
    _load().or_f16_to_f32_array(h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                _p(x, _f32p), h.size)
    return x


# --------------------------------------------------------------------------
# Q8_0 quantization and contractions
# --------------------------------------------------------------------------

def quantize_rows(x, k=None):
    """x: fp32 [n_rows][k] (2-D) or [k] -> uint8 [n_rows][k/32*34]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    n_rows, kk = x.shape
    if k is not None and k != kk:
        raise ValueError("k mismatch")
    out = np.empty((n_rows, kk // QK * BLOCK_BYTES), dtype=np.uint8)
    _check(_load().or_quantize_rows(_p(x, _f32p), kk, _p(out, _u8p), n_rows, kk),
           "quantize_rows")
    return out


def block_dot(wb, xb):
    wb = _blocks(wb, BLOCK_BYTES)
    xb = _blocks(xb, BLOCK_BYTES)
    return int(_load().or_block_dot(_p(wb, _u8p), _p(xb, _u8p)))


def matmul(w, x, n, k, m, n_begin=0, n_end=None):
    """Y[m][n] (fp64) = X[m][k] . W[n][k]^T with Q8_0 operands."""
    nb = k // QK
    w = _blocks(w, n * nb * BLOCK_BYTES)
    x = _blocks(x, m * nb * BLOCK_BYTES)
    if n_end is None:
        n_end = n
    y = np.zeros((m, n), dtype=np.float64)
    _check(_load().or_matmul(_p(w, _u8p), _p(x, _u8p), _p(y, _f64p), n, k, m,
                             n_begin, n_end), "matmul")
    return y


def matvec(w, x, n, k):
    return matmul(w, x, n, k, 1)[0]


def matmul_select(w, x, n, k, m, sel_m, sel_n):
    nb = k // QK
    w = _blocks(w, n * nb * BLOCK_BYTES)
    x = _blocks(x, m * nb * BLOCK_BYTES)
    sel_m = np.ascontiguousarray(sel_m, dtype=np.int64)
    sel_n = np.ascontiguousarray(sel_n, dtype=np.int64)
    y = np.empty(sel_m.size, dtype=np.float64)
    _check(_load().or_matmul_select(_p(w, _u8p), _p(x, _u8p), n, k, m, _p(sel_m, _i64p),
                                    _p(sel_n, _i64p), sel_m.size, _p(y, _f64p)),
           "matmul_select")
    return y


def matmul_rows(w, x, n, k, m, rows):
    """Y[:, rows] for a list of weight rows (fp64 [m][len(rows)])."""
    rows = np.asarray(rows, dtype=np.int64)
    sel_m = np.repeat(np.arange(m, dtype=np.int64), rows.size)
    sel_n = np.tile(rows, m)
    return matmul_select(w, x, n, k, m, sel_m, sel_n).reshape(m, rows.size)


def matmul_blocksums(w, x, n, k, m):
    nb = k // QK
    w = _blocks(w, n * nb * BLOCK_BYTES)
    x = _blocks(x, m * nb * BLOCK_BYTES)
    s = np.empty((m, n, nb), dtype=np.int32)
    _check(_load().or_matmul_blocksums(_p(w, _u8p), _p(x, _u8p), _p(s, _i32p), n, k, m),
           "matmul_blocksums")
    return s


# --------------------------------------------------------------------------
# Mixture of experts
# --------------------------------------------------------------------------

def mul_mat_id(w, rows_per_expert, row_off, n_rows, x, ids, k, n_expert):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n_tok, n_used = ids.shape
    nb = k // QK
    w = _blocks(w, n_expert * rows_per_expert * nb * BLOCK_BYTES)
    x = _blocks(x, n_tok * nb * BLOCK_BYTES)
    out = np.empty((n_tok, n_used, n_rows), dtype=np.float64)
    _check(_load().or_mul_mat_id(_p(w, _u8p), rows_per_expert, row_off, n_rows,
                                 _p(x, _u8p), _p(ids, _i32p), _p(out, _f64p), n_tok, k,
                                 n_expert, n_used), "mul_mat_id")
    return out


def fused_mul_silu(g, u):
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    h = np.empty_like(g)
    _load().or_fused_mul_silu(_p(g, _f64p), _p(u, _f64p), _p(h, _f64p), g.size)
    return h


def moe_up_gate_swiglu(w_ug, x, ids, n_embd, n_ff, n_expert):
    """h[t][u][j] (fp64) for the combined up_gate tensor, gate rows first."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n_tok, n_used = ids.shape
    nb = n_embd // QK
    w_ug = _blocks(w_ug, n_expert * 2 * n_ff * nb * BLOCK_BYTES)
    x = _blocks(x, n_tok * nb * BLOCK_BYTES)
    h = np.empty((n_tok, n_used, n_ff), dtype=np.float64)
    _check(_load().or_moe_up_gate_swiglu(_p(w_ug, _u8p), _p(x, _u8p), _p(ids, _i32p),
                                         _p(h, _f64p), n_tok, n_embd, n_ff, n_expert,
                                         n_used), "moe_up_gate_swiglu")
    return h


def moe_up_gate_swiglu_split(w_ug, x, ids, n_embd, n_ff, n_expert):
    """The fallback form: two row views of the combined tensor, mul_mat_id on
    each, then silu(gate)*up."""
    g = mul_mat_id(w_ug, 2 * n_ff, 0, n_ff, x, ids, n_embd, n_expert)
    u = mul_mat_id(w_ug, 2 * n_ff, n_ff, n_ff, x, ids, n_embd, n_expert)
    return fused_mul_silu(g, u).reshape(g.shape)


def up_gate_swiglu(w_ug, x, n_embd, n_ff):
    """Dense FFN up_gate: h[t][j] (fp64) = silu(W[j] . x_t) * (W[n_ff + j] . x_t)
    for one combined weight [2*n_ff][n_embd] (gate rows first) and Q8_0 rows
    x [m][n_embd/32] -- the MoE form with a single expert that every token
    uses (FUSED_UP_GATE beside MOE_FUSED_UP_GATE on the Gemma-4-on-Xeon page,
    section on the broken op paths)."""
    nb = n_embd // QK
    x = _blocks(x)
    m = x.size // (nb * BLOCK_BYTES)
    ids = np.zeros((m, 1), dtype=np.int32)
    return moe_up_gate_swiglu(w_ug, x, ids, n_embd, n_ff, 1)[:, 0, :]


def moe_route(ids, n_expert):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n_tok, n_used = ids.shape
    counts = np.empty(n_expert, dtype=np.int32)
    offsets = np.empty(n_expert + 1, dtype=np.int32)
    pairs = np.empty(max(n_tok * n_used, 1), dtype=np.int32)
    _check(_load().or_moe_route(_p(ids, _i32p), n_tok, n_used, n_expert, _p(counts, _i32p),
                                _p(offsets, _i32p), _p(pairs, _i32p)), "moe_route")
    return counts, offsets, pairs[: n_tok * n_used]


def moe_down_combine(w_d, h, ids, cw, n_ff, n_embd, n_expert, sel=None, return_hq=False):
    """out[t][n] (fp64) = sum_u cw[t][u] * down_{ids[t][u]}(q(h[t][u]))[n].

    h must be fp32 [n_tok][n_used][n_ff]: it is quantized in fp32.
    sel: optional list of output columns; out is then [n_tok][len(sel)]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    cw = np.ascontiguousarray(cw, dtype=np.float32)
    h = np.ascontiguousarray(h, dtype=np.float32)
    n_tok, n_used = ids.shape
    if h.size != n_tok * n_used * n_ff:
        raise ValueError("h shape")
    nb = n_ff // QK
    w_d = _blocks(w_d, n_expert * n_embd * nb * BLOCK_BYTES)
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int64)
        n_out = sel.size
        sel_p = _p(sel, _i64p)
    else:
        n_out = n_embd
        sel_p = None
    out = np.empty((n_tok, n_out), dtype=np.float64)
    hq = np.empty((n_tok, n_used, nb * BLOCK_BYTES), dtype=np.uint8) if return_hq else None
    scratch = np.empty(max(n_used, 1) * nb * BLOCK_BYTES, dtype=np.uint8)
    _check(_load().or_moe_down_combine(_p(w_d, _u8p), _p(h, _f32p), _p(ids, _i32p),
                                       _p(cw, _f32p), _p(out, _f64p),
                                       _p(hq, _u8p) if hq is not None else None,
                                       n_tok, n_ff, n_embd, n_expert, n_used, sel_p,
                                       n_out if sel is not None else 0,
                                       _p(scratch, _u8p)), "moe_down_combine")
    return (out, hq) if return_hq else out


def moe_ffn(w_ug, w_d, x_f32, ids, cw, n_embd, n_ff, n_expert):
    """Whole expert FFN from fp32 token activations: quantize x, up_gate +
    SwiGLU (fp64), round h to fp32, down + combine.  Returns (out, h64)."""
    xq = quantize_rows(x_f32)
    h = moe_up_gate_swiglu(w_ug, xq, ids, n_embd, n_ff, n_expert)
    out = moe_down_combine(w_d, h.astype(np.float32), ids, cw, n_ff, n_embd, n_expert)
    return out, h


# --------------------------------------------------------------------------
# Row-interleaved weight layout (R8): groups of 8 rows, scales then codes,
# both ordered by (block, row); see q8_oracle.c
# --------------------------------------------------------------------------

def r8_bytes(n, k):
    v = int(_load().or_r8_bytes(n, k))
    if v < 0:
        raise ValueError(f"oracle r8_bytes: status {v}")
    return v


def repack_r8(w, n, k):
    """Native rows uint8 [n][k/32*34] -> uint8 [r8_bytes(n, k)]."""
    nb = k // QK
    w = _blocks(w, n * nb * BLOCK_BYTES)
    out = np.empty(r8_bytes(n, k), dtype=np.uint8)
    _check(_load().or_repack_r8(_p(w, _u8p), _p(out, _u8p), n, k), "repack_r8")
    return out


def matvec_r8(w_r8, x, n, k):
    """y[n] (fp64) for weights in the R8 layout and one Q8_0 activation row."""
    nb = k // QK
    w_r8 = _blocks(w_r8, r8_bytes(n, k))
    x = _blocks(x, nb * BLOCK_BYTES)
    y = np.empty(n, dtype=np.float64)
    _check(_load().or_matvec_r8(_p(w_r8, _u8p), _p(x, _u8p), _p(y, _f64p), n, k),
           "matvec_r8")
    return y


# --------------------------------------------------------------------------
# Q8_1 activations and the K-quant weights (Q4_K = type 4, Q5_K = type 5);
# layouts in q8_oracle.c
# --------------------------------------------------------------------------

Q8_1_BLOCK_BYTES = 36
KQ_BLOCK_BYTES = {4: 144, 5: 176}
QKK = 256


def quantize_rows_q8_1(x):
    """x: fp32 [n_rows][k] (2-D) or [k] -> uint8 [n_rows][k/32*36]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    n_rows, k = x.shape
    out = np.empty((n_rows, k // QK * Q8_1_BLOCK_BYTES), dtype=np.uint8)
    _check(_load().or_quantize_rows_q8_1(_p(x, _f32p), k, _p(out, _u8p), n_rows, k),
           "quantize_rows_q8_1")
    return out


def kq_scale_min(b12, j):
    b12 = np.ascontiguousarray(b12, dtype=np.uint8)
    sc, m = ctypes.c_int(), ctypes.c_int()
    _load().or_kq_scale_min(_p(b12, _u8p), j, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def _kq_bytes(t):
    if t not in KQ_BLOCK_BYTES:
        raise ValueError(f"unknown K-quant type {t}")
    return KQ_BLOCK_BYTES[t]


def kq_dequantize(t, w, n, k):
    """Super-blocks uint8 [n][k/256*bytes] -> fp64 [n][k]."""
    _kq_bytes(t)
    w = _blocks(w, n * (k // QKK) * KQ_BLOCK_BYTES[t])
    out = np.empty((n, k), dtype=np.float64)
    _check(_load().or_kq_dequantize_rows(t, _p(w, _u8p), _p(out, _f64p), n, k), "kq_dequantize")
    return out


def kq_matvec(t, w, x, n, k):
    """y[n] (fp64) for K-quant weights of type t and one Q8_1 activation row."""
    _kq_bytes(t)
    w = _blocks(w, n * (k // QKK) * KQ_BLOCK_BYTES[t])
    x = _blocks(x, k // QK * Q8_1_BLOCK_BYTES)
    y = np.empty(n, dtype=np.float64)
    _check(_load().or_kq_matvec(t, _p(w, _u8p), _p(x, _u8p), _p(y, _f64p), n, k), "kq_matvec")
    return y


# --------------------------------------------------------------------------
# helpers for reading blocks (used by tests to build independent checks)
# --------------------------------------------------------------------------

def split_blocks(q):
    """uint8 [..., nb*34] -> (scale bits uint16 [..., nb], codes int8 [..., nb, 32])."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    lead = q.shape[:-1]
    nb = q.shape[-1] // BLOCK_BYTES
    b = q.reshape(lead + (nb, BLOCK_BYTES))
    d = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
    codes = b[..., 2:].view(np.int8)
    return d, codes
