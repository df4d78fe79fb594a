"""The C ABI: the library loads, exports every function include/q8moe.h
declares, and rejects bad arguments on the host with the documented status
before touching the GPU (these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8moe.h")

Q8_OK, Q8_E_NULL, Q8_E_SHAPE, Q8_E_ALIGN, Q8_E_UNSUPPORTED, Q8_E_WORKSPACE = 0, -1, -2, -3, -4, -5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    import moe_expert_ffn_q8_amd as q
    return q.raw


def test_exports_everything_declared(lib):
    names = declared_functions()
    assert len(names) >= 11, names
    for n in names:
        assert hasattr(lib, n), n
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr)
    import moe_expert_ffn_q8_amd as q
    assert set(names) == set(q.EXPORTS)


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6, -99):
        assert lib.q8_status_str(s)


A = 1 << 20          # a fake, suitably aligned address: never dereferenced
WS = 1 << 24         # a fake 256-byte-aligned workspace address (never dereferenced)


def test_quantize_rows_checks(lib):
    f = lib.q8_0_quantize_rows
    assert f(A, 64, A, 1, 33, None) == Q8_E_SHAPE          # k % 32
    assert f(A, 64, A, 1, 0, None) == Q8_E_SHAPE
    assert f(A, 16, A, 1, 32, None) == Q8_E_SHAPE          # stride < k
    assert f(A, 64, A, -1, 64, None) == Q8_E_SHAPE
    assert f(A, 64, A, 0, 64, None) == Q8_OK               # no rows: no-op
    assert f(None, 64, A, 1, 64, None) == Q8_E_NULL
    assert f(A + 4, 64, A, 1, 64, None) == Q8_E_ALIGN      # fp32 input needs 16 B
    assert f(A, 66, A, 2, 64, None) == Q8_E_ALIGN          # stride multiple of 4
    assert f(A, 64, A + 1, 1, 64, None) == Q8_E_ALIGN


def test_matvec_matmul_checks(lib):
    assert lib.q8_0_matvec(A, A, A, 10, 40, None) == Q8_E_SHAPE
    assert lib.q8_0_matvec(A, A, A, -1, 64, None) == Q8_E_SHAPE
    assert lib.q8_0_matvec(A, A, A, 0, 64, None) == Q8_OK
    assert lib.q8_0_matvec(None, A, A, 10, 64, None) == Q8_E_NULL
    assert lib.q8_0_matvec(A, None, A, 10, 64, None) == Q8_E_NULL
    assert lib.q8_0_matvec(A, A, None, 10, 64, None) == Q8_E_NULL
    assert lib.q8_0_matvec(A + 1, A, A, 10, 64, None) == Q8_E_ALIGN
    assert lib.q8_0_matvec(A, A, A + 2, 10, 64, None) == Q8_E_ALIGN
    assert lib.q8_0_matmul(A, A, A, 10, 64, -3, None) == Q8_E_SHAPE
    assert lib.q8_0_matmul(A, A, A, 10, 64, 0, None) == Q8_OK
    assert lib.q8_0_matmul_blocksums(A, A, A, None, 10, 64, 1, None) == Q8_E_NULL
    # any m: above 16 rows the sums come from the matrix-core kernel
    assert lib.q8_0_matmul_blocksums(A, A, A, A + 2, 10, 64, 17, None) == Q8_E_ALIGN


def test_batched_checks(lib):
    import moe_expert_ffn_q8_amd as q
    D = q.Q8MatmulDesc
    def call(*ds):
        arr = (D * len(ds))(*ds)
        return lib.q8_0_matmul_batched(arr, len(ds), None)
    ok = dict(w=A, x=A, y=A, n=8, k=64, m=1, batch=1, w_batch_stride=0, x_row_stride=2,
              x_batch_stride=0, y_row_stride=8, y_batch_stride=0)
    assert lib.q8_0_matmul_batched(None, 0, None) == Q8_OK
    assert lib.q8_0_matmul_batched(None, 1, None) == Q8_E_NULL
    assert lib.q8_0_matmul_batched(None, -1, None) == Q8_E_SHAPE
    assert call(D(**{**ok, "k": 48})) == Q8_E_SHAPE
    assert call(D(**{**ok, "m": 17})) == Q8_E_UNSUPPORTED
    assert call(D(**{**ok, "m": 2, "x_row_stride": 1})) == Q8_E_SHAPE
    assert call(D(**{**ok, "batch": 2, "w_batch_stride": 3})) == Q8_E_SHAPE
    assert call(D(**{**ok, "batch": 2, "w_batch_stride": 16, "y_batch_stride": 0})) == Q8_E_SHAPE
    assert call(D(**{**ok, "w": None})) == Q8_E_NULL
    assert call(D(**{**ok, "y": A + 2})) == Q8_E_ALIGN
    assert call(D(**{**ok, "n": 0})) == Q8_OK
    arr = (D * 33)(*([D(**{**ok, "n": 0})] * 33))
    assert lib.q8_0_matmul_batched(arr, 33, None) == Q8_E_UNSUPPORTED


def test_moe_checks(lib):
    import moe_expert_ffn_q8_amd as q
    ws_bytes = q.moe_workspace_bytes(4, 256, 64, 8, 2)
    assert ws_bytes >= 256
    assert q.moe_workspace_bytes(4, 250, 64, 8, 2) == 0
    assert q.moe_workspace_bytes(4, 256, 64, 8, 17) == 0
    ug = lib.moe_up_gate_swiglu
    args = [A, A, A, A, 4, 256, 64, 8, 2, A, ws_bytes, None]
    def with_(i, v):
        a = list(args)
        a[i] = v
        return ug(*a)
    assert with_(5, 250) == Q8_E_SHAPE              # n_embd % 32
    assert with_(6, 48) == Q8_E_SHAPE               # n_ff % 32
    assert with_(8, 0) == Q8_E_SHAPE                # n_used
    assert with_(8, 17) == Q8_E_UNSUPPORTED
    assert with_(4, 1025) == Q8_E_UNSUPPORTED       # too many slots
    assert with_(7, 0) == Q8_E_SHAPE
    assert with_(9, None) == Q8_E_WORKSPACE
    assert with_(10, ws_bytes - 1) == Q8_E_WORKSPACE
    assert with_(9, A + 16) == Q8_E_ALIGN
    assert with_(0, None) == Q8_E_NULL
    assert with_(3, A + 2) == Q8_E_ALIGN
    dc = lib.moe_down_combine
    dargs = [A, A, A, A, A, 4, 64, 256, 8, 2, A, ws_bytes, None]
    assert dc(*dargs[:4], None, *dargs[5:]) == Q8_E_NULL
    a = list(dargs); a[1] = A + 4
    assert dc(*a) == Q8_E_ALIGN                     # h needs 16 B
    a = list(dargs); a[11] = 8
    assert dc(*a) == Q8_E_WORKSPACE
    assert lib.moe_route(A, A, A, A, 4, 8, 2, None, 256, None) == Q8_E_WORKSPACE
    assert lib.moe_route(A, None, A, A, 4, 8, 2, A, 256, None) == Q8_E_NULL


def test_moe_prefill_checks(lib):
    """More than 16 tokens: the prefill path's workspace (routing tables, the
    quantized token rows, then the quantized h rows and the per-slot outputs)
    and its shape limits."""
    import moe_expert_ffn_q8_amd as q

    def a256(v):
        return (v + 255) // 256 * 256

    n_tok, n_embd, n_ff, n_expert, n_used = 512, 2048, 768, 128, 8
    slots = n_tok * n_used
    max_tiles = slots // 32 + n_expert + 1
    data = 256 + a256((n_expert + 1) * 4) + a256(slots * 4) + a256(max_tiles * 16)
    # quantized rows in the tile layout (32 code bytes per block, then fp32
    # scales): the token rows, then the slot rows of h, then the slot outputs
    up = a256(n_tok * (n_embd // 32) * 32) + a256(n_tok * (n_embd // 32) * 4)
    down = a256(slots * (n_ff // 32) * 32) + a256(slots * (n_ff // 32) * 4) \
        + a256(slots * n_embd * 4)
    ws = q.moe_workspace_bytes(n_tok, n_embd, n_ff, n_expert, n_used)
    assert ws == data + up + down
    assert ws > q.moe_workspace_bytes(16, n_embd, n_ff, n_expert, n_used)
    ug = lib.moe_up_gate_swiglu
    assert ug(A, A, A, A, n_tok, n_embd, n_ff, n_expert, n_used, A, ws - 1, None) == Q8_E_WORKSPACE
    assert ug(A, A, A, A, 8193, n_embd, n_ff, n_expert, n_used, A, 1 << 40, None) == Q8_E_UNSUPPORTED
    # 1600 slots with n_ff/32 = 3 (not a multiple of 4): no prefill path, too many slots
    assert ug(A, A, A, A, 200, 256, 96, 8, 8, A, 1 << 40, None) == Q8_E_UNSUPPORTED
    assert q.moe_workspace_bytes(200, 256, 96, 8, 8) == 0
    # 20 tokens x 8 with n_ff/32 = 3: 160 slots stay on the streaming kernels
    assert q.moe_workspace_bytes(20, 256, 96, 8, 8) == 256 + a256(160 * 256 * 4)


def test_moe_batched_checks(lib):
    """Grouped MoE calls: every descriptor is checked before anything is
    enqueued (no valid launch here: there is no GPU)."""
    import ctypes
    import moe_expert_ffn_q8_amd as q
    ws_bytes = q.moe_workspace_bytes(4, 256, 64, 8, 2)
    good = q.MoeUpGateDesc(A, A, A, A, A, ws_bytes)
    ug = lib.moe_up_gate_swiglu_batched

    def call(descs, n=None, shape=(4, 256, 64, 8, 2)):
        arr = (q.MoeUpGateDesc * max(len(descs), 1))(*descs)
        return ug(arr, len(descs) if n is None else n, *shape, None)

    assert call([good], n=-1) == Q8_E_SHAPE
    assert call([], n=0) == Q8_OK                      # nothing to do
    assert ug(None, 2, 4, 256, 64, 8, 2, None) == Q8_E_NULL
    assert call([good], shape=(4, 250, 64, 8, 2)) == Q8_E_SHAPE
    assert call([good], shape=(4, 256, 64, 8, 17)) == Q8_E_UNSUPPORTED
    bad_ws = q.MoeUpGateDesc(A, A, A, A, A, ws_bytes - 1)
    assert call([good, bad_ws]) == Q8_E_WORKSPACE     # the second descriptor fails
    bad_align = q.MoeUpGateDesc(A, A + 4, A, A, A, ws_bytes)
    assert call([good, good, bad_align]) == Q8_E_ALIGN
    bad_null = q.MoeUpGateDesc(A, A, None, A, A, ws_bytes)
    assert call([bad_null]) == Q8_E_NULL

    dn = lib.moe_down_combine_batched
    dgood = q.MoeDownDesc(A, A, A, A, A, A, ws_bytes)
    darr = (q.MoeDownDesc * 2)(dgood, q.MoeDownDesc(A, A, A, A, None, A, ws_bytes))
    assert dn(darr, 2, 4, 64, 256, 8, 2, None) == Q8_E_NULL
    darr = (q.MoeDownDesc * 2)(dgood, q.MoeDownDesc(A, A + 4, A, A, A, A, ws_bytes))
    assert dn(darr, 2, 4, 64, 256, 8, 2, None) == Q8_E_ALIGN
    assert dn(darr, -3, 4, 64, 256, 8, 2, None) == Q8_E_SHAPE
    assert dn(None, 0, 4, 64, 256, 8, 2, None) == Q8_OK
    assert ctypes.sizeof(q.MoeUpGateDesc) == 48 and ctypes.sizeof(q.MoeDownDesc) == 56


def test_matmul_f32_checks(lib):
    """fp32-activation products: host checks (no launch without a GPU)."""
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_0_matmul_f32_batched

    def call(**kw):
        base = dict(w=A, x=A, y=A, n=64, k=768, m=1, batch=1, w_batch_stride=0, x_row_stride=768,
                    x_batch_stride=0, y_row_stride=64, y_batch_stride=0)
        base.update(kw)
        d = q.Q8MatmulF32Desc(*[base[k] for k, _ in q.Q8MatmulF32Desc._fields_])
        arr = (q.Q8MatmulF32Desc * 1)(d)
        return f(arr, 1, None)

    assert call(k=100) == Q8_E_SHAPE                 # k % 32
    assert call(k=96) == Q8_E_UNSUPPORTED            # k/32 not a multiple of 8: no fused engine
    assert call(k=16384) == Q8_E_UNSUPPORTED         # longer rows than the engines take
    assert call(m=17) == Q8_E_UNSUPPORTED
    assert call(x=A + 4) == Q8_E_ALIGN               # fp32 rows need 16 B
    assert call(w=A + 2) == Q8_E_ALIGN
    assert call(m=2, x_row_stride=770) == Q8_E_ALIGN
    assert call(m=2, x_row_stride=512) == Q8_E_SHAPE
    assert call(batch=2, w_batch_stride=64 * 24, y_batch_stride=0) == Q8_E_SHAPE
    assert call(y=None) == Q8_E_NULL
    assert f(None, 1, None) == Q8_E_NULL
    assert f(None, 0, None) == Q8_OK
    assert f(None, -1, None) == Q8_E_SHAPE


def test_matmul_f32_step_checks(lib):
    """One-launch step: host checks and the workspace size (no launch without
    a GPU)."""
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_0_matmul_f32_step
    g = lib.q8_0_matmul_f32_step_ws_bytes

    def desc(**kw):
        base = dict(w=A, x=A, y=A, n=64, k=768, m=1, batch=1, w_batch_stride=0, x_row_stride=768,
                    x_batch_stride=0, y_row_stride=64, y_batch_stride=0)
        base.update(kw)
        return q.Q8MatmulF32Desc(*[base[k] for k, _ in q.Q8MatmulF32Desc._fields_])

    def arr(*ds):
        return (q.Q8MatmulF32Desc * len(ds))(*ds)

    def call(ws=WS, ws_bytes=1 << 20, **kw):
        return f(arr(desc(**kw)), 1, ws, ws_bytes, None)

    # workspace: 256 B header, each descriptor's quantized rows (256-aligned),
    # 256 B of counter per batch entry, an int32 flag per tile (256-aligned);
    # a tile is 64 / (k/128) rows
    assert g(arr(desc()), 1) == 256 + 1024 + 256 + 256         # 24 blocks = 816 B; 7 tiles
    two = arr(desc(batch=40, w_batch_stride=64 * 24, x_batch_stride=768, y_batch_stride=64),
              desc(n=10, k=2048, m=2, x_row_stride=2048, y_row_stride=10))
    img = (40 * 24 * 34 + 255) // 256 * 256 + (2 * 64 * 34 + 255) // 256 * 256
    tiles = 40 * 7 + 3                                          # R = 10 and R = 4
    assert g(two, 2) == 256 + img + 41 * 256 + (4 * tiles + 255) // 256 * 256
    assert g(arr(desc(m=3, x_row_stride=768, y_row_stride=64)), 1) == Q8_E_UNSUPPORTED
    assert g(None, 0) == 256
    assert call(m=3, x_row_stride=768) == Q8_E_UNSUPPORTED     # m <= 2 only
    assert call(k=96) == Q8_E_UNSUPPORTED
    assert call(k=100) == Q8_E_SHAPE
    assert call(x=A + 4) == Q8_E_ALIGN
    assert call(y=None) == Q8_E_NULL
    assert call(ws=None) == Q8_E_WORKSPACE
    assert call(ws_bytes=1791) == Q8_E_WORKSPACE
    assert call(ws=WS + 16) == Q8_E_ALIGN
    assert call(n=0, ws=None) == Q8_OK                          # nothing to do
    assert f(None, 0, None, 0, None) == Q8_OK
    assert f(None, 1, WS, 1 << 20, None) == Q8_E_NULL
    assert f(None, -1, WS, 1 << 20, None) == Q8_E_SHAPE


def test_up_gate_checks(lib):
    """Dense up_gate: host checks (no launch without a GPU)."""
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_0_up_gate_swiglu_batched

    def call(**kw):
        base = dict(w=A, x=A, h=A, n_ff=64, n_embd=768, m=1, batch=1, w_batch_stride=0,
                    x_row_stride=24, x_batch_stride=0, h_row_stride=64, h_batch_stride=0)
        base.update(kw)
        d = q.Q8UpGateDesc(*[base[k] for k, _ in q.Q8UpGateDesc._fields_])
        return f((q.Q8UpGateDesc * 1)(d), 1, None)

    assert call(n_embd=100) == Q8_E_SHAPE
    assert call(n_ff=-1) == Q8_E_SHAPE
    assert call(m=3) == Q8_E_UNSUPPORTED
    assert call(n_embd=96) == Q8_E_UNSUPPORTED          # k/32 not a multiple of 8
    assert call(n_embd=16384) == Q8_E_UNSUPPORTED
    assert call(w=A + 2) == Q8_E_ALIGN
    assert call(x=A + 1) == Q8_E_ALIGN
    assert call(m=2, x_row_stride=23) == Q8_E_SHAPE
    assert call(m=2, h_row_stride=63) == Q8_E_SHAPE
    assert call(batch=2, w_batch_stride=64 * 24) == Q8_E_SHAPE        # < 2 n_ff rows
    assert call(batch=2, w_batch_stride=2 * 64 * 24, h_batch_stride=0) == Q8_E_SHAPE
    assert call(batch=2, w_batch_stride=2 * 64 * 24 + 1, h_batch_stride=64) == Q8_E_ALIGN
    assert call(h=None) == Q8_E_NULL
    assert call(n_ff=0, h=None) == Q8_OK
    assert f(None, 0, None) == Q8_OK
    assert f(None, 1, None) == Q8_E_NULL
    many = (q.Q8UpGateDesc * 33)()
    assert f(many, 33, None) == Q8_E_UNSUPPORTED


def test_read_probe_checks(lib):
    f = lib.q8_read_probe
    assert f(A, -16, A, 4096, None) == Q8_E_SHAPE
    assert f(A, 0, None, 0, None) == Q8_OK
    assert f(None, 1024, A, 4096, None) == Q8_E_NULL
    assert f(A + 8, 1024, A, 4096, None) == Q8_E_ALIGN
    assert f(A, 1000, A, 4096, None) == Q8_E_ALIGN


def test_r8_checks(lib):
    assert lib.q8_0_r8_bytes(9, 64) == 2 * 8 * 2 * 34
    assert lib.q8_0_r8_bytes(16, 64) == 16 * 2 * 34
    assert lib.q8_0_r8_bytes(0, 64) == 0
    assert lib.q8_0_r8_bytes(4, 48) == Q8_E_SHAPE
    assert lib.q8_0_r8_bytes(-1, 64) == Q8_E_SHAPE
    rp = lib.q8_0_repack_r8
    assert rp(A, A, 10, 40, None) == Q8_E_SHAPE
    assert rp(A, A, -1, 64, None) == Q8_E_SHAPE
    assert rp(A, A, 0, 64, None) == Q8_OK
    assert rp(None, A, 10, 64, None) == Q8_E_NULL
    assert rp(A, None, 10, 64, None) == Q8_E_NULL
    assert rp(A + 1, A, 10, 64, None) == Q8_E_ALIGN
    assert rp(A, A + 8, 10, 64, None) == Q8_E_ALIGN        # the R8 buffer needs 16 B
    mv = lib.q8_0_matvec_r8
    assert mv(A, A, A, 10, 40, None) == Q8_E_SHAPE
    assert mv(A, A, A, -1, 64, None) == Q8_E_SHAPE
    assert mv(A, A, A, 0, 64, None) == Q8_OK
    assert mv(None, A, A, 10, 64, None) == Q8_E_NULL
    assert mv(A, None, A, 10, 64, None) == Q8_E_NULL
    assert mv(A, A, None, 10, 64, None) == Q8_E_NULL
    assert mv(A + 8, A, A, 10, 64, None) == Q8_E_ALIGN
    assert mv(A, A + 1, A, 10, 64, None) == Q8_E_ALIGN
    assert mv(A, A, A + 2, 10, 64, None) == Q8_E_ALIGN
    assert mv(A, A, A, 10, 32768 + 32, None) == Q8_E_UNSUPPORTED


def test_r8_batched_checks(lib):
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_0_matvec_r8_batched

    def call(*descs, n_desc=None):
        arr = (q.Q8R8Desc * max(1, len(descs)))(*descs)
        return f(arr, len(descs) if n_desc is None else n_desc, None)

    ok = q.Q8R8Desc(A, A, A, 64, 768, 2, 64 * 24 * 34, 24, 64)
    assert f(None, 0, None) == Q8_OK
    assert f(None, 1, None) == Q8_E_NULL
    assert call(ok, n_desc=-1) == Q8_E_SHAPE
    assert call(*([ok] * 33)) == Q8_E_UNSUPPORTED
    assert call(q.Q8R8Desc(A, A, A, 64, 40, 1, 0, 0, 0)) == Q8_E_SHAPE      # k % 32
    assert call(q.Q8R8Desc(A, A, A, -1, 64, 1, 0, 0, 0)) == Q8_E_SHAPE
    assert call(q.Q8R8Desc(None, None, None, 0, 64, 1, 0, 0, 0)) == Q8_OK   # empty
    assert call(q.Q8R8Desc(None, A, A, 8, 64, 1, 0, 0, 0)) == Q8_E_NULL
    # batch > 1: strides must separate the matrices and outputs
    assert call(q.Q8R8Desc(A, A, A, 64, 768, 2, 64 * 24 * 34 - 16, 24, 64)) == Q8_E_SHAPE
    assert call(q.Q8R8Desc(A, A, A, 64, 768, 2, 64 * 24 * 34, 24, 63)) == Q8_E_SHAPE
    assert call(q.Q8R8Desc(A, A, A, 64, 768, 2, 64 * 24 * 34 + 8, 24, 64)) == Q8_E_ALIGN
    assert call(q.Q8R8Desc(A + 8, A, A, 64, 768, 1, 0, 0, 0)) == Q8_E_ALIGN
    assert call(q.Q8R8Desc(A, A, A, 64, 32768 + 32, 1, 0, 0, 0)) == Q8_E_UNSUPPORTED


def test_r8_f32_batched_checks(lib):
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_0_matvec_r8_f32_batched

    def call(*descs):
        arr = (q.Q8R8F32Desc * max(1, len(descs)))(*descs)
        return f(arr, len(descs), None)

    assert f(None, 0, None) == Q8_OK
    assert call(q.Q8R8F32Desc(A, A + 8, A, 64, 768, 1, 0, 0, 0)) == Q8_E_ALIGN    # fp32 x: 16 B
    assert call(q.Q8R8F32Desc(A, A, A, 64, 768, 2, 64 * 24 * 34, 770, 64)) == Q8_E_ALIGN
    assert call(q.Q8R8F32Desc(A, A, A, 64, 768, 2, 64 * 24 * 34, -4, 64)) == Q8_E_SHAPE
    assert call(q.Q8R8F32Desc(A, A, A, 64, 40, 1, 0, 0, 0)) == Q8_E_SHAPE
    assert call(q.Q8R8F32Desc(A, A, A, 64, 32768 + 32, 1, 0, 0, 0)) == Q8_E_UNSUPPORTED


def test_kq_checks(lib):
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_1_quantize_rows
    assert f(A, 64, A, 1, 33, None) == Q8_E_SHAPE
    assert f(A, 16, A, 1, 32, None) == Q8_E_SHAPE
    assert f(A, 64, A, 0, 64, None) == Q8_OK
    assert f(None, 64, A, 1, 64, None) == Q8_E_NULL
    assert f(A + 4, 64, A, 1, 64, None) == Q8_E_ALIGN
    assert f(A, 64, A + 2, 1, 64, None) == Q8_E_ALIGN
    for mv in (lib.q4_k_matvec, lib.q5_k_matvec):
        assert mv(A, A, A, 10, 128, None) == Q8_E_SHAPE           # k % 256
        assert mv(A, A, A, -1, 256, None) == Q8_E_SHAPE
        assert mv(A, A, A, 0, 256, None) == Q8_OK
        assert mv(None, A, A, 10, 256, None) == Q8_E_NULL
        assert mv(A + 8, A, A, 10, 256, None) == Q8_E_ALIGN
        assert mv(A, A + 2, A, 10, 256, None) == Q8_E_ALIGN
        assert mv(A, A, A + 2, 10, 256, None) == Q8_E_ALIGN
        assert mv(A, A, A, 10, 8192 + 256, None) == Q8_E_UNSUPPORTED
    g = lib.kq_matvec_batched

    def call(t, *descs):
        arr = (q.KqMatvecDesc * max(1, len(descs)))(*descs)
        return g(t, arr, len(descs), None)

    assert call(6, q.KqMatvecDesc(A, A, A, 8, 256, 1, 0, 0, 0)) == Q8_E_UNSUPPORTED
    assert call(4, q.KqMatvecDesc(A, A, A, 8, 256, 2, 7, 8, 8)) == Q8_E_SHAPE     # w stride
    assert call(4, q.KqMatvecDesc(A, A, A, 8, 256, 2, 8, 8, 7)) == Q8_E_SHAPE     # y stride


def test_r8_mm_checks(lib):
    import moe_expert_ffn_q8_amd as q
    f = lib.q8_0_matmul_r8_batched

    def call(*descs):
        arr = (q.Q8R8MmDesc * max(1, len(descs)))(*descs)
        return f(arr, len(descs), None)

    D = q.Q8R8MmDesc
    assert f(None, 0, None) == Q8_OK
    assert call(D(A, A, A, 64, 768, 17, 1, 0, 24, 0, 64, 0)) == Q8_E_UNSUPPORTED     # m > 16
    assert call(D(A, A, A, 64, 768, 8, 1, 0, 23, 0, 64, 0)) == Q8_E_SHAPE            # x row stride
    assert call(D(A, A, A, 64, 768, 8, 1, 0, 24, 0, 63, 0)) == Q8_E_SHAPE            # y row stride
    assert call(D(A, A, A, 64, 768, 8, 2, 16, 24, 192, 64, 512)) == Q8_E_SHAPE        # w stride
    assert call(D(A, A, A, 64, 768, 8, 2, 64 * 24 * 34 + 8, 24, 192, 64, 512)) == Q8_E_ALIGN
    assert call(D(A + 8, A, A, 64, 768, 8, 1, 0, 24, 0, 64, 0)) == Q8_E_ALIGN
    assert call(D(A, A + 1, A, 64, 768, 8, 1, 0, 24, 0, 64, 0)) == Q8_E_ALIGN
    assert call(D(A, A, A, 64, 40, 8, 1, 0, 24, 0, 64, 0)) == Q8_E_SHAPE              # k % 32
    assert call(D(None, A, A, 64, 768, 8, 1, 0, 24, 0, 64, 0)) == Q8_E_NULL
    assert call(D(A, A, A, 64, 768, 0, 1, 0, 24, 0, 64, 0)) == Q8_OK                 # no rows


def test_moe_r8_checks(lib):
    import moe_expert_ffn_q8_amd as q
    f = lib.moe_r8_ffn_batched
    need = lib.moe_r8_workspace_bytes(1, 2048, 768, 128, 8)
    assert need == 256 + (8 * 24 * 34 + 255) // 256 * 256
    assert lib.moe_r8_workspace_bytes(1, 2048, 768 + 16, 128, 8) == 0      # n_ff % 32
    assert lib.moe_r8_workspace_bytes(1, 2048, 4096, 128, 8) == 0           # n_ff > 2048

    def call(d, n_tok=1, n_embd=2048, n_ff=768, n_expert=128, n_used=8):
        arr = (q.MoeR8FfnDesc * 1)(d)
        return f(arr, 1, n_tok, n_embd, n_ff, n_expert, n_used, None)

    D = q.MoeR8FfnDesc
    ok = D(A, A, A, A, A, A, A, WS, need)
    assert call(ok, n_ff=4096) == Q8_E_UNSUPPORTED
    assert call(ok, n_used=17) == Q8_E_UNSUPPORTED
    assert call(ok, n_embd=2047) == Q8_E_SHAPE
    assert call(D(A, A, A, A, A, A, A, WS, need - 1)) == Q8_E_WORKSPACE
    assert call(D(A, A, A, A, A, A, A, None, need)) == Q8_E_WORKSPACE
    assert call(D(A, A, A, A, A, A, A, WS + 16, need)) == Q8_E_ALIGN
    assert call(D(None, A, A, A, A, A, A, WS, need)) == Q8_E_NULL
    assert call(D(A, A + 8, A, A, A, A, A, WS, need)) == Q8_E_ALIGN
    assert call(D(A, A, A + 4, A, A, A, A, WS, need)) == Q8_E_ALIGN
    assert call(ok, n_tok=0) == Q8_OK
    # more than 16 tokens: the grouped path and its workspace (that of the
    # native-row prefill path); h rows need 16-byte alignment there
    pre = lib.moe_r8_workspace_bytes(512, 2048, 768, 128, 8)
    assert pre == lib.moe_workspace_bytes(512, 2048, 768, 128, 8)
    # 2..16 tokens: the fp32 slot rows of the combine after the error word
    assert lib.moe_r8_workspace_bytes(16, 2048, 768, 128, 8) == 256 + 128 * 2048 * 4
    big = D(A, A, A, A, A, A, A, WS, pre)
    assert call(D(A, A, A, A, A, A + 4, A, WS, pre), n_tok=512) == Q8_E_ALIGN     # h
    assert call(D(A, A, A, A, A, A, A, WS, pre - 1), n_tok=512) == Q8_E_WORKSPACE
    assert call(big, n_tok=8193) == Q8_E_UNSUPPORTED                            # too many tokens


def test_moe_r8_fused_checks(lib):
    """moe_r8_ffn_fused (one token, one layer, one launch): its workspace size
    (256 bytes of counters, then the block terms [n_used][n_ff/32][n_embd] in
    fp32), the shape limits (n_embd % 256) and every argument check before any
    launch."""
    import moe_expert_ffn_q8_amd as q
    f = lib.moe_r8_ffn_fused
    need = lib.moe_r8_fused_workspace_bytes(2048, 768, 128, 8)
    assert need == 256 + 8 * 24 * 2048 * 4
    assert lib.moe_r8_fused_workspace_bytes(2048 - 32, 768, 128, 8) == 0      # n_embd % 256
    assert lib.moe_r8_fused_workspace_bytes(2048, 4096, 128, 8) == 0          # n_ff > 2048
    assert lib.moe_r8_fused_workspace_bytes(2048, 768, 128, 17) == 0          # n_used > 16
    assert lib.moe_r8_fused_workspace_bytes(2048, 768, 0, 8) == 0

    def call(d, n_embd=2048, n_ff=768, n_expert=128, n_used=8):
        return f(ctypes.byref(d) if d is not None else None, n_embd, n_ff, n_expert, n_used, None)

    D = q.MoeR8FfnDesc
    ok = D(A, A, A, A, A, A, A, WS, need)
    assert call(None) == Q8_E_NULL
    assert call(ok, n_embd=2047) == Q8_E_SHAPE
    assert call(ok, n_ff=40) == Q8_E_SHAPE
    assert call(ok, n_used=0) == Q8_E_SHAPE
    assert call(ok, n_embd=2048 - 32) == Q8_E_UNSUPPORTED
    assert call(ok, n_used=17) == Q8_E_UNSUPPORTED
    assert call(D(A, A, A, A, A, A, A, WS, need - 1)) == Q8_E_WORKSPACE
    assert call(D(A, A, A, A, A, A, A, None, need)) == Q8_E_WORKSPACE
    assert call(D(A, A, A, A, A, A, A, WS + 16, need)) == Q8_E_ALIGN
    assert call(D(A, A, None, A, A, A, A, WS, need)) == Q8_E_NULL
    assert call(D(A, A + 8, A, A, A, A, A, WS, need)) == Q8_E_ALIGN
    assert call(D(A, A, A + 4, A, A, A, A, WS, need)) == Q8_E_ALIGN
    assert call(D(A, A, A, A, A, A + 2, A, WS, need)) == Q8_E_ALIGN


def test_moe_r8_noalloc_checks(lib):
    """The no-alloc variant: the shape and descriptor checks of
    moe_r8_ffn_batched (its ws fields ignored), decode shapes only, and a
    clear status when the layers' workspaces exceed the library's 48 MiB
    array -- all before any HIP call."""
    import moe_expert_ffn_q8_amd as q
    f = lib.moe_r8_ffn_batched_noalloc
    D = q.MoeR8FfnDesc

    def call(ds, n_tok=1, n_embd=2048, n_ff=768, n_expert=128, n_used=8):
        arr = (D * max(1, len(ds)))(*ds)
        return f(arr, len(ds), n_tok, n_embd, n_ff, n_expert, n_used, None)

    ok = D(A, A, A, A, A, A, A, None, 0)            # no workspace: ignored
    assert call([ok], n_ff=4096) == Q8_E_UNSUPPORTED
    assert call([ok], n_embd=2047) == Q8_E_SHAPE
    assert call([D(None, A, A, A, A, A, A, None, 0)]) == Q8_E_NULL
    assert call([D(A, A, A + 4, A, A, A, A, None, 0)]) == Q8_E_ALIGN
    assert call([ok], n_tok=0) == Q8_OK
    assert call([]) == Q8_OK
    assert call([ok], n_tok=17) == Q8_E_UNSUPPORTED   # the prefill path: not in this variant
    # 16 tokens x 16 slots, n_embd 2048: error word + fp32 slot rows
    # (2,097,152 bytes) per layer -> 23 layers fit
    per = (lib.moe_r8_workspace_bytes(16, 2048, 2048, 64, 16) + 255) // 256 * 256
    assert per == 256 + 256 * 2048 * 4
    fit = (48 << 20) // per
    assert fit == 23
    assert call([ok] * (fit + 1), 16, 2048, 2048, 64, 16) == Q8_E_WORKSPACE
    assert call([ok] * 3 + [D(A, A, A, A, A, None, A, None, 0)], 16, 2048, 2048, 64, 16) == Q8_E_NULL
