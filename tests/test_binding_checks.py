"""The Python binding checks every tensor against the sizes its shape
arguments imply (and that all tensors of a call share one device) before it
calls the library, since the C ABI takes bare pointers and cannot see an
undersized buffer.  These run without a GPU: the tensors are stand-ins that
report a GPU device, a size and a fake address, and every call here must stop
at the binding's check (a ValueError naming the operand), before any pointer
reaches the library."""
import pytest
import torch

import moe_expert_ffn_q8_amd as q

QK, BB = 32, 34


class FakeGpu:
    """Duck-typed GPU tensor: only what the binding's checks read."""
    _next = 1 << 30

    def __init__(self, shape, dtype, device=0):
        self.shape = torch.Size(shape if isinstance(shape, tuple) else (shape,))
        self.dtype = dtype
        self.device = torch.device("cuda", device)
        self.is_cuda = True
        self._ptr = FakeGpu._next
        FakeGpu._next += 1 << 28

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self._ptr

    def dim(self):
        return len(self.shape)

    def stride(self, i=None):
        st, acc = [], 1
        for s in reversed(self.shape):
            st.append(acc)
            acc *= s
        st = tuple(reversed(st))
        return st if i is None else st[i]


def u8(n, dev=0):
    return FakeGpu(n, torch.uint8, dev)


def f32(shape, dev=0):
    return FakeGpu(shape, torch.float32, dev)


def i32(shape, dev=0):
    return FakeGpu(shape, torch.int32, dev)


def rejects(fn, *args, match=None, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_dense_products_reject_undersized_operands():
    n, k, m = 64, 256, 4
    nb = k // QK
    w, x, y = u8(n * nb * BB), u8(nb * BB), f32(n)
    rejects(q.q8_0_matvec, u8(n * nb * BB - 1), x, n, k, y, match="w")
    rejects(q.q8_0_matvec, w, u8(nb * BB - 2), n, k, y, match="x")
    rejects(q.q8_0_matvec, w, x, n, k, f32(n - 1), match="y")
    rejects(q.q8_0_matvec, w, x, n, k, f32(n, dev=1), match="several devices")
    xm = u8(m * nb * BB)
    rejects(q.q8_0_matmul, w, u8((m - 1) * nb * BB), n, k, m, f32((m, n)), match="x")
    rejects(q.q8_0_matmul, w, xm, n, k, m, f32((m, n - 1)), match="y")
    rejects(q.q8_0_matmul_blocksums, w, u8(nb * BB), n, k, m, match="x")
    rejects(q.q8_0_quantize_rows, f32((3, k)), u8(3 * nb * BB - 1), match="y")


def test_r8_products_reject_undersized_operands():
    n, k = 20, 512
    nb = k // QK
    rb = q.q8_0_r8_bytes(n, k)
    assert rb == 3 * 272 * nb        # 20 rows pad to 3 groups of 8
    rejects(q.q8_0_repack_r8, u8(n * nb * BB), n, k, u8(rb - 16), match="out")
    rejects(q.q8_0_matvec_r8, u8(rb - 1), u8(nb * BB), n, k, f32(n), match="w_r8")
    # descriptors: a batch of 3 matrices needs 2 strides plus one matrix
    wr = u8(2 * rb + rb)
    rejects(q.make_r8_desc, u8(2 * rb + rb - 1), u8(3 * nb * BB), f32(3 * n), n, k, batch=3,
            w_batch_stride=rb, x_batch_stride=nb, y_batch_stride=n, match="w_r8")
    rejects(q.make_r8_desc, wr, u8(3 * nb * BB), f32(3 * n - 1), n, k, batch=3,
            w_batch_stride=rb, x_batch_stride=nb, y_batch_stride=n, match="y")
    rejects(q.make_r8_f32_desc, wr, f32(3 * k - 4), f32(3 * n), n, k, batch=3,
            w_batch_stride=rb, x_batch_stride=k, y_batch_stride=n, match="x")
    # an element offset past what the tensor holds
    rejects(q.make_r8_f32_desc, wr, (f32(4 * k), 2 * k), f32(3 * n), n, k, batch=3,
            w_batch_stride=rb, x_batch_stride=k, y_batch_stride=n, match="x")
    rejects(q.make_r8_mm_desc, wr, u8(8 * nb * BB - 1), f32(8 * n), n, k, m=8, match="x")


def test_descriptor_builders_reject_undersized_operands():
    n, k, m, batch = 48, 256, 2, 5
    nb = k // QK
    w = u8(batch * n * nb * BB)
    rejects(q.make_desc, u8(batch * n * nb * BB - BB), u8(batch * m * nb * BB),
            f32(batch * m * n), n, k, m=m, batch=batch, w_batch_stride=n * nb,
            x_batch_stride=m * nb, y_batch_stride=m * n, match="w")
    rejects(q.make_f32_desc, w, f32(batch * m * k - 1), f32(batch * m * n), n, k, m=m,
            batch=batch, w_batch_stride=n * nb, x_batch_stride=m * k, y_batch_stride=m * n,
            match="x")
    rejects(q.make_up_gate_desc, u8(2 * n * nb * BB - 1), u8(nb * BB), f32(n), n, k, match="w")
    rejects(q.make_kq_desc, u8(n * (k // 256) * 176 - 1), u8(nb * 36), f32(n), n, k, t=5,
            match="w")
    # a row stride that reaches past the activation tensor
    rejects(q.make_desc, w, u8(2 * nb * BB), f32(2 * n), n, k, m=2, x_row_stride=2 * nb,
            match="x")


def test_moe_calls_reject_undersized_operands():
    T, U, E, n_embd, n_ff = 3, 4, 8, 256, 128
    nbe, nbf = n_embd // QK, n_ff // QK
    wug = u8(E * 2 * n_ff * nbe * BB)
    wd = u8(E * n_embd * nbf * BB)
    x, ids, h = f32((T, n_embd)), i32((T, U)), f32((T, U, n_ff))
    cw, out, ws = f32((T, U)), f32((T, n_embd)), u8(1 << 20)
    rejects(q.moe_up_gate_swiglu, u8(E * 2 * n_ff * nbe * BB - 1), x, ids, n_embd, n_ff, E, ws,
            h, match="w_up_gate")
    rejects(q.moe_up_gate_swiglu, wug, f32((T - 1, n_embd)), ids, n_embd, n_ff, E, ws, h,
            match="x")
    rejects(q.moe_up_gate_swiglu, wug, x, ids, n_embd, n_ff, E, ws, f32((T, U, n_ff - 1)),
            match="h")
    rejects(q.moe_up_gate_swiglu, wug, x, ids, n_embd, n_ff, E, u8(1 << 20, dev=1), h,
            match="several devices")
    rejects(q.moe_down_combine, u8(E * n_embd * nbf * BB - 1), h, ids, cw, n_ff, n_embd, E, ws,
            out, match="w_down")
    rejects(q.moe_down_combine, wd, h, ids, f32((T, U - 1)), n_ff, n_embd, E, ws, out, match="cw")
    rejects(q.moe_down_combine, wd, h, ids, cw, n_ff, n_embd, E, ws, f32((T, n_embd - 1)),
            match="out")
    layer = dict(w_up_gate=wug, x=x, ids=ids, h=h, ws=ws)
    bad = dict(layer, ids=i32((T, U - 1)))       # a second layer with another routing shape
    rejects(q.moe_up_gate_swiglu_batched, [layer, bad], n_embd, n_ff, E, match="ids")
    dl = dict(w_down=wd, h=h, ids=ids, cw=cw, out=out, ws=ws)
    rejects(q.moe_down_combine_batched, [dl, dict(dl, w_down=u8(10))], n_ff, n_embd, E,
            match="w_down")


def test_moe_r8_rejects_undersized_operands():
    T, U, E, n_embd, n_ff = 2, 4, 8, 256, 128
    ug_rows, dn_rows = E * 2 * n_ff, E * n_embd
    layer = dict(w_up_gate_r8=u8(q.q8_0_r8_bytes(ug_rows, n_embd)),
                 w_down_r8=u8(q.q8_0_r8_bytes(dn_rows, n_ff)), x=f32((T, n_embd)),
                 ids=i32((T, U)), cw=f32((T, U)), h=f32((T, U, n_ff)), out=f32((T, n_embd)),
                 ws=u8(1 << 20))
    rejects(q.moe_r8_ffn_batched, [dict(layer, w_down_r8=u8(q.q8_0_r8_bytes(dn_rows, n_ff) - 16))],
            n_embd, n_ff, E, match="w_down_r8")
    rejects(q.moe_r8_ffn_batched, [layer, dict(layer, h=f32((T, U, n_ff - 32)))], n_embd, n_ff, E,
            match="h")
