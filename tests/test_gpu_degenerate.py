"""Degenerate sizes through the entry points the hot path uses: no rows, no
outputs, no tokens and empty batch entries return success and touch no output
byte (nor the workspace), and empty entries inside a batched launch leave the
other entries' results within the parity bound."""
import pytest

from gpu_cases import acts_q8, assert_rows_close, to_gpu, weights_q8

pytestmark = pytest.mark.gpu

SENT = 12345.0


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def sentinel(n):
    import torch
    return torch.full((n,), SENT, dtype=torch.float32, device="cuda")


def untouched(t):
    return bool((t == SENT).all().item())


def test_quantize_no_rows(q):
    import torch
    x = torch.randn(4, 768, device="cuda")
    y = torch.full((4 * 24 * 34,), 0xAB, dtype=torch.uint8, device="cuda")
    q.q8_0_quantize_rows(x[:0], y=y, k=768)
    torch.cuda.synchronize()
    assert bool((y == 0xAB).all().item())


def test_products_without_outputs(q, orc):
    import torch
    n, k, m = 64, 768, 20
    w = to_gpu(weights_q8(orc, n, k, "deg", n, k))
    x = to_gpu(acts_q8(orc, m, k, "deg-x", m, k))
    y = sentinel(n * m)
    q.q8_0_matvec(w, x, 0, k, y=y)
    q.q8_0_matmul(w, x, n, k, 0, y=y)
    q.q8_0_matmul(w, x, 0, k, m, y=y)
    wr = q.q8_0_repack_r8(w, n, k)
    q.q8_0_matvec_r8(wr, x, 0, k, y=y)
    torch.cuda.synchronize()
    assert untouched(y)


def test_batched_launch_with_empty_entries(q, orc):
    """Native rows (the streaming and small-batch engines) and R8 rows: empty
    descriptors (n = 0, m = 0, batch = 0) around real ones leave their own
    outputs untouched and the real entries within the parity bound."""
    import torch
    k = 768
    for n, m in [(300, 1), (129, 8)]:
        w = weights_q8(orc, n, k, "deg-b", n, k)
        x = acts_q8(orc, m, k, "deg-bx", n, m)
        wg, xg = to_gpu(w), to_gpu(x)
        y = sentinel(n * m + 64)
        spare = sentinel(64)
        descs = [q.make_desc(wg, xg, spare, 0, k, m=m),
                 q.make_desc(wg, xg, y, n, k, m=m),
                 q.make_desc(wg, xg, spare, n, k, m=0),
                 q.make_desc(wg, xg, spare, n, k, m=m, batch=0)]
        q.q8_0_matmul_batched(descs, y)
        torch.cuda.synchronize()
        assert_rows_close(y[:n * m].view(m, n).cpu().numpy(), orc.matmul(w, x, n, k, m))
        assert untouched(y[n * m:]) and untouched(spare), (n, m)
    n = 300
    w = weights_q8(orc, n, k, "deg-r", n, k)
    x = acts_q8(orc, 1, k, "deg-rx", n)
    wr = q.q8_0_repack_r8(to_gpu(w), n, k)
    xg = to_gpu(x)
    y = sentinel(n + 64)
    spare = sentinel(64)
    descs = [q.make_r8_desc(wr, xg, spare, 0, k),
             q.make_r8_desc(wr, xg, y, n, k),
             q.make_r8_desc(wr, xg, spare, n, k, batch=0)]
    q.q8_0_matvec_r8_batched(descs, y)
    torch.cuda.synchronize()
    assert_rows_close(y[:n].view(1, n).cpu().numpy(), orc.matmul(w, x, n, k, 1))
    assert untouched(y[n:]) and untouched(spare)


@pytest.mark.parametrize("r8", [False, True])
def test_expert_ffn_without_tokens(q, orc, r8):
    import torch
    n_embd, n_ff, E, U = 256, 64, 8, 2
    ids = torch.empty((0, U), dtype=torch.int32, device="cuda")
    x = torch.randn(1, n_embd, device="cuda")
    cw = torch.empty((0, U), dtype=torch.float32, device="cuda")
    h = sentinel(U * n_ff)
    out = sentinel(n_embd)
    wug = to_gpu(weights_q8(orc, E * 2 * n_ff, n_embd, "deg-ug"))
    wd = to_gpu(weights_q8(orc, E * n_embd, n_ff, "deg-dn"))
    if r8:
        ws = q.moe_r8_workspace(1, n_embd, n_ff, E, U, "cuda")
        ws.fill_(0x5A)
        q.moe_r8_ffn_batched([dict(w_up_gate_r8=q.q8_0_repack_r8(wug, E * 2 * n_ff, n_embd),
                                   w_down_r8=q.q8_0_repack_r8(wd, E * n_embd, n_ff), x=x[:0],
                                   ids=ids, cw=cw, h=h, out=out, ws=ws)], n_embd, n_ff, E)
    else:
        ws = q.moe_workspace(1, n_embd, n_ff, E, U, "cuda")
        ws.fill_(0x5A)
        q.moe_up_gate_swiglu(wug, x[:0], ids, n_embd, n_ff, E, ws, h=h)
        q.moe_down_combine(wd, h, ids, cw, n_ff, n_embd, E, ws, out=out)
    torch.cuda.synchronize()
    assert untouched(h) and untouched(out)
    assert bool((ws == 0x5A).all().item())
