"""The library allocates nothing and never synchronizes, so its launches can
be captured in a HIP graph.  A captured decode step (quantize + batched
products) and a captured MoE layer are replayed several times, with eager work
and synchronizations in between; every replay must equal the eager result bit
for bit."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_graph_replay_decode_step():
    import torch
    import moe_expert_ffn_q8_amd as q
    dev = "cuda"
    shapes = [(768, 768, 6), (2048, 768, 2), (768, 2048, 3)]
    ws, descs = [], []
    k_total = sum(k * b for _, k, b in shapes)
    xf = torch.from_numpy(synth.normal_f32((1, k_total), 1.0, "graph", "x")).to(dev)
    xq = q.q8_empty(1, k_total, dev)
    n_out = sum(n * b for n, _, b in shapes)
    y = torch.empty((1, n_out), dtype=torch.float32, device=dev)
    xoff = yoff = 0
    for i, (n, k, b) in enumerate(shapes):
        w = q.q8_0_quantize_rows(torch.from_numpy(
            synth.normal_f32((n * b, k), 0.02, "graph", "w", i)).to(dev))
        ws.append(w)
        descs.append(q.make_desc(w, (xq, xoff), (y, yoff), n, k, batch=b, w_batch_stride=n * k // 32,
                                 x_batch_stride=k // 32, y_batch_stride=n))
        xoff += b * k // 32
        yoff += b * n

    def step():
        q.q8_0_quantize_rows(xf, y=xq)
        q.q8_0_matmul_batched(descs, y)

    step()
    torch.cuda.synchronize()
    ref = y.clone()
    g = _capture(step)
    for rep in range(4):
        y.fill_(float("nan"))
        xq.zero_()
        torch.cuda.synchronize()
        junk = torch.randn(1000, device=dev).sum()       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), rep
        del junk


def test_graph_replay_moe_layer():
    import torch
    import moe_expert_ffn_q8_amd as q
    import oracle
    dev = "cuda"
    T, E, U, n_embd, n_ff = 4, 16, 4, 512, 256
    wug = torch.from_numpy(oracle.quantize_rows(
        synth.normal_f32((E * 2 * n_ff, n_embd), 0.02, "graph", "ug"))).to(dev)
    wd = torch.from_numpy(oracle.quantize_rows(
        synth.normal_f32((E * n_embd, n_ff), 0.02, "graph", "dn"))).to(dev)
    xf = torch.from_numpy(synth.normal_f32((T, n_embd), 1.0, "graph", "xt")).to(dev)
    ids = torch.from_numpy(synth.expert_ids(T, U, E, "graph", "ids")).to(dev)
    cw = torch.from_numpy(synth.combine_weights(T, U, "graph", "cw")).to(dev)
    ws = q.moe_workspace(T, n_embd, n_ff, E, U, dev)
    h = torch.empty((T, U, n_ff), dtype=torch.float32, device=dev)
    out = torch.empty((T, n_embd), dtype=torch.float32, device=dev)

    def layer():
        q.moe_up_gate_swiglu(wug, xf, ids, n_embd, n_ff, E, ws, h=h)
        q.moe_down_combine(wd, h, ids, cw, n_ff, n_embd, E, ws, out=out)

    layer()
    torch.cuda.synchronize()
    ref_h, ref_out = h.clone(), out.clone()
    g = _capture(layer)
    for rep in range(4):
        h.fill_(float("nan"))
        out.fill_(float("nan"))
        ws.fill_(0x55)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), ref_h.view(torch.int32)), rep
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), rep
        assert q.moe_error_word(ws) == 0
