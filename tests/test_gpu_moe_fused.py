"""GPU parity of the one-launch expert FFN over R8 expert weights
(moe_r8_ffn_fused: one token, one layer): h bit for bit against
moe_r8_ffn_batched (the same up_gate arithmetic); out against the oracle's
down + combine fed the GPU's own h, and against moe_r8_ffn_batched, within
the parity bound (the same block terms summed in another order); repeated
calls on one workspace (its counters return to zero), bitwise repeatability,
HIP graph replays, out-of-range ids."""
import numpy as np
import pytest

import synth
from gpu_cases import assert_rows_close, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _layer(q, orc, n_embd, n_ff, n_expert, n_used, tag, ids=None):
    import torch
    w_ug = orc.quantize_rows(synth.normal_f32((n_expert * 2 * n_ff, n_embd), 0.02, tag, "ug"))
    w_d = orc.quantize_rows(synth.normal_f32((n_expert * n_embd, n_ff), 0.02, tag, "down"))
    xf = synth.normal_f32((1, n_embd), 1.0, tag, "x")
    if ids is None:
        ids = synth.expert_ids(1, n_used, n_expert, tag, "ids")
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    cw = synth.combine_weights(1, n_used, tag, "cw")
    d = dict(w_up_gate_r8=q.q8_0_repack_r8(to_gpu(w_ug), n_expert * 2 * n_ff, n_embd),
             w_down_r8=q.q8_0_repack_r8(to_gpu(w_d), n_expert * n_embd, n_ff),
             x=to_gpu(xf), ids=to_gpu(ids), cw=to_gpu(cw),
             h=torch.full((1, n_used, n_ff), float("nan"), device="cuda"),
             out=torch.full((1, n_embd), float("nan"), device="cuda"),
             ws=q.moe_r8_fused_workspace(n_embd, n_ff, n_expert, n_used, "cuda"))
    return d, dict(w_ug=w_ug, w_d=w_d, xq=orc.quantize_rows(xf), ids=ids, cw=cw)


def _batched(q, d, n_embd, n_ff, n_expert, n_used):
    import torch
    b = dict(d, h=torch.empty_like(d["h"]), out=torch.empty_like(d["out"]),
             ws=q.moe_r8_workspace(1, n_embd, n_ff, n_expert, n_used, "cuda"))
    q.moe_r8_ffn_batched([b], n_embd, n_ff, n_expert)
    return b


def _counters_zero(d):
    return bool((d["ws"][4:12] == 0).all().item())


SHAPES = [(256, 96, 8, 2), (512, 128, 16, 4), (768, 256, 32, 8), (2048, 768, 128, 8),
          (1024, 2048, 32, 16), (256, 32, 4, 1), (512, 64, 4, 3)]


@pytest.mark.parametrize("n_embd,n_ff,n_expert,n_used", SHAPES)
def test_fused_matches_oracle_and_two_launch_form(q, orc, n_embd, n_ff, n_expert, n_used):
    print(f"case: fused {n_embd} {n_ff} {n_expert} {n_used}", flush=True)
    d, c = _layer(q, orc, n_embd, n_ff, n_expert, n_used, f"fz-{n_embd}-{n_ff}-{n_expert}-{n_used}")
    q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
    b = _batched(q, d, n_embd, n_ff, n_expert, n_used)
    assert q.moe_error_word(d["ws"]) == 0
    assert _counters_zero(d)
    h = d["h"].cpu().numpy()
    assert np.array_equal(h.view(np.uint32), b["h"].cpu().numpy().view(np.uint32))
    out_ref = orc.moe_down_combine(c["w_d"], h, c["ids"], c["cw"], n_ff, n_embd, n_expert)
    out = d["out"].cpu().numpy()
    assert_rows_close(out, out_ref)
    assert_rows_close(out, b["out"].cpu().numpy())


def test_fused_repeated_calls_one_workspace(q, orc):
    """Three calls with different token rows on one workspace: each within the
    bound of the oracle, the counters back at zero after each, and a repeat
    of the first input gives the first output bit for bit."""
    import torch
    n_embd, n_ff, n_expert, n_used = 2048, 768, 128, 8
    d, c = _layer(q, orc, n_embd, n_ff, n_expert, n_used, "fz-rep")
    outs = []
    for i in range(3):
        xf = synth.normal_f32((1, n_embd), 1.0, "fz-rep", "x", i)
        d["x"].copy_(torch.from_numpy(xf))
        q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
        assert q.moe_error_word(d["ws"]) == 0 and _counters_zero(d)
        h = d["h"].cpu().numpy()
        h_ref = orc.moe_up_gate_swiglu(c["w_ug"], orc.quantize_rows(xf), c["ids"], n_embd, n_ff,
                                       n_expert)
        assert_rows_close(h.reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
        out = d["out"].cpu().numpy()
        assert_rows_close(out, orc.moe_down_combine(c["w_d"], h, c["ids"], c["cw"], n_ff, n_embd,
                                                    n_expert))
        outs.append(out.copy())
    d["x"].copy_(torch.from_numpy(synth.normal_f32((1, n_embd), 1.0, "fz-rep", "x", 0)))
    q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
    assert np.array_equal(d["out"].cpu().numpy().view(np.uint32), outs[0].view(np.uint32))


def test_fused_graph_replays(q, orc):
    """The call captured in a HIP graph: every replay, with eager work of the
    same call in between, gives the eager result bit for bit."""
    import torch
    n_embd, n_ff, n_expert, n_used = 2048, 768, 128, 8
    d, _ = _layer(q, orc, n_embd, n_ff, n_expert, n_used, "fz-graph")
    q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
    torch.cuda.synchronize()
    ref = d["out"].clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
    torch.cuda.synchronize()
    for _ in range(3):
        d["out"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["out"].view(torch.int32), ref.view(torch.int32))
        q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
        torch.cuda.synchronize()
        assert torch.equal(d["out"].view(torch.int32), ref.view(torch.int32))
    assert _counters_zero(d)


def test_fused_invalid_id(q, orc):
    """An out-of-range id: bit 0 of the error word, NaN h row for its slot,
    NaN outputs; the next call with valid ids clears the word."""
    n_embd, n_ff, n_expert, n_used = 512, 128, 16, 4
    ids = np.array([[3, 16, 0, 7]], dtype=np.int32)
    d, c = _layer(q, orc, n_embd, n_ff, n_expert, n_used, "fz-bad", ids=ids)
    q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
    assert q.moe_error_word(d["ws"]) == 1
    assert _counters_zero(d)
    h = d["h"].cpu().numpy()
    assert np.all(np.isnan(h[0, 1])) and not np.any(np.isnan(h[0, [0, 2, 3]]))
    assert np.all(np.isnan(d["out"].cpu().numpy()))
    d["ids"].copy_(d["ids"].new_tensor([[3, 15, 0, 7]]))
    q.moe_r8_ffn_fused(d, n_embd, n_ff, n_expert)
    assert q.moe_error_word(d["ws"]) == 0
    c["ids"] = np.array([[3, 15, 0, 7]], dtype=np.int32)
    h = d["h"].cpu().numpy()
    assert_rows_close(d["out"].cpu().numpy(),
                      orc.moe_down_combine(c["w_d"], h, c["ids"], c["cw"], n_ff, n_embd, n_expert))


def test_fused_limits(q):
    assert q.raw.moe_r8_fused_workspace_bytes(224, 64, 8, 2) == 0      # n_embd % 256 != 0
    assert q.raw.moe_r8_fused_workspace_bytes(256, 64, 8, 2) == 256 + 2 * 2 * 256 * 4
