"""GPU parity of the decode expert FFN over R8 expert weights
(moe_r8_ffn_batched) against the oracle, with the stage-boundary protocol of
the native expert FFN: h per (t,u) row against the oracle's h from the same
quantized token rows; out against the oracle's down + combine fed the GPU's
own h; error word and NaN rows for out-of-range ids."""
import numpy as np
import pytest

import synth
from gpu_cases import assert_rows_close, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, tag, ids=None):
    import torch
    w_ug = orc.quantize_rows(synth.normal_f32((n_expert * 2 * n_ff, n_embd), 0.02, tag, "ug"))
    w_d = orc.quantize_rows(synth.normal_f32((n_expert * n_embd, n_ff), 0.02, tag, "down"))
    xf = synth.normal_f32((n_tok, n_embd), 1.0, tag, "x")
    if ids is None:
        ids = synth.expert_ids(n_tok, n_used, n_expert, tag, "ids")
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    cw = synth.combine_weights(n_tok, n_used, tag, "cw")
    d = dict(w_up_gate_r8=q.q8_0_repack_r8(to_gpu(w_ug), n_expert * 2 * n_ff, n_embd),
             w_down_r8=q.q8_0_repack_r8(to_gpu(w_d), n_expert * n_embd, n_ff),
             x=to_gpu(xf), ids=to_gpu(ids), cw=to_gpu(cw),
             h=torch.full((n_tok, n_used, n_ff), float("nan"), device="cuda"),
             out=torch.full((n_tok, n_embd), float("nan"), device="cuda"),
             ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda").fill_(0x7F))
    return d, dict(w_ug=w_ug, w_d=w_d, xq=orc.quantize_rows(xf), ids=ids, cw=cw)


def _check(q, orc, d, c, n_tok, n_embd, n_ff, n_expert, n_used):
    assert q.moe_error_word(d["ws"]) == 0
    h = d["h"].cpu().numpy()
    h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"], c["ids"], n_embd, n_ff, n_expert)
    assert_rows_close(h.reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    out_ref = orc.moe_down_combine(c["w_d"], h, c["ids"], c["cw"], n_ff, n_embd, n_expert)
    assert_rows_close(d["out"].cpu().numpy(), out_ref)


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used", [
    (1, 256, 96, 8, 2), (1, 512, 128, 16, 4), (3, 768, 256, 32, 8), (16, 512, 192, 16, 8),
    (1, 2048, 768, 128, 8), (16, 2048, 768, 128, 8), (1, 1024, 2048, 32, 16), (4, 224, 32, 4, 3)])
def test_moe_r8_ffn(q, orc, n_tok, n_embd, n_ff, n_expert, n_used):
    d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, f"r8moe-{n_tok}-{n_embd}-{n_ff}-{n_expert}-{n_used}")
    q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
    _check(q, orc, d, c, n_tok, n_embd, n_ff, n_expert, n_used)


def test_moe_r8_ffn_repeated_experts(q, orc):
    """Every token names the same 4 experts: 6 slots per expert, served by its
    owner in two passes over the rows (4 slots, then 2)."""
    n_tok, n_embd, n_ff, n_expert, n_used = 6, 512, 128, 4, 4
    ids = np.tile(np.array([2, 0, 3, 1], dtype=np.int32), (n_tok, 1))
    d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, "r8moe-rep", ids=ids)
    q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
    _check(q, orc, d, c, n_tok, n_embd, n_ff, n_expert, n_used)


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used,same", [
    (16, 2048, 768, 32, 8, False), (16, 2048, 768, 32, 8, True), (5, 512, 96, 8, 3, False)])
def test_moe_r8_gather_matches_one_token_calls(q, orc, n_tok, n_embd, n_ff, n_expert, n_used,
                                               same):
    """Several tokens go through the expert-major kernels (each active expert
    read once per call); per slot the arithmetic and its order are those of the
    one-token kernels, so h and out equal, bit for bit, one call per token.
    same: every token names experts 0..n_used-1 (16 slots per expert, 4 passes
    over its rows)."""
    import torch
    print(f"case: r8 gather {n_tok} {n_embd} {n_ff} {n_expert} {n_used} same={same}", flush=True)
    tag = f"r8gt-{n_tok}-{n_embd}-{same}"
    ids = None
    if same:
        ids = np.tile(np.arange(n_used, dtype=np.int32), (n_tok, 1))
    d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, tag, ids=ids)
    q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
    torch.cuda.synchronize()
    for t in range(n_tok):
        one = dict(d, x=d["x"][t:t + 1].contiguous(), ids=d["ids"][t:t + 1].contiguous(),
                   cw=d["cw"][t:t + 1].contiguous(),
                   h=torch.full((1, n_used, n_ff), 5.0, device="cuda"),
                   out=torch.full((1, n_embd), 5.0, device="cuda"),
                   ws=q.moe_r8_workspace(1, n_embd, n_ff, n_expert, n_used, "cuda"))
        q.moe_r8_ffn_batched([one], n_embd, n_ff, n_expert)
        assert torch.equal(one["h"][0].view(torch.int32), d["h"][t].view(torch.int32)), t
        assert torch.equal(one["out"][0].view(torch.int32), d["out"][t].view(torch.int32)), t
    _check(q, orc, d, c, n_tok, n_embd, n_ff, n_expert, n_used)


def test_moe_r8_gather_grouped_matches_chained(q, orc):
    """30 layers of 16 tokens in one call take longer streams per wave than one
    layer per call (the work per wave follows the layers in the call); h and
    out are the same bits either way.  The layers share one set of weights
    (own ids, rows and combine weights each); layer 0 is also checked against
    the oracle."""
    import torch
    n_layers, n_tok, n_embd, n_ff, n_expert, n_used = 30, 16, 512, 256, 128, 8
    print("case: r8 gather 30 layers grouped vs chained", flush=True)
    d0, c0 = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, "r8gt-30")
    layers = []
    for l in range(n_layers):
        key = ("r8gt-30", str(l))
        ids = np.ascontiguousarray(synth.expert_ids(n_tok, n_used, n_expert, *key, "ids"),
                                   dtype=np.int32)
        layers.append(dict(d0, x=to_gpu(synth.normal_f32((n_tok, n_embd), 1.0, *key, "x")),
                           ids=to_gpu(ids), cw=to_gpu(synth.combine_weights(n_tok, n_used, *key, "cw")),
                           h=torch.full((n_tok, n_used, n_ff), float("nan"), device="cuda"),
                           out=torch.full((n_tok, n_embd), float("nan"), device="cuda"),
                           ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")))
    q.moe_r8_ffn_batched(layers, n_embd, n_ff, n_expert)
    torch.cuda.synchronize()
    for l, d in enumerate(layers):
        one = dict(d, h=torch.full_like(d["h"], 2.0), out=torch.full_like(d["out"], 2.0))
        q.moe_r8_ffn_batched([one], n_embd, n_ff, n_expert)
        assert torch.equal(one["h"].view(torch.int32), d["h"].view(torch.int32)), l
        assert torch.equal(one["out"].view(torch.int32), d["out"].view(torch.int32)), l
    ids0 = layers[0]["ids"].cpu().numpy()
    c = dict(c0, xq=orc.quantize_rows(layers[0]["x"].cpu().numpy()), ids=ids0,
             cw=layers[0]["cw"].cpu().numpy())
    _check(q, orc, layers[0], c, n_tok, n_embd, n_ff, n_expert, n_used)


def test_moe_r8_ffn_layers(q, orc):
    """Three independent layers in one call."""
    shape = (2, 512, 160, 8, 4)
    pairs = [_layer(q, orc, *shape, f"r8moe-l{i}") for i in range(3)]
    q.moe_r8_ffn_batched([d for d, _ in pairs], shape[1], shape[2], shape[3])
    for d, c in pairs:
        _check(q, orc, d, c, *shape)


def test_moe_r8_ffn_invalid_ids(q, orc):
    n_tok, n_embd, n_ff, n_expert, n_used = 4, 256, 64, 8, 3
    ids = synth.expert_ids(n_tok, n_used, n_expert, "r8moe-bad", "ids")
    ids[1, 2] = n_expert + 5
    ids[3, 0] = -1
    d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, "r8moe-bad", ids=ids)
    q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
    assert q.moe_error_word(d["ws"]) == 1
    h = d["h"].cpu().numpy()
    out = d["out"].cpu().numpy()
    assert np.all(np.isnan(h[1, 2])) and np.all(np.isnan(h[3, 0]))
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[3]))
    good = [0, 2]
    ok_ids = c["ids"][good]
    h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"][good], ok_ids, n_embd, n_ff, n_expert)
    assert_rows_close(h[good].reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    out_ref = orc.moe_down_combine(c["w_d"], h[good], ok_ids, c["cw"][good], n_ff, n_embd,
                                   n_expert)
    assert_rows_close(out[good], out_ref)
    # the next valid call clears the word
    d2, c2 = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, "r8moe-bad2")
    d2["ws"] = d["ws"]
    q.moe_r8_ffn_batched([d2], n_embd, n_ff, n_expert)
    _check(q, orc, d2, c2, n_tok, n_embd, n_ff, n_expert, n_used)


# More than 16 tokens: routing into tiles and the grouped int8 matrix-core
# products over the R8 weights.
@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used", [
    (17, 256, 128, 8, 2),       # fewest tokens on this path
    (40, 512, 256, 16, 4),      # several column blocks
    (64, 128, 384, 1, 1),       # one expert: two full tiles, waves past the output
    (200, 256, 384, 32, 8),     # ragged tiles
    (24, 4096, 256, 4, 2),      # up_gate K of 128 blocks: the token tile in two parts
    (30, 256, 2560, 3, 2),      # down K of 80 blocks: a full part and a padded one
    (300, 256, 128, 2, 2),      # two experts with about ten tiles each
    (40, 256, 128, 1024, 16)])  # the most experts, 16 slots per token, most experts idle
def test_moe_r8_ffn_prefill(q, orc, n_tok, n_embd, n_ff, n_expert, n_used):
    d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used,
                  f"r8pre-{n_tok}-{n_embd}-{n_ff}-{n_expert}-{n_used}")
    q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
    _check(q, orc, d, c, n_tok, n_embd, n_ff, n_expert, n_used)


def test_moe_r8_ffn_prefill_layers_and_invalid(q, orc):
    """Two layers of 40 tokens in one call, the second with out-of-range ids
    (NaN h rows and output rows, error word 1 in that layer's workspace)."""
    shape = (40, 512, 128, 8, 4)
    ids = synth.expert_ids(40, 4, 8, "r8pre-bad", "ids")
    ids[5, 1] = 8
    ids[33, 3] = -2
    d0, c0 = _layer(q, orc, *shape, "r8pre-l0")
    d1, c1 = _layer(q, orc, *shape, "r8pre-bad", ids=ids)
    q.moe_r8_ffn_batched([d0, d1], shape[1], shape[2], shape[3])
    _check(q, orc, d0, c0, *shape)
    assert q.moe_error_word(d1["ws"]) == 1
    h = d1["h"].cpu().numpy()
    out = d1["out"].cpu().numpy()
    assert np.all(np.isnan(h[5, 1])) and np.all(np.isnan(h[33, 3]))
    assert np.all(np.isnan(out[5])) and np.all(np.isnan(out[33]))
    good = np.array([t for t in range(40) if t not in (5, 33)])
    h_ref = orc.moe_up_gate_swiglu(c1["w_ug"], c1["xq"][good], c1["ids"][good], shape[1],
                                   shape[2], shape[3])
    assert_rows_close(h[good].reshape(-1, shape[2]), h_ref.reshape(-1, shape[2]))
    out_ref = orc.moe_down_combine(c1["w_d"], h[good], c1["ids"][good], c1["cw"][good], shape[2],
                                   shape[1], shape[3])
    assert_rows_close(out[good], out_ref)


def test_moe_r8_ffn_prefill_full_layer(q, orc):
    """The Gemma-4-26B-A4B expert FFN shape at 512 tokens: h and out bit for bit
    equal to the native-row prefill path on the same weights (both sum each
    element's exact block products in ascending block order), and sampled
    tokens against the oracle."""
    n_tok, n_embd, n_ff, n_expert, n_used = 512, 2048, 768, 128, 8
    d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, "r8pre-full")
    q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
    assert q.moe_error_word(d["ws"]) == 0
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    h_nat = torch_nan_like(d["h"])
    q.moe_up_gate_swiglu(to_gpu(c["w_ug"]), d["x"], d["ids"], n_embd, n_ff, n_expert, ws, h=h_nat)
    out_nat = torch_nan_like(d["out"])
    q.moe_down_combine(to_gpu(c["w_d"]), h_nat, d["ids"], d["cw"], n_ff, n_embd, n_expert, ws,
                       out=out_nat)
    import torch
    assert torch.equal(d["h"], h_nat)
    assert torch.equal(d["out"], out_nat)
    sel = np.array([0, 3, 200, 511])
    h = d["h"].cpu().numpy()
    h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"][sel], c["ids"][sel], n_embd, n_ff,
                                   n_expert)
    assert_rows_close(h[sel].reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    out_ref = orc.moe_down_combine(c["w_d"], h[sel], c["ids"][sel], c["cw"][sel], n_ff, n_embd,
                                   n_expert)
    assert_rows_close(d["out"].cpu().numpy()[sel], out_ref)


def torch_nan_like(t):
    import torch
    return torch.full_like(t, float("nan"))


def test_moe_r8_ffn_workspace_reuse(q, orc):
    """One workspace (sized for the largest call) across calls of different
    sizes and paths: 200 tokens, then 40, then 4 (decode kernels), then 40
    with an out-of-range id, then 40 again: every call's results and error
    word are its own."""
    import torch
    n_embd, n_ff, n_expert, n_used = 256, 128, 16, 4
    ws = q.moe_r8_workspace(200, n_embd, n_ff, n_expert, n_used, "cuda")
    assert ws.numel() >= q.moe_r8_workspace(40, n_embd, n_ff, n_expert, n_used, "cuda").numel()
    for i, n_tok in enumerate([200, 40, 4, 40, 40]):
        ids = None
        if i == 3:
            ids = synth.expert_ids(n_tok, n_used, n_expert, "r8ws-bad", "ids")
            ids[7, 2] = n_expert
        d, c = _layer(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, f"r8ws-{i}", ids=ids)
        d["ws"] = ws
        q.moe_r8_ffn_batched([d], n_embd, n_ff, n_expert)
        if i == 3:
            assert q.moe_error_word(ws) == 1
            assert bool(torch.isnan(d["out"][7]).all())
            assert bool(torch.isnan(d["h"][7, 2]).all())
            # every other result of the call is intact: the valid tokens' h
            # and out, and token 7's h rows of its valid slots
            sel = np.array([t for t in range(n_tok) if t != 7])
            h = d["h"].cpu().numpy()
            h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"][sel], c["ids"][sel], n_embd, n_ff,
                                           n_expert)
            assert_rows_close(h[sel].reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
            ok = [0, 1, 3]
            h7 = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"][7:8],
                                        np.ascontiguousarray(c["ids"][7:8, ok]), n_embd, n_ff,
                                        n_expert)
            assert_rows_close(h[7, ok], h7.reshape(-1, n_ff))
            out_ref = orc.moe_down_combine(c["w_d"], h[sel], c["ids"][sel], c["cw"][sel], n_ff,
                                           n_embd, n_expert)
            assert_rows_close(d["out"].cpu().numpy()[sel], out_ref)
            continue
        _check(q, orc, d, c, n_tok, n_embd, n_ff, n_expert, n_used)
