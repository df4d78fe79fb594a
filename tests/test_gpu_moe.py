"""GPU parity of the expert FFN (moe_route, moe_up_gate_swiglu,
moe_down_combine) against the oracle.

Protocol (stage boundaries): routing is compared exactly; h is compared per
(t,u) row against the oracle's h computed from the same quantized token rows;
down+combine is compared against the oracle fed the GPU's own h (fp32), so
both sides quantize the same h values with the same rule.  An end-to-end check
(oracle from fp32 x alone) is also made: any output row off by more than the
tolerance must be explained by h codes that flip between GPU h and oracle h at
a rounding boundary."""
import numpy as np
import pytest

import synth
from gpu_cases import TOL, assert_rows_close, nan_like, to_gpu
from qref import rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, tag, ids=None):
    w_ug = orc.quantize_rows(synth.normal_f32((n_expert * 2 * n_ff, n_embd), 0.02, tag, "ug"))
    w_d = orc.quantize_rows(synth.normal_f32((n_expert * n_embd, n_ff), 0.02, tag, "down"))
    xf = synth.normal_f32((n_tok, n_embd), 1.0, tag, "x")
    if ids is None:
        ids = synth.expert_ids(n_tok, n_used, n_expert, tag, "ids")
    cw = synth.combine_weights(n_tok, n_used, tag, "cw")
    return w_ug, w_d, xf, np.ascontiguousarray(ids, dtype=np.int32), cw


def _run(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, tag, ids=None):
    w_ug, w_d, xf, ids, cw = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, tag, ids)
    xq = orc.quantize_rows(xf)
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    ws.fill_(0x7F)
    h = nan_like((n_tok, n_used, n_ff))
    q.moe_up_gate_swiglu(to_gpu(w_ug), to_gpu(xf), to_gpu(ids), n_embd, n_ff, n_expert, ws, h=h)
    assert q.moe_error_word(ws) == 0
    h_gpu = h.cpu().numpy()
    h_ref = orc.moe_up_gate_swiglu(w_ug, xq, ids, n_embd, n_ff, n_expert)
    assert_rows_close(h_gpu.reshape(n_tok * n_used, n_ff), h_ref.reshape(n_tok * n_used, n_ff))

    ws.fill_(0x7F)
    out = nan_like((n_tok, n_embd))
    q.moe_down_combine(to_gpu(w_d), h, to_gpu(ids), to_gpu(cw), n_ff, n_embd, n_expert, ws,
                       out=out)
    assert q.moe_error_word(ws) == 0
    out_gpu = out.cpu().numpy()
    out_ref = orc.moe_down_combine(w_d, h_gpu, ids, cw, n_ff, n_embd, n_expert)
    assert_rows_close(out_gpu, out_ref)
    return dict(w_ug=w_ug, w_d=w_d, xf=xf, xq=xq, ids=ids, cw=cw, h_gpu=h_gpu, h_ref=h_ref,
                out_gpu=out_gpu)


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used", [
    (1, 256, 64, 8, 2), (3, 512, 96, 6, 4), (16, 256, 128, 32, 8), (5, 768, 160, 4, 4),
    (2, 2048, 768, 16, 8), (1, 4096, 256, 4, 1), (7, 256, 32, 1, 1),
    (1, 256, 256, 8, 8),      # row-major down (8 slots)
    (2, 512, 512, 8, 8),      # row-major down (16 slots, two per wave)
    (3, 256, 256, 8, 8),      # expert-major down, several slots per expert
    (9, 768, 256, 64, 4),     # up_gate with 4 tokens per chunk
    (40, 256, 256, 4, 2)])    # many slots per expert: several chunks
def test_moe_small(q, orc, n_tok, n_embd, n_ff, n_expert, n_used):
    _run(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, f"moe-{n_tok}-{n_embd}-{n_ff}")


def test_moe_duplicate_ids(q, orc):
    """ids need not be distinct: a token may name the same expert twice."""
    ids = np.array([[2, 2, 0], [1, 2, 2], [0, 0, 0]], dtype=np.int32)
    _run(q, orc, 3, 256, 64, 4, 3, "moe-dup", ids=ids)


def _route_check(q, orc, ids, n_expert):
    ws = q.moe_workspace(ids.shape[0], 256, 64, n_expert, ids.shape[1], "cuda")
    c, o, p = q.moe_route(to_gpu(ids), n_expert, ws)
    rc, ro, rp = orc.moe_route(ids, n_expert)
    assert np.array_equal(c.cpu().numpy(), rc)
    assert np.array_equal(o.cpu().numpy(), ro)
    assert np.array_equal(p.cpu().numpy(), rp)


@pytest.mark.parametrize("n_tok,n_used,n_expert", [(1, 8, 128), (16, 8, 128), (100, 8, 128),
                                                   (5, 3, 7), (64, 16, 1000)])
def test_route_exact(q, orc, n_tok, n_used, n_expert):
    ids = synth.expert_ids(n_tok, n_used, n_expert, "route", n_tok, n_used)
    _route_check(q, orc, ids, n_expert)


@pytest.mark.parametrize("n_tok,n_embd,n_ff", [
    (3, 256, 64),      # generic up_gate and down kernels (64/32 = 2 blocks per row)
    (3, 256, 256),     # fast up_gate, row-major down with the fused combine
    (10, 512, 256),    # fast up_gate (several tokens per expert), expert-major down
    (12, 320, 256)])   # generic up_gate (10 blocks per row), expert-major down
def test_invalid_ids_flagged(q, orc, n_tok, n_embd, n_ff):
    n_expert, n_used = 4, 2
    w_ug, w_d, xf, _, cw = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used,
                                 f"moe-bad-{n_tok}-{n_embd}-{n_ff}")
    ids = (np.arange(n_tok * n_used).reshape(n_tok, n_used) % n_expert).astype(np.int32)
    ids[1, 1] = 7                                                  # out of range
    xq = orc.quantize_rows(xf)
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    h = q.moe_up_gate_swiglu(to_gpu(w_ug), to_gpu(xf), to_gpu(ids), n_embd, n_ff, n_expert, ws)
    assert q.moe_error_word(ws) == 1
    hh = h.cpu().numpy()
    assert np.all(np.isnan(hh[1, 1]))
    ref = orc.moe_up_gate_swiglu(w_ug, xq, np.where(ids < n_expert, ids, 0), n_embd, n_ff,
                                 n_expert)
    for t in range(n_tok):
        for u in range(n_used):
            if (t, u) != (1, 1):
                assert rel_l2_rows(hh[t, u][None], ref[t, u][None])[0] <= TOL
    hh[1, 1] = 0.0
    out = q.moe_down_combine(to_gpu(w_d), to_gpu(hh), to_gpu(ids), to_gpu(cw), n_ff, n_embd,
                             n_expert, ws).cpu().numpy()
    assert q.moe_error_word(ws) == 1
    assert np.all(np.isnan(out[1]))
    good = [t for t in range(n_tok) if t != 1]
    assert np.all(np.isfinite(out[good]))
    ref_out = orc.moe_down_combine(w_d, hh[good], ids[good], cw[good], n_ff, n_embd, n_expert)
    assert_rows_close(out[good], ref_out)
    c, o, p = q.moe_route(to_gpu(ids), n_expert, ws)
    assert q.moe_error_word(ws) == 1
    assert int(o.cpu()[-1]) == n_tok * n_used - 1
    # a clean call clears the word again
    q.moe_route(to_gpu(np.zeros((1, 2), np.int32)), n_expert, ws)
    assert q.moe_error_word(ws) == 0


def _flip_explained(orc, h_gpu, h_ref64, n_ff):
    """Codes of q(h) that differ between GPU h and the oracle's own h must sit
    at a rounding boundary: |h/d - (n + 1/2)| tiny or the block amax moved."""
    a = h_gpu.reshape(-1, n_ff).astype(np.float32)
    b = h_ref64.reshape(-1, n_ff).astype(np.float32)
    qa = orc.quantize_rows(a)
    qb = orc.quantize_rows(b)
    if np.array_equal(qa, qb):
        return 0
    da, ca = orc.split_blocks(qa)
    db, cb = orc.split_blocks(qb)
    flips = 0
    bb = b.reshape(b.shape[0], -1, 32).astype(np.float64)
    for r, blk in zip(*np.nonzero((ca != cb).any(axis=2) | (da != db))):
        amax = np.abs(bb[r, blk]).max()
        d32 = np.float32(amax) / np.float32(127)
        ratio = bb[r, blk] / np.float64(d32)
        diff = ca[r, blk].astype(int) != cb[r, blk].astype(int)
        near_half = np.abs(np.abs(ratio - np.trunc(ratio)) - 0.5) < 1e-3
        amax_moved = da[r, blk] != db[r, blk]
        assert amax_moved or np.all(near_half[diff]), (r, blk, ratio[diff])
        flips += int(diff.sum())
    return flips


def test_moe_end_to_end_flips_explained(q, orc):
    n_tok, n_embd, n_ff, n_expert, n_used = 16, 512, 256, 32, 8
    r = _run(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, "moe-e2e")
    flips = _flip_explained(orc, r["h_gpu"], r["h_ref"], n_ff)
    out_e2e = orc.moe_down_combine(r["w_d"], r["h_ref"].astype(np.float32), r["ids"], r["cw"],
                                   n_ff, n_embd, n_expert)
    err = rel_l2_rows(r["out_gpu"], out_e2e)
    if flips == 0:
        assert err.max() <= TOL
    print(f"end-to-end: {flips} flipped h codes, max row error {err.max():.2e}")


@pytest.mark.parametrize("n_tok", [1, 16])
def test_moe_full_layer_shape(q, orc, n_tok):
    """One layer at the full expert shape: n_embd 2048, n_ff 768, 128 experts,
    8 active per token, batch 1 and 16."""
    _run(q, orc, n_tok, 2048, 768, 128, 8, f"c4-layer-{n_tok}")


def _batched_layers(q, orc, n_layers, n_tok, n_embd, n_ff, n_expert, n_used, tag, bad_layer=None):
    import torch
    layers, refs = [], []
    for l in range(n_layers):
        w_ug, w_d, xf, ids, cw = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, f"{tag}-{l}")
        if l == bad_layer:
            ids = ids.copy()
            ids[0, 0] = n_expert           # out of range: this layer only
        ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
        ws.fill_(0x7F)
        layers.append(dict(w_up_gate=to_gpu(w_ug), x=to_gpu(xf), ids=to_gpu(ids),
                           h=nan_like((n_tok, n_used, n_ff)), ws=ws, w_down=to_gpu(w_d),
                           cw=to_gpu(cw), out=nan_like((n_tok, n_embd))))
        refs.append(dict(w_ug=w_ug, w_d=w_d, xq=orc.quantize_rows(xf), ids=ids, cw=cw))
    return layers, refs


@pytest.mark.parametrize("n_layers,n_tok,n_embd,n_ff,n_expert,n_used", [
    (3, 1, 512, 256, 16, 8),      # decode: row-major down kernel
    (5, 4, 256, 128, 8, 4),       # expert-major down + combine
    (33, 1, 256, 64, 8, 2),       # more descriptors than one launch takes
    (2, 3, 256, 96, 6, 4)])       # generic kernels (k/32 not a multiple of 8)
def test_moe_batched_layers(q, orc, n_layers, n_tok, n_embd, n_ff, n_expert, n_used):
    """Grouped calls over independent layers: each layer's h and output match
    the oracle, and are bitwise equal to the single-layer calls."""
    import torch
    layers, refs = _batched_layers(q, orc, n_layers, n_tok, n_embd, n_ff, n_expert, n_used,
                                   f"mb-{n_layers}-{n_tok}-{n_ff}")
    q.moe_up_gate_swiglu_batched(layers, n_embd, n_ff, n_expert)
    q.moe_down_combine_batched(layers, n_ff, n_embd, n_expert)
    torch.cuda.synchronize()
    for d, r in zip(layers, refs):
        assert q.moe_error_word(d["ws"]) == 0
        h_gpu = d["h"].cpu().numpy()
        h_ref = orc.moe_up_gate_swiglu(r["w_ug"], r["xq"], r["ids"], n_embd, n_ff, n_expert)
        assert_rows_close(h_gpu.reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
        out_ref = orc.moe_down_combine(r["w_d"], h_gpu, r["ids"], r["cw"], n_ff, n_embd, n_expert)
        assert_rows_close(d["out"].cpu().numpy(), out_ref)
        # same bits as the single-layer calls
        h1 = nan_like(tuple(d["h"].shape))
        q.moe_up_gate_swiglu(d["w_up_gate"], d["x"], d["ids"], n_embd, n_ff, n_expert, d["ws"],
                             h=h1)
        o1 = nan_like(tuple(d["out"].shape))
        q.moe_down_combine(d["w_down"], h1, d["ids"], d["cw"], n_ff, n_embd, n_expert, d["ws"],
                           out=o1)
        assert torch.equal(h1, d["h"]) and torch.equal(o1, d["out"])


def test_moe_batched_invalid_id_one_layer(q, orc):
    """An out-of-range id in one layer sets that layer's error word and NaNs
    only; the other layers are unaffected."""
    import torch
    n_layers, n_tok, n_embd, n_ff, n_expert, n_used = 3, 1, 256, 64, 8, 4
    layers, refs = _batched_layers(q, orc, n_layers, n_tok, n_embd, n_ff, n_expert, n_used,
                                   "mb-bad", bad_layer=1)
    q.moe_up_gate_swiglu_batched(layers, n_embd, n_ff, n_expert)
    q.moe_down_combine_batched(layers, n_ff, n_embd, n_expert)
    torch.cuda.synchronize()
    for l, (d, r) in enumerate(zip(layers, refs)):
        h = d["h"].cpu().numpy()
        out = d["out"].cpu().numpy()
        if l == 1:
            assert q.moe_error_word(d["ws"]) == 1
            assert np.all(np.isnan(h[0, 0])) and np.all(np.isnan(out[0]))
            assert not np.any(np.isnan(h[0, 1:]))
        else:
            assert q.moe_error_word(d["ws"]) == 0
            assert not np.any(np.isnan(h)) and not np.any(np.isnan(out))
            out_ref = orc.moe_down_combine(r["w_d"], h, r["ids"], r["cw"], n_ff, n_embd, n_expert)
            assert_rows_close(out, out_ref)
