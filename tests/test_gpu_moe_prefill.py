"""GPU parity of the expert FFN's prefill path (more than 16 tokens per call:
routing into tiles, quantization, grouped int8 matrix-core GEMMs, combine)
against the oracle, with the stage-boundary protocol of the decode tests: h
per (t,u) row against the oracle's h from the same quantized token rows,
down+combine against the oracle fed the GPU's own h; fp32 within 1e-5
per-row relative L2, every output written (outputs pre-filled with NaN)."""
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


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used", [
    (17, 256, 128, 8, 2),       # fewest tokens on this path
    (40, 512, 256, 16, 4),      # several column blocks of 128
    (64, 128, 384, 1, 1),       # one expert: two full tiles of 32 slots, three column blocks
    (200, 256, 384, 32, 8),     # ragged tiles (counts not multiples of 32)
    (100, 384, 128, 5, 3),      # few experts, several tiles each
    (24, 4096, 256, 4, 2),      # up_gate K of 128 blocks: the token tile staged in two parts
    (30, 256, 2560, 3, 2),      # down K of 80 blocks: a full part and a padded one
    (300, 256, 128, 2, 2),      # two experts with about ten tiles each
    (40, 256, 128, 1024, 16)])  # the most experts, 16 slots per token, most experts idle
def test_prefill_small(q, orc, n_tok, n_embd, n_ff, n_expert, n_used):
    w_ug, w_d, xf, ids, cw = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used,
                                   f"pre-{n_tok}-{n_embd}-{n_ff}")
    xq = orc.quantize_rows(xf)
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    ws.fill_(0x7F)
    h = nan_like((n_tok, n_used, n_ff))
    q.moe_up_gate_swiglu(to_gpu(w_ug), to_gpu(xf), to_gpu(ids), n_embd, n_ff, n_expert, ws, h=h)
    assert q.moe_error_word(ws) == 0
    h_gpu = h.cpu().numpy()
    h_ref = orc.moe_up_gate_swiglu(w_ug, xq, ids, n_embd, n_ff, n_expert)
    assert_rows_close(h_gpu.reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    ws.fill_(0x7F)
    out = nan_like((n_tok, n_embd))
    q.moe_down_combine(to_gpu(w_d), h, to_gpu(ids), to_gpu(cw), n_ff, n_embd, n_expert, ws,
                       out=out)
    assert q.moe_error_word(ws) == 0
    out_ref = orc.moe_down_combine(w_d, h_gpu, ids, cw, n_ff, n_embd, n_expert)
    assert_rows_close(out.cpu().numpy(), out_ref)


def test_prefill_duplicates_and_invalid(q, orc):
    """ids need not be distinct (a token may name an expert twice); an id out
    of range sets the error word, NaNs its h row and its token's output row,
    and leaves every other row exact."""
    n_tok, n_embd, n_ff, n_expert, n_used = 33, 256, 128, 7, 3
    ids = (np.arange(n_tok * n_used).reshape(n_tok, n_used) * 5 % n_expert).astype(np.int32)
    ids[3] = [2, 2, 2]
    ids[5, 1] = 99
    ids[20, 0] = -1
    w_ug, w_d, xf, _, cw = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, "pre-bad", ids)
    xq = orc.quantize_rows(xf)
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    h = q.moe_up_gate_swiglu(to_gpu(w_ug), to_gpu(xf), to_gpu(ids), n_embd, n_ff, n_expert, ws)
    assert q.moe_error_word(ws) == 1
    hh = h.cpu().numpy()
    assert np.all(np.isnan(hh[5, 1])) and np.all(np.isnan(hh[20, 0]))
    safe = np.where((ids >= 0) & (ids < n_expert), ids, 0).astype(np.int32)
    ref = orc.moe_up_gate_swiglu(w_ug, xq, safe, n_embd, n_ff, n_expert)
    for t in range(n_tok):
        for u in range(n_used):
            if (t, u) not in ((5, 1), (20, 0)):
                assert rel_l2_rows(hh[t, u][None], ref[t, u][None])[0] <= TOL, (t, u)
    hh[5, 1] = 0.0
    hh[20, 0] = 0.0
    out = q.moe_down_combine(to_gpu(w_d), to_gpu(hh), to_gpu(ids), to_gpu(cw), n_ff, n_embd,
                             n_expert, ws).cpu().numpy()
    assert q.moe_error_word(ws) == 1
    assert np.all(np.isnan(out[5])) and np.all(np.isnan(out[20]))
    ref_out = orc.moe_down_combine(w_d, hh, safe, cw, n_ff, n_embd, n_expert)
    keep = [t for t in range(n_tok) if t not in (5, 20)]
    assert_rows_close(out[keep], ref_out[keep])


def test_prefill_full_layer_sampled(q, orc):
    """The Gemma-4-26B-A4B expert FFN shape (n_embd 2048, n_ff 768, 128 experts,
    top-8) at 512 tokens: h rows and output rows of sampled tokens against the
    oracle (the oracle runs on the selected tokens only: each token's rows
    depend on that token alone)."""
    n_tok, n_embd, n_ff, n_expert, n_used = 512, 2048, 768, 128, 8
    w_ug, w_d, xf, ids, cw = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, "pre-full")
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    h = nan_like((n_tok, n_used, n_ff))
    q.moe_up_gate_swiglu(to_gpu(w_ug), to_gpu(xf), to_gpu(ids), n_embd, n_ff, n_expert, ws, h=h)
    out = nan_like((n_tok, n_embd))
    q.moe_down_combine(to_gpu(w_d), h, to_gpu(ids), to_gpu(cw), n_ff, n_embd, n_expert, ws,
                       out=out)
    assert q.moe_error_word(ws) == 0
    h_gpu = h.cpu().numpy()
    out_gpu = out.cpu().numpy()
    assert not np.isnan(h_gpu).any() and not np.isnan(out_gpu).any()
    sel = np.array([0, 1, 77, 255, 300, 511])
    xq = orc.quantize_rows(xf[sel])
    h_ref = orc.moe_up_gate_swiglu(w_ug, xq, ids[sel], n_embd, n_ff, n_expert)
    assert_rows_close(h_gpu[sel].reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    out_ref = orc.moe_down_combine(w_d, h_gpu[sel], ids[sel], cw[sel], n_ff, n_embd, n_expert)
    assert_rows_close(out_gpu[sel], out_ref)
