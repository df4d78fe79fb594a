"""Pins for the oracle's mixture-of-experts pieces.

- Fused up_gate + SwiGLU over the combined [n_embd, 2*n_ff, n_expert] tensor
  (gate rows first) equals the fallback of the Gemma-4-on-Xeon page (three-part
  fix, runtime graph fallback): two row views, mul_mat_id on each, then
  silu(gate)*up -- bit for bit, and also equals separately stored gate and up
  tensors.
- Against a dequantize-then-fp64 brute force written with numpy.
- Special cases: one expert / one slot reduce to the dense matmul; one-hot
  combine weights select one slot; a joint permutation of the slots leaves the
  output unchanged up to fp64 rounding.
- Routing: invariants and a brute-force sort.
"""
import math

import numpy as np
import pytest

import synth
from qref import dequant


def _moe_case(n_tok, n_embd, n_ff, n_expert, n_used, tag):
    w_ug_f = synth.normal_f32((n_expert * 2 * n_ff, n_embd), 0.02, "test", tag, "ug")
    w_d_f = synth.normal_f32((n_expert * n_embd, n_ff), 0.02, "test", tag, "down")
    x_f = synth.normal_f32((n_tok, n_embd), 1.0, "test", tag, "x")
    ids = synth.expert_ids(n_tok, n_used, n_expert, "test", tag, "ids")
    cw = synth.combine_weights(n_tok, n_used, "test", tag, "cw")
    return w_ug_f, w_d_f, x_f, ids, cw


def _silu(g):
    return g / (1.0 + np.exp(-g))


def test_fused_equals_split_bitwise(orc):
    n_tok, n_embd, n_ff, n_expert, n_used = 3, 256, 96, 6, 4
    w_ug_f, _, x_f, ids, _ = _moe_case(n_tok, n_embd, n_ff, n_expert, n_used, "split")
    w_ug = orc.quantize_rows(w_ug_f)
    x = orc.quantize_rows(x_f)
    fused = orc.moe_up_gate_swiglu(w_ug, x, ids, n_embd, n_ff, n_expert)
    split = orc.moe_up_gate_swiglu_split(w_ug, x, ids, n_embd, n_ff, n_expert)
    assert np.array_equal(fused, split)
    # separately stored gate and up tensors (no views)
    nb34 = n_embd // 32 * 34
    w3 = w_ug.reshape(n_expert, 2 * n_ff, nb34)
    gate = np.ascontiguousarray(w3[:, :n_ff])
    up = np.ascontiguousarray(w3[:, n_ff:])
    g = orc.mul_mat_id(gate, n_ff, 0, n_ff, x, ids, n_embd, n_expert)
    u = orc.mul_mat_id(up, n_ff, 0, n_ff, x, ids, n_embd, n_expert)
    assert np.array_equal(fused, orc.fused_mul_silu(g, u).reshape(g.shape))


def test_up_gate_vs_dequantized(orc):
    n_tok, n_embd, n_ff, n_expert, n_used = 4, 512, 64, 8, 3
    w_ug_f, _, x_f, ids, _ = _moe_case(n_tok, n_embd, n_ff, n_expert, n_used, "ugdq")
    w_ug = orc.quantize_rows(w_ug_f)
    x = orc.quantize_rows(x_f)
    h = orc.moe_up_gate_swiglu(w_ug, x, ids, n_embd, n_ff, n_expert)
    W = dequant(w_ug, n_embd).reshape(n_expert, 2 * n_ff, n_embd)
    X = dequant(x, n_embd)
    for t in range(n_tok):
        for u in range(n_used):
            e = ids[t, u]
            g = W[e, :n_ff] @ X[t]
            up = W[e, n_ff:] @ X[t]
            np.testing.assert_allclose(h[t, u], _silu(g) * up, rtol=1e-11, atol=1e-14)


def test_up_gate_gate_half_first(orc):
    """Zero the up half of one expert: its outputs vanish; zero the gate half:
    silu(0) = 0 makes them vanish too; the rows are not swapped."""
    n_tok, n_embd, n_ff, n_expert, n_used = 2, 128, 32, 3, 2
    w_ug_f, _, x_f, _, _ = _moe_case(n_tok, n_embd, n_ff, n_expert, n_used, "half")
    ids = np.array([[0, 1], [1, 2]], dtype=np.int32)
    w3 = w_ug_f.reshape(n_expert, 2 * n_ff, n_embd).copy()
    w3[1, n_ff:] = 0.0          # expert 1: up half zero
    w3[2, :n_ff] = 0.0          # expert 2: gate half zero
    w_ug = orc.quantize_rows(w3.reshape(-1, n_embd))
    x = orc.quantize_rows(x_f)
    h = orc.moe_up_gate_swiglu(w_ug, x, ids, n_embd, n_ff, n_expert)
    assert np.all(h[0, 1] == 0) and np.all(h[1, 0] == 0) and np.all(h[1, 1] == 0)
    assert np.all(h[0, 0] != 0)
    # values that quantize exactly (max = 127 * 2^k, so d = 2^k): gate weight
    # 31.75, up weight and activation 127/128 -> h = silu(31.75*a) * a*a
    w3 = np.zeros((1, 2 * n_ff, n_embd), dtype=np.float32)
    a = 127.0 / 128
    xf = np.zeros((1, n_embd), dtype=np.float32); xf[0, 0] = a
    w3[0, :n_ff, 0] = 31.75
    w3[0, n_ff:, 0] = a
    h = orc.moe_up_gate_swiglu(orc.quantize_rows(w3.reshape(-1, n_embd)),
                               orc.quantize_rows(xf), np.zeros((1, 1), np.int32),
                               n_embd, n_ff, 1)
    g = 31.75 * a
    np.testing.assert_allclose(h[0, 0], g / (1 + np.exp(-g)) * a * a, rtol=1e-15)


def test_single_expert_reduces_to_dense(orc):
    n_tok, n_embd, n_ff = 5, 256, 64
    w_ug_f, w_d_f, x_f, _, _ = _moe_case(n_tok, n_embd, n_ff, 1, 1, "dense")
    w_ug = orc.quantize_rows(w_ug_f)
    w_d = orc.quantize_rows(w_d_f)
    x = orc.quantize_rows(x_f)
    ids = np.zeros((n_tok, 1), dtype=np.int32)
    h = orc.moe_up_gate_swiglu(w_ug, x, ids, n_embd, n_ff, 1)
    g = orc.matmul(w_ug, x, 2 * n_ff, n_embd, n_tok)
    assert np.array_equal(h[:, 0, :], orc.fused_mul_silu(g[:, :n_ff].copy(),
                                                        g[:, n_ff:].copy()).reshape(n_tok, n_ff))
    h32 = h.astype(np.float32)
    out = orc.moe_down_combine(w_d, h32, ids, np.ones((n_tok, 1), np.float32), n_ff, n_embd, 1)
    hq = orc.quantize_rows(h32.reshape(n_tok, n_ff))
    assert np.array_equal(out, orc.matmul(w_d, hq, n_embd, n_ff, n_tok))


def test_down_combine_one_hot_and_hq(orc):
    n_tok, n_embd, n_ff, n_expert, n_used = 3, 128, 96, 5, 4
    _, w_d_f, _, ids, _ = _moe_case(n_tok, n_embd, n_ff, n_expert, n_used, "onehot")
    w_d = orc.quantize_rows(w_d_f)
    h = synth.normal_f32((n_tok, n_used, n_ff), 0.5, "test", "onehot", "h")
    for k in range(n_used):
        cw = np.zeros((n_tok, n_used), np.float32); cw[:, k] = 1.0
        out, hq = orc.moe_down_combine(w_d, h, ids, cw, n_ff, n_embd, n_expert, return_hq=True)
        assert np.array_equal(hq.reshape(n_tok * n_used, -1),
                              orc.quantize_rows(h.reshape(n_tok * n_used, n_ff)))
        W = w_d.reshape(n_expert, n_embd, -1)
        for t in range(n_tok):
            y = orc.matvec(W[ids[t, k]], hq[t, k], n_embd, n_ff)
            assert np.array_equal(out[t], y)


def test_down_combine_vs_dequantized_and_permutation(orc):
    n_tok, n_embd, n_ff, n_expert, n_used = 4, 256, 128, 10, 8
    _, w_d_f, _, ids, cw = _moe_case(n_tok, n_embd, n_ff, n_expert, n_used, "dc")
    w_d = orc.quantize_rows(w_d_f)
    h = synth.normal_f32((n_tok, n_used, n_ff), 0.3, "test", "dc", "h")
    out, hq = orc.moe_down_combine(w_d, h, ids, cw, n_ff, n_embd, n_expert, return_hq=True)
    W = dequant(w_d, n_ff).reshape(n_expert, n_embd, n_ff)
    H = dequant(hq.reshape(-1, hq.shape[-1]), n_ff).reshape(n_tok, n_used, n_ff)
    ref = np.zeros((n_tok, n_embd))
    for t in range(n_tok):
        for u in range(n_used):
            ref[t] += float(cw[t, u]) * (W[ids[t, u]] @ H[t, u])
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-13)
    perm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    out_p = orc.moe_down_combine(w_d, h[:, perm], ids[:, perm], cw[:, perm], n_ff, n_embd,
                                 n_expert)
    np.testing.assert_allclose(out_p, out, rtol=1e-12, atol=1e-14)
    sel = [0, 255, 17, 17]
    assert np.array_equal(orc.moe_down_combine(w_d, h, ids, cw, n_ff, n_embd, n_expert, sel=sel),
                          out[:, sel])


@pytest.mark.parametrize("n_tok,n_used,n_expert", [(1, 8, 128), (16, 8, 128), (5, 3, 4),
                                                   (7, 1, 2)])
def test_route(orc, n_tok, n_used, n_expert):
    ids = synth.expert_ids(n_tok, n_used, n_expert, "test", "route", n_tok)
    counts, offsets, pairs = orc.moe_route(ids, n_expert)
    assert counts.sum() == n_tok * n_used
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(pairs), np.arange(n_tok * n_used))      # each slot once
    flat = ids.reshape(-1)
    brute = sorted(range(n_tok * n_used), key=lambda s: (flat[s], s))
    assert list(pairs) == brute
    for e in range(n_expert):
        assert np.all(flat[pairs[offsets[e]:offsets[e + 1]]] == e)


def test_route_rejects_bad_ids(orc):
    with pytest.raises(ValueError):
        orc.moe_route(np.array([[0, 5]], dtype=np.int32), 5)
    with pytest.raises(ValueError):
        orc.moe_route(np.array([[-1, 2]], dtype=np.int32), 5)


def _q8_block(d_bits, codes):
    """One hand-built Q8_0 block: binary16 scale bits + 32 int8 codes."""
    b = np.zeros(34, dtype=np.uint8)
    b[0:2] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    b[2:] = np.asarray(codes, dtype=np.int8).view(np.uint8)
    return b


def test_dense_up_gate_exact_case(orc):
    """Dense up_gate on hand-built blocks (scales 1.0 and 0.5, binary16 0x3C00 and
    0x3800): gate row j sums to 32*(j+1), up row j to -32*(j+1) against an
    all-ones activation, so h = silu(32(j+1)) * (-32(j+1)); swapping the halves
    would give silu(-32(j+1)) * 32(j+1) (about -0) instead."""
    n_ff, n_embd = 3, 64
    ones = np.ones(32, dtype=np.int8)
    rows = []
    for j in range(n_ff):          # gate rows: (j+1) * ones at scale 1.0, second block zero
        rows.append(np.concatenate([_q8_block(0x3C00, (j + 1) * ones), _q8_block(0, 0 * ones)]))
    for j in range(n_ff):          # up rows: -2(j+1) * ones at scale 0.5 in the second block
        rows.append(np.concatenate([_q8_block(0, 0 * ones), _q8_block(0x3800, -2 * (j + 1) * ones)]))
    w = np.concatenate(rows)
    x = np.concatenate([_q8_block(0x3C00, ones), _q8_block(0x3C00, ones)])
    h = orc.up_gate_swiglu(w, x, n_embd, n_ff)
    assert h.shape == (1, n_ff)
    for j in range(n_ff):
        g, u = 32.0 * (j + 1), -32.0 * (j + 1)
        np.testing.assert_allclose(h[0, j], g / (1.0 + math.exp(-g)) * u, rtol=1e-15)


def test_dense_up_gate_vs_dequantized_and_split(orc):
    """Dense up_gate against dequantize-then-fp64 numpy, and equal bit for bit
    to the split form (oracle products of the two halves, then silu * up)."""
    m, n_embd, n_ff = 3, 768, 80
    w_f = synth.normal_f32((2 * n_ff, n_embd), 0.02, "test", "dense-ug", "w")
    x_f = synth.normal_f32((m, n_embd), 1.0, "test", "dense-ug", "x")
    w = orc.quantize_rows(w_f)
    x = orc.quantize_rows(x_f)
    h = orc.up_gate_swiglu(w, x, n_embd, n_ff)
    W = dequant(w, n_embd)
    X = dequant(x, n_embd)
    g = X @ W[:n_ff].T
    up = X @ W[n_ff:].T
    np.testing.assert_allclose(h, _silu(g) * up, rtol=1e-11, atol=1e-14)
    gg = orc.matmul(w, x, 2 * n_ff, n_embd, m)
    split = orc.fused_mul_silu(gg[:, :n_ff].copy(), gg[:, n_ff:].copy()).reshape(m, n_ff)
    assert np.array_equal(h, split)
