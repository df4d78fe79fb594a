"""The expert FFN checked at its stage boundaries with the validation exports
of the kernels the product calls run (q8v_moe_up_gate, q8v_moe_hq,
q8v_moe_r8_ffn):
  B  the routing the kernels served and every gate / up block sum, exact;
     h within 1e-5 per (t,u) row against the oracle's h from the same
     quantized token rows;
  C  the quantized h rows the down products used, byte for byte against the
     oracle's quantization of the GPU's h; every down block sum exact; out
     within 1e-5 per token against the oracle fed the GPU's h;
  D  (full layer shapes) the oracle's whole FFN from the fp32 token rows alone
     against the GPU's out: codes of q(h) that differ between the two h must
     each sit at a rounding boundary, and every token without such a code is
     within 1e-5.
The validation calls' h and out are bitwise those of the product calls."""
import functools

import numpy as np
import pytest

import synth
from gpu_cases import TOL, assert_rows_close, to_gpu
from qref import rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


@functools.lru_cache(maxsize=2)
def _weights(n_embd, n_ff, n_expert, tag):
    import oracle
    w_ug = oracle.quantize_rows(synth.normal_f32((n_expert * 2 * n_ff, n_embd), 0.02, tag, "ug"))
    w_d = oracle.quantize_rows(synth.normal_f32((n_expert * n_embd, n_ff), 0.02, tag, "down"))
    return w_ug, w_d


def _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, tag, wtag=None):
    w_ug, w_d = _weights(n_embd, n_ff, n_expert, wtag or tag)
    xf = synth.normal_f32((n_tok, n_embd), 1.0, tag, "x")
    ids = np.ascontiguousarray(synth.expert_ids(n_tok, n_used, n_expert, tag, "ids"), np.int32)
    cw = synth.combine_weights(n_tok, n_used, tag, "cw")
    return dict(w_ug=w_ug, w_d=w_d, xf=xf, xq=orc.quantize_rows(xf), ids=ids, cw=cw)


def _expert(w, e, rows, nb):
    return w.reshape(-1, nb * 34)[e * rows:(e + 1) * rows]


def _check_ug_sums(orc, c, sums, n_embd, n_ff, slots):
    nbe = n_embd // 32
    n_used = c["ids"].shape[1]
    for s in slots:
        t, u = divmod(int(s), n_used)
        e = int(c["ids"][t, u])
        ref = orc.matmul_blocksums(_expert(c["w_ug"], e, 2 * n_ff, nbe), c["xq"][t:t + 1],
                                   2 * n_ff, n_embd, 1)[0]
        assert np.array_equal(sums[s], ref), f"gate/up block sums of slot {s}"


def _check_dn_sums(orc, c, sums, hq_ref, n_embd, n_ff, slots):
    nbf = n_ff // 32
    n_used = c["ids"].shape[1]
    for s in slots:
        t, u = divmod(int(s), n_used)
        e = int(c["ids"][t, u])
        ref = orc.matmul_blocksums(_expert(c["w_d"], e, n_embd, nbf), hq_ref[s:s + 1],
                                   n_embd, n_ff, 1)[0]
        assert np.array_equal(sums[s], ref), f"down block sums of slot {s}"


def _flips_explained(orc, h_gpu, h_ref32, n_ff):
    """Codes of q(h) that differ between the GPU's h and the oracle's own h:
    each must be at a rounding boundary (the oracle's h/d within 1e-4 of
    n + 1/2) or in a block whose scale moved.  Returns (flipped codes, the
    (t*n_used+u) rows that hold them)."""
    qa, qb = orc.quantize_rows(h_gpu.reshape(-1, n_ff)), orc.quantize_rows(h_ref32.reshape(-1, n_ff))
    da, ca = orc.split_blocks(qa)
    db, cb = orc.split_blocks(qb)
    bb = h_ref32.reshape(qa.shape[0], -1, 32).astype(np.float64)
    flips, rows = 0, set()
    for r, blk in zip(*np.nonzero((ca != cb).any(axis=2) | (da != db))):
        diff = ca[r, blk].astype(int) != cb[r, blk].astype(int)
        d32 = np.float32(np.abs(h_ref32.reshape(qa.shape[0], -1, 32)[r, blk]).max()) / np.float32(127)
        ratio = bb[r, blk] / np.float64(d32)
        near_half = np.abs(np.abs(ratio - np.trunc(ratio)) - 0.5) < 1e-4
        assert da[r, blk] != db[r, blk] or np.all(near_half[diff]), (r, blk, ratio[diff])
        flips += int(diff.sum())
        rows.add(int(r))
    return flips, rows


def _stages(q, orc, c, n_embd, n_ff, n_expert, sample=None, stage_d=False):
    import torch
    n_tok, n_used = c["ids"].shape
    slots = np.arange(n_tok * n_used) if sample is None else sample
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    wug, wd, xg, idg, cwg = (to_gpu(c["w_ug"]), to_gpu(c["w_d"]), to_gpu(c["xf"]),
                             to_gpu(c["ids"]), to_gpu(c["cw"]))
    # stage B
    h, sums, counts, offsets, pairs = q.q8v_moe_up_gate(wug, xg, idg, n_embd, n_ff, n_expert, ws)
    assert q.moe_error_word(ws) == 0
    rc, ro, rp = orc.moe_route(c["ids"], n_expert)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(pairs.cpu().numpy(), rp)
    _check_ug_sums(orc, c, sums.cpu().numpy(), n_embd, n_ff, slots)
    del sums
    h_gpu = h.cpu().numpy()
    h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"], c["ids"], n_embd, n_ff, n_expert)
    assert_rows_close(h_gpu.reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    h1 = q.moe_up_gate_swiglu(wug, xg, idg, n_embd, n_ff, n_expert, ws)
    assert torch.equal(h1.view(torch.int32), h.view(torch.int32))
    # stage C: the oracle is fed the GPU's h
    out, hq, dsums = q.q8v_moe_hq(wd, h, idg, cwg, n_ff, n_embd, n_expert, ws)
    assert q.moe_error_word(ws) == 0
    hq_ref = orc.quantize_rows(h_gpu.reshape(-1, n_ff))
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    _check_dn_sums(orc, c, dsums.cpu().numpy(), hq_ref, n_embd, n_ff, slots)
    del dsums
    out_gpu = out.cpu().numpy()
    assert_rows_close(out_gpu, orc.moe_down_combine(c["w_d"], h_gpu, c["ids"], c["cw"], n_ff,
                                                    n_embd, n_expert))
    o1 = q.moe_down_combine(wd, h, idg, cwg, n_ff, n_embd, n_expert, ws)
    assert torch.equal(o1.view(torch.int32), out.view(torch.int32))
    if stage_d:
        h32 = h_ref.astype(np.float32)
        out_ind = orc.moe_down_combine(c["w_d"], h32, c["ids"], c["cw"], n_ff, n_embd, n_expert)
        flips, rows = _flips_explained(orc, h_gpu, h32, n_ff)
        flipped_tok = {r // n_used for r in rows}
        err = rel_l2_rows(out_gpu, out_ind)
        clean = [t for t in range(n_tok) if t not in flipped_tok]
        assert err[clean].max(initial=0.0) <= TOL
        print(f"stage D: {n_tok} tokens, {flips} flipped h codes in {len(rows)} h rows "
              f"({len(flipped_tok)} tokens), max row error {err.max():.2e} "
              f"(tokens without flips {err[clean].max(initial=0.0):.2e})", flush=True)


@pytest.mark.parametrize("n_tok", [1, 16])
def test_stages_full_layer_decode(q, orc, n_tok):
    """The 30-layer MoE workload's layer shape (n_embd 2048, n_ff 768, 128
    experts, top-8) at 1 and 16 tokens: every slot's sums, stage D."""
    print(f"case: stages, full layer, {n_tok} tokens", flush=True)
    c = _case(orc, n_tok, 2048, 768, 128, 8, f"stg-{n_tok}", wtag="stg-w")
    _stages(q, orc, c, 2048, 768, 128, stage_d=True)


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used", [
    (3, 512, 256, 8, 8), (2, 512, 512, 8, 8), (9, 768, 256, 64, 4), (40, 256, 256, 4, 2)])
def test_stages_decode_shapes(q, orc, n_tok, n_embd, n_ff, n_expert, n_used):
    """The row-major down kernel (24 and 16 slots... of up to 16: 3 tokens x 8
    takes the expert-major down kernel, 2 x 8 the row-major one), chunks of 4
    token rows (9 tokens), and 40 tokens over 4 experts (the grouped path,
    several tiles per expert)."""
    print(f"case: stages {n_tok} {n_embd} {n_ff} {n_expert} {n_used}", flush=True)
    c = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, f"stg-s-{n_tok}-{n_embd}-{n_ff}")
    _stages(q, orc, c, n_embd, n_ff, n_expert)


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used", [
    (40, 512, 256, 16, 4), (200, 256, 128, 8, 8), (17, 1024, 384, 32, 2),
    (700, 256, 128, 16, 8), (1100, 128, 128, 64, 8)])
def test_stages_prefill(q, orc, n_tok, n_embd, n_ff, n_expert, n_used):
    """More than 16 tokens: the grouped matrix-core path; its routing is the
    ascending (t,u) order within each expert (5600 and 8800 slots: the
    routing reads the ids in 2 and 3 passes of 4096)."""
    print(f"case: stages prefill {n_tok} {n_embd} {n_ff} {n_expert} {n_used}", flush=True)
    c = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, f"stg-p-{n_tok}-{n_embd}")
    _stages(q, orc, c, n_embd, n_ff, n_expert)


def test_stages_prefill_full_layer(q, orc):
    """512 tokens of the full layer shape (4096 slots, all 128 experts): the
    routing exact, the sums of 24 sampled slots, h and out sampled."""
    print("case: stages prefill, full layer, 512 tokens", flush=True)
    c = _case(orc, 512, 2048, 768, 128, 8, "stg-p512", wtag="stg-w")
    sample = np.unique(np.concatenate([[0, 4095], np.random.default_rng(3).integers(0, 4096, 22)]))
    import torch
    n_embd, n_ff, n_expert, n_used = 2048, 768, 128, 8
    ws = q.moe_workspace(512, n_embd, n_ff, n_expert, n_used, "cuda")
    wug, xg, idg = to_gpu(c["w_ug"]), to_gpu(c["xf"]), to_gpu(c["ids"])
    h, sums, counts, offsets, pairs = q.q8v_moe_up_gate(wug, xg, idg, n_embd, n_ff, n_expert, ws)
    rc, ro, rp = orc.moe_route(c["ids"], n_expert)
    assert np.array_equal(counts.cpu().numpy(), rc) and np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(pairs.cpu().numpy(), rp)
    ss = sums.cpu().numpy()
    del sums
    _check_ug_sums(orc, c, ss, n_embd, n_ff, sample)
    h_gpu = h.cpu().numpy()
    toks = np.unique(sample // n_used)
    h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"][toks], c["ids"][toks], n_embd, n_ff, n_expert)
    assert_rows_close(h_gpu[toks].reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    out, hq, dsums = q.q8v_moe_hq(to_gpu(c["w_d"]), h, idg, to_gpu(c["cw"]), n_ff, n_embd,
                                  n_expert, ws)
    hq_ref = orc.quantize_rows(h_gpu.reshape(-1, n_ff))
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    _check_dn_sums(orc, c, dsums.cpu().numpy(), hq_ref, n_embd, n_ff, sample)
    assert_rows_close(out.cpu().numpy()[toks], orc.moe_down_combine(
        c["w_d"], h_gpu[toks], c["ids"][toks], c["cw"][toks], n_ff, n_embd, n_expert))


def test_stages_generic_kernels(q, orc):
    """Shapes on the generic kernels (n_embd/32 not a multiple of 8): sums and
    q(h) as everywhere; these kernels do not group slots by expert, so the
    routing output is refused."""
    n_tok, n_embd, n_ff, n_expert, n_used = 3, 256 + 32, 96, 6, 4
    c = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, "stg-gen")
    ws = q.moe_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")
    with pytest.raises(q.Q8Error):
        q.q8v_moe_up_gate(to_gpu(c["w_ug"]), to_gpu(c["xf"]), to_gpu(c["ids"]), n_embd, n_ff,
                          n_expert, ws)
    h, sums, _, _, _ = q.q8v_moe_up_gate(to_gpu(c["w_ug"]), to_gpu(c["xf"]), to_gpu(c["ids"]),
                                         n_embd, n_ff, n_expert, ws, route=False)
    _check_ug_sums(orc, c, sums.cpu().numpy(), n_embd, n_ff, range(n_tok * n_used))
    h_gpu = h.cpu().numpy()
    out, hq, dsums = q.q8v_moe_hq(to_gpu(c["w_d"]), h, to_gpu(c["ids"]), to_gpu(c["cw"]), n_ff,
                                  n_embd, n_expert, ws)
    hq_ref = orc.quantize_rows(h_gpu.reshape(-1, n_ff))
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    _check_dn_sums(orc, c, dsums.cpu().numpy(), hq_ref, n_embd, n_ff, range(n_tok * n_used))


def _r8_layer(q, c, n_embd, n_ff, n_expert):
    import torch
    n_tok, n_used = c["ids"].shape
    return dict(w_up_gate_r8=q.q8_0_repack_r8(to_gpu(c["w_ug"]), n_expert * 2 * n_ff, n_embd),
                w_down_r8=q.q8_0_repack_r8(to_gpu(c["w_d"]), n_expert * n_embd, n_ff),
                x=to_gpu(c["xf"]), ids=to_gpu(c["ids"]), cw=to_gpu(c["cw"]),
                h=torch.full((n_tok, n_used, n_ff), float("nan"), device="cuda"),
                out=torch.full((n_tok, n_embd), float("nan"), device="cuda"),
                ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda"))


@pytest.mark.parametrize("n_tok,n_embd,n_ff,n_expert,n_used,full", [
    (1, 2048, 768, 128, 8, True), (16, 2048, 768, 128, 8, True), (3, 768, 256, 32, 8, False),
    (40, 512, 256, 16, 4, False), (700, 256, 128, 16, 8, False)])
def test_stages_r8(q, orc, n_tok, n_embd, n_ff, n_expert, n_used, full):
    """The expert FFN over R8 expert weights (decode kernels up to 16 tokens,
    the matrix-core path above): sums of both products, q(h), the routing the
    kernels grouped slots by (2 tokens or more); h and out bitwise those of
    moe_r8_ffn_batched."""
    import torch
    print(f"case: stages r8 {n_tok} {n_embd} {n_ff} {n_expert} {n_used}", flush=True)
    c = _case(orc, n_tok, n_embd, n_ff, n_expert, n_used, f"stg-r8-{n_tok}-{n_embd}",
              wtag="stg-w" if full else None)
    d = _r8_layer(q, c, n_embd, n_ff, n_expert)
    grouped = n_tok > 1
    ug, dn, hq, counts, offsets, pairs = q.q8v_moe_r8_ffn(d, n_embd, n_ff, n_expert, route=grouped)
    assert q.moe_error_word(d["ws"]) == 0
    if grouped:
        rc, ro, rp = orc.moe_route(c["ids"], n_expert)
        assert np.array_equal(counts.cpu().numpy(), rc)
        assert np.array_equal(offsets.cpu().numpy(), ro)
        assert np.array_equal(pairs.cpu().numpy(), rp)
    else:
        with pytest.raises(q.Q8Error):
            q.q8v_moe_r8_ffn(d, n_embd, n_ff, n_expert, route=True)
    slots = range(n_tok * n_used)
    _check_ug_sums(orc, c, ug.cpu().numpy(), n_embd, n_ff, slots)
    h_gpu = d["h"].cpu().numpy()
    hq_ref = orc.quantize_rows(h_gpu.reshape(-1, n_ff))
    assert np.array_equal(hq.cpu().numpy(), hq_ref)
    _check_dn_sums(orc, c, dn.cpu().numpy(), hq_ref, n_embd, n_ff, slots)
    h_ref = orc.moe_up_gate_swiglu(c["w_ug"], c["xq"], c["ids"], n_embd, n_ff, n_expert)
    assert_rows_close(h_gpu.reshape(-1, n_ff), h_ref.reshape(-1, n_ff))
    assert_rows_close(d["out"].cpu().numpy(), orc.moe_down_combine(
        c["w_d"], h_gpu, c["ids"], c["cw"], n_ff, n_embd, n_expert))
    d2 = dict(d, h=torch.full_like(d["h"], 3.0), out=torch.full_like(d["out"], 3.0))
    q.moe_r8_ffn_batched([d2], n_embd, n_ff, n_expert)
    assert torch.equal(d2["h"].view(torch.int32), d["h"].view(torch.int32))
    assert torch.equal(d2["out"].view(torch.int32), d["out"].view(torch.int32))
