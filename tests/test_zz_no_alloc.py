"""moe_r8_ffn_batched_noalloc (the expert FFN over R8 weights with the
library's own per-device workspace) against moe_r8_ffn_batched on the same
inputs: h and out bit for bit, on two calls in a row, the second smaller
(fewer layers and tokens) with an out-of-range id, so that it must not see
anything the first call left in the shared array."""
import numpy as np
import pytest

import synth
from gpu_cases import to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _blocks(rows, k, *key):
    """Random Q8_0 rows: codes uniform in [-127, 127], binary16 scales of the
    size N(0, 0.02) weights give (amax/127 of 32 normals: about 4e-4)."""
    g = synth.rng(*key)
    b = g.integers(-127, 128, size=(rows, k // 32, 34), dtype=np.int64).astype(np.int8)
    b = b.view(np.uint8)
    d = (g.uniform(0.5, 1.5, size=(rows, k // 32)) * 4e-4).astype(np.float16).view(np.uint16)
    b[..., 0], b[..., 1] = d & 0xFF, d >> 8
    return np.ascontiguousarray(b.reshape(rows, -1))


def _layers(q, n_layers, n_tok, n_embd, n_ff, n_expert, n_used, tag, bad=None):
    import torch
    out = []
    for i in range(n_layers):
        key = (tag, str(i))
        wug = _blocks(n_expert * 2 * n_ff, n_embd, *key, "ug")
        wd = _blocks(n_expert * n_embd, n_ff, *key, "dn")
        ids = synth.expert_ids(n_tok, n_used, n_expert, *key, "ids")
        if bad is not None and i == 0:
            ids[bad] = n_expert
        wug_g, wd_g = to_gpu(wug), to_gpu(wd)
        out.append(dict(
            w_up_gate_r8=q.q8_0_repack_r8(wug_g, n_expert * 2 * n_ff, n_embd),
            w_down_r8=q.q8_0_repack_r8(wd_g, n_expert * n_embd, n_ff),
            x=to_gpu(synth.normal_f32((n_tok, n_embd), 1.0, *key, "x")),
            ids=to_gpu(np.ascontiguousarray(ids, dtype=np.int32)),
            cw=to_gpu(synth.combine_weights(n_tok, n_used, *key, "cw")),
            h=torch.full((n_tok, n_used, n_ff), float("nan"), device="cuda"),
            out=torch.full((n_tok, n_embd), float("nan"), device="cuda"),
            ws=q.moe_r8_workspace(n_tok, n_embd, n_ff, n_expert, n_used, "cuda")))
    return out


def _same_bits(a, b):
    import torch
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _run_and_compare(q, layers, n_embd, n_ff, n_expert):
    import torch
    ref = [dict(d, h=torch.full_like(d["h"], 7.0), out=torch.full_like(d["out"], 7.0))
           for d in layers]
    q.moe_r8_ffn_batched(ref, n_embd, n_ff, n_expert)
    q.moe_r8_ffn_batched_noalloc(layers, n_embd, n_ff, n_expert)
    torch.cuda.synchronize()
    for d, r in zip(layers, ref):
        assert _same_bits(d["h"], r["h"])
        assert _same_bits(d["out"], r["out"])
    return ref


def test_noalloc_matches_workspace_entry_point(q):
    import torch
    n_embd, n_ff, n_expert, n_used = 1024, 256, 16, 8
    print("case: 3 layers x 8 tokens, then 1 layer x 2 tokens with an out-of-range id", flush=True)
    big = _layers(q, 3, 8, n_embd, n_ff, n_expert, n_used, "noalloc-big")
    ref = _run_and_compare(q, big, n_embd, n_ff, n_expert)
    for r in ref:
        assert q.moe_error_word(r["ws"]) == 0
        assert bool(torch.isfinite(r["out"]).all())
    small = _layers(q, 1, 2, n_embd, n_ff, n_expert, n_used, "noalloc-small", bad=(1, 3))
    ref = _run_and_compare(q, small, n_embd, n_ff, n_expert)
    assert q.moe_error_word(ref[0]["ws"]) == 1
    d = small[0]
    assert bool(torch.isnan(d["h"][1, 3]).all()) and bool(torch.isnan(d["out"][1]).all())
    assert bool(torch.isfinite(d["out"][0]).all())


def test_noalloc_one_token_full_layer_shape(q):
    """The decode shape of the 30-layer MoE workload (n_embd 2048, n_ff 768,
    top-8) at one token, two layers, then the same call again with one layer."""
    n_embd, n_ff, n_expert, n_used = 2048, 768, 16, 8
    print("case: 2 layers x 1 token (2048 / 768), then 1 layer", flush=True)
    layers = _layers(q, 2, 1, n_embd, n_ff, n_expert, n_used, "noalloc-c4")
    _run_and_compare(q, layers, n_embd, n_ff, n_expert)
    _run_and_compare(q, layers[1:], n_embd, n_ff, n_expert)


def test_noalloc_rejects_beyond_its_array(q):
    """More layers than the library's 48 MiB array holds: Q8_E_WORKSPACE, and
    more than 16 tokens (the prefill path): Q8_E_UNSUPPORTED."""
    from moe_expert_ffn_q8_amd import MoeR8FfnDesc
    lib = q.raw
    A = 1 << 20
    n_tok, n_embd, n_ff, n_expert, n_used = 16, 2048, 2048, 64, 16
    per = (q.raw.moe_r8_workspace_bytes(n_tok, n_embd, n_ff, n_expert, n_used) + 255) // 256 * 256
    n_fit = (48 << 20) // per
    descs = (MoeR8FfnDesc * (n_fit + 1))(*[MoeR8FfnDesc(A, A, A, A, A, A, A, None, 0)
                                           for _ in range(n_fit + 1)])
    assert lib.moe_r8_ffn_batched_noalloc(descs, n_fit + 1, n_tok, n_embd, n_ff, n_expert, n_used,
                                          None) == -5
    assert lib.moe_r8_ffn_batched_noalloc(descs, 1, 17, 2048, 768, 128, 8, None) == -4
