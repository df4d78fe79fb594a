"""Seeded synthetic inputs for the Q8_0 decode path.

This module is shared by the tests, the benchmark and the oracle's callers.  It
only draws random numbers: it holds none of the method's arithmetic (no
quantization, no dot products).  Everything is deterministic in the key.

Streams: every tensor gets its own generator, keyed by a tuple of integers or
strings (base seed, workload, layer, tensor name, step ...).  Strings are mapped
to integers with CRC-32 so the key is stable across processes.

CPU (numpy) generators: PCG64 seeded through numpy's SeedSequence.  Normals are
drawn in fp64, scaled by sigma in fp64, then rounded once to fp32.

GPU generators (for the large benchmark inputs): torch's Philox generator on
the device, seeded from the same key; these are not bit-identical to the numpy
streams, and nothing compares them with the numpy streams.
"""
import zlib

import numpy as np

BASE_SEED = 0


def _key_ints(key):
    out = []
    for k in key:
        if isinstance(k, str):
            out.append(zlib.crc32(k.encode("utf-8")))
        else:
            out.append(int(k) & 0xFFFFFFFF)
    return out


def rng(*key):
    """numpy Generator for a key."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(_key_ints(key))))


def normal_f32(shape, sigma, *key):
    """N(0, sigma^2) values as fp32 (drawn in fp64, scaled, rounded once)."""
    g = rng(*key)
    return (g.standard_normal(size=shape, dtype=np.float64) * float(sigma)).astype(np.float32)


def expert_ids(n_tok, n_used, n_expert, *key):
    """int32 [n_tok][n_used]: n_used distinct experts per token, uniform."""
    g = rng(*key)
    ids = np.empty((n_tok, n_used), dtype=np.int32)
    for t in range(n_tok):
        ids[t] = g.choice(n_expert, size=n_used, replace=False)
    return ids


def combine_weights(n_tok, n_used, *key):
    """fp32 [n_tok][n_used]: softmax over each token's N(0,1) logits (fp64)."""
    g = rng(*key)
    z = g.standard_normal(size=(n_tok, n_used), dtype=np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def key_seed(*key):
    """A 63-bit integer seed derived from a key (for torch generators)."""
    ss = np.random.SeedSequence(_key_ints(key))
    return int(ss.generate_state(2, dtype=np.uint32)[0]) << 31 | int(
        ss.generate_state(2, dtype=np.uint32)[1] >> 1)


def normal_f32_torch(shape, sigma, device, *key, chunk=1 << 26):
    """N(0, sigma^2) fp32 tensor drawn on `device` with torch's generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(key_seed(*key))
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e].normal_(mean=0.0, std=float(sigma), generator=gen)
    return out


# K-quant super-blocks (256 values): random bytes everywhere except the two
# binary16 super-block scales, which get positive values of the size that
# N(0, 0.02) weights would give (d ~ 0.02/40 for the 6-bit scales, dmin ~
# 0.02/20 for the mins).  Byte counts per super-block: 144 (Q4_K), 176 (Q5_K).
KQ_BYTES = {4: 144, 5: 176}


def kq_blocks(t, n, k, *key):
    """uint8 [n][k/256 * bytes] random super-blocks of type t (4 or 5)."""
    g = rng(*key)
    w = g.integers(0, 256, size=(n, k // 256, KQ_BYTES[t]), dtype=np.uint8)
    d = (g.uniform(0.5, 1.5, size=(n, k // 256)) * (0.02 / 40)).astype(np.float16).view(np.uint16)
    dm = (g.uniform(0.5, 1.5, size=(n, k // 256)) * (0.02 / 20)).astype(np.float16).view(np.uint16)
    w[..., 0], w[..., 1] = d & 0xFF, d >> 8
    w[..., 2], w[..., 3] = dm & 0xFF, dm >> 8
    return w.reshape(n, -1)


def kq_blocks_torch(t, n, k, device, *key):
    """The same kind of super-blocks drawn on `device` with torch's generator
    (not bit-identical to kq_blocks)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(key_seed(*key))
    nb = KQ_BYTES[t]
    w = torch.randint(0, 256, (n, k // 256, nb), dtype=torch.uint8, device=device, generator=gen)
    u = torch.empty((n, k // 256, 2), dtype=torch.float32, device=device).uniform_(0.5, 1.5,
                                                                                 generator=gen)
    u[..., 0] *= 0.02 / 40
    u[..., 1] *= 0.02 / 20
    w[..., 0:4] = u.to(torch.float16).contiguous().view(torch.uint8).view(n, k // 256, 4)
    return w.view(n, -1)
