"""Independent numpy readers used by the tests to check the oracle and the GPU
path: they parse 34-byte Q8_0 blocks with numpy's own float16 and compute in
fp64 with numpy's matmul.  No oracle code is used here."""
import numpy as np

BLOCK_BYTES = 34


def parse(q, nb):
    q = np.ascontiguousarray(q, dtype=np.uint8).reshape(-1, nb, BLOCK_BYTES)
    d = q[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    c = q[..., 2:].view(np.int8).astype(np.int64)
    return d, c


def dequant(q, k):
    """Q8_0 rows -> fp64 [rows][k] (exact: fp16 * int8 fits fp64)."""
    nb = k // 32
    d, c = parse(q, nb)
    return (d[..., None] * c).reshape(-1, k)


def blocksums(w, x, n, k, m):
    nb = k // 32
    _, cw = parse(w, nb)
    _, cx = parse(x, nb)
    return np.einsum("nbj,mbj->mnb", cw.reshape(n, nb, 32), cx.reshape(m, nb, 32))


def matmul(w, x, n, k, m):
    return dequant(x, k).reshape(m, k) @ dequant(w, k).reshape(n, k).T


def rel_l2_rows(got, ref):
    """per-row ||got - ref|| / ||ref|| in fp64 (rows = leading index)."""
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)
