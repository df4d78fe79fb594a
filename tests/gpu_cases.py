"""Shared helpers of the GPU parity tests (inputs from synth, quantized by the
oracle on the CPU; comparison in fp64 per output row)."""
import numpy as np

import synth
from qref import rel_l2_rows

TOL = 1e-5      # max relative error of each output row, in L2


def weights_q8(orc, n, k, *key, sigma=0.02):
    wf = synth.normal_f32((n, k), sigma, *key)
    return orc.quantize_rows(wf)


def acts_q8(orc, m, k, *key):
    xf = synth.normal_f32((m, k), 1.0, *key)
    return orc.quantize_rows(xf)


def to_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nan_like(shape):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def assert_rows_close(got, ref, tol=TOL):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), "non-finite output (an element was not written?)"
    err = rel_l2_rows(got, ref)
    assert err.max() <= tol, f"max per-row relative L2 error {err.max():.3e} > {tol}"
    return err
