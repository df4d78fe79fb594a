"""GPU parity of q8_0_matmul_f32_step (a decode step in one launch: the first
workgroups quantize every activation row once into the workspace, the product
tiles wait for their rows).  Against the two-launch form (q8_0_quantize_rows +
q8_0_matmul_batched) bit for bit, against the oracle within 1e-5 per-row
relative L2; the workspace image must hold the quantizer's bytes, and every
counter must be back at zero after each call (so calls and graph replays can
reuse the workspace)."""
import numpy as np
import pytest

import synth

from gpu_cases import assert_rows_close, nan_like, to_gpu, weights_q8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def align256(v):
    return (v + 255) // 256 * 256


class Step:
    """Products of several widths over one fp32 activation buffer [m][k_total]
    (the decode-step layout: each product reads its own slice)."""

    def __init__(self, q, orc, specs, m, tag):
        import torch
        self.q, self.specs, self.m = q, specs, m
        self.k_total = sum(k * b for _, k, b in specs)
        self.n_out = sum(n * b for n, _, b in specs)
        self.w_host, self.w = [], []
        for i, (n, k, b) in enumerate(specs):
            w = weights_q8(orc, b * n, k, tag, "w", i)
            self.w_host.append(w)
            self.w.append(to_gpu(w))
        self.x = torch.empty((m, self.k_total), dtype=torch.float32, device="cuda")
        self.y = nan_like((m, self.n_out))
        self.descs = []
        xoff = yoff = 0
        for (n, k, b), w in zip(specs, self.w):
            nb = k // 32
            self.descs.append(q.make_f32_desc(
                w, (self.x, xoff), (self.y, yoff), n, k, m=m, batch=b, w_batch_stride=n * nb,
                x_row_stride=self.k_total, x_batch_stride=k, y_row_stride=self.n_out,
                y_batch_stride=n))
            xoff += b * k
            yoff += b * n
        self.ws = q.q8_0_matmul_f32_step_workspace(self.descs, "cuda")
        self.img0 = 256
        self.img_end = 256 + sum(align256(b * m * (k // 32) * 34) for _, k, b in specs)

    def run(self):
        self.q.q8_0_matmul_f32_step(self.descs, self.ws)

    def two_launch(self):
        """The same products through q8_0_quantize_rows + q8_0_matmul_batched."""
        import torch
        q = self.q
        xq = q.q8_0_quantize_rows(self.x)
        y2 = nan_like((self.m, self.n_out))
        nb_total = self.k_total // 32
        descs, xoff, yoff = [], 0, 0
        for (n, k, b), w in zip(self.specs, self.w):
            nb = k // 32
            descs.append(q.make_desc(w, (xq, xoff // 32), (y2, yoff), n, k, m=self.m, batch=b,
                                     w_batch_stride=n * nb, x_row_stride=nb_total,
                                     x_batch_stride=nb, y_row_stride=self.n_out,
                                     y_batch_stride=n))
            xoff += b * k
            yoff += b * n
        q.q8_0_matmul_batched(descs, y2)
        torch.cuda.synchronize()
        return xq, y2

    def check_workspace(self, xq):
        """Error word zero, counters and flags zero, image = the quantizer's
        bytes."""
        ws = self.ws.cpu().numpy()
        assert ws[:4].view(np.int32)[0] == 0
        assert not ws[self.img_end:].any()
        xq = xq.cpu().numpy()
        off = self.img0
        xoff = 0
        for n, k, b in self.specs:
            nb = k // 32
            size = b * self.m * nb * 34
            img = ws[off:off + size].reshape(b, self.m, nb * 34)
            for e in range(b):
                for r in range(self.m):
                    expect = xq[r, (xoff + e * nb) * 34:(xoff + (e + 1) * nb) * 34]
                    assert np.array_equal(img[e, r], expect), (n, k, e, r)
            off += align256(size)
            xoff += b * nb


SPECS = [(96, 768, 5), (160, 2048, 2), (50, 256, 1), (700, 768, 1), (64, 4096, 1), (3, 8192, 2)]


@pytest.mark.parametrize("m", [1, 2])
def test_step_matches_two_launch_and_oracle(q, orc, m):
    """Several widths (ragged last tiles, k from 256 to 8192, one-row and
    three-row products): the one-launch step equals the two-launch form bit
    for bit and the oracle within tolerance; the workspace holds the
    quantizer's bytes and its counters are back at zero."""
    import torch
    st = Step(q, orc, SPECS, m, f"step-{m}")
    xf = synth.normal_f32((m, st.k_total), 1.0, "step-x", m)
    st.x.copy_(torch.from_numpy(xf))
    st.run()
    torch.cuda.synchronize()
    xq, y2 = st.two_launch()
    assert torch.equal(st.y.view(torch.int32), y2.view(torch.int32))
    st.check_workspace(xq)
    xq_ref = orc.quantize_rows(xf)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    yy = st.y.cpu().numpy()
    xoff = yoff = 0
    for (n, k, b), w in zip(SPECS, st.w_host):
        nb = k // 32
        for e in range(b):
            xe = np.ascontiguousarray(xq_ref[:, (xoff + e * nb) * 34:(xoff + (e + 1) * nb) * 34])
            ref = orc.matmul(w[e * n:(e + 1) * n], xe, n, k, m)
            assert_rows_close(yy[:, yoff + e * n:yoff + (e + 1) * n], ref)
        xoff += b * nb
        yoff += b * n


def test_step_reuses_workspace(q, orc):
    """Consecutive calls with new activations on one workspace (no clearing in
    between): every call equals the two-launch form, so no call reads rows
    left by the previous one."""
    import torch
    st = Step(q, orc, SPECS[:4], 1, "step-reuse")
    for rep in range(4):
        st.x.copy_(torch.from_numpy(synth.normal_f32((1, st.k_total), 1.0, "step-reuse-x", rep)))
        st.y.fill_(float("nan"))
        st.run()
        torch.cuda.synchronize()
        xq, y2 = st.two_launch()
        assert torch.equal(st.y.view(torch.int32), y2.view(torch.int32)), rep
        st.check_workspace(xq)


def test_step_graph_replays(q, orc):
    """The step captured in a HIP graph and replayed with new activations copied
    in between (eager work and synchronizations between replays): every replay
    equals the eager two-launch result for its input."""
    import torch
    st = Step(q, orc, [(768, 768, 6), (2048, 768, 2), (768, 2048, 3)], 1, "step-graph")
    st.x.copy_(torch.from_numpy(synth.normal_f32((1, st.k_total), 1.0, "step-graph-x", -1)))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    for rep in range(4):
        st.x.copy_(torch.from_numpy(synth.normal_f32((1, st.k_total), 1.0, "step-graph-x", rep)))
        st.y.fill_(float("nan"))
        junk = torch.randn(1000, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        xq, y2 = st.two_launch()
        assert torch.equal(st.y.view(torch.int32), y2.view(torch.int32)), rep
        st.check_workspace(xq)
        del junk


def test_step_llama_decode_shapes(q, orc):
    """The full Llama-2-110M-shaped decode step (85 products: 48 x 768x768,
    24 x 2048x768, 12 x 768x2048, the 32000x768 classifier) in one launch:
    bitwise equal to the two-launch form; sampled outputs of every stack
    against the oracle."""
    import torch
    specs = [(768, 768, 48), (2048, 768, 24), (768, 2048, 12), (32000, 768, 1)]
    st = Step(q, orc, specs, 1, "step-llama")
    xf = synth.normal_f32((1, st.k_total), 1.0, "step-llama-x")
    st.x.copy_(torch.from_numpy(xf))
    st.run()
    torch.cuda.synchronize()
    xq, y2 = st.two_launch()
    assert torch.equal(st.y.view(torch.int32), y2.view(torch.int32))
    st.check_workspace(xq)
    xq_ref = orc.quantize_rows(xf)
    yy = st.y.cpu().numpy()
    rng = np.random.default_rng(7)
    xoff = yoff = 0
    for (n, k, b), w in zip(specs, st.w_host):
        nb = k // 32
        for e in sorted(set([0, b - 1, int(rng.integers(b))])):
            rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 30)]))
            xe = np.ascontiguousarray(xq_ref[:, (xoff + e * nb) * 34:(xoff + (e + 1) * nb) * 34])
            wr = np.ascontiguousarray(w[e * n:(e + 1) * n][rows])
            ref = orc.matmul(wr, xe, len(rows), k, 1)
            assert_rows_close(yy[:, yoff + e * n + rows], ref)
        xoff += b * nb
        yoff += b * n
