"""The attention forward and the ring merge captured into a HIP graph: the entry points only
enqueue kernels on the caller's stream (no allocation, no synchronization, no memset), so
a captured sequence replays to the eager result.  Each replay is preceded by eager work
and a synchronization, and every replay is compared bit for bit with the eager run."""
import math

import numpy as np
import pytest
import torch

import synthetic
from gpu_utils import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def test_graph_capture_varlen_forward_and_merge(mi):
    lengths = [300, 0, 1, 129, 64, 517, 2]
    w = synthetic.varlen_inputs(401, Nq=8, Nkv=2, D=128, dtype="bf16", lengths_q=lengths)
    T = w["Tq"]
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    cu = torch.from_numpy(w["cu_q"]).to("cuda:0")
    sc = 1 / math.sqrt(128)
    # two partial results (a causal forward and a banded forward over the same keys) and
    # their merge: three launches whose inputs are written inside the graph
    out1, out2, out = (torch.empty_like(q) for _ in range(3))
    m1, l1, m2, l2, mo, lo = (torch.empty((8, T), device="cuda:0") for _ in range(6))
    side = torch.cuda.Stream()

    def work():
        mi.attn_fwd_varlen(q, k, v, out1, m1, l1, cu, cu, w["B"], T, T, 517, 517, 8, 2, 128,
                           "bf16", sc, "causal", stream=torch.cuda.current_stream())
        mi.attn_fwd_varlen(q, k, v, out2, m2, l2, cu, cu, w["B"], T, T, 517, 517, 8, 2, 128,
                           "bf16", sc, "band", 40, 0, stream=torch.cuda.current_stream())
        # TND merge: one "batch" of T positions with N = 8 heads (stats [N, T])
        mi.attn_lse_merge(out1, m1, l1, out2, m2, l2, out, mo, lo, 1, 8, T, 128, "bf16", "BSND",
                          stream=torch.cuda.current_stream())

    with torch.cuda.stream(side):
        work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out1, m1, l1, out, mo, lo)]

    g = torch.cuda.CUDAGraph()
    for t in (out1, out2, out, m1, l1, m2, l2, mo, lo):
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        work()
    for rep in range(3):
        # eager work between the replays: clobber every output, then synchronize
        for t in (out1, out2, out):
            t.fill_(float("nan"))
        for t in (m1, l1, m2, l2, mo, lo):
            t.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out1, m1, l1, out, mo, lo), eager):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), rep
    assert np.isfinite(out.float().cpu().numpy()).all()


def test_graph_capture_general_kernel(mi):
    """The head-dim-general kernel (fp32 at D 128, and bf16 at D 200 with a smaller V head
    dim) captured into a graph: every replay equals the eager run bit for bit."""
    lengths = [150, 0, 1, 65, 33]
    wf = synthetic.varlen_inputs(402, Nq=4, Nkv=2, D=128, dtype="f32", lengths_q=lengths)
    wb = synthetic.varlen_inputs(403, Nq=4, Nkv=2, D=200, dtype="bf16", lengths_q=lengths)
    T = wf["Tq"]
    qf, kf, vf = (dev(wf[x], "f32") for x in ("q", "k", "v"))
    qb, kb, vb = (dev(wb[x], "bf16") for x in ("q", "k", "v"))
    vb = vb[..., :120].contiguous()
    cu = torch.from_numpy(wf["cu_q"]).to("cuda:0")
    of, ob = torch.empty_like(qf), torch.empty((T, 4, 120), dtype=torch.bfloat16, device="cuda:0")
    mf, lf, mb, lb = (torch.empty((4, T), device="cuda:0") for _ in range(4))
    side = torch.cuda.Stream()

    def work():
        s = torch.cuda.current_stream()
        mi.attn_fwd_varlen(qf, kf, vf, of, mf, lf, cu, cu, wf["B"], T, T, 150, 150, 4, 2, 128,
                           "f32", 1 / math.sqrt(128), "causal", stream=s)
        mi.attn_fwd_varlen_ext(qb, kb, vb, ob, mb, lb, cu, cu, wb["B"], T, T, 150, 150, 4, 2, 200,
                               120, "bf16", 1 / math.sqrt(200), "band", 30, 5, None, None, stream=s)

    with torch.cuda.stream(side):
        work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (of, mf, lf, ob, mb, lb)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        work()
    for rep in range(3):
        for t in (of, ob):
            t.fill_(float("nan"))
        for t in (mf, lf, mb, lb):
            t.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((of, mf, lf, ob, mb, lb), eager):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), rep
    assert np.isfinite(of.cpu().numpy()).all()
