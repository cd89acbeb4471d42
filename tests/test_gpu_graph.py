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
