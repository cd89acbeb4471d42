"""GPU parity of attn_fwd / attn_fwd_varlen against the CPU fp64 oracle.

Both sides read the same seeded inputs (synthetic.py); the HIP results are compared
element by element with the oracle at the tolerances of tests/gpu_utils.py.  Sizes span
several 128-row / 64-key tiles with ragged tails; the full-size packed workload is
checked on whole sequences x sampled heads.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import (check_out, check_stats, dev, empty_like_storage, host_values,
                       nan_stats)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _run_dense(mi, w, scale, mask, pre=0, nxt=0):
    B, Nq, Nkv, Sq, Skv, D = (w[x] for x in ("B", "Nq", "Nkv", "Sq", "Skv", "D"))
    dt, lay = w["dtype"], w["layout"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    out = empty_like_storage(q.shape, dt)
    m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    mi.attn_fwd(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, dt, lay, scale, mask, pre, nxt)
    torch.cuda.synchronize()
    return host_values(out), host_values(m), host_values(l)


def _oracle_dense(w, scale, mask, pre=0, nxt=0):
    dt, lay = w["dtype"], w["layout"]
    q = synthetic.to_bnsd(synthetic.storage_values(w["q"], dt), lay, w["Nq"])
    k = synthetic.to_bnsd(synthetic.storage_values(w["k"], dt), lay, w["Nkv"])
    v = synthetic.to_bnsd(synthetic.storage_values(w["v"], dt), lay, w["Nkv"])
    return oracle.attn(q, k, v, scale, mask, pre, nxt)


def _compare_dense(mi, w, scale, mask, pre=0, nxt=0):
    go, gm, gl = _run_dense(mi, w, scale, mask, pre, nxt)
    wo, wm, wl = _oracle_dense(w, scale, mask, pre, nxt)
    go = synthetic.to_bnsd(go, w["layout"], w["Nq"])
    err = check_out(go, wo, w["dtype"])
    check_stats(gm, gl, wm, wl)
    return err


def test_dense_f32_b1n1s128d64(mi):
    w = synthetic.make("dense_f32_b1n1s128d64")
    _compare_dense(mi, w, 1 / math.sqrt(64), "none")


def test_dense_bf16_b8n8s128d64(mi):
    w = synthetic.make("dense_bf16_b8n8s128d64")
    _compare_dense(mi, w, 1 / math.sqrt(64), "none")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("layout", ["BNSD", "BSND", "BSH", "SBH"])
@pytest.mark.parametrize("mask,pre,nxt", [("none", 0, 0), ("causal", 0, 0), ("band", 70, 33),
                                          ("band", 1 << 62, -150)])
def test_dense_layouts_masks(mi, dtype, D, layout, mask, pre, nxt):
    # Sq = 300, Skv = 333: 3 query tiles (last ragged), 6 key tiles (last ragged); GQA 4/2
    w = synthetic.dense_inputs(11, 2, 4, 2, 300, 333, D, dtype, layout)
    _compare_dense(mi, w, 1 / math.sqrt(D), mask, pre, nxt)


@pytest.mark.parametrize("Nq,Nkv", [(8, 1), (6, 3), (5, 5)])
def test_dense_gqa_mqa(mi, Nq, Nkv):
    w = synthetic.dense_inputs(12, 1, Nq, Nkv, 257, 190, 128, "bf16", "BSND")
    _compare_dense(mi, w, 1 / math.sqrt(128), "causal")


@pytest.mark.parametrize("Sq,Skv", [(1, 1), (1, 700), (129, 1), (64, 64)])
def test_dense_edge_lengths(mi, Sq, Skv):
    w = synthetic.dense_inputs(13, 1, 2, 2, Sq, Skv, 64, "bf16", "BNSD")
    _compare_dense(mi, w, 0.125, "none")
    _compare_dense(mi, w, 0.125, "causal")


def _run_varlen(mi, w, scale, mask, pre=0, nxt=0):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    out = empty_like_storage(q.shape, dt)
    m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
    mi.attn_fwd_varlen(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"],
                       int(w["lengths_q"].max()), int(w["lengths_kv"].max()), w["Nq"], w["Nkv"],
                       w["D"], dt, scale, mask, pre, nxt)
    torch.cuda.synchronize()
    return host_values(out), host_values(m), host_values(l)


@pytest.mark.parametrize("mask,pre,nxt", [("causal", 0, 0), ("none", 0, 0), ("band", 200, 7)])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_varlen_small(mi, mask, pre, nxt, dtype):
    lengths = [300, 0, 1, 129, 64, 517, 2]   # zero-length, single-row and ragged sequences
    w = synthetic.varlen_inputs(21, Nq=8, Nkv=2, D=128, dtype=dtype, lengths_q=lengths)
    go, gm, gl = _run_varlen(mi, w, 1 / math.sqrt(128), mask, pre, nxt)
    q, k, v = (synthetic.storage_values(w[x], dtype) for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 1 / math.sqrt(128), mask, pre, nxt)
    check_out(go, wo, dtype)
    check_stats(gm, gl, wm, wl)


@pytest.mark.parametrize("D", [32, 96])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_varlen_other_head_dims(mi, D, dtype):
    lengths = [300, 0, 1, 129, 64, 517, 2]
    w = synthetic.varlen_inputs(25 + D, Nq=8, Nkv=2, D=D, dtype=dtype, lengths_q=lengths)
    go, gm, gl = _run_varlen(mi, w, 1 / math.sqrt(D), "causal")
    q, k, v = (synthetic.storage_values(w[x], dtype) for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 1 / math.sqrt(D), "causal")
    check_out(go, wo, dtype)
    check_stats(gm, gl, wm, wl)


def test_varlen_q_kv_lengths_differ(mi):
    w = synthetic.varlen_inputs(22, Nq=4, Nkv=4, D=64, dtype="bf16",
                                lengths_q=[100, 7, 260], lengths_kv=[50, 300, 260])
    go, gm, gl = _run_varlen(mi, w, 0.125, "causal")
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 0.125, "causal")
    check_out(go, wo, "bf16")
    check_stats(gm, gl, wm, wl)


@pytest.fixture(scope="module")
def metric_run(mi):
    """The full packed workload: 16 sequences (T = 33,064), Nq 32, Nkv 8, D 128, causal."""
    w = synthetic.make(synthetic.METRIC_WORKLOAD)
    go, gm, gl = _run_varlen(mi, w, 1 / math.sqrt(128), "causal")
    return w, go, gm, gl


def test_varlen_full_workload_every_element(metric_run):
    """The full packed workload, every output element and every statistic (16 sequences x
    32 heads: 1,058,048 rows) against one oracle run over all of it."""
    w, go, gm, gl = metric_run
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 1 / math.sqrt(128), "causal",
                                    threads=oracle.max_threads())
    err = check_out(go, wo, "bf16", "full workload")
    em, el = check_stats(gm, gl, wm, wl)
    print(f"full workload bf16: out {err:.3e}, softmax_max {em:.2e}, softmax_sum {el:.2e}")


def test_varlen_full_workload_f16_every_element(mi):
    """The full packed workload's shape and lengths (same seed) with fp16 storage, every
    element against the oracle."""
    w = synthetic.varlen_inputs(0, Nq=32, Nkv=8, D=128, dtype="f16", B=16)
    assert w["Tq"] == synthetic.make(synthetic.METRIC_WORKLOAD)["Tq"]
    go, gm, gl = _run_varlen(mi, w, 1 / math.sqrt(128), "causal")
    q, k, v = (synthetic.storage_values(w[x], "f16") for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 1 / math.sqrt(128), "causal",
                                    threads=oracle.max_threads())
    err = check_out(go, wo, "f16", "full workload f16")
    em, el = check_stats(gm, gl, wm, wl)
    print(f"full workload f16: out {err:.3e}, softmax_max {em:.2e}, softmax_sum {el:.2e}")


def test_varlen_full_workload_properties(metric_run):
    """Every output row of the full workload is finite with softmax_sum >= 1; row 0 of each
    sequence sees one key, so its output is V[0] and its softmax_sum is 1 up to the
    kernel's exponent of the max logit itself: exp2 of the fused multiply-add
    scale*log2(e)*s - round(scale*log2(e)*s), the rounding residue of one product (at most
    half an ulp of the scaled logit), which leaves the sum within 2^-22 of 1 rather than
    exactly 1."""
    w, go, gm, gl = metric_run
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gm)) and np.all(np.isfinite(gl))
    assert np.all(gl >= 1.0 - 1e-6)
    v = synthetic.storage_values(w["v"], "bf16")
    cu = np.concatenate([[0], w["cu_q"]])
    G = w["Nq"] // w["Nkv"]
    for b in range(w["B"]):
        r0 = int(cu[b])
        assert np.all(np.abs(gl[:, r0] - 1.0) <= 2.0 ** -22)
        for h in range(w["Nq"]):
            assert np.max(np.abs(go[r0, h] - v[r0, h // G])) <= 2 ** -8 * np.max(np.abs(v[r0, h // G]))


def test_varlen_deterministic(mi):
    w = synthetic.varlen_inputs(23, Nq=8, Nkv=2, D=128, dtype="bf16", lengths_q=[1000, 333, 77])
    a = _run_varlen(mi, w, 0.088, "causal")
    b = _run_varlen(mi, w, 0.088, "causal")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_outputs_do_not_spill_past_their_buffers(mi):
    """Canaries on both sides of out / stats stay untouched."""
    w = synthetic.varlen_inputs(24, Nq=4, Nkv=4, D=64, dtype="bf16", lengths_q=[130, 61])
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    pad = 4096
    n_out = q.numel()
    buf = torch.full((n_out + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda:0")
    sbuf = torch.full((2 * (w["Nq"] * w["Tq"]) + 3 * pad,), 7.0, dtype=torch.float32, device="cuda:0")
    out = buf[pad:pad + n_out]
    m = sbuf[pad:pad + w["Nq"] * w["Tq"]]
    l = sbuf[2 * pad + w["Nq"] * w["Tq"]:2 * pad + 2 * w["Nq"] * w["Tq"]]
    mi.attn_fwd_varlen(q, k, v, out, m, l, cq, cq, w["B"], w["Tq"], w["Tq"], 130, 130, 4, 4, 64,
                       "bf16", 0.125, "causal")
    torch.cuda.synchronize()
    hb = host_values(buf)
    hs = host_values(sbuf)
    assert np.all(hb[:pad] == 7.0) and np.all(hb[pad + n_out:] == 7.0)
    assert np.all(hs[:pad] == 7.0)
    nm = w["Nq"] * w["Tq"]
    assert np.all(hs[pad + nm:2 * pad + nm] == 7.0) and np.all(hs[2 * pad + 2 * nm:] == 7.0)


def test_stats_pointers_may_be_null(mi):
    w = synthetic.dense_inputs(25, 1, 2, 2, 100, 100, 64, "bf16", "BNSD")
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, "bf16")
    mi.attn_fwd(q, k, v, out, None, None, 1, 2, 2, 100, 100, 64, "bf16", "BNSD", 0.125, "causal")
    torch.cuda.synchronize()
    wo, _, _ = _oracle_dense(w, 0.125, "causal")
    check_out(host_values(out), wo, "bf16")


def test_package_imported_before_torch():
    """A fresh process that imports the package before torch launches kernels correctly
    (the package loads torch's HIP runtime before the library)."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import scaled_dot_product_02_amd as mi\n"
        "import torch\n"
        "q = torch.ones(1, 2, 128, 64, device='cuda', dtype=torch.bfloat16)\n"
        "o = torch.zeros_like(q)\n"
        "mi.attn_fwd(q, q, q, o, None, None, 1, 2, 2, 128, 128, 64, 'bf16', 'BNSD', 0.125, 'causal')\n"
        "torch.cuda.synchronize()\n"
        "assert bool((o.float() == 1).all()), 'attention of constant V must return V'\n"
        "print('ok')\n" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
