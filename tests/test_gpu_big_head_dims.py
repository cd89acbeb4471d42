"""GPU parity at head dims 160, 192, 224 and 256 (bf16 / fp16 on the matrix cores, with
4-wave workgroups and 32-key tiles) against the CPU fp64 oracle: dense layouts x masks at
ragged sizes with GQA, packed batches with empty and single-row sequences, bottom-right
causal with a prefix, and the fused update."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import check_out, check_stats, dev, empty_like_storage, host_values, nan_stats

pytestmark = pytest.mark.gpu

BIG = 1 << 40


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _bnsd(w, x, n):
    return synthetic.to_bnsd(synthetic.storage_values(w[x], w["dtype"]), w["layout"], n)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [160, 192, 224, 256])
@pytest.mark.parametrize("layout", ["BNSD", "SBH"])
@pytest.mark.parametrize("mask,pre,nxt", [("none", 0, 0), ("causal", 0, 0), ("band", 70, 33)])
def test_dense(mi, dtype, D, layout, mask, pre, nxt):
    # Sq 300, Skv 333: 3 query tiles of 128 rows (ragged), 11 key tiles of 32 (ragged); GQA 4/2
    B, Nq, Nkv, Sq, Skv = 2, 4, 2, 300, 333
    w = synthetic.dense_inputs(301 + D, B, Nq, Nkv, Sq, Skv, D, dtype, layout)
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, dtype)
    m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    sc = 1 / math.sqrt(D)
    mi.attn_fwd(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, dtype, layout, sc, mask, pre, nxt)
    torch.cuda.synchronize()
    wo, wm, wl = oracle.attn(_bnsd(w, "q", Nq), _bnsd(w, "k", Nkv), _bnsd(w, "v", Nkv), sc, mask, pre, nxt)
    check_out(synthetic.to_bnsd(host_values(out), layout, Nq), wo, dtype)
    check_stats(host_values(m), host_values(l), wm, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [160, 256])
def test_varlen(mi, dtype, D):
    lengths = [300, 0, 1, 129, 64, 517, 2]
    w = synthetic.varlen_inputs(311, Nq=8, Nkv=2, D=D, dtype=dtype, lengths_q=lengths)
    sc = 1 / math.sqrt(D)
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    out = empty_like_storage(q.shape, dtype)
    m, l = nan_stats((8, w["Tq"])), nan_stats((8, w["Tq"]))
    mi.attn_fwd_varlen(q, k, v, out, m, l, cq, cq, w["B"], w["Tq"], w["Tq"], 517, 517, 8, 2, D,
                       dtype, sc, "causal")
    torch.cuda.synchronize()
    qo, ko, vo = (synthetic.storage_values(w[x], dtype) for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(qo, ko, vo, w["cu_q"], w["cu_kv"], sc, "causal")
    check_out(host_values(out), wo, dtype)
    check_stats(host_values(m), host_values(l), wm, wl)


def test_bottom_right_prefix(mi):
    B, Nq, Nkv, Sq, Skv, D, dtype = 3, 4, 2, 300, 520, 192, "bf16"
    w = synthetic.dense_inputs(321, B, Nq, Nkv, Sq, Skv, D, dtype, "BSND")
    prefix = np.array([0, 100, 600])
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, dtype)
    m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    sc = 1 / math.sqrt(D)
    mi.attn_fwd_ext(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, D, dtype, "BSND", sc, "causal_br",
                    0, 0, torch.from_numpy(prefix).to("cuda:0"), None)
    torch.cuda.synchronize()
    keep = np.stack([oracle.keep_band(Sq, Skv, BIG, 0, "bottom_right") |
                     (np.arange(Skv)[None, :] < min(P, Skv)) for P in prefix])
    wo, wm, wl = oracle.attn_keep(_bnsd(w, "q", Nq), _bnsd(w, "k", Nkv), _bnsd(w, "v", Nkv), keep, sc)
    check_out(synthetic.to_bnsd(host_values(out), "BSND", Nq), wo, dtype)
    check_stats(host_values(m), host_values(l), wm, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_update(mi, dtype):
    """The fused ring update at D 256: a random prior (5% empty rows) merged with one chunk."""
    B, Nq, Nkv, Sq, Skv, D, layout = 2, 4, 2, 300, 333, 256, "BNSD"
    w = synthetic.dense_inputs(331, B, Nq, Nkv, Sq, Skv, D, dtype, layout)
    rng = np.random.default_rng(332)
    o = rng.standard_normal((B, Nq, Sq, D), dtype=np.float32)
    pm = (rng.standard_normal((B, Nq, Sq)) * 3).astype(np.float32)
    pl = rng.uniform(0.5, 50.0, (B, Nq, Sq)).astype(np.float32)
    e = rng.random((B, Nq, Sq)) < 0.05
    pm[e], pl[e] = -np.inf, 0.0
    o_st = synthetic.to_storage(o, dtype)
    o_or = synthetic.storage_values(o_st, dtype).astype(np.float64)
    o_or[e] = 0.0
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, dtype)
    mo, lo = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    sc = 1 / math.sqrt(D)
    mi.attn_fwd_update(q, k, v, dev(o_st, dtype), torch.from_numpy(pm).to("cuda:0"),
                       torch.from_numpy(pl).to("cuda:0"), out, mo, lo, B, Nq, Nkv, Sq, Skv, D,
                       dtype, layout, sc, "causal", 0, 0)
    torch.cuda.synchronize()
    wo, wm, wl = oracle.attn_update(_bnsd(w, "q", Nq), _bnsd(w, "k", Nkv), _bnsd(w, "v", Nkv),
                                    o_or, pm, pl, sc, "causal", 0, 0)
    check_out(host_values(out), wo, dtype)
    check_stats(host_values(mo), host_values(lo), wm, wl)


def test_mha_head_dim_256(mi):
    """The MHA module with 2 heads of 256 (embed 512) in bf16, eval mode."""
    B, S, E, N = 2, 200, 512, 2
    torch.manual_seed(1)
    m = mi.MultiHeadAttention(E, N, dropout=0.0, dtype=torch.bfloat16, device="cuda:0")
    m.eval()
    x = torch.randn((B, S, E), device="cuda:0").to(torch.bfloat16)
    hv = lambda t: host_values(t.detach())
    with torch.no_grad():
        got = hv(m(x))
    rnd = lambda a: synthetic.storage_values(synthetic.to_storage(np.asarray(a), "bf16"), "bf16").astype(np.float64)
    want = oracle.mha_self_attn(hv(x), hv(m.qkv_proj.weight), hv(m.qkv_proj.bias),
                                hv(m.out_proj.weight), hv(m.out_proj.bias), N, round_to=rnd)
    err = np.max(np.abs(got - want)) / np.max(np.abs(want))
    assert err <= 2.0 ** -6, err
