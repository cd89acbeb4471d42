"""GPU parity of the mask modes against the CPU fp64 oracle's explicit visibility matrices:
bottom-right causal and band (attn_fwd, attn_fwd_varlen, attn_fwd_update), the prefix
(attn_fwd_varlen_ext / attn_fwd_ext), and an explicit mask tensor (any dtype; rows of
whole 4-byte words on the tiled kernel for bf16 / fp16, other rows and fp32 on the
head-dim-general kernel).  Sizes span several tiles with ragged ends; Sq > Skv gives empty
rows.
"""
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


def _dense_gpu(mi, w, scale, mask, pre=0, nxt=0, prefix=None, amask=None):
    B, Nq, Nkv, Sq, Skv, D = (w[x] for x in ("B", "Nq", "Nkv", "Sq", "Skv", "D"))
    Dv = w.get("Dv", D)
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    out = empty_like_storage(synthetic.storage_shape(w["layout"], B, Nq, Sq, Dv), dt)
    m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    pf = None if prefix is None else torch.from_numpy(np.asarray(prefix, np.int64)).to("cuda:0")
    am = None if amask is None else torch.from_numpy(np.ascontiguousarray(amask, np.uint8)).to("cuda:0")
    mi.attn_fwd_ext(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, Dv, dt, w["layout"], scale,
                       mask, pre, nxt, pf, am)
    torch.cuda.synchronize()
    return synthetic.to_bnsd(host_values(out), w["layout"], Nq), host_values(m), host_values(l)


def _check_dense(mi, w, scale, mask, keep, pre=0, nxt=0, prefix=None, amask=None):
    go, gm, gl = _dense_gpu(mi, w, scale, mask, pre, nxt, prefix, amask)
    wo, wm, wl = oracle.attn_keep(_bnsd(w, "q", w["Nq"]), _bnsd(w, "k", w["Nkv"]),
                                  _bnsd(w, "v", w["Nkv"]), keep, scale)
    check_out(go, wo, w["dtype"])
    check_stats(gm, gl, wm, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Skv", [(300, 333), (333, 300), (257, 257)])
@pytest.mark.parametrize("mask,pre,nxt", [("causal_br", 0, 0), ("band_br", 70, 33),
                                          ("band_br", BIG, -40)])
def test_dense_bottom_right(mi, dtype, D, Sq, Skv, mask, pre, nxt):
    w = synthetic.dense_inputs(81, 2, 4, 2, Sq, Skv, D, dtype, "BSND")
    p = BIG if mask == "causal_br" else pre
    n = 0 if mask == "causal_br" else nxt
    keep = oracle.keep_band(Sq, Skv, p, n, "bottom_right")
    _check_dense(mi, w, 1 / math.sqrt(D), mask, keep, pre, nxt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mask,align", [("causal_br", "bottom_right"), ("causal", "top_left")])
def test_dense_prefix(mi, dtype, mask, align):
    B, Sq, Skv, D = 3, 300, 520, 128
    w = synthetic.dense_inputs(82, B, 4, 2, Sq, Skv, D, dtype, "BNSD")
    prefix = np.array([0, 100, 600])       # 600 is clamped to Skv
    keep = np.stack([oracle.keep_band(Sq, Skv, BIG, 0, align) |
                     (np.arange(Skv)[None, :] < min(P, Skv)) for P in prefix])
    _check_dense(mi, w, 1 / math.sqrt(D), mask, keep, prefix=prefix)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,pre,nxt", [("none", 0, 0), ("causal", 0, 0), ("band_br", 50, 20)])
@pytest.mark.parametrize("Skv", [150, 152])
def test_dense_explicit_mask(mi, dtype, D, mask, pre, nxt, Skv):
    """Mask rows of 152 bytes (4-byte words) run on the matrix cores for bf16 / fp16; rows
    of 150 bytes take the head-dim-general kernel."""
    Sq = 200
    w = synthetic.dense_inputs(83, 2, 4, 2, Sq, Skv, D, dtype, "BSH")
    rng = np.random.default_rng(84)
    amask = rng.random((Sq, Skv)) < 0.3          # True = masked out
    amask[7] = True                               # a fully masked row: the empty result
    if mask == "none":
        band = np.ones((Sq, Skv), dtype=bool)
    elif mask == "causal":
        band = oracle.keep_band(Sq, Skv, BIG, 0)
    else:
        band = oracle.keep_band(Sq, Skv, pre, nxt, "bottom_right")
    _check_dense(mi, w, 1 / math.sqrt(D), mask, band & ~amask, pre, nxt, amask=amask)


def _varlen_gpu(mi, w, scale, mask, pre=0, nxt=0, prefix=None, amask=None):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    Dv = w.get("Dv", w["D"])
    out = empty_like_storage((w["Tq"], w["Nq"], Dv), dt)
    m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
    pf = None if prefix is None else torch.from_numpy(np.asarray(prefix, np.int64)).to("cuda:0")
    am = None if amask is None else torch.from_numpy(np.ascontiguousarray(amask, np.uint8)).to("cuda:0")
    mi.attn_fwd_varlen_ext(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"],
                              int(w["lengths_q"].max()), int(w["lengths_kv"].max()), w["Nq"],
                              w["Nkv"], w["D"], Dv, dt, scale, mask, pre, nxt, pf, am)
    torch.cuda.synchronize()
    return host_values(out), host_values(m), host_values(l)


def _check_varlen(mi, w, scale, mask, keep_of, pre=0, nxt=0, prefix=None, amask=None):
    go, gm, gl = _varlen_gpu(mi, w, scale, mask, pre, nxt, prefix, amask)
    q, k, v = (synthetic.storage_values(w[x], w["dtype"]) for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen_keep(q, k, v, w["cu_q"], w["cu_kv"], keep_of, scale)
    check_out(go, wo, w["dtype"])
    check_stats(gm, gl, wm, wl)


LQ = [300, 0, 1, 129, 64, 517, 2, 40]
LK = [333, 5, 7, 129, 300, 600, 0, 20]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mask,pre,nxt", [("causal_br", 0, 0), ("band_br", 90, 10)])
def test_varlen_bottom_right(mi, dtype, mask, pre, nxt):
    """Per-sequence bottom-right alignment: the offset Skv_b - Sq_b differs by sequence
    (zero-length queries, zero-length keys, Sq > Skv and Sq < Skv)."""
    w = synthetic.varlen_inputs(85, Nq=8, Nkv=2, D=128, dtype=dtype, lengths_q=LQ, lengths_kv=LK)
    p = BIG if mask == "causal_br" else pre
    n = 0 if mask == "causal_br" else nxt
    _check_varlen(mi, w, 1 / math.sqrt(128), mask,
                  lambda b, sq, sk: oracle.keep_band(sq, sk, p, n, "bottom_right"), pre, nxt)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_varlen_prefix_bottom_right_causal(mi, dtype):
    """The prefix mode: keys j < prefix[b] plus bottom-right causal."""
    w = synthetic.varlen_inputs(86, Nq=8, Nkv=2, D=64, dtype=dtype, lengths_q=LQ, lengths_kv=LK)
    prefix = [200, 3, 0, 129, 64, 333, 0, 25]
    _check_varlen(mi, w, 0.125, "causal_br",
                  lambda b, sq, sk: oracle.keep_prefix_causal(sq, sk, min(prefix[b], sk)),
                  prefix=prefix)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("lk", [LK, LK[:5] + [601] + LK[6:]])
def test_varlen_explicit_mask(mi, dtype, lk):
    w = synthetic.varlen_inputs(87, Nq=8, Nkv=2, D=128, dtype=dtype, lengths_q=LQ, lengths_kv=lk)
    mq, mk = max(LQ), max(lk)
    amask = np.random.default_rng(88).random((mq, mk)) < 0.25
    _check_varlen(mi, w, 1 / math.sqrt(128), "causal",
                  lambda b, sq, sk: oracle.keep_band(sq, sk, BIG, 0) & ~amask[:sq, :sk],
                  amask=amask)


def _with_dv(w, Dv, seed):
    """The inputs with V redrawn at head dim Dv (same recipe: standard normal float32, then
    the storage type)."""
    rng = np.random.default_rng(seed)
    if "layout" in w:
        shape = synthetic.storage_shape(w["layout"], w["B"], w["Nkv"], w["Skv"], Dv)
    else:
        shape = (w["Tkv"], w["Nkv"], Dv)
    v = synthetic.to_storage(rng.standard_normal(shape, dtype=np.float32), w["dtype"])
    return dict(w, v=v, Dv=Dv)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D,Dv", [(64, 32), (96, 64), (128, 64), (128, 96)])
@pytest.mark.parametrize("layout", ["BNSD", "SBH"])
def test_dense_value_head_dim_below_qk(mi, dtype, D, Dv, layout):
    """qD == kD >= vD: the value / output head dim below the query / key one."""
    w = _with_dv(synthetic.dense_inputs(91, 2, 4, 2, 300, 333, D, dtype, layout), Dv, 92)
    keep = oracle.keep_band(300, 333, BIG, 0)
    _check_dense(mi, w, 1 / math.sqrt(D), "causal", keep)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_value_head_dim_below_qk(mi, dtype):
    w = _with_dv(synthetic.varlen_inputs(93, Nq=8, Nkv=2, D=128, dtype=dtype, lengths_q=LQ,
                                         lengths_kv=LK), 64, 94)
    _check_varlen(mi, w, 1 / math.sqrt(128), "causal_br",
                  lambda b, sq, sk: oracle.keep_band(sq, sk, BIG, 0, "bottom_right"))


def test_update_bottom_right(mi):
    """The fused ring update takes the bottom-right modes too (offset chunk diagonal)."""
    B, Nq, Nkv, Sq, Skv, D = 1, 4, 2, 300, 200, 128
    w = synthetic.dense_inputs(89, B, Nq, Nkv, Sq, Skv, D, "bf16", "BNSD")
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    rng = np.random.default_rng(90)
    po = rng.standard_normal((B, Nq, Sq, D), dtype=np.float32)
    po_st = synthetic.to_storage(po, "bf16")
    pm = (rng.standard_normal((B, Nq, Sq)) * 2).astype(np.float32)
    pl = rng.uniform(1, 20, (B, Nq, Sq)).astype(np.float32)
    out = empty_like_storage(q.shape, "bf16")
    mo, lo = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    mi.attn_fwd_update(q, k, v, dev(po_st, "bf16"), torch.from_numpy(pm).to("cuda:0"),
                       torch.from_numpy(pl).to("cuda:0"), out, mo, lo, B, Nq, Nkv, Sq, Skv, D,
                       "bf16", "BNSD", 0.1, "causal_br")
    torch.cuda.synchronize()
    keep = oracle.keep_band(Sq, Skv, BIG, 0, "bottom_right")
    o_c, m_c, l_c = oracle.attn_keep(_bnsd(w, "q", Nq), _bnsd(w, "k", Nkv), _bnsd(w, "v", Nkv), keep, 0.1)
    wo, wm, wl = oracle.merge(synthetic.storage_values(po_st, "bf16"), pm, pl, o_c, m_c, l_c)
    check_out(host_values(out), wo, "bf16")
    check_stats(host_values(mo), host_values(lo), wm, wl)


def test_metric_lengths_with_prefix(mi):
    """The full packed workload's lengths (seed 0), bottom-right causal plus a per-sequence
    prefix, on the MFMA path; sampled sequences x heads against the oracle."""
    w = synthetic.make(synthetic.METRIC_WORKLOAD)
    lengths = w["lengths_q"]
    prefix = [int(L) // 3 for L in lengths]
    go, gm, gl = _varlen_gpu(mi, w, 1 / math.sqrt(128), "causal_br", prefix=prefix)
    cu = np.concatenate([[0], w["cu_q"]])
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    for b, h in [(14, 5), (7, 0), (3, 31)]:
        sl = slice(int(cu[b]), int(cu[b + 1]))
        L = int(lengths[b])
        keep = oracle.keep_prefix_causal(L, L, prefix[b])
        wo, wm, wl = oracle.attn_keep(q[sl, h][None, None], k[sl, h // 4][None, None],
                                      v[sl, h // 4][None, None], keep, 1 / math.sqrt(128))
        check_out(go[sl, h], wo[0, 0], "bf16", f"seq {b} head {h}")
        check_stats(gm[h, sl], gl[h, sl], wm[0, 0], wl[0, 0])
