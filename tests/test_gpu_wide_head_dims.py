"""GPU parity of the head-dim-general forward against the CPU fp64 oracle: head dims the
tiled kernels are not built for (any 1 <= Dv <= D <= 768, multiples of 8 or not), in every
dtype, with the layouts, masks, packed batches, the fused update, the explicit mask tensor
and dropout.  Sizes span several 32- / 64-row tiles and 32-key tiles with ragged tails."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import check_out, check_stats, dev, empty_like_storage, host_values, nan_stats
from test_gpu_masks import _check_dense, _check_varlen, _with_dv

pytestmark = pytest.mark.gpu

BIG = 1 << 40


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _band(mask, pre, nxt, Sq, Skv):
    if mask == "none":
        return np.ones((Sq, Skv), dtype=bool)
    if mask == "causal":
        return oracle.keep_band(Sq, Skv, BIG, 0)
    return oracle.keep_band(Sq, Skv, pre, nxt)


# (D, Dv): odd and non-multiple-of-8 dims (scalar loads), dims between the tiled ones, and
# up to the spec's 768, with V head dims below the Q/K one
DIMS = [(1, 1), (8, 8), (40, 40), (80, 48), (100, 100), (200, 200), (288, 288), (320, 160),
        (384, 384), (512, 512), (640, 600), (768, 768), (768, 520), (97, 9)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D,Dv", DIMS)
@pytest.mark.parametrize("layout,mask,pre,nxt", [("BNSD", "none", 0, 0), ("BSND", "causal", 0, 0),
                                                 ("SBH", "band", 45, 20)])
def test_dense(mi, dtype, D, Dv, layout, mask, pre, nxt):
    B, Nq, Nkv, Sq, Skv = 2, 4, 2, 150, 170
    w = synthetic.dense_inputs(500 + D, B, Nq, Nkv, Sq, Skv, D, dtype, layout)
    if Dv != D:
        w = _with_dv(w, Dv, 600 + Dv)
    _check_dense(mi, w, 1 / math.sqrt(D), mask, _band(mask, pre, nxt, Sq, Skv), pre, nxt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D,Dv", [(160, 160), (256, 256), (128, 64)])
def test_tiled_dims_on_the_general_path(mi, dtype, D, Dv):
    """Head dims of the tiled kernels in combinations they are not built for: fp32 at 160
    and 256, and a mask tensor with 256 or with Dv < D."""
    Sq, Skv = 130, 152
    w = synthetic.dense_inputs(510 + D, 2, 4, 2, Sq, Skv, D, dtype, "BSND")
    if Dv != D:
        w = _with_dv(w, Dv, 610)
    amask = np.random.default_rng(511).random((Sq, Skv)) < 0.3
    amask[5] = True
    _check_dense(mi, w, 1 / math.sqrt(D), "causal", oracle.keep_band(Sq, Skv, BIG, 0) & ~amask,
                 amask=amask)
    _check_dense(mi, w, 1 / math.sqrt(D), "band", oracle.keep_band(Sq, Skv, 40, 40), 40, 40)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D,Dv", [(72, 72), (448, 300), (768, 768)])
def test_varlen(mi, dtype, D, Dv):
    lq = [150, 0, 1, 65, 33, 200, 2]
    lk = [170, 5, 0, 65, 100, 210, 3]
    w = synthetic.varlen_inputs(520 + D, Nq=4, Nkv=2, D=D, dtype=dtype, lengths_q=lq, lengths_kv=lk)
    w = dict(w, lengths_q=np.asarray(lq), lengths_kv=np.asarray(lk))
    if Dv != D:
        w = _with_dv(w, Dv, 620)
    _check_varlen(mi, w, 1 / math.sqrt(D), "causal_br",
                  lambda b, sq, sk: oracle.keep_band(sq, sk, BIG, 0, "bottom_right"))
    amask = np.random.default_rng(521).random((200, 210)) < 0.25
    _check_varlen(mi, w, 1 / math.sqrt(D), "band", lambda b, sq, sk: oracle.keep_band(sq, sk, 30, 9)
                  & ~amask[:sq, :sk], 30, 9, amask=amask)


def test_prefix_bottom_right(mi):
    B, Nq, Nkv, Sq, Skv, D = 3, 2, 1, 100, 180, 300
    w = synthetic.dense_inputs(530, B, Nq, Nkv, Sq, Skv, D, "bf16", "BNSD")
    prefix = np.array([0, 150, 400])
    keep = np.stack([oracle.keep_band(Sq, Skv, BIG, 0, "bottom_right") |
                     (np.arange(Skv)[None, :] < min(P, Skv)) for P in prefix])
    _check_dense(mi, w, 1 / math.sqrt(D), "causal_br", keep, prefix=prefix)


@pytest.mark.parametrize("dtype,D", [("bf16", 320), ("f16", 100), ("f32", 200), ("f32", 768)])
def test_update(mi, dtype, D):
    """The fused ring update: a random prior (5% empty rows) merged with one chunk."""
    B, Nq, Nkv, Sq, Skv, layout = 2, 4, 2, 150, 170, "BNSD"
    w = synthetic.dense_inputs(540 + D, B, Nq, Nkv, Sq, Skv, D, dtype, layout)
    rng = np.random.default_rng(541)
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
    bn = lambda x, n: synthetic.to_bnsd(synthetic.storage_values(w[x], dtype), layout, n)
    wo, wm, wl = oracle.attn_update(bn("q", Nq), bn("k", Nkv), bn("v", Nkv), o_or, pm, pl, sc,
                                    "causal", 0, 0)
    check_out(host_values(out), wo, dtype)
    check_stats(host_values(mo), host_values(lo), wm, wl)


@pytest.mark.parametrize("dtype,D", [("bf16", 256), ("f16", 200), ("f32", 80), ("bf16", 768)])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_dropout(mi, dtype, D, mask):
    B, Nq, Nkv, Sq, Skv, p = 2, 4, 2, 150, 170, 0.25
    w = synthetic.dense_inputs(550 + D, B, Nq, Nkv, Sq, Skv, D, dtype, "BSND")
    seed, offset = 0x0123_4567_89AB_CDEF, 3
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, dtype)
    m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    sc = 1 / math.sqrt(D)
    mi.attn_fwd_ext(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, D, dtype, "BSND", sc, mask,
                    0, 0, None, None, p, seed, offset)
    torch.cuda.synchronize()
    bn = lambda x, n: synthetic.to_bnsd(synthetic.storage_values(w[x], dtype), "BSND", n)
    wo, wm, wl = oracle.attn_dropout(bn("q", Nq), bn("k", Nkv), bn("v", Nkv), sc, mask, 0, 0,
                                     float(np.float32(p)), seed, offset)
    check_out(synthetic.to_bnsd(host_values(out), "BSND", Nq), wo, dtype)
    check_stats(host_values(m), host_values(l), wm, wl)


def test_mha_head_dim_80(mi):
    """The MHA module with 8 heads of 80 (embed 640) in bf16, eval mode."""
    B, S, E, N = 2, 150, 640, 8
    torch.manual_seed(2)
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
