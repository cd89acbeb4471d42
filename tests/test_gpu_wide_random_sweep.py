"""A seeded random sweep (150 cases) of the head-dim-general forward against the CPU fp64
oracle: each case draws Q/K and V head dims (1 <= Dv <= D <= 768, odd sizes included, dims
the tiled kernels serve excluded so every case runs on the general kernel), dtype, GQA
ratio, dense layout or packed batch (zero lengths included), a mask mode with random band
widths and, for some cases, an explicit mask tensor.  The oracle sees each mask as an
explicit visibility matrix (oracle.keep_band, pinned against np.tril and torch's SDPA)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import check_out, check_stats, dev, empty_like_storage, host_values, nan_stats

pytestmark = pytest.mark.gpu

BIG = 1 << 40
N_CASES = 150
TILED = {32, 64, 96, 128, 160, 192, 224, 256}


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = ["bf16", "f16", "f32"][rng.integers(0, 3)]
    while True:
        D = int(rng.integers(1, 769))
        Dv = D if rng.random() < 0.5 else int(rng.integers(1, D + 1))
        if not (D in TILED and Dv == D):
            break
    Nkv = int(rng.integers(1, 3))
    Nq = Nkv * int(rng.integers(1, 4))
    mask = ["none", "causal", "band", "causal_br", "band_br"][rng.integers(0, 5)]
    pre, nxt = 0, 0
    if mask.startswith("band"):
        pre = int(rng.integers(-40, 200))
        nxt = int(rng.integers(max(-40, -pre), 200))
    return dict(dtype=dtype, D=D, Dv=Dv, Nq=Nq, Nkv=Nkv, mask=mask, pre=pre, nxt=nxt,
                varlen=bool(rng.integers(0, 2)), amask=bool(rng.random() < 0.3), rng=rng)


def _keep(mask, pre, nxt, Sq, Skv):
    if mask == "none":
        return np.ones((Sq, Skv), dtype=bool)
    p, n = (BIG, 0) if mask.startswith("causal") else (pre, nxt)
    return oracle.keep_band(Sq, Skv, p, n, "bottom_right" if mask.endswith("_br") else "top_left")


def _v(rng, shape, dt):
    return synthetic.to_storage(rng.standard_normal(shape, dtype=np.float32), dt)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(mi, i):
    c = _case(i)
    rng, dt, D, Dv, Nq, Nkv = c["rng"], c["dtype"], c["D"], c["Dv"], c["Nq"], c["Nkv"]
    sc = float(rng.uniform(0.5, 1.5)) / math.sqrt(D)
    if not c["varlen"]:
        B = int(rng.integers(1, 3))
        Sq, Skv = int(rng.integers(1, 200)), int(rng.integers(1, 200))
        layout = ["BNSD", "BSND", "BSH", "SBH"][rng.integers(0, 4)]
        w = synthetic.dense_inputs(8000 + i, B, Nq, Nkv, Sq, Skv, D, dt, layout)
        w["v"] = _v(rng, synthetic.storage_shape(layout, B, Nkv, Skv, Dv), dt)
        am = rng.random((Sq, Skv)) < 0.3 if c["amask"] else None
        q, k, v = (dev(w[x], dt) for x in ("q", "k", "v"))
        out = empty_like_storage(synthetic.storage_shape(layout, B, Nq, Sq, Dv), dt)
        m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
        amd = None if am is None else torch.from_numpy(am.astype(np.uint8)).to("cuda:0")
        mi.attn_fwd_ext(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, Dv, dt, layout, sc, c["mask"],
                        c["pre"], c["nxt"], None, amd)
        torch.cuda.synchronize()
        bn = lambda x, n: synthetic.to_bnsd(synthetic.storage_values(w[x], dt), layout, n)
        keep = _keep(c["mask"], c["pre"], c["nxt"], Sq, Skv)
        if am is not None:
            keep = keep & ~am
        wo, wm, wl = oracle.attn_keep(bn("q", Nq), bn("k", Nkv), bn("v", Nkv), keep, sc)
        check_out(synthetic.to_bnsd(host_values(out), layout, Nq), wo, dt, f"case {i} {c}")
        check_stats(host_values(m), host_values(l), wm, wl)
    else:
        B = int(rng.integers(1, 5))
        lq = rng.integers(0, 160, size=B)
        lk = rng.integers(0, 160, size=B)
        lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)
        w = synthetic.varlen_inputs(9000 + i, Nq=Nq, Nkv=Nkv, D=D, dtype=dt, lengths_q=lq, lengths_kv=lk)
        w["v"] = _v(rng, (w["Tkv"], Nkv, Dv), dt)
        mq, mk = int(lq.max()), int(lk.max())
        am = rng.random((mq, mk)) < 0.3 if c["amask"] else None
        q, k, v = (dev(w[x], dt) for x in ("q", "k", "v"))
        cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
        ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
        Tq, Tkv = w["Tq"], w["Tkv"]
        out = empty_like_storage((Tq, Nq, Dv), dt)
        m, l = nan_stats((Nq, Tq)), nan_stats((Nq, Tq))
        amd = None if am is None else torch.from_numpy(am.astype(np.uint8)).to("cuda:0")
        mi.attn_fwd_varlen_ext(q, k, v, out, m, l, cq, ck, B, Tq, Tkv, mq, mk, Nq, Nkv, D, Dv, dt,
                               sc, c["mask"], c["pre"], c["nxt"], None, amd)
        torch.cuda.synchronize()
        qo, ko, vo = (synthetic.storage_values(w[x], dt) for x in ("q", "k", "v"))

        def keep_of(b, sq, skv):
            kp = _keep(c["mask"], c["pre"], c["nxt"], sq, skv)
            return kp if am is None else kp & ~am[:sq, :skv]
        wo, wm, wl = oracle.attn_varlen_keep(qo, ko, vo, w["cu_q"], w["cu_kv"], keep_of, sc)
        check_out(host_values(out), wo, dt, f"case {i} {c}")
        check_stats(host_values(m), host_values(l), wm, wl)
