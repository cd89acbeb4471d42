"""A seeded random sweep of attn_fwd_ext / attn_fwd_varlen_ext against the CPU fp64 oracle.

Each case draws its own combination of: dense or packed batch, dtype, head dim (32..256;
fp32 up to 128), GQA ratio and head counts, layout, mask mode with random band widths
(empty rows included), Sq != Skv, and packed batches whose query and key lengths differ
per sequence (zero lengths included).  The oracle sees each mask as an explicit visibility
matrix (oracle.keep_band, pinned against np.tril and torch's SDPA), so the combinations
the structured tests do not pair up are checked against the same definition."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import check_out, check_stats, dev, empty_like_storage, host_values, nan_stats

pytestmark = pytest.mark.gpu

BIG = 1 << 40
N_CASES = 160


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _case(i):
    rng = np.random.default_rng(1000 + i)
    dtype = ["bf16", "f16", "f32"][rng.integers(0, 3)]
    dims = [32, 64, 96, 128] + ([] if dtype == "f32" else [160, 192, 224, 256])
    D = int(rng.choice(dims))
    Nkv = int(rng.integers(1, 5))
    Nq = Nkv * int(rng.integers(1, 5))
    mask = ["none", "causal", "band", "causal_br", "band_br"][rng.integers(0, 5)]
    pre, nxt = 0, 0
    if mask.startswith("band"):
        pre = int(rng.integers(-60, 400))
        nxt = int(rng.integers(max(-60, -pre), 400))
    return dict(dtype=dtype, D=D, Nq=Nq, Nkv=Nkv, mask=mask, pre=pre, nxt=nxt,
                varlen=bool(rng.integers(0, 2)), rng=rng)


def _keep(mask, pre, nxt, Sq, Skv):
    if mask == "none":
        return np.ones((Sq, Skv), dtype=bool)
    p, n = (BIG, 0) if mask.startswith("causal") else (pre, nxt)
    return oracle.keep_band(Sq, Skv, p, n, "bottom_right" if mask.endswith("_br") else "top_left")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(mi, i):
    c = _case(i)
    rng, dt, D, Nq, Nkv = c["rng"], c["dtype"], c["D"], c["Nq"], c["Nkv"]
    sc = float(rng.uniform(0.5, 1.5)) / math.sqrt(D)
    if not c["varlen"]:
        B = int(rng.integers(1, 4))
        Sq, Skv = int(rng.integers(1, 401)), int(rng.integers(1, 401))
        layout = ["BNSD", "BSND", "BSH", "SBH"][rng.integers(0, 4)]
        w = synthetic.dense_inputs(2000 + i, B, Nq, Nkv, Sq, Skv, D, dt, layout)
        q, k, v = (dev(w[x], dt) for x in ("q", "k", "v"))
        out = empty_like_storage(q.shape, dt)
        m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
        mi.attn_fwd_ext(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, D, dt, layout, sc, c["mask"],
                        c["pre"], c["nxt"], None, None)
        torch.cuda.synchronize()
        bn = lambda x, n: synthetic.to_bnsd(synthetic.storage_values(w[x], dt), layout, n)
        wo, wm, wl = oracle.attn_keep(bn("q", Nq), bn("k", Nkv), bn("v", Nkv),
                                      _keep(c["mask"], c["pre"], c["nxt"], Sq, Skv), sc)
        check_out(synthetic.to_bnsd(host_values(out), layout, Nq), wo, dt, f"case {i} {c}")
        check_stats(host_values(m), host_values(l), wm, wl)
    else:
        B = int(rng.integers(1, 7))
        lq = rng.integers(0, 301, size=B)
        lk = rng.integers(0, 301, size=B)
        lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)
        w = synthetic.varlen_inputs(3000 + i, Nq=Nq, Nkv=Nkv, D=D, dtype=dt, lengths_q=lq, lengths_kv=lk)
        q, k, v = (dev(w[x], dt) for x in ("q", "k", "v"))
        cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
        ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
        Tq, Tkv = w["Tq"], w["Tkv"]
        out = empty_like_storage(q.shape, dt)
        m, l = nan_stats((Nq, Tq)), nan_stats((Nq, Tq))
        mi.attn_fwd_varlen_ext(q, k, v, out, m, l, cq, ck, B, Tq, Tkv, int(lq.max()), int(lk.max()),
                               Nq, Nkv, D, D, dt, sc, c["mask"], c["pre"], c["nxt"], None, None)
        torch.cuda.synchronize()
        qo, ko, vo = (synthetic.storage_values(w[x], dt) for x in ("q", "k", "v"))
        wo, wm, wl = oracle.attn_varlen_keep(qo, ko, vo, w["cu_q"], w["cu_kv"],
                                             lambda b, sq, skv: _keep(c["mask"], c["pre"], c["nxt"], sq, skv), sc)
        check_out(host_values(out), wo, dt, f"case {i} {c}")
        check_stats(host_values(m), host_values(l), wm, wl)
