"""GPU parity at the edges of the accepted argument ranges: a packed batch of T = 2^20 tokens
(the varlen operator's bound of 1M tokens, read as 2^20), the library's largest batch of 2048
sequences, 256 query heads (the operator's bound on N), a single-head sequence of 131,072
keys, and SBH batches whose row stride crosses the tiled kernel's 32-bit tile range.
Sampled rows are checked against the oracle, each computed from its own visible keys."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import check_out, check_stats, dev, empty_like_storage, host_values, nan_stats

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _varlen(mi, w, scale, mask="causal"):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    out = empty_like_storage(q.shape, dt)
    m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
    mi.attn_fwd_varlen(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"],
                       int(w["lengths_q"].max()), int(w["lengths_kv"].max()), w["Nq"], w["Nkv"],
                       w["D"], dt, scale, mask)
    torch.cuda.synchronize()
    return host_values(out), host_values(m), host_values(l)


def test_packed_batch_of_2_20_tokens(mi):
    """Two causal sequences of 2^19 tokens (T = 2^20), one head, D 64: rows at the start,
    the end and the boundary of each sequence."""
    L = 1 << 19
    w = synthetic.varlen_inputs(111, Nq=1, Nkv=1, D=64, dtype="bf16", lengths_q=[L, L])
    assert w["Tq"] == 1 << 20
    go, gm, gl = _varlen(mi, w, 0.125)
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    for s0 in (0, L):
        for i in (0, 1, 4097, L // 2 + 3, L - 1):
            r = s0 + i
            wo, wm, wl = oracle.attn(q[r:r + 1, 0][None, None], k[s0:r + 1, 0][None, None],
                                     v[s0:r + 1, 0][None, None], 0.125, "none")
            check_out(go[r:r + 1, 0], wo[0, 0], "bf16", f"row {r}")
            check_stats(gm[0, r:r + 1], gl[0, r:r + 1], wm[0, 0], wl[0, 0])
    assert np.all(np.isfinite(go)) and np.all(gl >= 1.0 - 1e-6)


def test_2048_sequences(mi):
    """The largest accepted batch: 2048 sequences of 0..64 tokens, some empty."""
    rng = np.random.default_rng(112)
    lengths = rng.integers(0, 65, size=2048)
    lengths[0] = 64
    w = synthetic.varlen_inputs(113, Nq=2, Nkv=1, D=32, dtype="bf16", lengths_q=lengths)
    go, gm, gl = _varlen(mi, w, 1 / math.sqrt(32))
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 1 / math.sqrt(32), "causal")
    check_out(go, wo, "bf16")
    check_stats(gm, gl, wm, wl)


@pytest.mark.parametrize("Nkv", [256, 8, 1])
def test_256_query_heads(mi, Nkv):
    w = synthetic.dense_inputs(114, 1, 256, Nkv, 100, 130, 64, "bf16", "BSND")
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, "bf16")
    m, l = nan_stats((1, 256, 100)), nan_stats((1, 256, 100))
    mi.attn_fwd(q, k, v, out, m, l, 1, 256, Nkv, 100, 130, 64, "bf16", "BSND", 0.125, "causal")
    torch.cuda.synchronize()
    qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], "bf16"), "BSND", n)
                  for x, n in (("q", 256), ("k", Nkv), ("v", Nkv)))
    wo, wm, wl = oracle.attn(qo, ko, vo, 0.125, "causal")
    check_out(synthetic.to_bnsd(host_values(out), "BSND", 256), wo, "bf16")
    check_stats(host_values(m), host_values(l), wm, wl)


def test_single_head_131072_keys(mi):
    """Dense BNSD, one head, Sq = Skv = 131,072, D 128, causal: rows near the start, the
    middle and the end (the last one sees every key)."""
    S = 1 << 17
    w = synthetic.dense_inputs(115, 1, 1, 1, S, S, 128, "bf16", "BNSD")
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, "bf16")
    m, l = nan_stats((1, 1, S)), nan_stats((1, 1, S))
    mi.attn_fwd(q, k, v, out, m, l, 1, 1, 1, S, S, 128, "bf16", "BNSD", 1 / math.sqrt(128), "causal")
    torch.cuda.synchronize()
    go, gm, gl = host_values(out), host_values(m), host_values(l)
    qo, ko, vo = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    for i in (0, 255, 256, 70001, S - 1):
        wo, wm, wl = oracle.attn(qo[:, :, i:i + 1], ko[:, :, :i + 1], vo[:, :, :i + 1],
                                 1 / math.sqrt(128), "none")
        check_out(go[:, :, i:i + 1], wo, "bf16", f"row {i}")
        check_stats(gm[:, :, i:i + 1], gl[:, :, i:i + 1], wm, wl)


@pytest.mark.parametrize("B,route", [(16383, "tiled"), (32768, "general")])
def test_sbh_row_stride_beyond_32_bit_tiles(mi, B, route):
    """SBH bf16, S 64, N 8, D 128: the K / V row stride is B * 1024 elements.  At B 32768 a
    64-row tile spans 2^32 bytes, past the tiled kernel's 32-bit buffer range, so the call
    must run on the general kernel (64-bit indexing); just below the bound it stays tiled.
    Sampled batch entries (every head) against the oracle."""
    S, N, D = 64, 8, 128
    assert mi.attn_fwd_route(B, N, N, S, S, D, D, "bf16", "SBH", "causal") == route
    q = synthetic.device_normal((S, B, N * D), 116, "bf16")
    k = synthetic.device_normal((S, B, N * D), 117, "bf16")
    v = synthetic.device_normal((S, B, N * D), 118, "bf16")
    out = torch.full_like(q, float("nan"))
    m, l = nan_stats((B, N, S)), nan_stats((B, N, S))
    scale = 1 / math.sqrt(D)
    mi.attn_fwd(q, k, v, out, m, l, B, N, N, S, S, D, "bf16", "SBH", scale, "causal")
    torch.cuda.synchronize()
    for b in (0, 1, B // 2 + 7, B - 1):
        # the stored bits of batch entry b, read back: (S, N*D) -> (1, N, S, D)
        pick = lambda t: host_values(t[:, b]).reshape(S, N, D).transpose(1, 0, 2)[None]
        wo, wm, wl = oracle.attn(pick(q), pick(k), pick(v), scale, "causal")
        check_out(pick(out), wo, "bf16", f"batch entry {b}")
        check_stats(host_values(m[b])[None], host_values(l[b])[None], wm, wl)
    del q, k, v, out
    torch.cuda.empty_cache()
