"""GPU parity of attn_fwd_update / attn_fwd_varlen_update (attention over one key chunk
merged into a running result in the kernel's epilogue) against the CPU fp64 oracle.

Checked: random priors (with empty rows whose output buffer holds NaN, which must not be
read) x masks x layouts x dtypes x head dims at ragged sizes; in-place accumulation; a
four-chunk causal ring at full size (S 8192, N 32, D 128, SBH bf16) against full causal
attention (GPU) and the oracle (sampled heads); a packed batch whose keys arrive in five
chunks, each packed with its own cumulative lengths.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import TOL_OUT, check_out, check_stats, dev, empty_like_storage, host_values, nan_stats

pytestmark = pytest.mark.gpu

BIG = 1 << 40   # pre_tokens that excludes nothing


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _prior(seed, shape_out, stats_shape, dtype, empty_frac=0.05):
    """Random running result: out N(0,1) (float32, storage layout), max N(0,9), sum
    U(0.5, 50); a fraction of rows is empty (max -inf, sum 0).  Returns (out, m, l, empty)."""
    rng = np.random.default_rng(seed)
    o = rng.standard_normal(shape_out, dtype=np.float32)
    m = (rng.standard_normal(stats_shape, dtype=np.float32) * 3).astype(np.float32)
    l = rng.uniform(0.5, 50.0, stats_shape).astype(np.float32)
    e = rng.random(stats_shape) < empty_frac
    m[e], l[e] = -np.inf, 0.0
    return o, m, l, e


def _dense_case(seed, dtype, layout, D, B=2, Nq=4, Nkv=2, Sq=300, Skv=333):
    """Q/K/V of one chunk and a random prior: (inputs, prior out on the GPU with NaN in its
    empty rows, prior out for the oracle with 0 there, prior max, prior sum)."""
    w = synthetic.dense_inputs(seed, B, Nq, Nkv, Sq, Skv, D, dtype, layout)
    st = synthetic.storage_shape(layout, B, Nq, Sq, D)
    o, m, l, e = _prior(seed + 1000, st, (B, Nq, Sq), dtype)
    o_st = synthetic.to_storage(o, dtype)
    o_oracle = synthetic.to_bnsd(synthetic.storage_values(o_st, dtype), layout, Nq).copy()
    o_oracle[e] = 0.0
    # GPU copy: NaN in the empty rows (their weight is 0 and the kernel must not read them)
    o_gpu = dev(o_st, dtype)
    nan_rows = torch.from_numpy(synthetic.from_bnsd(np.broadcast_to(e[..., None], (B, Nq, Sq, D)).astype(np.float32), layout)).to("cuda:0")
    o_gpu = torch.where(nan_rows.reshape(o_gpu.shape) > 0, torch.full_like(o_gpu, float("nan")), o_gpu)
    return w, o_gpu, o_oracle, m, l


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("layout", ["BNSD", "SBH"])
@pytest.mark.parametrize("mask,pre,nxt", [("none", 0, 0), ("causal", 0, 0), ("band", 70, 33),
                                          ("band", BIG, -150)])
def test_update_random_prior(mi, dtype, D, layout, mask, pre, nxt):
    B, Nq, Nkv, Sq, Skv = 2, 4, 2, 300, 333
    w, o_gpu, o_or, m, l = _dense_case(51 + D, dtype, layout, D)
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    out = empty_like_storage(q.shape, dtype)
    mo, lo = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    mg, lg = torch.from_numpy(m).to("cuda:0"), torch.from_numpy(l).to("cuda:0")
    sc = 1 / math.sqrt(D)
    mi.attn_fwd_update(q, k, v, o_gpu, mg, lg, out, mo, lo, B, Nq, Nkv, Sq, Skv, D, dtype, layout,
                       sc, mask, pre, nxt)
    torch.cuda.synchronize()
    qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], dtype), layout, n)
                  for x, n in (("q", Nq), ("k", Nkv), ("v", Nkv)))
    wo, wm, wl = oracle.attn_update(qo, ko, vo, o_or, m, l, sc, mask, pre, nxt)
    check_out(synthetic.to_bnsd(host_values(out), layout, Nq), wo, dtype)
    check_stats(host_values(mo), host_values(lo), wm, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_update_in_place(mi, dtype):
    """out / stats alias the prior (the usual accumulation)."""
    B, Nq, Nkv, Sq, Skv, D, layout = 2, 4, 2, 300, 333, 128, "BSND"
    w, o_gpu, o_or, m, l = _dense_case(61, dtype, layout, D)
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    mg, lg = torch.from_numpy(m).to("cuda:0"), torch.from_numpy(l).to("cuda:0")
    mi.attn_fwd_update(q, k, v, o_gpu, mg, lg, o_gpu, mg, lg, B, Nq, Nkv, Sq, Skv, D, dtype,
                       layout, 0.088, "band", 100, 20)
    torch.cuda.synchronize()
    qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], dtype), layout, n)
                  for x, n in (("q", Nq), ("k", Nkv), ("v", Nkv)))
    wo, wm, wl = oracle.attn_update(qo, ko, vo, o_or, m, l, 0.088, "band", 100, 20)
    check_out(synthetic.to_bnsd(host_values(o_gpu), layout, Nq), wo, dtype)
    check_stats(host_values(mg), host_values(lg), wm, wl)


def test_update_rows_without_keys_keep_the_prior_exactly(mi):
    """A chunk that no row of the first 150 sees (band next = -150): those rows' output is
    the prior's stored value, bit for bit, and their statistics are unchanged."""
    B, Nq, Nkv, Sq, Skv, D, layout = 1, 2, 2, 300, 100, 64, "BNSD"
    w, o_gpu, o_or, m, l = _dense_case(62, "bf16", layout, D, B, Nq, Nkv, Sq, Skv)
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    mg, lg = torch.from_numpy(m).to("cuda:0"), torch.from_numpy(l).to("cuda:0")
    prior = host_values(o_gpu)
    out = empty_like_storage(q.shape, "bf16")
    mo, lo = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
    mi.attn_fwd_update(q, k, v, o_gpu, mg, lg, out, mo, lo, B, Nq, Nkv, Sq, Skv, D, "bf16", layout,
                       0.125, "band", BIG, -150)
    torch.cuda.synchronize()
    go = host_values(out)
    keep = l[:, :, :150] > 0
    assert np.array_equal(go[:, :, :150][keep], prior[:, :, :150][keep])
    assert np.all(go[:, :, :150][~keep] == 0)
    assert np.array_equal(host_values(mo)[:, :, :150], m[:, :, :150].astype(np.float64))
    assert np.array_equal(host_values(lo)[:, :, :150], l[:, :, :150].astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_in_place_update_by_a_chunk_the_first_tiles_do_not_see(mi, dtype):
    """In place, band(inf, -400): rows < 400 see no key, so whole 256-row tiles have nothing
    to do (the MFMA kernel skips them).  Those rows keep the prior bit for bit, rows with an
    empty prior (NaN in the buffer) become 0 / -inf / 0, and every row matches the oracle."""
    B, Nq, Nkv, Sq, Skv, D, layout = 1, 4, 2, 600, 100, 128, "BSND"
    w, o_gpu, o_or, m, l = _dense_case(63, dtype, layout, D, B, Nq, Nkv, Sq, Skv)
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    mg, lg = torch.from_numpy(m).to("cuda:0"), torch.from_numpy(l).to("cuda:0")
    prior = synthetic.to_bnsd(host_values(o_gpu), layout, Nq).copy()
    mi.attn_fwd_update(q, k, v, o_gpu, mg, lg, o_gpu, mg, lg, B, Nq, Nkv, Sq, Skv, D, dtype,
                       layout, 0.1, "band", BIG, -400)
    torch.cuda.synchronize()
    go = synthetic.to_bnsd(host_values(o_gpu), layout, Nq)
    gm, gl = host_values(mg), host_values(lg)
    qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], dtype), layout, n)
                  for x, n in (("q", Nq), ("k", Nkv), ("v", Nkv)))
    wo, wm, wl = oracle.attn_update(qo, ko, vo, o_or, m, l, 0.1, "band", BIG, -400)
    check_out(go, wo, dtype)
    check_stats(gm, gl, wm, wl)
    keep = l[:, :, :400] > 0
    assert np.array_equal(go[:, :, :400][keep], prior[:, :, :400][keep])
    assert np.all(go[:, :, :400][~keep] == 0)
    assert np.array_equal(gm[:, :, :400], m[:, :, :400].astype(np.float64))
    assert np.array_equal(gl[:, :, :400], l[:, :, :400].astype(np.float64))


def test_four_chunk_ring_equals_full_attention(mi):
    """S = 8192, N = 32, D = 128, SBH bf16: causal attention accumulated in place over four
    key chunks of 2048 (chunk j: band(inf, -2048 j)), starting from an empty result whose
    output buffer holds NaN, equals full causal attention: GPU vs GPU everywhere, and the
    oracle on sampled heads."""
    S, N, D, C = 8192, 32, 128, 2048
    w = synthetic.make("ring_merge_sbh_bf16_s8192_n32_d128")
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    sc = 1 / math.sqrt(D)
    out = empty_like_storage(q.shape, "bf16")
    m = torch.full((1, N, S), -float("inf"), device="cuda:0")
    l = torch.zeros((1, N, S), device="cuda:0")
    for j in range(S // C):
        kk, vv = k[j * C:(j + 1) * C].contiguous(), v[j * C:(j + 1) * C].contiguous()
        mi.attn_fwd_update(q, kk, vv, out, m, l, out, m, l, 1, N, N, S, C, D, "bf16", "SBH", sc,
                           "band", BIG, -j * C)
    full = empty_like_storage(q.shape, "bf16")
    mf, lf = nan_stats((1, N, S)), nan_stats((1, N, S))
    mi.attn_fwd(q, k, v, full, mf, lf, 1, N, N, S, S, D, "bf16", "SBH", sc, "causal")
    torch.cuda.synchronize()
    g_out = synthetic.to_bnsd(host_values(out), "SBH", N)
    g_full = synthetic.to_bnsd(host_values(full), "SBH", N)
    assert np.all(np.isfinite(g_out))
    assert np.max(np.abs(g_out - g_full)) <= TOL_OUT["bf16"]
    gm, gl = host_values(m), host_values(l)
    check_stats(gm, gl, host_values(mf), host_values(lf))
    qv, kv, vv = (synthetic.to_bnsd(synthetic.storage_values(w[x], "bf16"), "SBH", N)
                  for x in ("q", "k", "v"))
    rows = np.r_[0:128, 2040:2060, 4095:4100, 6100:6200, 8100:8192]
    for head in (3, 30):
        wo, wm, wl = oracle.attn(qv[:, head:head + 1], kv[:, head:head + 1], vv[:, head:head + 1],
                                 sc, "causal")
        check_out(g_out[:, head:head + 1, rows], wo[:, :, rows], "bf16", f"head {head}")
        check_stats(gm[:, head:head + 1, rows], gl[:, head:head + 1, rows], wm[:, :, rows],
                    wl[:, :, rows])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_varlen_chunked_ring_equals_full_attention(mi, dtype):
    """A packed batch whose keys arrive in chunks of 128 per sequence (chunk j = keys
    [128 j, 128 j + 128) of every sequence, packed with its own cumulative lengths),
    accumulated in place from an empty result, against the oracle's full causal attention."""
    lengths = np.array([300, 0, 1, 129, 517, 2])
    Nq, Nkv, D, C = 8, 2, 128, 128
    w = synthetic.varlen_inputs(71, Nq=Nq, Nkv=Nkv, D=D, dtype=dtype, lengths_q=lengths)
    T, B = w["Tq"], len(lengths)
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    starts = np.concatenate([[0], w["cu_q"][:-1]])
    out = empty_like_storage(q.shape, dtype)
    m = torch.full((Nq, T), -float("inf"), device="cuda:0")
    l = torch.zeros((Nq, T), device="cuda:0")
    sc = 1 / math.sqrt(D)
    for j in range(int(math.ceil(lengths.max() / C))):
        rows = [np.arange(s + min(C * j, n), s + min(C * (j + 1), n)) for s, n in zip(starts, lengths)]
        lk = np.array([len(r) for r in rows], dtype=np.int64)
        idx = torch.from_numpy(np.concatenate(rows).astype(np.int64)).to("cuda:0")
        kk, vv = k[idx].contiguous(), v[idx].contiguous()
        ck = torch.from_numpy(np.cumsum(lk)).to("cuda:0")
        mi.attn_fwd_varlen_update(q, kk, vv, out, m, l, out, m, l, cq, ck, B, T, int(lk.sum()),
                                  int(lengths.max()), int(max(lk.max(), 1)), Nq, Nkv, D, dtype, sc,
                                  "band", BIG, -C * j)
    torch.cuda.synchronize()
    qo, ko, vo = (synthetic.storage_values(w[x], dtype) for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen(qo, ko, vo, w["cu_q"], w["cu_kv"], sc, "causal")
    check_out(host_values(out), wo, dtype)
    check_stats(host_values(m), host_values(l), wm, wl)
