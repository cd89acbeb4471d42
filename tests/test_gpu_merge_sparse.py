"""GPU parity of attn_lse_merge and sparse_csr_attn against the CPU fp64 oracle.

The merge kernel is checked on seeded random partials (same values on both sides), and
end to end: two GPU partial forwards over the halves of K/V merged on the GPU against
the oracle's full causal attention.  The sparse kernel is checked on small patterns and
on the full-size band + random pattern (B 2, N 8, S 4096, D 64).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import (TOL_OUT, check_out, check_stats, dev, empty_like_storage, host_values,
                       nan_stats)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "paddle_sparse_attention_example.json")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _partials(seed, B, N, S, D, dtype, layout, sums="positive", empty_frac=0.0):
    """Seeded random partial results (out in `layout`, stats [B,N,S])."""
    rng = np.random.default_rng(seed)
    st = synthetic.storage_shape(layout, B, N, S, D)
    o1 = rng.standard_normal(st, dtype=np.float32)
    o2 = rng.standard_normal(st, dtype=np.float32)
    m1 = rng.standard_normal((B, N, S), dtype=np.float32) * 3
    m2 = rng.standard_normal((B, N, S), dtype=np.float32) * 3
    if sums == "positive":
        l1 = rng.uniform(0.5, 50.0, (B, N, S)).astype(np.float32)
        l2 = rng.uniform(0.5, 50.0, (B, N, S)).astype(np.float32)
    else:
        l1 = rng.standard_normal((B, N, S), dtype=np.float32)
        l2 = rng.standard_normal((B, N, S), dtype=np.float32)
    if empty_frac:
        e1 = rng.random((B, N, S)) < empty_frac
        e2 = rng.random((B, N, S)) < empty_frac
        m1[e1], l1[e1] = -np.inf, 0.0
        m2[e2], l2[e2] = -np.inf, 0.0
    o1, o2 = synthetic.to_storage(o1, dtype), synthetic.to_storage(o2, dtype)
    return o1, m1, l1, o2, m2, l2


def _merge_gpu(mi, parts, B, N, S, D, dtype, layout, alias=False):
    o1, m1, l1, o2, m2, l2 = parts
    t = [dev(o1, dtype), dev(m1, "f32"), dev(l1, "f32"), dev(o2, dtype), dev(m2, "f32"), dev(l2, "f32")]
    if alias:
        out, mo, lo = t[0], t[1], t[2]
    else:
        out, mo, lo = empty_like_storage(t[0].shape, dtype), nan_stats((B, N, S)), nan_stats((B, N, S))
    mi.attn_lse_merge(*t, out, mo, lo, B, N, S, D, dtype, layout)
    torch.cuda.synchronize()
    return host_values(out), host_values(mo), host_values(lo)


def _merge_oracle(parts, N, dtype, layout):
    o1, m1, l1, o2, m2, l2 = parts
    a = synthetic.to_bnsd(synthetic.storage_values(o1, dtype), layout, N)
    b = synthetic.to_bnsd(synthetic.storage_values(o2, dtype), layout, N)
    return oracle.merge(a, m1, l1, b, m2, l2)


@pytest.mark.parametrize("layout", ["SBH", "BNSD", "BSND"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [128, 64, 1, 12])
def test_merge_random_partials(mi, layout, dtype, D):
    B, N, S = 2, 4, 333
    parts = _partials(31 + D, B, N, S, D, dtype, layout, empty_frac=0.05)
    go, gm, gl = _merge_gpu(mi, parts, B, N, S, D, dtype, layout)
    wo, wm, wl = _merge_oracle(parts, N, dtype, layout)
    check_out(synthetic.to_bnsd(go, layout, N), wo, dtype)
    assert np.array_equal(gm, wm.astype(np.float32).astype(np.float64))  # max is exact
    check_stats(gm, gl, wm, wl)


def test_merge_ring_update_example_shape(mi):
    """The ring-update page's example shape: out [2048, 1, 12] bf16 (N = 12, D = 1) with
    random stats whose sums may be negative.  Rows whose merged sum is near zero are
    ill-conditioned (the weights blow up); the comparison is relative there."""
    B, N, S, D = 1, 12, 2048, 1
    parts = _partials(41, B, N, S, D, "bf16", "SBH", sums="randn")
    go, gm, gl = _merge_gpu(mi, parts, B, N, S, D, "bf16", "SBH")
    wo, wm, wl = _merge_oracle(parts, N, "bf16", "SBH")
    go = synthetic.to_bnsd(go, "SBH", N)
    ok = np.abs(wl) > 1e-2
    err = np.abs(go - wo)[..., 0][ok] / np.maximum(1.0, np.abs(wo[..., 0][ok]))
    assert np.max(err) <= 2 ** -7
    assert np.array_equal(gm, wm.astype(np.float32).astype(np.float64))
    assert np.max(np.abs(gl - wl) / np.maximum(1.0, np.abs(wl))) <= 1e-5


def test_merge_in_place(mi):
    B, N, S, D = 1, 32, 8192, 128
    parts = _partials(42, B, N, S, D, "bf16", "SBH", empty_frac=0.01)
    go, gm, gl = _merge_gpu(mi, parts, B, N, S, D, "bf16", "SBH", alias=True)
    wo, wm, wl = _merge_oracle(parts, N, "bf16", "SBH")
    check_out(synthetic.to_bnsd(go, "SBH", N), wo, "bf16")
    check_stats(gm, gl, wm, wl)


def test_ring_halves_merge_equals_full_attention(mi):
    """S = 8192, N = 32, D = 128, SBH bf16: partial A = causal over K/V[:4096], partial B =
    band(pre=inf, next=-4096) over K/V[4096:] (rows < 4096 see nothing there); the merge
    must equal full causal attention.  Oracle on sampled heads; GPU-vs-GPU everywhere."""
    S, N, D, h = 8192, 32, 128, 4096
    w = synthetic.make("ring_merge_sbh_bf16_s8192_n32_d128")
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    sc = 1 / math.sqrt(D)
    outs = []
    for (ks, mask, pre, nxt) in ((slice(0, h), "causal", 0, 0), (slice(h, S), "band", 1 << 62, -h),
                                 (slice(0, S), "causal", 0, 0)):
        kk, vv = k[ks].contiguous(), v[ks].contiguous()
        o = empty_like_storage(q.shape, "bf16")
        m, l = nan_stats((1, N, S)), nan_stats((1, N, S))
        mi.attn_fwd(q, kk, vv, o, m, l, 1, N, N, S, kk.shape[0], D, "bf16", "SBH", sc, mask, pre, nxt)
        outs.append((o, m, l))
    (oa, ma, la), (ob, mb, lb), (of, mf, lf) = outs
    out, mo, lo = empty_like_storage(q.shape, "bf16"), nan_stats((1, N, S)), nan_stats((1, N, S))
    mi.attn_lse_merge(oa, ma, la, ob, mb, lb, out, mo, lo, 1, N, S, D, "bf16", "SBH")
    torch.cuda.synchronize()
    hb_l = host_values(lb)
    assert np.all(hb_l[:, :, :h] == 0) and np.all(host_values(mb)[:, :, :h] == -np.inf)
    g_out = synthetic.to_bnsd(host_values(out), "SBH", N)
    g_full = synthetic.to_bnsd(host_values(of), "SBH", N)
    assert np.max(np.abs(g_out - g_full)) <= TOL_OUT["bf16"]
    check_stats(host_values(mo), host_values(lo), host_values(mf), host_values(lf))
    # oracle on sampled heads: rows of both halves
    qv = synthetic.to_bnsd(synthetic.storage_values(w["q"], "bf16"), "SBH", N)
    kv = synthetic.to_bnsd(synthetic.storage_values(w["k"], "bf16"), "SBH", N)
    vv = synthetic.to_bnsd(synthetic.storage_values(w["v"], "bf16"), "SBH", N)
    for head in (0, 21):
        rows = np.r_[0:256, 4000:4200, 8000:8192]
        sel = np.zeros(S, dtype=bool)
        sel[rows] = True
        wo, wm, wl = oracle.attn(qv[:, head:head + 1], kv[:, head:head + 1], vv[:, head:head + 1], sc, "causal")
        check_out(g_out[:, head:head + 1, sel], wo[:, :, sel], "bf16", f"head {head}")
        check_stats(host_values(mo)[:, head:head + 1, sel], host_values(lo)[:, head:head + 1, sel],
                    wm[:, :, sel], wl[:, :, sel])


def _sparse_gpu(mi, w, scale, dtype="f32"):
    q, k, v = (dev(w[x], dtype) for x in ("q", "k", "v"))
    off = torch.from_numpy(np.ascontiguousarray(w["offset"])).to("cuda:0")
    col = torch.from_numpy(np.ascontiguousarray(w["columns"])).to("cuda:0")
    out = empty_like_storage(q.shape, dtype)
    mi.sparse_csr_attn(q, k, v, out, off, col, w["nnz"], w["B"], w["N"], w["S"], w["D"], dtype, scale)
    torch.cuda.synchronize()
    return host_values(out)


# head dims: the compile-time sizes (32, 64, 96, 128) and every run-time class (values per
# lane 1, 2, 4, 8, 12), odd dims (scalar K reads) and even ones, up to the 768 limit
SPARSE_DIMS = [1, 2, 3, 8, 17, 32, 64, 77, 96, 100, 128, 130, 200, 256, 257, 384, 511, 512,
               513, 640, 766, 768]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("D", SPARSE_DIMS)
def test_sparse_small(mi, D, dtype):
    """Band 16 + 80 random columns per row, S 300 (a ragged last block of rows)."""
    w = synthetic.sparse_inputs(51 + D, 2, 3, 300, D, band=16, n_random=80, dtype=dtype)
    # the entry point takes a float scale: the oracle gets the same float value
    sc = float(np.float32(1 / math.sqrt(D)))
    go = _sparse_gpu(mi, w, sc, dtype)
    wo, _, _ = oracle.sparse(w["q"], w["k"], w["v"], w["offset"], w["columns"], sc)
    check_out(go, wo, dtype, f"D {D}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("D", [64, 768])
def test_sparse_band_wider_than_the_window(mi, D, dtype):
    """A band of 300 keys: at D 64 the LDS window holds the 128 keys before each row of a
    block, at D 768 only a few (fp32 15, fp64 3), so most entries are gathered from global
    memory next to window reads, in the same chunks."""
    w = synthetic.sparse_inputs(60 + D, 1, 2, 700, D, band=300, n_random=20, dtype=dtype)
    sc = float(np.float32(1 / math.sqrt(D)))
    go = _sparse_gpu(mi, w, sc, dtype)
    wo, _, _ = oracle.sparse(w["q"], w["k"], w["v"], w["offset"], w["columns"], sc)
    check_out(go, wo, dtype, f"D {D}")


def test_sparse_no_locality(mi):
    """Every row lists 150 uniformly random columns of the whole slice (unsorted, repeats
    allowed): entries in and out of the window in the same chunk."""
    rng = np.random.default_rng(61)
    S, D, N = 500, 64, 2
    q, k, v = (rng.standard_normal((1, N, S, D), dtype=np.float32) for _ in range(3))
    cnt = 150
    offset = np.broadcast_to(np.arange(S + 1, dtype=np.int32) * cnt, (1, N, S + 1)).copy()
    columns = rng.integers(0, S, size=(1, N, S * cnt)).astype(np.int32)
    w = dict(q=q, k=k, v=v, offset=offset, columns=columns, nnz=S * cnt, B=1, N=N, S=S, D=D)
    go = _sparse_gpu(mi, w, 0.125)
    wo, _, _ = oracle.sparse(q, k, v, offset, columns, 0.125)
    check_out(go, wo, "f32")


def test_sparse_unaligned_key_pointer(mi):
    """A K pointer 4 bytes past a 16-byte boundary takes the scalar-read kernel."""
    w = synthetic.sparse_inputs(62, 1, 2, 200, 64, band=32, n_random=30, dtype="f32")
    q, v = dev(w["q"], "f32"), dev(w["v"], "f32")
    kbuf = torch.zeros(w["k"].size + 1, dtype=torch.float32, device="cuda:0")
    kbuf[1:] = torch.from_numpy(np.ascontiguousarray(w["k"]).reshape(-1)).to("cuda:0")
    k = kbuf[1:]
    assert k.data_ptr() % 16 == 4
    off = torch.from_numpy(np.ascontiguousarray(w["offset"])).to("cuda:0")
    col = torch.from_numpy(np.ascontiguousarray(w["columns"])).to("cuda:0")
    out = empty_like_storage(q.shape, "f32")
    mi.sparse_csr_attn(q, k, v, out, off, col, w["nnz"], 1, 2, 200, 64, "f32", 0.125)
    torch.cuda.synchronize()
    wo, _, _ = oracle.sparse(w["q"], w["k"], w["v"], w["offset"], w["columns"], 0.125)
    check_out(host_values(out), wo, "f32")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_sparse_paddle_example(mi, dtype):
    """The Paddle sparse_attention worked example on the GPU at its own shape [1, 1, 4, 2],
    against the output the page prints (fp32 to 8 decimals) and the oracle."""
    fx = json.load(open(GOLDEN))
    npdt = np.float32 if dtype == "f32" else np.float64
    x = np.array(fx["query"], dtype=npdt).reshape(fx["shape"])
    assert np.array_equal(x, np.array(fx["key"], npdt).reshape(fx["shape"]))
    w = dict(q=x, k=x, v=x, offset=np.array(fx["offset"], np.int32).reshape(1, 1, 5),
             columns=np.array(fx["columns"], np.int32).reshape(1, 1, 8), nnz=8, B=1, N=1, S=4, D=2)
    sc = float(np.float32(1 / math.sqrt(2)))
    go = _sparse_gpu(mi, w, sc, dtype)
    printed = np.array(fx["printed_output"])
    assert np.max(np.abs(go[0, 0] - printed)) < 1e-6
    wo, _, _ = oracle.sparse(w["q"], w["k"], w["v"], w["offset"], w["columns"], sc)
    check_out(go, wo, dtype)


def test_sparse_empty_rows_and_duplicates(mi):
    rng = np.random.default_rng(52)
    S, D = 70, 64
    q, k, v = (rng.standard_normal((1, 2, S, D), dtype=np.float32) for _ in range(3))
    offs, cols = [], []
    for n in range(2):
        off, col = [0], []
        for i in range(S):
            cnt = 0 if i % 5 == 0 else int(rng.integers(1, 150))
            col += list(rng.integers(0, S, size=cnt))    # repeats allowed
            off.append(len(col))
        offs.append(off)
        cols.append(col)
    nnz = max(len(c) for c in cols)
    columns = np.zeros((1, 2, nnz), np.int32)
    for n in range(2):
        columns[0, n, :len(cols[n])] = cols[n]
    w = dict(q=q, k=k, v=v, offset=np.array(offs, np.int32).reshape(1, 2, S + 1), columns=columns,
             nnz=nnz, B=1, N=2, S=S, D=D)
    go = _sparse_gpu(mi, w, 0.125)
    wo, _, _ = oracle.sparse(q, k, v, w["offset"], columns, 0.125)
    check_out(go, wo, "f32")
    assert np.all(go[0, :, ::5] == 0)


@pytest.fixture(scope="module")
def sparse_full(mi):
    w = synthetic.make("csr_sparse_f32_b2n8s4096d64")
    return w, _sparse_gpu(mi, w, 1 / math.sqrt(64))


def test_sparse_full_workload(sparse_full):
    w, go = sparse_full
    assert w["nnz"] == 768096
    wo, _, _ = oracle.sparse(w["q"], w["k"], w["v"], w["offset"], w["columns"], 1 / math.sqrt(64))
    check_out(go, wo, "f32")


def test_sparse_full_workload_f64(mi):
    """The full CSR workload (same seed and pattern) with fp64 inputs and arithmetic."""
    w = synthetic.sparse_inputs(0, 2, 8, 4096, 64, band=128, n_random=64, dtype="f64")
    assert w["nnz"] == 768096
    go = _sparse_gpu(mi, w, 0.125, "f64")
    wo, _, _ = oracle.sparse(w["q"], w["k"], w["v"], w["offset"], w["columns"], 0.125)
    check_out(go, wo, "f64")


def test_sparse_deterministic(mi, sparse_full):
    w, go = sparse_full
    assert np.array_equal(_sparse_gpu(mi, w, 1 / math.sqrt(64)), go)
