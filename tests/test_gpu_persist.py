"""GPU parity of the persistent causal forward (one workgroup per CU walking a static list of
work items of R rows x HPI query heads).

Every case runs twice through the C ABI, once on the persistent kernel and once with
MIATTN_PERSIST=0 on the tiled kernel, and the two results must be identical bit for bit:
each output row is computed by the same per-row arithmetic in both (the same key tiles in
the same order, the same lazy rescale), only the grouping of rows into workgroups and the
schedule differ.  The cases that only this path has (GQA groups packed into one item,
items that see no key, many sequences, both causal alignments) are also compared with the
CPU fp64 oracle at the tolerances of tests/gpu_utils.py.
"""
import math
import os

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


def _both(run):
    """run() on the persistent kernel and on the tiled one."""
    os.environ.pop("MIATTN_PERSIST", None)
    a = run()
    os.environ["MIATTN_PERSIST"] = "0"
    try:
        b = run()
    finally:
        os.environ.pop("MIATTN_PERSIST", None)
    return a, b


def _varlen_run(mi, w, mask="causal"):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    mq = max(1, int(w["lengths_q"].max()))
    mk = max(1, int(w["lengths_kv"].max()))
    scale = 1 / math.sqrt(w["D"])

    def run():
        out = empty_like_storage(q.shape, dt)
        m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
        mi.attn_fwd_varlen(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"], mq, mk,
                           w["Nq"], w["Nkv"], w["D"], dt, scale, mask)
        torch.cuda.synchronize()
        return host_values(out), host_values(m), host_values(l)
    return run


def _assert_identical(a, b, what):
    for x, y, name in zip(a, b, ("out", "softmax_max", "softmax_sum")):
        assert np.array_equal(x, y, equal_nan=False), f"{what}: {name} differs from the tiled kernel"


def _oracle_varlen(w, mask):
    q, k, v = (synthetic.storage_values(w[x], w["dtype"]) for x in ("q", "k", "v"))
    if mask == "causal":
        return oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 1 / math.sqrt(w["D"]), "causal")
    return oracle.attn_varlen_keep(
        q, k, v, w["cu_q"], w["cu_kv"],
        lambda b, sq, sk: oracle.keep_band(sq, sk, 1 << 62, 0, "bottom_right"), 1 / math.sqrt(w["D"]))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_full_workload_matches_tiled_bit_for_bit(mi, dtype):
    """The 16-sequence packed causal GQA workload (T = 33,064, Nq 32, Nkv 8, D 128)."""
    w = synthetic.varlen_inputs(0, Nq=32, Nkv=8, D=128, dtype=dtype, B=16)
    assert mi.attn_fwd_route(1, 32, 8, 4096, 4096, 128, 128, dtype, "BSND", "causal") == "persistent"
    a, b = _both(_varlen_run(mi, w))
    _assert_identical(a, b, f"full workload {dtype}")


@pytest.mark.parametrize("Nq,Nkv", [(8, 8), (8, 4), (8, 2), (8, 1), (16, 1), (6, 2), (12, 2), (24, 8)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", ["causal", "causal_br"])
def test_gqa_packing_against_oracle_and_tiled(mi, Nq, Nkv, D, mask):
    """GQA ratios 1, 2, 4, 8, 16, 3, 6, 3 (heads per item 1, 2, 4, 8, 8, 1, 2, 1); query and
    key lengths that differ per sequence, with zeros on either side (items without a key)."""
    lq = [300, 0, 1, 129, 64, 517, 2, 65, 190]
    lk = [300, 40, 0, 200, 64, 400, 2, 65, 3]
    w = synthetic.varlen_inputs(400 + Nq + 10 * Nkv + D, Nq=Nq, Nkv=Nkv, D=D, dtype="bf16",
                                lengths_q=lq, lengths_kv=lk)
    a, b = _both(_varlen_run(mi, w, mask))
    _assert_identical(a, b, f"Nq {Nq} Nkv {Nkv} D {D} {mask}")
    wo, wm, wl = _oracle_varlen(w, mask)
    check_out(a[0], wo, "bf16", f"Nq {Nq} Nkv {Nkv} D {D} {mask}")
    check_stats(a[1], a[2], wm, wl)


def test_512_sequences(mi):
    """The largest packed batch the persistent kernel takes (its workgroups sort the
    sequence lengths in LDS), lengths 0..300."""
    rng = np.random.default_rng(410)
    lengths = rng.integers(0, 301, size=512)
    w = synthetic.varlen_inputs(411, Nq=4, Nkv=1, D=64, dtype="f16", lengths_q=lengths)
    a, b = _both(_varlen_run(mi, w))
    _assert_identical(a, b, "512 sequences")
    wo, wm, wl = _oracle_varlen(w, "causal")
    check_out(a[0], wo, "f16")
    check_stats(a[1], a[2], wm, wl)


def test_513_sequences_take_the_tiled_kernel(mi):
    """One sequence more than the persistent kernel sorts: the tiled kernel serves it, with
    the same result."""
    rng = np.random.default_rng(412)
    lengths = rng.integers(0, 70, size=513)
    w = synthetic.varlen_inputs(413, Nq=2, Nkv=2, D=128, dtype="bf16", lengths_q=lengths)
    a, b = _both(_varlen_run(mi, w))
    _assert_identical(a, b, "513 sequences")


@pytest.mark.parametrize("layout", ["BNSD", "SBH", "BSND"])
@pytest.mark.parametrize("Nq,Nkv", [(4, 4), (8, 2)])
def test_dense_batches(mi, layout, Nq, Nkv):
    """Dense causal batches (every sequence the same length): 3 x 700 queries over 700 keys
    top-left, and 3 x 300 queries over 700 keys bottom-right."""
    for Sq, Skv, mask in ((700, 700, "causal"), (300, 700, "causal_br")):
        w = synthetic.dense_inputs(420 + Sq + Nq, 3, Nq, Nkv, Sq, Skv, 128, "bf16", layout)
        q, k, v = dev(w["q"], "bf16"), dev(w["k"], "bf16"), dev(w["v"], "bf16")

        def run():
            out = empty_like_storage(q.shape, "bf16")
            m, l = nan_stats((3, Nq, Sq)), nan_stats((3, Nq, Sq))
            mi.attn_fwd(q, k, v, out, m, l, 3, Nq, Nkv, Sq, Skv, 128, "bf16", layout,
                        1 / math.sqrt(128), mask)
            torch.cuda.synchronize()
            return host_values(out), host_values(m), host_values(l)
        a, b = _both(run)
        _assert_identical(a, b, f"dense {layout} {Sq}x{Skv} {mask}")
        qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], "bf16"), layout, n)
                      for x, n in (("q", Nq), ("k", Nkv), ("v", Nkv)))
        keep = oracle.keep_band(Sq, Skv, 1 << 62, 0, "bottom_right" if mask == "causal_br" else "top_left")
        wo, wm, wl = oracle.attn_keep(qo, ko, vo, keep, 1 / math.sqrt(128))
        check_out(synthetic.to_bnsd(a[0], layout, Nq), wo, "bf16", f"dense {layout} {mask}")
        check_stats(a[1], a[2], wm, wl)


def test_stats_may_be_null_and_outputs_stay_in_bounds(mi):
    """NULL statistics on the persistent path, and canaries around the output buffer."""
    w = synthetic.varlen_inputs(430, Nq=8, Nkv=2, D=128, dtype="bf16", lengths_q=[333, 64, 1])
    q, k, v = (dev(w[x], "bf16") for x in ("q", "k", "v"))
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    pad = 8192
    buf = torch.full((q.numel() + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda:0")
    out = buf[pad:pad + q.numel()].view(q.shape)
    mi.attn_fwd_varlen(q, k, v, out, None, None, cq, cq, 3, w["Tq"], w["Tq"], 333, 333, 8, 2, 128,
                       "bf16", 1 / math.sqrt(128), "causal")
    torch.cuda.synchronize()
    hb = host_values(buf)
    assert np.all(hb[:pad] == 7.0) and np.all(hb[pad + q.numel():] == 7.0)
    wo, _, _ = _oracle_varlen(w, "causal")
    check_out(host_values(out), wo, "bf16")


def test_deterministic(mi):
    w = synthetic.varlen_inputs(431, Nq=16, Nkv=4, D=128, dtype="bf16", lengths_q=[1000, 333, 77, 2048])
    run = _varlen_run(mi, w)
    a, b = run(), run()
    _assert_identical(a, b, "repeat")


def _varlen_band_run(mi, w, mask, pre, nxt):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    mq = max(1, int(w["lengths_q"].max()))
    mk = max(1, int(w["lengths_kv"].max()))
    scale = 1 / math.sqrt(w["D"])

    def run():
        out = empty_like_storage(q.shape, dt)
        m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
        mi.attn_fwd_varlen(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"], mq, mk,
                           w["Nq"], w["Nkv"], w["D"], dt, scale, mask, pre, nxt)
        torch.cuda.synchronize()
        return host_values(out), host_values(m), host_values(l)
    return run


# masks whose visible keys start at key 0: no mask, and bands without a lower bound whose
# upper bound moves the causal diagonal up (33), down (-70: rows near the top see nothing)
# or, bottom-right aligned, by -5
OPEN_MASKS = [("none", 0, 0), ("band", 1 << 40, 33), ("band", 1 << 40, -70), ("band_br", 1 << 40, -5)]


@pytest.mark.parametrize("mask,pre,nxt", OPEN_MASKS)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nkv", [(8, 2), (6, 6)])
def test_open_masks_against_oracle_and_tiled(mi, mask, pre, nxt, D, Nq, Nkv):
    """Packed batches with query and key lengths that differ per sequence (zeros included):
    the persistent kernel equals the tiled one bit for bit and the oracle within tolerance."""
    lq = [300, 0, 1, 129, 64, 517, 2, 65, 190]
    lk = [300, 40, 0, 200, 64, 400, 2, 65, 3]
    w = synthetic.varlen_inputs(500 + D + Nq + len(mask) + (nxt & 0xff), Nq=Nq, Nkv=Nkv, D=D,
                                dtype="bf16", lengths_q=lq, lengths_kv=lk)
    a, b = _both(_varlen_band_run(mi, w, mask, pre, nxt))
    _assert_identical(a, b, f"{mask} {pre} {nxt} D {D}")
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    align = "bottom_right" if mask.endswith("_br") else "top_left"
    nxt_o = (1 << 62) if mask == "none" else nxt
    wo, wm, wl = oracle.attn_varlen_keep(
        q, k, v, w["cu_q"], w["cu_kv"],
        lambda bb, sq, sk: oracle.keep_band(sq, sk, 1 << 62, nxt_o, align), 1 / math.sqrt(D))
    check_out(a[0], wo, "bf16", f"{mask} {nxt} D {D}")
    check_stats(a[1], a[2], wm, wl)


@pytest.mark.parametrize("layout", ["BNSD", "SBH"])
def test_dense_no_mask(mi, layout):
    """Dense batches without a mask (the multi-head module's attention), 3 x 700 queries
    over 900 keys, GQA 8 / 2, D 64 in fp16 and D 128 in bf16."""
    for D, dt in ((64, "f16"), (128, "bf16")):
        assert mi.attn_fwd_route(3, 8, 2, 700, 900, D, D, dt, layout, "none") == "persistent"
        w = synthetic.dense_inputs(530 + D, 3, 8, 2, 700, 900, D, dt, layout)
        q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)

        def run():
            out = empty_like_storage(q.shape, dt)
            m, l = nan_stats((3, 8, 700)), nan_stats((3, 8, 700))
            mi.attn_fwd(q, k, v, out, m, l, 3, 8, 2, 700, 900, D, dt, layout, 1 / math.sqrt(D), "none")
            torch.cuda.synchronize()
            return host_values(out), host_values(m), host_values(l)
        a, b = _both(run)
        _assert_identical(a, b, f"dense none {layout} D {D}")
        qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], dt), layout, n)
                      for x, n in (("q", 8), ("k", 2), ("v", 2)))
        wo, wm, wl = oracle.attn(qo, ko, vo, 1 / math.sqrt(D), "none")
        check_out(synthetic.to_bnsd(a[0], layout, 8), wo, dt, f"dense none {layout} D {D}")
        check_stats(a[1], a[2], wm, wl)


def _varlen_prefix_run(mi, w, mask, prefix):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    pf = torch.from_numpy(np.asarray(prefix, np.int64)).to("cuda:0")
    mq = max(1, int(w["lengths_q"].max()))
    mk = max(1, int(w["lengths_kv"].max()))
    D = w["D"]

    def run():
        out = empty_like_storage(q.shape, dt)
        m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
        mi.attn_fwd_varlen_ext(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"], mq, mk,
                               w["Nq"], w["Nkv"], D, D, dt, 1 / math.sqrt(D), mask, 0, 0, pf, None)
        torch.cuda.synchronize()
        return host_values(out), host_values(m), host_values(l)
    return run


def _keep_prefix(mask, prefix):
    """Visibility of sequence b under causal (top-left) or bottom-right causal plus the prefix
    clamped to [0, Skv] (the oracle's own definitions)."""
    def keep(b, sq, sk):
        pfx = min(max(int(prefix[b]), 0), sk)
        if mask == "causal_br":
            return oracle.keep_prefix_causal(sq, sk, pfx)
        return oracle.keep_band(sq, sk, 1 << 62, 0) | (np.arange(sk)[None, :] < pfx)
    return keep


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nkv", [(8, 2), (6, 6)])
def test_prefix_against_oracle_and_tiled(mi, mask, D, Nq, Nkv):
    """A per-sequence prefix (keys below it visible from every row) on packed batches whose
    query and key lengths differ per sequence: prefixes of 0, inside the first key tile,
    across tiles, past the keys (clamped) and negative (clamped to 0), so that some items
    see more key tiles than their causal diagonal and some rows see only prefix keys.  The
    persistent kernel equals the tiled one bit for bit and the oracle within tolerance."""
    lq = [300, 0, 1, 129, 64, 517, 2, 65, 190]
    lk = [300, 40, 0, 200, 64, 400, 2, 65, 3]
    prefix = [200, 7, 5, 150, 0, 333, -4, 64, 900]
    w = synthetic.varlen_inputs(540 + D + Nq + len(mask), Nq=Nq, Nkv=Nkv, D=D, dtype="bf16",
                                lengths_q=lq, lengths_kv=lk)
    a, b = _both(_varlen_prefix_run(mi, w, mask, prefix))
    _assert_identical(a, b, f"prefix {mask} D {D}")
    q, k, v = (synthetic.storage_values(w[x], "bf16") for x in ("q", "k", "v"))
    wo, wm, wl = oracle.attn_varlen_keep(q, k, v, w["cu_q"], w["cu_kv"], _keep_prefix(mask, prefix),
                                         1 / math.sqrt(D))
    check_out(a[0], wo, "bf16", f"prefix {mask} D {D}")
    check_stats(a[1], a[2], wm, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_full_workload_prefix_matches_tiled_bit_for_bit(mi, dtype):
    """The 16-sequence packed causal GQA workload with a prefix of a third of each sequence
    (bottom-right causal): persistent and tiled kernels agree bit for bit; sampled
    (sequence, head) slices against the oracle."""
    w = synthetic.varlen_inputs(0, Nq=32, Nkv=8, D=128, dtype=dtype, B=16)
    prefix = [int(L) // 3 for L in w["lengths_kv"]]
    a, b = _both(_varlen_prefix_run(mi, w, "causal_br", prefix))
    _assert_identical(a, b, f"full workload prefix {dtype}")
    q, k, v = (synthetic.storage_values(w[x], dtype) for x in ("q", "k", "v"))
    cu = w["cu_q"]
    keep = _keep_prefix("causal_br", prefix)
    for s, h in ((0, 0), (5, 17), (11, 31), (15, 8)):
        lo, hi = (int(cu[s - 1]) if s else 0), int(cu[s])
        if hi == lo:
            continue
        hk = h // 4
        wo, wm, wl = oracle.attn_keep(q[lo:hi, h][None, None], k[lo:hi, hk][None, None],
                                      v[lo:hi, hk][None, None], keep(s, hi - lo, hi - lo),
                                      1 / math.sqrt(128))
        check_out(a[0][lo:hi, h], wo[0, 0], dtype, f"prefix seq {s} head {h}")
        check_stats(a[1][h, lo:hi], a[2][h, lo:hi], wm[0, 0], wl[0, 0])


@pytest.mark.parametrize("layout", ["BNSD", "SBH"])
def test_dense_prefix_against_oracle_and_tiled(mi, layout):
    """Dense batches with a prefix per batch entry (0, inside the diagonal, past Skv),
    causal top-left with Sq < Skv, GQA 8 / 2, D 128 bf16."""
    B, Nq, Nkv, Sq, Skv, D = 3, 8, 2, 500, 700, 128
    prefix = [0, 300, 1000]
    w = synthetic.dense_inputs(560, B, Nq, Nkv, Sq, Skv, D, "bf16", layout)
    q, k, v = dev(w["q"], "bf16"), dev(w["k"], "bf16"), dev(w["v"], "bf16")
    pf = torch.from_numpy(np.asarray(prefix, np.int64)).to("cuda:0")

    def run():
        out = empty_like_storage(q.shape, "bf16")
        m, l = nan_stats((B, Nq, Sq)), nan_stats((B, Nq, Sq))
        mi.attn_fwd_ext(q, k, v, out, m, l, B, Nq, Nkv, Sq, Skv, D, D, "bf16", layout,
                        1 / math.sqrt(D), "causal", 0, 0, pf, None)
        torch.cuda.synchronize()
        return host_values(out), host_values(m), host_values(l)
    a, b = _both(run)
    _assert_identical(a, b, f"dense prefix {layout}")
    qo, ko, vo = (synthetic.to_bnsd(synthetic.storage_values(w[x], "bf16"), layout, n)
                  for x, n in (("q", Nq), ("k", Nkv), ("v", Nkv)))
    keep = np.stack([_keep_prefix("causal", prefix)(bb, Sq, Skv) for bb in range(B)])
    wo, wm, wl = oracle.attn_keep(qo, ko, vo, keep, 1 / math.sqrt(D))
    check_out(synthetic.to_bnsd(a[0], layout, Nq), wo, "bf16", f"dense prefix {layout}")
    check_stats(a[1], a[2], wm, wl)


def _varlen_dropout_run(mi, w, mask, p, seed, offset, prefix=None):
    dt = w["dtype"]
    q, k, v = dev(w["q"], dt), dev(w["k"], dt), dev(w["v"], dt)
    cq = torch.from_numpy(w["cu_q"]).to("cuda:0")
    ck = torch.from_numpy(w["cu_kv"]).to("cuda:0")
    pf = None if prefix is None else torch.from_numpy(np.asarray(prefix, np.int64)).to("cuda:0")
    mq = max(1, int(w["lengths_q"].max()))
    mk = max(1, int(w["lengths_kv"].max()))
    D = w["D"]

    def run():
        out = empty_like_storage(q.shape, dt)
        m, l = nan_stats((w["Nq"], w["Tq"])), nan_stats((w["Nq"], w["Tq"]))
        mi.attn_fwd_varlen_ext(q, k, v, out, m, l, cq, ck, w["B"], w["Tq"], w["Tkv"], mq, mk,
                               w["Nq"], w["Nkv"], D, D, dt, 1 / math.sqrt(D), mask, 0, 0, pf, None,
                               p, seed, offset)
        torch.cuda.synchronize()
        return host_values(out), host_values(m), host_values(l)
    return run


@pytest.mark.parametrize("mask", ["causal", "causal_br"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nkv", [(8, 2), (6, 6)])
def test_dropout_matches_tiled_bit_for_bit(mi, mask, D, Nq, Nkv):
    """Dropout on the persistent kernel draws the tiled kernel's Philox4x32-10 counters
    (key block, sequence-local row, head + 256 sequence, offset): on packed batches with
    ragged lengths (zeros included), with and without a prefix, both kernels drop the same
    entries and give identical outputs and statistics."""
    lq = [300, 0, 1, 129, 64, 517, 2, 65, 190]
    lk = [300, 40, 0, 200, 64, 400, 2, 65, 3]
    w = synthetic.varlen_inputs(580 + D + Nq + len(mask), Nq=Nq, Nkv=Nkv, D=D, dtype="bf16",
                                lengths_q=lq, lengths_kv=lk)
    for prefix in (None, [200, 7, 5, 150, 0, 333, -4, 64, 900]):
        a, b = _both(_varlen_dropout_run(mi, w, mask, 0.2, 0x1234567890ABCDEF, 77, prefix))
        _assert_identical(a, b, f"dropout {mask} D {D} prefix {prefix is not None}")
        assert np.all(np.isfinite(a[0]))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_full_workload_dropout_matches_tiled_bit_for_bit(mi, dtype):
    """The 16-sequence packed causal GQA workload with dropout 0.1 (4 heads per item):
    persistent and tiled kernels agree bit for bit."""
    w = synthetic.varlen_inputs(0, Nq=32, Nkv=8, D=128, dtype=dtype, B=16)
    a, b = _both(_varlen_dropout_run(mi, w, "causal", 0.1, 2026, 0))
    _assert_identical(a, b, f"full workload dropout {dtype}")
