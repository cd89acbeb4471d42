"""Pins of the CPU fp64 oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle (wrong or missing scale,
a dropped term, a wrong sign or index in the mask, a transposed operand, a wrong GQA
mapping, a wrong CSR indexing, a wrong merge weight) fails at least one test:

- the Paddle sparse_attention worked example (printed values + closed forms);
- closed forms (Q = 0 gives plain means and integer sums; constant V returns V;
  a single visible key returns that key's value);
- invariants (probabilities sum to 1, key permutation, GQA == replicated MHA,
  band limits, varlen == per-sequence dense, merge split identity);
- a library cross-check: torch's CPU scaled_dot_product_attention in float64
  (the function the "flash attention的调用" page calls), with masks built by
  np.tril / np.triu or by explicit enumeration, and torch.logsumexp for the stats.

CPU only; no GPU, no HIP library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _torch_sdpa(q, k, v, scale, keep=None):
    """torch CPU float64 SDPA with an optional boolean keep-mask [Sq, Skv] and GQA."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = None if keep is None else torch.from_numpy(keep)
    gqa = q.shape[1] != k.shape[1]
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=gqa)
    return out.numpy()


def _torch_stats(q, k, scale, keep=None):
    """(max, sum at that max) of the scaled, masked logits via torch.amax / logsumexp."""
    G = q.shape[1] // k.shape[1]
    tk = torch.from_numpy(np.ascontiguousarray(np.repeat(k, G, axis=1)))
    s = scale * torch.matmul(torch.from_numpy(np.ascontiguousarray(q)), tk.transpose(-1, -2))
    if keep is not None:
        s = s.masked_fill(~torch.from_numpy(keep), -math.inf)
    m = s.amax(-1)
    lse = torch.logsumexp(s, -1)
    return m.numpy(), torch.exp(lse - m).numpy()


def _band_keep(Sq, Skv, pre, nxt):
    """keep[i, j] <=> -pre <= j - i <= next, built with np.tril / np.triu."""
    ones = np.ones((Sq, Skv), dtype=bool)
    return np.triu(ones, k=-pre) & np.tril(ones, k=nxt)


# ------------------------------------------------------------------------------------
# Paddle sparse_attention worked example
# ------------------------------------------------------------------------------------

def _paddle_example():
    with open(os.path.join(GOLDEN, "paddle_sparse_attention_example.json")) as f:
        g = json.load(f)
    x = lambda key: np.array(g[key], dtype=np.float64).reshape(1, 1, 4, 2)
    off = np.array(g["offset"], dtype=np.int32).reshape(1, 1, 5)
    col = np.array(g["columns"], dtype=np.int32).reshape(1, 1, 8)
    return x("query"), x("key"), x("value"), off, col, np.array(g["printed_output"])


def test_paddle_example_matches_printed_output():
    q, k, v, off, col, printed = _paddle_example()
    out, m, l = oracle.sparse(q, k, v, off, col, scale=1 / math.sqrt(2))
    # printed values are float32 results shown to 8 decimals (1 fp32 ulp ~ 2.4e-7 here)
    assert np.max(np.abs(out[0, 0] - printed)) < 5e-7


def test_paddle_example_closed_form():
    q, k, v, off, col, _ = _paddle_example()
    out, m, l = oracle.sparse(q, k, v, off, col, scale=1 / math.sqrt(2))
    a = 2 / (1 + math.exp(-math.sqrt(2)))       # rows 0, 2: logits 1/sqrt2 and 3/sqrt2
    b = 2 / (1 + math.exp(-5 * math.sqrt(2)))   # rows 1, 3: logits 3/sqrt2 and 13/sqrt2
    want = np.array([[a, 1 + a], [b, 1 + b], [a, 1 + a], [b, 1 + b]])
    assert np.max(np.abs(out[0, 0] - want)) < 1e-14
    assert np.allclose(m[0, 0], [3 / math.sqrt(2), 13 / math.sqrt(2)] * 2, rtol=0, atol=1e-14)
    assert np.allclose(l[0, 0], [1 + math.exp(-math.sqrt(2)), 1 + math.exp(-5 * math.sqrt(2))] * 2,
                       rtol=0, atol=1e-14)


@pytest.mark.parametrize("wrong_scale", [1.0, 0.5, 1 / 4])
def test_paddle_example_rejects_other_scales(wrong_scale):
    """The printed output discriminates the 1/sqrt(d) scale from no scale or 1/d."""
    q, k, v, off, col, printed = _paddle_example()
    out, _, _ = oracle.sparse(q, k, v, off, col, scale=wrong_scale)
    assert np.max(np.abs(out[0, 0] - printed)) > 1e-2


def test_dense_reading_of_paddle_example():
    """The same example through dense attention with the CSR pattern as a band:
    rows 0,1 see keys {0,1}; rows 2,3 see keys {2,3}."""
    q, k, v, _, _, printed = _paddle_example()
    out01, _, _ = oracle.attn(q[:, :, :2], k[:, :, :2], v[:, :, :2], scale=1 / math.sqrt(2))
    out23, _, _ = oracle.attn(q[:, :, 2:], k[:, :, 2:], v[:, :, 2:], scale=1 / math.sqrt(2))
    got = np.concatenate([out01[0, 0], out23[0, 0]])
    assert np.max(np.abs(got - printed)) < 5e-7


# ------------------------------------------------------------------------------------
# closed forms
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("mask,pre,nxt", [("none", 0, 0), ("causal", 0, 0), ("band", 3, 2),
                                          ("band", 0, 0), ("band", 9, -4)])
def test_zero_query_gives_means_and_counts(mask, pre, nxt):
    rng = np.random.default_rng(1)
    B, N, Sq, Skv, D = 2, 3, 11, 13, 5
    q = np.zeros((B, N, Sq, D))
    k, v = _rand(rng, B, N, Skv, D), _rand(rng, B, N, Skv, D)
    out, m, l = oracle.attn(q, k, v, 0.3, mask, pre, nxt)
    for i in range(Sq):
        if mask == "none":
            js = list(range(Skv))
        elif mask == "causal":
            js = list(range(min(i + 1, Skv)))
        else:
            js = [j for j in range(Skv) if i - pre <= j <= i + nxt]
        if not js:
            assert np.all(out[:, :, i] == 0) and np.all(m[:, :, i] == -np.inf)
            assert np.all(l[:, :, i] == 0)
            continue
        assert np.all(m[:, :, i] == 0.0)
        assert np.all(l[:, :, i] == float(len(js)))
        assert np.max(np.abs(out[:, :, i] - v[:, :, js].mean(axis=2))) < TOL


def test_constant_value_rows_return_the_constant():
    rng = np.random.default_rng(2)
    q, k = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 9, 4)
    c = rng.standard_normal(4)
    v = np.broadcast_to(c, (1, 2, 9, 4)).copy()
    out, _, _ = oracle.attn(q, k, v, 0.5, "causal")
    assert np.max(np.abs(out - c)) < TOL


def test_single_visible_key_and_probabilities():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 3)
    # band(0, 0): each row sees only its own key
    out, m, l, p = oracle.attn(q, k, v, 0.7, "band", 0, 0, return_probs=True)
    assert np.array_equal(out, v)
    assert np.all(l == 1.0)
    assert np.allclose(m[0, 0], 0.7 * np.einsum("sd,sd->s", q[0, 0], k[0, 0]), atol=TOL, rtol=0)
    # causal: row 0 returns V[0]; probability rows sum to 1 and vanish above the diagonal
    out, m, l, p = oracle.attn(q, k, v, 0.7, "causal", return_probs=True)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0])
    assert np.max(np.abs(p.sum(-1) - 1)) < TOL
    assert np.all(np.triu(p[0, 0], k=1) == 0)


# ------------------------------------------------------------------------------------
# library cross-check: torch CPU float64 scaled_dot_product_attention
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,Nq,Nkv,Sq,Skv,D", [(1, 1, 1, 16, 16, 8), (2, 4, 4, 9, 17, 5),
                                               (2, 8, 2, 20, 20, 16), (1, 6, 1, 7, 3, 4),
                                               (3, 4, 2, 33, 31, 12)])
@pytest.mark.parametrize("mask", ["none", "causal", "band"])
def test_oracle_matches_torch_sdpa_fp64(B, Nq, Nkv, Sq, Skv, D, mask):
    rng = np.random.default_rng(B * 1000 + Sq * 10 + D)
    q, k, v = _rand(rng, B, Nq, Sq, D), _rand(rng, B, Nkv, Skv, D), _rand(rng, B, Nkv, Skv, D)
    scale = 1 / math.sqrt(D)
    pre, nxt = (0, 0)
    if mask == "causal":
        keep = np.tril(np.ones((Sq, Skv), dtype=bool))
    elif mask == "band":
        pre, nxt = 3, 2
        keep = _band_keep(Sq, Skv, pre, nxt)
    else:
        keep = None
    out, m, l = oracle.attn(q, k, v, scale, mask, pre, nxt)
    rows = np.ones(Sq, dtype=bool) if keep is None else keep.any(1)
    want = _torch_sdpa(q, k, v, scale, keep)
    assert np.max(np.abs(out[:, :, rows] - want[:, :, rows])) < TOL
    wm, wl = _torch_stats(q, k, scale, keep)
    assert np.max(np.abs(m[:, :, rows] - wm[:, :, rows])) < TOL
    assert np.max(np.abs(l[:, :, rows] / wl[:, :, rows] - 1)) < TOL
    assert np.all(out[:, :, ~rows] == 0) and np.all(m[:, :, ~rows] == -np.inf)
    assert np.all(l[:, :, ~rows] == 0)


@pytest.mark.parametrize("S", [1, 4, 6])
def test_band_every_pre_next_against_enumeration(S):
    """Every (pre, next) in [-S, S]^2 with pre + next >= 0 (non-empty band), the visible
    set enumerated pair by pair, checked through torch SDPA."""
    rng = np.random.default_rng(S)
    D = 3
    q, k, v = _rand(rng, 1, 2, S, D), _rand(rng, 1, 2, S, D), _rand(rng, 1, 2, S, D)
    for pre in range(-S, S + 1):
        for nxt in range(-S, S + 1):
            if pre + nxt < 0:
                continue
            keep = np.array([[(i - pre) <= j <= (i + nxt) for j in range(S)] for i in range(S)])
            out, m, l = oracle.attn(q, k, v, 0.9, "band", pre, nxt)
            rows = keep.any(1)
            if rows.any():
                want = _torch_sdpa(q, k, v, 0.9, keep)
                assert np.max(np.abs(out[:, :, rows] - want[:, :, rows])) < TOL, (pre, nxt)
            assert np.all(out[:, :, ~rows] == 0) and np.all(l[:, :, ~rows] == 0)
    # causal is band(+inf, 0); a band wider than the sequence is "none"
    a = oracle.attn(q, k, v, 0.9, "causal")
    b = oracle.attn(q, k, v, 0.9, "band", 1 << 62, 0)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    a = oracle.attn(q, k, v, 0.9, "none")
    b = oracle.attn(q, k, v, 0.9, "band", S, S)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_key_permutation_invariance():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 2, 10, 6), _rand(rng, 2, 2, 14, 6), _rand(rng, 2, 2, 14, 6)
    perm = rng.permutation(14)
    a = oracle.attn(q, k, v, 0.4)
    b = oracle.attn(q, k[:, :, perm], v[:, :, perm], 0.4)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < TOL


def test_gqa_equals_replicated_heads():
    """kv head of query head h is h // (Nq/Nkv): GQA equals MHA with K/V repeated."""
    rng = np.random.default_rng(6)
    Nq, Nkv = 8, 2
    q, k, v = _rand(rng, 2, Nq, 12, 4), _rand(rng, 2, Nkv, 12, 4), _rand(rng, 2, Nkv, 12, 4)
    a = oracle.attn(q, k, v, 0.5, "causal")
    b = oracle.attn(q, np.repeat(k, Nq // Nkv, axis=1), np.repeat(v, Nq // Nkv, axis=1), 0.5, "causal")
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # an interleaved mapping (h % Nkv) gives something else
    c = oracle.attn(q, np.tile(k, (1, Nq // Nkv, 1, 1)), np.tile(v, (1, Nq // Nkv, 1, 1)), 0.5, "causal")
    assert np.max(np.abs(a[0] - c[0])) > 1e-3


# ------------------------------------------------------------------------------------
# packed variable-length batches
# ------------------------------------------------------------------------------------

def test_cumulative_end_offsets_convention():
    # aclnnFlashAttentionVarLenScore constraints: lengths [2,2,0,2,2] are passed as [2,4,4,6,8]
    assert synthetic.cumulative_ends([2, 2, 0, 2, 2]).tolist() == [2, 4, 4, 6, 8]


@pytest.mark.parametrize("mask,pre,nxt", [("causal", 0, 0), ("none", 0, 0), ("band", 4, 1)])
def test_varlen_equals_dense_per_sequence(mask, pre, nxt):
    lengths = [5, 0, 9, 1, 12]
    w = synthetic.varlen_inputs(7, Nq=4, Nkv=2, D=8, dtype="f32", lengths_q=lengths)
    q, k, v = (w[x].astype(np.float64) for x in ("q", "k", "v"))
    out, m, l = oracle.attn_varlen(q, k, v, w["cu_q"], w["cu_kv"], 0.35, mask, pre, nxt)
    assert out.shape == (sum(lengths), 4, 8) and m.shape == (4, sum(lengths))
    t0 = 0
    for L in lengths:
        if L:
            sl = slice(t0, t0 + L)
            do, dm, dl = oracle.attn(q[sl].transpose(1, 0, 2)[None], k[sl].transpose(1, 0, 2)[None],
                                     v[sl].transpose(1, 0, 2)[None], 0.35, mask, pre, nxt)
            assert np.array_equal(out[sl], do[0].transpose(1, 0, 2))
            assert np.array_equal(m[:, sl], dm[0]) and np.array_equal(l[:, sl], dl[0])
        t0 += L


def test_varlen_rejects_bad_offsets():
    q = np.zeros((4, 1, 2))
    with pytest.raises(ValueError):
        oracle.attn_varlen(q, q, q, [3, 2], [3, 2], 1.0)   # not monotone
    with pytest.raises(ValueError):
        oracle.attn_varlen(q, q, q, [1, 3], [1, 3], 1.0)   # last != T


# ------------------------------------------------------------------------------------
# explicit visibility matrices: bottom-right alignment, prefix, explicit masks, Dv < D
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("Sq,Skv", [(5, 9), (9, 5), (7, 7), (1, 6), (6, 1)])
def test_keep_bottom_right_causal_is_the_shifted_lower_triangle(Sq, Skv):
    """Bottom-right causal = ones.tril(diagonal = Skv - Sq) (the lower triangle whose
    diagonal ends at the last query / last key pair); equal to top-left when Sq = Skv."""
    want = np.tril(np.ones((Sq, Skv), dtype=bool), k=Skv - Sq)
    assert np.array_equal(oracle.keep_band(Sq, Skv, 1 << 62, 0, "bottom_right"), want)
    tl = np.tril(np.ones((Sq, Skv), dtype=bool))
    assert np.array_equal(oracle.keep_band(Sq, Skv, 1 << 62, 0, "top_left"), tl)
    # a bottom-right band is the top-left band with next and pre shifted by Skv - Sq
    assert np.array_equal(oracle.keep_band(Sq, Skv, 2, 1, "bottom_right"),
                          _band_keep(Sq, Skv, 2 - (Skv - Sq), 1 + (Skv - Sq)))


@pytest.mark.parametrize("Sq,Skv,P", [(6, 10, 4), (6, 10, 0), (10, 6, 3), (10, 6, 0), (8, 8, 8)])
def test_keep_prefix_causal_counts(Sq, Skv, P):
    """Row i sees the first P keys and the bottom-right causal keys: that is
    clip(max(P, i + Skv - Sq + 1), 0, Skv) keys, all of them a prefix of the key range."""
    keep = oracle.keep_prefix_causal(Sq, Skv, P)
    for i in range(Sq):
        n = min(Skv, max(P, i + Skv - Sq + 1, 0))
        assert keep[i].sum() == n and keep[i, :n].all()


@pytest.mark.parametrize("Dv", [5, 3])
def test_attn_keep_matches_torch_sdpa_fp64(Dv):
    """Random explicit masks (some rows empty), GQA, and a value head dim Dv <= D."""
    rng = np.random.default_rng(14)
    B, Nq, Nkv, Sq, Skv, D = 2, 4, 2, 9, 13, 5
    q, k, v = _rand(rng, B, Nq, Sq, D), _rand(rng, B, Nkv, Skv, D), _rand(rng, B, Nkv, Skv, Dv)
    keep = rng.random((Sq, Skv)) < 0.4
    keep[3] = False
    out, m, l = oracle.attn_keep(q, k, v, keep, 0.37)
    rows = keep.any(1)
    want = _torch_sdpa(q, k, v, 0.37, keep)
    assert out.shape == (B, Nq, Sq, Dv)
    assert np.max(np.abs(out[:, :, rows] - want[:, :, rows])) < TOL
    wm, wl = _torch_stats(q, k, 0.37, keep)
    assert np.max(np.abs(m[:, :, rows] - wm[:, :, rows])) < TOL
    assert np.max(np.abs(l[:, :, rows] / wl[:, :, rows] - 1)) < TOL
    assert np.all(out[:, :, 3] == 0) and np.all(m[:, :, 3] == -np.inf) and np.all(l[:, :, 3] == 0)


def test_attn_keep_zero_query_means_over_prefix_causal():
    rng = np.random.default_rng(15)
    Sq, Skv, P = 7, 10, 5
    q = np.zeros((1, 2, Sq, 4))
    k, v = _rand(rng, 1, 2, Skv, 4), _rand(rng, 1, 2, Skv, 4)
    keep = oracle.keep_prefix_causal(Sq, Skv, P)
    out, m, l = oracle.attn_keep(q, k, v, keep, 0.5)
    for i in range(Sq):
        js = np.nonzero(keep[i])[0]
        assert np.all(l[:, :, i] == len(js)) and np.all(m[:, :, i] == 0)
        assert np.max(np.abs(out[:, :, i] - v[:, :, js].mean(axis=2))) < TOL


def test_attn_varlen_keep_equals_positional_masks():
    """The per-sequence visibility path with top-left band matrices equals the positional
    band path (two independent routes through the oracle)."""
    rng = np.random.default_rng(16)
    lq, lk = np.array([5, 0, 7, 3]), np.array([6, 4, 2, 3])
    q, k, v = _rand(rng, lq.sum(), 4, 3), _rand(rng, lk.sum(), 2, 3), _rand(rng, lk.sum(), 2, 3)
    cq, ck = np.cumsum(lq), np.cumsum(lk)
    a = oracle.attn_varlen(q, k, v, cq, ck, 0.8, "band", 2, 1)
    b = oracle.attn_varlen_keep(q, k, v, cq, ck, lambda bi, sq, sk: oracle.keep_band(sq, sk, 2, 1),
                                0.8)
    for x, y in zip(a, b):
        assert np.max(np.abs(np.where(np.isinf(x), 0, x) - np.where(np.isinf(y), 0, y))) < TOL
        assert np.array_equal(np.isinf(x), np.isinf(y))


# ------------------------------------------------------------------------------------
# dropout: Philox4x32-10 and the keep decision
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("ctr,key,want", [
    # known-answer vectors of Philox4x32-10 published with the generator's reference
    # implementation (Random123)
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
])
def test_philox4x32_10_known_answers(ctr, key, want):
    got = oracle.philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in got) == want


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_keep_rate(p):
    keep = oracle.dropout_keep(2024, 3, 1, 5, 512, 2048, p)
    want = 1 - oracle.dropout_threshold(p) / 256
    assert abs(keep.mean() - want) < 0.004            # ~4 sigma for 2^20 draws
    # rows, columns and heads draw different bytes
    assert not np.array_equal(keep[0], keep[1]) and not np.array_equal(keep[:, 0], keep[:, 16])
    assert not np.array_equal(keep, oracle.dropout_keep(2024, 3, 1, 6, 512, 2048, p))


def test_dropout_zero_is_plain_attention_and_stats_are_undropped():
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 2, 4, 20, 8), _rand(rng, 2, 2, 33, 8), _rand(rng, 2, 2, 33, 8)
    plain = oracle.attn(q, k, v, 0.3, "causal")
    got = oracle.attn_dropout(q, k, v, 0.3, "causal", 0, 0, 0.0, 99, 0)
    assert np.max(np.abs(got[0] - plain[0])) < TOL
    drop = oracle.attn_dropout(q, k, v, 0.3, "causal", 0, 0, 0.4, 99, 0)
    assert np.array_equal(drop[1], plain[1]) and np.array_equal(drop[2], plain[2])
    assert np.max(np.abs(drop[0] - plain[0])) > 0.01


def test_dropout_is_unbiased_over_offsets():
    """E[dropout(P) V] = P V: the mean over 400 offsets approaches the plain output."""
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 32, 4), _rand(rng, 1, 1, 32, 4)
    plain = oracle.attn(q, k, v, 0.2)[0]
    acc = np.zeros_like(plain)
    for off in range(400):
        acc += oracle.attn_dropout(q, k, v, 0.2, "none", 0, 0, 0.25, 7, off)[0]
    assert np.max(np.abs(acc / 400 - plain)) < 0.04


# ------------------------------------------------------------------------------------
# merge of partial results (ring-attention update)
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("split", [0, 1, 7, 16, 23, 24])
def test_merge_split_identity(split):
    """merge(attn over K[:split], attn over K[split:]) == attn over all of K."""
    rng = np.random.default_rng(8 + split)
    q, k, v = _rand(rng, 2, 3, 10, 5), _rand(rng, 2, 3, 24, 5), _rand(rng, 2, 3, 24, 5)
    full = oracle.attn(q, k, v, 0.45)
    a = oracle.attn(q, k[:, :, :split], v[:, :, :split], 0.45)
    b = oracle.attn(q, k[:, :, split:], v[:, :, split:], 0.45)
    out, m, l = oracle.merge(*a, *b)
    assert np.max(np.abs(out - full[0])) < TOL
    assert np.array_equal(m, full[1])
    assert np.max(np.abs(l / full[2] - 1)) < TOL


def test_merge_ring_halves_with_offset_band():
    """The two-chunk causal split: chunk A = keys [0, S/2) causal, chunk B = keys
    [S/2, S) visible from query i iff S/2 + j <= i, i.e. band(pre=inf, next=-S/2)."""
    rng = np.random.default_rng(9)
    S, h = 16, 8
    q, k, v = _rand(rng, 1, 2, S, 4), _rand(rng, 1, 2, S, 4), _rand(rng, 1, 2, S, 4)
    full = oracle.attn(q, k, v, 0.5, "causal")
    a = oracle.attn(q, k[:, :, :h], v[:, :, :h], 0.5, "causal")
    b = oracle.attn(q, k[:, :, h:], v[:, :, h:], 0.5, "band", 1 << 62, -h)
    assert np.all(b[1][:, :, :h] == -np.inf) and np.all(b[2][:, :, :h] == 0)
    out, m, l = oracle.merge(*a, *b)
    assert np.max(np.abs(out - full[0])) < TOL
    assert np.array_equal(m, full[1])
    assert np.max(np.abs(l / full[2] - 1)) < TOL


def test_merge_closed_forms_on_random_stats():
    """Random stats of the ring-update page's example shape (S=2048, N=12, D=1;
    sums may be negative): the max is the larger max, equal outputs stay, equal
    maxes add the sums, an empty partial returns the other one."""
    rng = np.random.default_rng(10)
    B, N, S, D = 1, 12, 2048, 1
    o1, o2 = _rand(rng, B, N, S, D), _rand(rng, B, N, S, D)
    m1, m2 = _rand(rng, B, N, S), _rand(rng, B, N, S)
    l1, l2 = _rand(rng, B, N, S), _rand(rng, B, N, S)
    out, m, l = oracle.merge(o1, m1, l1, o2, m2, l2)
    assert np.array_equal(m, np.maximum(m1, m2))
    out_same, _, _ = oracle.merge(o1, m1, l1, o1, m2, l2)
    ok = np.abs(l) > 1e-3
    assert np.max(np.abs(out_same - o1)[ok]) < 1e-9
    # the oracle forms the merge through logarithms (log-sum-exp identity), so identities
    # hold to a few ulp of the values involved rather than bit for bit
    out_eq, m_eq, l_eq = oracle.merge(o1, m1, l1, o2, m1, l2)
    assert np.max(np.abs(l_eq - (l1 + l2))) < 1e-13
    lpos1, lpos2 = np.abs(l1) + 0.1, np.abs(l2) + 0.1
    out_eq, _, _ = oracle.merge(o1, m1, lpos1, o2, m1, lpos2)
    want = (lpos1[..., None] * o1 + lpos2[..., None] * o2) / (lpos1 + lpos2)[..., None]
    assert np.max(np.abs(out_eq - want)) < 1e-12
    empty_m, empty_l = np.full((B, N, S), -np.inf), np.zeros((B, N, S))
    o, mm, ll = oracle.merge(o1, m1, lpos1, np.zeros_like(o2), empty_m, empty_l)
    assert np.array_equal(o, o1) and np.array_equal(mm, m1)
    assert np.max(np.abs(ll / lpos1 - 1)) < 8 * 2.0 ** -52
    o, mm, ll = oracle.merge(o1, empty_m, empty_l, o2, empty_m, empty_l)
    assert np.all(o == 0) and np.all(mm == -np.inf) and np.all(ll == 0)


@pytest.mark.parametrize("mask,pre,nxt,cuts", [("causal", 0, 0, [0, 5, 6, 13, 24]),
                                                ("none", 0, 0, [0, 8, 16, 24]),
                                                ("band", 7, 3, [0, 1, 11, 12, 24])])
def test_update_over_key_chunks_equals_full_attention(mask, pre, nxt, cuts):
    """Ring accumulation: starting from an empty result, attn_update over consecutive key
    chunks [c0, c1), [c1, c2), ... with the band shifted by each chunk's start (keys
    j0 + j' seen from query i iff -pre <= j0 + j' - i <= next) gives attention over all
    keys.  Causal is band(inf, 0).  Empty chunks (13 -> 13) and one-key chunks included."""
    rng = np.random.default_rng(11)
    S, Skv = 20, 24
    q, k, v = _rand(rng, 2, 4, S, 6), _rand(rng, 2, 2, Skv, 6), _rand(rng, 2, 2, Skv, 6)
    full = oracle.attn(q, k, v, 0.4, mask, pre, nxt)
    p_lo = (1 << 62) if mask in ("causal", "none") else pre
    n_hi = 0 if mask == "causal" else ((1 << 62) if mask == "none" else nxt)
    out = np.full(q.shape, 12345.0)     # an empty prior's output is never used
    m = np.full((2, 4, S), -np.inf)
    l = np.zeros((2, 4, S))
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        if c1 == c0:
            continue
        o_c = oracle.attn_update(q, k[:, :, c0:c1], v[:, :, c0:c1], np.where(l[..., None] > 0, out, 0.0),
                                 m, l, 0.4, "band", p_lo + c0, n_hi - c0)
        out, m, l = o_c
    assert np.max(np.abs(out - full[0])) < TOL
    assert np.array_equal(m == -np.inf, full[1] == -np.inf)
    fin = full[1] > -np.inf
    assert np.max(np.abs(m[fin] - full[1][fin])) < TOL
    assert np.max(np.abs(l[fin] / full[2][fin] - 1)) < TOL
    assert np.all(l[~fin] == 0)


def test_varlen_update_over_key_chunks_equals_full_attention():
    """The packed form: each sequence's keys split into chunks, each chunk packed with its
    own cumulative lengths (one ring step's shard), accumulated with attn_varlen_update."""
    rng = np.random.default_rng(12)
    lq = np.array([9, 0, 1, 14])
    cu = np.cumsum(lq)
    T = int(cu[-1])
    q, k, v = _rand(rng, T, 4, 5), _rand(rng, T, 2, 5), _rand(rng, T, 2, 5)
    full = oracle.attn_varlen(q, k, v, cu, cu, 0.6, "causal")
    starts = np.concatenate([[0], cu[:-1]])
    out = np.zeros_like(q)
    m = np.full((4, T), -np.inf)
    l = np.zeros((4, T))
    C = 4
    for j in range(4):                     # chunk j holds keys [4j, 4j + 4) of each sequence
        rows = [np.arange(s + min(C * j, n), s + min(C * (j + 1), n)) for s, n in zip(starts, lq)]
        lk = np.array([len(r) for r in rows])
        idx = np.concatenate(rows).astype(np.int64)
        out, m, l = oracle.attn_varlen_update(q, k[idx], v[idx], out, m, l, cu, np.cumsum(lk),
                                              0.6, "band", 1 << 62, -C * j)
    assert np.max(np.abs(out - full[0])) < TOL
    fin = full[1] > -np.inf
    assert np.array_equal(m[~fin], full[1][~fin])
    assert np.max(np.abs(m[fin] - full[1][fin])) < TOL
    assert np.max(np.abs(l[fin] / full[2][fin] - 1)) < TOL


def test_update_with_empty_prior_is_plain_attention():
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 2, 9, 4), _rand(rng, 1, 2, 11, 4), _rand(rng, 1, 2, 11, 4)
    want = oracle.attn(q, k, v, 0.7, "band", 2, 1)
    got = oracle.attn_update(q, k, v, np.zeros_like(q), np.full((1, 2, 9), -np.inf),
                             np.zeros((1, 2, 9)), 0.7, "band", 2, 1)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    ok = want[2] > 0   # the sum passes through log and exp: a few ulp
    assert np.array_equal(got[2][~ok], want[2][~ok])
    assert np.max(np.abs(got[2][ok] / want[2][ok] - 1)) < 8 * 2.0 ** -52


# ------------------------------------------------------------------------------------
# CSR sparse attention
# ------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_sparse_matches_torch_with_dense_mask(seed):
    """Random CSR patterns (rows of K all distinct) vs torch SDPA with the same pattern
    as a boolean mask; a stored duplicate counts twice, i.e. adds log(2) to its logit."""
    rng = np.random.default_rng(100 + seed)
    B, N, S, D = 1, 2, 8, 4
    q, k, v = _rand(rng, B, N, S, D), _rand(rng, B, N, S, D), _rand(rng, B, N, S, D)
    dup = seed % 2 == 1
    offs, cols, bias = [], [], np.full((B, N, S, S), -np.inf)
    for n in range(N):
        off, col = [0], []
        for i in range(S):
            cnt = int(rng.integers(0, S + 1)) if i % 3 else int(rng.integers(1, S + 1))
            row = list(rng.choice(S, size=cnt, replace=False))
            if dup and row:
                row.append(row[0])
            rng.shuffle(row)
            for c in row:
                bias[0, n, i, c] = np.logaddexp(bias[0, n, i, c], 0.0)
            col += row
            off.append(len(col))
        offs.append(off)
        cols.append(col)
    nnz = max(len(c) for c in cols)
    columns = np.zeros((B, N, nnz), dtype=np.int32)
    for n in range(N):
        columns[0, n, :len(cols[n])] = cols[n]
    offset = np.array(offs, dtype=np.int32).reshape(B, N, S + 1)
    out, m, l = oracle.sparse(q, k, v, offset, columns, 0.6)
    rows = np.isfinite(bias).any(-1)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(bias), scale=0.6).numpy()
    assert np.max(np.abs(out[rows] - want[rows])) < TOL
    assert np.all(out[~rows] == 0) and np.all(l[~rows] == 0)


def test_sparse_equals_dense_for_causal_pattern():
    rng = np.random.default_rng(11)
    S = 12
    q, k, v = _rand(rng, 2, 3, S, 5), _rand(rng, 2, 3, S, 5), _rand(rng, 2, 3, S, 5)
    offset = np.tile(np.array([i * (i + 1) // 2 for i in range(S + 1)], dtype=np.int32), (2, 3, 1))
    columns = np.tile(np.concatenate([np.arange(i + 1) for i in range(S)]).astype(np.int32), (2, 3, 1))
    a = oracle.sparse(q, k, v, offset, columns, 0.3)
    b = oracle.attn(q, k, v, 0.3, "causal")
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) < TOL


def test_sparse_rejects_out_of_range_columns():
    q = np.zeros((1, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.sparse(q, q, q, np.array([[[0, 1, 2]]], np.int32), np.array([[[0, 2]]], np.int32), 1.0)


# ---- the multi-head self-attention module ("flash attention的调用", MultiHeadAttention) ----

def _mha_torch(x, w_qkv, b_qkv, w_out, b_out, N, attend=None):
    """The module's forward written with torch's float64 CPU primitives: linear layers,
    chunk into thirds, per-head SDPA, heads merged, output linear layer."""
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float64))
    B, S, E = x.shape
    q, k, v = torch.nn.functional.linear(t(x), t(w_qkv), t(b_qkv)).chunk(3, dim=-1)
    q, k, v = (a.reshape(B, S, N, E // N).transpose(1, 2) for a in (q, k, v))
    mask = None if attend is None else torch.from_numpy(attend)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    o = o.transpose(1, 2).reshape(B, S, E)
    return torch.nn.functional.linear(o, t(w_out), t(b_out)).numpy()


@pytest.mark.parametrize("B,S,E,N,bias", [(2, 9, 16, 2, True), (1, 5, 24, 3, False), (3, 4, 8, 1, True)])
def test_mha_matches_torch_module(B, S, E, N, bias):
    rng = np.random.default_rng(B * 100 + S)
    x = rng.standard_normal((B, S, E))
    w_qkv, w_out = rng.standard_normal((3 * E, E)) / 3, rng.standard_normal((E, E)) / 3
    b_qkv = rng.standard_normal(3 * E) if bias else None
    b_out = rng.standard_normal(E) if bias else None
    got = oracle.mha_self_attn(x, w_qkv, b_qkv, w_out, b_out, N)
    want = _mha_torch(x, w_qkv, b_qkv, w_out, b_out, N)
    assert np.max(np.abs(got - want)) <= TOL


def test_mha_with_mask_matches_torch_module():
    rng = np.random.default_rng(7)
    B, S, E, N = 2, 8, 16, 4
    x = rng.standard_normal((B, S, E))
    w_qkv, w_out = rng.standard_normal((3 * E, E)) / 3, rng.standard_normal((E, E)) / 3
    b_qkv, b_out = rng.standard_normal(3 * E), rng.standard_normal(E)
    keep = rng.random((S, S)) < 0.6
    keep[np.arange(S), rng.integers(0, S, S)] = True   # every row keeps at least one key
    got = oracle.mha_self_attn(x, w_qkv, b_qkv, w_out, b_out, N, keep=keep)
    want = _mha_torch(x, w_qkv, b_qkv, w_out, b_out, N, attend=keep)
    assert np.max(np.abs(got - want)) <= TOL


def test_mha_brute_force_loops():
    """B 1, S 3, E 4, N 2 by explicit loops over every index (no matrix library)."""
    rng = np.random.default_rng(11)
    S, E, N = 3, 4, 2
    D = E // N
    x = rng.standard_normal((1, S, E))
    w_qkv, b_qkv = rng.standard_normal((3 * E, E)), rng.standard_normal(3 * E)
    w_out, b_out = rng.standard_normal((E, E)), rng.standard_normal(E)
    proj = [[b_qkv[f] + sum(x[0, s, c] * w_qkv[f, c] for c in range(E)) for f in range(3 * E)]
            for s in range(S)]
    o = [[0.0] * E for _ in range(S)]
    for h in range(N):
        for i in range(S):
            sc = [sum(proj[i][h * D + d] * proj[j][E + h * D + d] for d in range(D)) / math.sqrt(D)
                  for j in range(S)]
            mx = max(sc)
            ws = [math.exp(a - mx) for a in sc]
            tot = sum(ws)
            for d in range(D):
                o[i][h * D + d] = sum(ws[j] * proj[j][2 * E + h * D + d] for j in range(S)) / tot
    want = np.array([[b_out[f] + sum(o[s][c] * w_out[f, c] for c in range(E)) for f in range(E)]
                     for s in range(S)])[None]
    got = oracle.mha_self_attn(x, w_qkv, b_qkv, w_out, b_out, N)
    assert np.max(np.abs(got - want)) <= TOL
