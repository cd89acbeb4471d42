"""Seeded synthetic inputs for the attention forward, shared by the tests and the bench.

This module draws random numbers and lays them out; it holds none of the attention
arithmetic.  Both the HIP path and the CPU oracle receive exactly the values produced
here (for bf16 and fp16 the oracle receives the exact widening of the stored 2-byte values).

Recipe (one fresh ``numpy.random.default_rng(seed)`` per workload, seed 0 unless a test
says otherwise; draws in this fixed order):

1. sequence lengths (packed-batch workloads only): ``rng.integers(lo, hi + 1, size=B)``;
2. Q, K, V: ``rng.standard_normal(shape, dtype=float32)`` each, in the storage layout;
3. CSR columns (sparse workloads only), per (b, n) b-major, per row i ascending.

bf16 and fp16 storage are produced by round-to-nearest-even from those float32 draws.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# bf16 storage helpers (input preparation only)
# ----------------------------------------------------------------------------------------


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite normal draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's cast rounds to nearest, ties to even);
    return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_from_f16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of binary16 bit patterns to float32."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def storage_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of a stored tensor (float32 array, or bf16 / fp16 bit patterns)."""
    if dtype == "bf16":
        return f32_from_bf16_bits(arr).astype(np.float64)
    if dtype == "f16":
        return f32_from_f16_bits(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in the storage form of `dtype` (bits for the 2-byte types)."""
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "f16":
        return f16_bits_from_f32(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


# ----------------------------------------------------------------------------------------
# layouts: storage shape of a (B, N, S, D) tensor, and the view back to (B, N, S, D)
# ----------------------------------------------------------------------------------------

LAYOUTS = ("BNSD", "BSND", "BSH", "SBH")


def device_normal(shape, seed: int, dtype: str, device: str = "cuda:0"):
    """N(0, 1) draws made on the device (torch's counter-based generator, seeded), stored in
    `dtype`: for inputs of several GiB that the host would take long to draw and upload.
    Returns a torch tensor; its values reach the oracle by reading back the stored bits."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(tdt)


def storage_shape(layout: str, B: int, N: int, S: int, D: int):
    if layout == "BNSD":
        return (B, N, S, D)
    if layout == "BSND":
        return (B, S, N, D)
    if layout == "BSH":
        return (B, S, N * D)
    if layout == "SBH":
        return (S, B, N * D)
    raise ValueError(layout)


def to_bnsd(arr: np.ndarray, layout: str, N: int) -> np.ndarray:
    """View a stored tensor in logical (B, N, S, D) order (no copy, no arithmetic)."""
    if layout == "BNSD":
        return arr
    if layout == "BSND":
        return arr.transpose(0, 2, 1, 3)
    if layout == "BSH":
        B, S, H = arr.shape
        return arr.reshape(B, S, N, H // N).transpose(0, 2, 1, 3)
    if layout == "SBH":
        S, B, H = arr.shape
        return arr.reshape(S, B, N, H // N).transpose(1, 2, 0, 3)
    raise ValueError(layout)


def from_bnsd(arr: np.ndarray, layout: str) -> np.ndarray:
    """Inverse of :func:`to_bnsd`: a contiguous array in the storage layout."""
    B, N, S, D = arr.shape
    if layout == "BNSD":
        out = arr
    elif layout == "BSND":
        out = arr.transpose(0, 2, 1, 3)
    elif layout == "BSH":
        out = arr.transpose(0, 2, 1, 3).reshape(B, S, N * D)
    elif layout == "SBH":
        out = arr.transpose(2, 0, 1, 3).reshape(S, B, N * D)
    else:
        raise ValueError(layout)
    return np.ascontiguousarray(out)


# ----------------------------------------------------------------------------------------
# packed variable-length batches
# ----------------------------------------------------------------------------------------


def cumulative_ends(lengths) -> np.ndarray:
    """Cumulative sequence lengths as END offsets with no leading zero (int64).

    This is the convention of the aclnnFlashAttentionVarLenScore constraints: lengths
    [2, 2, 0, 2, 2] are passed as [2, 4, 4, 6, 8].
    """
    return np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int64)


def draw_lengths(rng: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


# ----------------------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------------------


def dense_inputs(seed: int, B: int, Nq: int, Nkv: int, Sq: int, Skv: int, D: int,
                 dtype: str = "bf16", layout: str = "BNSD") -> dict:
    """Q [B,Nq,Sq,D], K/V [B,Nkv,Skv,D] drawn in the storage ``layout``."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, storage_shape(layout, B, Nq, Sq, D), dtype)
    k = _draw(rng, storage_shape(layout, B, Nkv, Skv, D), dtype)
    v = _draw(rng, storage_shape(layout, B, Nkv, Skv, D), dtype)
    return dict(q=q, k=k, v=v, B=B, Nq=Nq, Nkv=Nkv, Sq=Sq, Skv=Skv, D=D, dtype=dtype, layout=layout)


def varlen_inputs(seed: int, Nq: int, Nkv: int, D: int, dtype: str = "bf16", *,
                  B: int | None = None, len_lo: int = 1, len_hi: int = 4096,
                  lengths_q=None, lengths_kv=None) -> dict:
    """Packed TND batch.  Lengths are drawn first (unless given), then Q, K, V."""
    rng = np.random.default_rng(seed)
    if lengths_q is None:
        lengths_q = draw_lengths(rng, B, len_lo, len_hi)
    lengths_q = np.asarray(lengths_q, dtype=np.int64)
    lengths_kv = lengths_q if lengths_kv is None else np.asarray(lengths_kv, dtype=np.int64)
    Tq, Tkv = int(lengths_q.sum()), int(lengths_kv.sum())
    q = _draw(rng, (Tq, Nq, D), dtype)
    k = _draw(rng, (Tkv, Nkv, D), dtype)
    v = _draw(rng, (Tkv, Nkv, D), dtype)
    return dict(q=q, k=k, v=v, lengths_q=lengths_q, lengths_kv=lengths_kv,
                cu_q=cumulative_ends(lengths_q), cu_kv=cumulative_ends(lengths_kv),
                Tq=Tq, Tkv=Tkv, B=len(lengths_q), Nq=Nq, Nkv=Nkv, D=D, dtype=dtype)


def csr_band_random(rng: np.random.Generator, S: int, band: int, n_random: int):
    """One (b, n) CSR pattern: row i keeps the causal local band {max(0,i-band+1) .. i}
    plus min(n_random, i-band+1) distinct columns drawn uniformly without replacement
    from the earlier columns [0, i-band]; columns of a row are sorted ascending.
    Returns (offset int32 [S+1] row pointer, columns int32 [nnz])."""
    offset = np.zeros(S + 1, dtype=np.int64)
    cols = []
    for i in range(S):
        lo = max(0, i - band + 1)
        row = []
        n_before = i - band + 1  # size of [0, i-band]
        if n_before > 0 and n_random > 0:
            pick = rng.choice(n_before, size=min(n_random, n_before), replace=False)
            row.append(np.sort(pick).astype(np.int64))
        row.append(np.arange(lo, i + 1, dtype=np.int64))
        r = np.concatenate(row)
        cols.append(r)
        offset[i + 1] = offset[i] + len(r)
    return offset.astype(np.int32), np.concatenate(cols).astype(np.int32)


def sparse_inputs(seed: int, B: int, N: int, S: int, D: int, band: int, n_random: int,
                  dtype: str = "f32") -> dict:
    """Q/K/V [B,N,S,D] then a band+random CSR pattern per (b, n).

    Every (b, n) pattern of this recipe has the same nnz, so ``columns`` is [B,N,nnz]
    as the Paddle sparse_attention API expects."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, N, S, D), dtype)
    k = _draw(rng, (B, N, S, D), dtype)
    v = _draw(rng, (B, N, S, D), dtype)
    offs, cols = [], []
    for _b in range(B):
        for _n in range(N):
            o, c = csr_band_random(rng, S, band, n_random)
            offs.append(o)
            cols.append(c)
    nnz = len(cols[0])
    assert all(len(c) == nnz for c in cols)
    offset = np.stack(offs).reshape(B, N, S + 1)
    columns = np.stack(cols).reshape(B, N, nnz)
    return dict(q=q, k=k, v=v, offset=offset, columns=columns, nnz=nnz,
                B=B, N=N, S=S, D=D, dtype=dtype)


# ----------------------------------------------------------------------------------------
# the five named workloads (full sizes) and small variants the oracle finishes in seconds
# ----------------------------------------------------------------------------------------

WORKLOADS = {
    "dense_f32_b1n1s128d64": dict(kind="dense", B=1, Nq=1, Nkv=1, Sq=128, Skv=128, D=64,
                                  dtype="f32", layout="BNSD", mask="none"),
    "dense_bf16_b8n8s128d64": dict(kind="dense", B=8, Nq=8, Nkv=8, Sq=128, Skv=128, D=64,
                                   dtype="bf16", layout="BNSD", mask="none"),
    "varlen_causal_gqa_bf16_b16_t33064_nq32_nkv8_d128": dict(
        kind="varlen", B=16, len_lo=1, len_hi=4096, Nq=32, Nkv=8, D=128, dtype="bf16",
        mask="causal"),
    "ring_merge_sbh_bf16_s8192_n32_d128": dict(kind="merge", B=1, N=32, S=8192, D=128,
                                               dtype="bf16", layout="SBH"),
    "csr_sparse_f32_b2n8s4096d64": dict(kind="sparse", B=2, N=8, S=4096, D=64, band=128,
                                        n_random=64, dtype="f32"),
}

METRIC_WORKLOAD = "varlen_causal_gqa_bf16_b16_t33064_nq32_nkv8_d128"


def make(name: str, seed: int = 0) -> dict:
    """Inputs of a named workload (see WORKLOADS)."""
    w = WORKLOADS[name]
    if w["kind"] == "dense":
        return dense_inputs(seed, w["B"], w["Nq"], w["Nkv"], w["Sq"], w["Skv"], w["D"],
                            w["dtype"], w["layout"])
    if w["kind"] == "varlen":
        return varlen_inputs(seed, w["Nq"], w["Nkv"], w["D"], w["dtype"], B=w["B"],
                             len_lo=w["len_lo"], len_hi=w["len_hi"])
    if w["kind"] == "merge":
        # One Q/K/V of the full causal problem; the two partials split K/V in halves.
        return dense_inputs(seed, w["B"], w["N"], w["N"], w["S"], w["S"], w["D"],
                            w["dtype"], w["layout"])
    if w["kind"] == "sparse":
        return sparse_inputs(seed, w["B"], w["N"], w["S"], w["D"], w["band"], w["n_random"],
                             w["dtype"])
    raise ValueError(name)
