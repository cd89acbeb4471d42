"""CPU fp64 oracle for the attention forward (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline leg
are the only callers.  The product path (the HIP library and its binding) never imports
this package, and this package imports nothing from the product path.

All functions take and return float64 numpy arrays in a canonical layout:
dense tensors (B, N, S, D), packed tensors (T, N, D), stats (B, N, S) or (N, T).
Layout conversions are the caller's (they are views, not arithmetic).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c to load (the sanitizer build of the CPU test run)
_BUILT = os.path.join(_HERE, "liboracle.so")
_LIB = os.environ.get("ORACLE_LIB") or _BUILT

MASKS = {"none": 0, "causal": 1, "band": 2}
_lib = None


def build() -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", _BUILT + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_BUILT + ".tmp", _BUILT)
    return _BUILT


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        if "ORACLE_LIB" in os.environ:
            raise ImportError(f"ORACLE_LIB={_LIB} does not exist")
        build()
    lib = ctypes.CDLL(_LIB)
    P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_attn.argtypes = [P] * 7 + [I64] * 6 + [D, I, I64, I64, I]
    lib.oracle_attn_varlen.argtypes = [P] * 8 + [I64] * 6 + [D, I, I64, I64, I]
    lib.oracle_merge.argtypes = [P] * 9 + [I64] * 4 + [I]
    lib.oracle_sparse.argtypes = [P] * 8 + [I64] * 5 + [D, I]
    lib.oracle_attn_keep.argtypes = [P] * 7 + [I64] * 7 + [D, I]
    for f in (lib.oracle_attn, lib.oracle_attn_varlen, lib.oracle_merge, lib.oracle_sparse,
              lib.oracle_attn_keep):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _clamp_tokens(x: int) -> int:
    # Positions are < 2**40 in any workload here; clamping keeps pre/next in int64
    # without changing which keys are visible.
    lim = 1 << 62
    return int(max(-lim, min(lim, int(x))))


def attn(q, k, v, scale: float, mask: str = "none", pre: int = 0, next: int = 0,
         threads: int = 0, return_probs: bool = False):
    """Dense attention.  q (B,Nq,Sq,D), k/v (B,Nkv,Skv,D) -> out (B,Nq,Sq,D),
    softmax_max (B,Nq,Sq), softmax_sum (B,Nq,Sq) [, probs (B,Nq,Sq,Skv)]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Sq, D = q.shape
    Bk, Nkv, Skv, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch")
    out = np.empty_like(q)
    m = np.empty((B, Nq, Sq))
    l = np.empty((B, Nq, Sq))
    probs = np.empty((B, Nq, Sq, Skv)) if return_probs else None
    rc = _load().oracle_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(m), _ptr(l),
                             _ptr(probs) if probs is not None else None,
                             B, Nq, Nkv, Sq, Skv, D, float(scale), MASKS[mask],
                             _clamp_tokens(pre), _clamp_tokens(next), threads)
    if rc != 0:
        raise ValueError("oracle_attn: invalid arguments")
    return (out, m, l, probs) if return_probs else (out, m, l)


def attn_varlen(q, k, v, cu_q, cu_kv, scale: float, mask: str = "none", pre: int = 0,
                next: int = 0, threads: int = 0):
    """Packed attention.  q (Tq,Nq,D), k/v (Tkv,Nkv,D), cu_* END offsets (B,) ->
    out (Tq,Nq,D), softmax_max (Nq,Tq), softmax_sum (Nq,Tq)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int64)
    cu_kv = np.ascontiguousarray(cu_kv, dtype=np.int64)
    Tq, Nq, D = q.shape
    Tkv, Nkv, _ = k.shape
    out = np.empty_like(q)
    m = np.empty((Nq, Tq))
    l = np.empty((Nq, Tq))
    rc = _load().oracle_attn_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(m), _ptr(l),
                                    _ptr(cu_q), _ptr(cu_kv), len(cu_q), Tq, Tkv, Nq, Nkv, D,
                                    float(scale), MASKS[mask], _clamp_tokens(pre),
                                    _clamp_tokens(next), threads)
    if rc != 0:
        raise ValueError("oracle_attn_varlen: invalid arguments")
    return out, m, l


# ------------------------------------------------------------------------------------
# explicit visibility matrices ("keep": True where key j is visible from query i), for the
# mask modes of aclnnFlashAttentionVarLenScore (sparseMode, preTokens / nextTokens,
# prefixOptional, attenMaskOptional), written from the readings stated with each.
# ------------------------------------------------------------------------------------

def keep_band(Sq: int, Skv: int, pre: int, next: int, align: str = "top_left") -> np.ndarray:
    """Band -pre <= j - i <= next.  top_left: positions as they are; bottom_right: the
    diagonal moved to the last query / last key pair, i.e. j - i - (Skv - Sq)."""
    i = np.arange(Sq, dtype=np.int64)[:, None]
    j = np.arange(Skv, dtype=np.int64)[None, :]
    d = j - i - ((Skv - Sq) if align == "bottom_right" else 0)
    return (d >= -int(pre)) & (d <= int(next))


def keep_prefix_causal(Sq: int, Skv: int, prefix: int) -> np.ndarray:
    """Bottom-right causal plus a prefix: key j is visible from query i when
    j - i <= Skv - Sq, or when j < prefix (the first `prefix` keys are seen by every row)."""
    i = np.arange(Sq, dtype=np.int64)[:, None]
    j = np.arange(Skv, dtype=np.int64)[None, :]
    return (j - i <= Skv - Sq) | (j < int(prefix))


def attn_keep(q, k, v, keep, scale: float, threads: int = 0):
    """Dense attention over an explicit visibility matrix.  q (B,Nq,Sq,D), k (B,Nkv,Skv,D),
    v (B,Nkv,Skv,Dv), keep (Sq,Skv) or (B,Sq,Skv) bool -> out (B,Nq,Sq,Dv),
    softmax_max (B,Nq,Sq), softmax_sum (B,Nq,Sq)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Sq, D = q.shape
    _, Nkv, Skv, Dv = v.shape
    if k.shape != (B, Nkv, Skv, D) or v.shape[:3] != (B, Nkv, Skv):
        raise ValueError("shape mismatch")
    keep = np.broadcast_to(np.asarray(keep, dtype=bool), (B, Sq, Skv))
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    out = np.empty((B, Nq, Sq, Dv))
    m = np.empty((B, Nq, Sq))
    l = np.empty((B, Nq, Sq))
    rc = _load().oracle_attn_keep(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(m), _ptr(l),
                                  _ptr(keep), B, Nq, Nkv, Sq, Skv, D, Dv, float(scale), threads)
    if rc != 0:
        raise ValueError("oracle_attn_keep: invalid arguments")
    return out, m, l


def attn_varlen_keep(q, k, v, cu_q, cu_kv, keep_of, scale: float, threads: int = 0):
    """Packed attention with a visibility matrix per sequence: keep_of(b, Sq_b, Skv_b) ->
    bool (Sq_b, Skv_b).  q (Tq,Nq,D), k (Tkv,Nkv,D), v (Tkv,Nkv,Dv) -> out (Tq,Nq,Dv),
    softmax_max (Nq,Tq), softmax_sum (Nq,Tq).  Each sequence is the dense definition on its
    own rows (the packing of the varlen operator page)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, Nq, _ = q.shape
    Dv = v.shape[2]
    out = np.zeros((Tq, Nq, Dv))
    m = np.full((Nq, Tq), -np.inf)
    l = np.zeros((Nq, Tq))
    q0 = kv0 = 0
    for b, (qe, ke) in enumerate(zip(np.asarray(cu_q), np.asarray(cu_kv))):
        qe, ke = int(qe), int(ke)
        if qe > q0:
            qb = q[q0:qe].transpose(1, 0, 2)[None]
            kb = k[kv0:ke].transpose(1, 0, 2)[None]
            vb = v[kv0:ke].transpose(1, 0, 2)[None]
            if ke > kv0:
                o, mm, ll = attn_keep(qb, kb, vb, keep_of(b, qe - q0, ke - kv0), scale, threads)
                out[q0:qe] = o[0].transpose(1, 0, 2)
                m[:, q0:qe] = mm[0]
                l[:, q0:qe] = ll[0]
        q0, kv0 = qe, ke
    return out, m, l


# ------------------------------------------------------------------------------------
# dropout on the attention probabilities (the dropout_p of the MultiHeadAttention page and
# the SDPA-pitfalls blog).  The pages specify no generator; both sides implement the
# counter-based Philox4x32-10 from its published definition (Salmon, Moraes, Dror, Shaw,
# "Parallel random numbers: as easy as 1, 2, 3", SC 2011): 10 rounds of two 32x32->64
# multiplications by 0xD2511F53 and 0xCD9E8D57 with the Weyl key schedule 0x9E3779B9,
# 0xBB67AE85.
# ------------------------------------------------------------------------------------

def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 of the counters (uint32 arrays, broadcast) under key (k0, k1):
    four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint32) for x in (c0, c1, c2, c3)]
    c = [np.broadcast_to(x, np.broadcast(*c).shape).copy() for x in c]
    key = [int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF]
    for r in range(10):
        p0 = np.uint64(0xD2511F53) * c[0].astype(np.uint64)
        p1 = np.uint64(0xCD9E8D57) * c[2].astype(np.uint64)
        hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), p0.astype(np.uint32)
        hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), p1.astype(np.uint32)
        c = [hi1 ^ c[1] ^ np.uint32(key[0]), lo1, hi0 ^ c[3] ^ np.uint32(key[1]), lo0]
        key = [(key[0] + 0x9E3779B9) & 0xFFFFFFFF, (key[1] + 0xBB67AE85) & 0xFFFFFFFF]
    return c


def dropout_threshold(p: float) -> int:
    """Byte threshold of dropout probability p (0 <= p < 1): a probability is dropped when
    its random byte is below round(256 p); kept ones are scaled by 256 / (256 - thr)."""
    return int(round(float(p) * 256.0))


def dropout_keep(seed: int, offset: int, b: int, h: int, Sq: int, Skv: int, p: float):
    """Keep matrix [Sq, Skv] of (sequence / batch entry b, query head h): the random byte of
    (i, j) is byte j % 4 of word (j % 16) // 4 of Philox4x32-10 with counter
    (j // 16, i, h + 256 b, offset) and key (seed low 32 bits, seed high 32 bits)."""
    i = np.arange(Sq, dtype=np.uint32)[:, None]
    j = np.arange(Skv, dtype=np.uint32)[None, :]
    w = philox4x32_10(j // 16, i, np.uint32(h + 256 * b), np.uint32(offset), seed, seed >> 32)
    word = np.choose((j % 16) // 4, w) if Skv and Sq else np.zeros((Sq, Skv), np.uint32)
    byte = (word >> (8 * (j % 4))) & np.uint32(0xFF)
    return byte >= np.uint32(dropout_threshold(p))


def attn_dropout(q, k, v, scale: float, mask: str, pre: int, next: int, p: float, seed: int,
                 offset: int, batch_index=None, threads: int = 0):
    """Dense attention with dropout on the probabilities: out = (P * keep * 256 / (256 -
    thr)) V, with P the oracle's softmax probabilities; the statistics are those of P.
    batch_index[b] gives the b used in the counter (default b)."""
    out, m, l, probs = attn(q, k, v, scale, mask, pre, next, threads, return_probs=True)
    B, Nq, Sq, _ = out.shape
    Skv = probs.shape[-1]
    G = Nq // k.shape[1]
    thr = dropout_threshold(p)
    vv = _f64(v)
    res = np.empty_like(out)
    for b in range(B):
        bi = b if batch_index is None else int(batch_index[b])
        for h in range(Nq):
            keep = dropout_keep(seed, offset, bi, h, Sq, Skv, p)
            pd = probs[b, h] * keep * (256.0 / (256 - thr))
            res[b, h] = pd @ vv[b, h // G]
    return res, m, l


def attn_varlen_dropout(q, k, v, cu_q, cu_kv, scale: float, mask: str, pre: int, next: int,
                        p: float, seed: int, offset: int, threads: int = 0):
    """Packed attention with dropout: each sequence b is attn_dropout on its own rows, with
    sequence index b in the counter.  Shapes as attn_varlen."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, Nq, D = q.shape
    out = np.zeros_like(q)
    m = np.full((Nq, Tq), -np.inf)
    l = np.zeros((Nq, Tq))
    q0 = kv0 = 0
    for b, (qe, ke) in enumerate(zip(np.asarray(cu_q), np.asarray(cu_kv))):
        qe, ke = int(qe), int(ke)
        if qe > q0 and ke > kv0:
            o, mm, ll = attn_dropout(q[q0:qe].transpose(1, 0, 2)[None], k[kv0:ke].transpose(1, 0, 2)[None],
                                     v[kv0:ke].transpose(1, 0, 2)[None], scale, mask, pre, next, p,
                                     seed, offset, batch_index=[b], threads=threads)
            out[q0:qe] = o[0].transpose(1, 0, 2)
            m[:, q0:qe] = mm[0]
            l[:, q0:qe] = ll[0]
        q0, kv0 = qe, ke
    return out, m, l


def merge(o1, m1, l1, o2, m2, l2, threads: int = 0):
    """Merge two partials.  o* (B,N,S,D), m*/l* (B,N,S) -> out, softmax_max, softmax_sum."""
    o1, o2 = _f64(o1), _f64(o2)
    m1, l1, m2, l2 = _f64(m1), _f64(l1), _f64(m2), _f64(l2)
    B, N, S, D = o1.shape
    out = np.empty_like(o1)
    mo = np.empty((B, N, S))
    lo = np.empty((B, N, S))
    rc = _load().oracle_merge(_ptr(o1), _ptr(m1), _ptr(l1), _ptr(o2), _ptr(m2), _ptr(l2),
                              _ptr(out), _ptr(mo), _ptr(lo), B, N, S, D, threads)
    if rc != 0:
        raise ValueError("oracle_merge: invalid arguments")
    return out, mo, lo


def attn_update(q, k, v, prev_out, prev_max, prev_sum, scale: float, mask: str = "none",
                pre: int = 0, next: int = 0, threads: int = 0):
    """Attention of q over one key chunk, merged into a running result: the ring-attention
    update ("npu_ring_attention_update对外接口", equivalent small-operator logic) of
    (prev_out, prev_max, prev_sum) with attn(q, k, v).  Shapes as attn / merge."""
    o, m, l = attn(q, k, v, scale, mask, pre, next, threads)
    return merge(prev_out, prev_max, prev_sum, o, m, l, threads)


def attn_varlen_update(q, k, v, prev_out, prev_max, prev_sum, cu_q, cu_kv, scale: float,
                       mask: str = "none", pre: int = 0, next: int = 0, threads: int = 0):
    """attn_update over a packed batch: out (Tq,Nq,D), stats (Nq,Tq) as attn_varlen."""
    o, m, l = attn_varlen(q, k, v, cu_q, cu_kv, scale, mask, pre, next, threads)
    # the packed result is the dense (1, Nq, Tq, D) view for the elementwise merge
    bnsd = lambda x: np.ascontiguousarray(_f64(x).transpose(1, 0, 2))[None]
    out, mo, lo = merge(bnsd(prev_out), _f64(prev_max)[None], _f64(prev_sum)[None],
                        bnsd(o), m[None], l[None], threads)
    return np.ascontiguousarray(out[0].transpose(1, 0, 2)), mo[0], lo[0]


def sparse(q, k, v, offset, columns, scale: float, threads: int = 0):
    """CSR-sparse attention.  q/k/v (B,N,S,D), offset int32 (B,N,S+1), columns int32
    (B,N,nnz) -> out (B,N,S,D), softmax_max (B,N,S), softmax_sum (B,N,S)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    offset = np.ascontiguousarray(offset, dtype=np.int32)
    columns = np.ascontiguousarray(columns, dtype=np.int32)
    B, N, S, D = q.shape
    nnz = columns.shape[-1]
    out = np.empty_like(q)
    m = np.empty((B, N, S))
    l = np.empty((B, N, S))
    rc = _load().oracle_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(m), _ptr(l),
                               _ptr(offset), _ptr(columns), nnz, B, N, S, D, float(scale),
                               threads)
    if rc != 0:
        raise ValueError("oracle_sparse: invalid arguments")
    return out, m, l


def mha_self_attn(x, w_qkv, b_qkv, w_out, b_out, N: int, keep=None, dropout=None,
                  round_to=None, threads: int = 0):
    """Forward of the multi-head self-attention module of "flash attention的调用" (its
    MultiHeadAttention example): [q | k | v] = x W_qkv^T + b_qkv with the 3E outputs split
    into thirds, each reshaped to N heads of D = E / N columns; per head softmax(q k^T /
    sqrt(D)) v (no causal mask); the heads concatenated back; out = o W_out^T + b_out.

    x (B,S,E); w_qkv (3E,E); b_qkv (3E,) or None; w_out (E,E); b_out (E,) or None.
    keep: optional (S,S) bool visibility (True = the pair takes part).
    dropout: optional (p, seed, offset), applied as attn_dropout (batch b, head h counters).
    round_to: optional function applied where a storage type would round (the projections'
    outputs and the attention output), so that a low-precision product can be compared
    against the same roundings.  Returns out (B,S,E) in float64."""
    x = _f64(x)
    B, S, E = x.shape
    if E % N:
        raise ValueError("E must be a multiple of N")
    D = E // N
    qkv = x @ _f64(w_qkv).T
    if b_qkv is not None:
        qkv = qkv + _f64(b_qkv)
    if round_to is not None:
        qkv = round_to(qkv)
    q, k, v = (np.ascontiguousarray(qkv[..., i * E:(i + 1) * E].reshape(B, S, N, D).transpose(0, 2, 1, 3))
               for i in range(3))
    scale = 1.0 / np.sqrt(D)
    if dropout is not None:
        p, seed, offset = dropout
        o = attn_dropout(q, k, v, scale, "none", 0, 0, p, seed, offset, threads=threads)[0]
    elif keep is not None:
        o = attn_keep(q, k, v, keep, scale, threads)[0]
    else:
        o = attn(q, k, v, scale, "none", threads=threads)[0]
    o = o.transpose(0, 2, 1, 3).reshape(B, S, E)
    if round_to is not None:
        o = round_to(o)
    y = o @ _f64(w_out).T
    if b_out is not None:
        y = y + _f64(b_out)
    return y


def max_threads() -> int:
    """Threads the oracle uses when threads=0 (the OpenMP default of this process)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
