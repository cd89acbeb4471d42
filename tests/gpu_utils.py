"""Helpers of the GPU parity tests: device upload/download and the tolerance checks.

Tolerances (stated once, used everywhere):
  fp32 outputs:                    max |gpu - oracle| <= 1e-5
  bf16 outputs (fp32 accumulation): max |gpu - oracle| <= 2e-2
  fp16 outputs (fp32 accumulation): max |gpu - oracle| <= 5e-3  (derived: the softmax weights
    and the output are each rounded once to binary16, unit roundoff u = 2^-11, with |v|, |out|
    <= 5 for these normal draws, so the error is below 2 * 5 * u = 4.9e-3)
  fp64 outputs (fp64 arithmetic):  max |gpu - oracle| <= 1e-10  (derived: score rounding
    ~ D * 2^-53 * sum|q_d k_d| < 1e-12 for these draws, times |v| <= 5, with margin)
  softmax_max:  |gpu - oracle| <= 1e-4 * max(1, |oracle|)   (-inf must match exactly)
  softmax_sum:  |gpu - oracle| <= 1e-4 * oracle              (0 must match exactly)
"""
from __future__ import annotations

import numpy as np
import torch

import synthetic

TOL_OUT = {"f32": 1e-5, "bf16": 2e-2, "f16": 5e-3, "f64": 1e-10}
TOL_STAT = 1e-4


def dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload a stored array (float32, or bf16 / fp16 bit patterns) to cuda:0 unchanged."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to("cuda:0")


def host_values(t: torch.Tensor) -> np.ndarray:
    """float64 values of a device tensor (exact widening of bf16 / fp16 / fp32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synthetic.f32_from_bf16_bits(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    if t.dtype == torch.float16:
        return t.numpy().astype(np.float64)
    return t.numpy().astype(np.float64)


def empty_like_storage(shape, dtype: str) -> torch.Tensor:
    """Output buffer pre-filled with NaN so that an unwritten element fails the checks."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
           "f64": torch.float64}[dtype]
    return torch.full(shape, float("nan"), dtype=tdt, device="cuda:0")


def nan_stats(shape) -> torch.Tensor:
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda:0")


def check_out(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "out"):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values (unwritten or NaN)"
    err = np.max(np.abs(got - want)) if got.size else 0.0
    assert err <= TOL_OUT[dtype], f"{what}: max abs err {err:.3e} > {TOL_OUT[dtype]}"
    return err


def check_stats(gm: np.ndarray, gl: np.ndarray, wm: np.ndarray, wl: np.ndarray):
    assert gm.shape == wm.shape and gl.shape == wl.shape
    empty = wl == 0
    assert np.all(gm[empty] == -np.inf), "softmax_max of empty rows must be -inf"
    assert np.all(gl[empty] == 0), "softmax_sum of empty rows must be 0"
    ne = ~empty
    if ne.any():
        em = np.abs(gm[ne] - wm[ne]) / np.maximum(1.0, np.abs(wm[ne]))
        el = np.abs(gl[ne] - wl[ne]) / wl[ne]
        assert np.max(em) <= TOL_STAT, f"softmax_max rel err {np.max(em):.3e}"
        assert np.max(el) <= TOL_STAT, f"softmax_sum rel err {np.max(el):.3e}"
        return float(np.max(em)), float(np.max(el))
    return 0.0, 0.0
