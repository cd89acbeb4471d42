"""mha_self_attn_fwd_noalloc (the multi-head module without a workspace: intermediates in a
static device array, projections on the library's own GEMM kernel) against
mha_self_attn_fwd through the C ABI, on two calls in a row where the second is smaller (the
array keeps the first call's contents), and against the CPU fp64 oracle.  Tolerances as
tests/test_gpu_mha.py (relative to the largest output; the two entry points differ only in
the summation order of the projections)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_utils import dev, empty_like_storage, host_values
from test_gpu_mha import RTOL, _check, _inputs, _rounder

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mi():
    import scaled_dot_product_02_amd as m
    return m


def _both(mi, stored, B, S, E, N, dtype, mask=None, p=0.0, seed=0, offset=0):
    d = {k: None if v is None else dev(v, dtype) for k, v in stored.items()}
    ref = empty_like_storage((B, S, E), dtype)
    nbytes = mi.mha_workspace_bytes(B, S, E, dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    mi.mha_self_attn_fwd(d["x"], d["w_qkv"], d["b_qkv"], d["w_out"], d["b_out"], ref, ws, nbytes,
                         B, S, E, N, dtype, atten_mask=mask, dropout_p=p, seed=seed, offset=offset)
    got = empty_like_storage((B, S, E), dtype)
    mi.mha_self_attn_fwd_noalloc(d["x"], d["w_qkv"], d["b_qkv"], d["w_out"], d["b_out"], got,
                                 B, S, E, N, dtype, atten_mask=mask, dropout_p=p, seed=seed,
                                 offset=offset)
    torch.cuda.synchronize()
    return host_values(got), host_values(ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_noalloc_matches_workspace_entry_point_twice(mi, dtype):
    """A larger call, then a smaller one (other heads, no bias) on the same scratch."""
    for seed, (B, S, E, N, bias) in ((301, (2, 300, 512, 8, True)), (302, (1, 129, 256, 2, False))):
        stored, vals = _inputs(seed, B, S, E, dtype, bias)
        got, ref = _both(mi, stored, B, S, E, N, dtype)
        _check(got, ref, dtype, f"noalloc vs workspace entry point, B {B} S {S} E {E}")
        want = oracle.mha_self_attn(vals["x"], vals["w_qkv"], vals["b_qkv"], vals["w_out"],
                                    vals["b_out"], N, round_to=_rounder(dtype))
        _check(got, want, dtype, f"noalloc vs oracle, B {B} S {S} E {E}")


def test_noalloc_mask_and_dropout(mi):
    B, S, E, N = 2, 192, 256, 4
    stored, _ = _inputs(303, B, S, E, "bf16")
    am = torch.from_numpy((np.random.default_rng(304).random((S, S)) < 0.3).astype(np.uint8)).to("cuda:0")
    got, ref = _both(mi, stored, B, S, E, N, "bf16", mask=am)
    _check(got, ref, "bf16", "mask tensor")
    got, ref = _both(mi, stored, B, S, E, N, "bf16", p=0.2, seed=77, offset=5)
    _check(got, ref, "bf16", "dropout")


def test_noalloc_rejects_problems_beyond_its_scratch(mi):
    # bf16: 4 planes of B*S*E*2 bytes; B*S*E = 8 Mi elements fits exactly, one row more does not
    E = 512
    with pytest.raises(mi.MiattnError) as e:
        mi.mha_self_attn_fwd_noalloc(256, 256, None, 256, None, 256, 1, (8 << 20) // E + 1, E, 8,
                                     "bf16", stream=0)
    assert mi.STATUS[e.value.status] == "MIATTN_ERR_SCRATCH"
