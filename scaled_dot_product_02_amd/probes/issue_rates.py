"""Issue rates of one and two waves per SIMD on matrix and vector instructions, from the
probe miattn_probe_issue (include/miattn_probes.h), as a markdown table.

    python -m scaled_dot_product_02_amd.probes.issue_rates [--iters N]

Each workgroup (one per CU) times its waves with the shader clock; a pattern's time is the
span from the first wave's start to the last wave's end, per round of the pattern.  In the
two-stream patterns (one wave of MFMAs and one of vector work on each SIMD) the table also
gives each role's own time and checks, from the SIMD id each wave reports, that every SIMD
held one wave of each role.
"""
from __future__ import annotations

import argparse
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(os.path.dirname(HERE), "libmiattn_probes.so")

PATTERNS = [
    (0, "16 v_mfma_f32_32x32x16_bf16"),
    (9, "16 v_mfma_f32_32x32x16_bf16 on one accumulator (dependent chain)"),
    (1, "64 v_fma_f32"),
    (10, "64 v_fma_f32 in one dependent chain"),
    (2, "32 v_exp_f32"),
    (11, "32 v_exp_f32, each followed by a v_add_f32 of its result"),
    (3, "16 MFMA, each followed by 2 v_fma_f32 + 2 v_exp_f32 (one stream)"),
    (5, "16 MFMA, each followed by 4 v_fma_f32 + 2 v_exp_f32 (one stream)"),
    (4, "per SIMD: one wave 16 MFMA, the other 32 v_fma_f32 + 32 v_exp_f32"),
    (6, "per SIMD: one wave 16 MFMA at s_setprio 3, the other 32 v_fma_f32 + 32 v_exp_f32"),
    (7, "per SIMD: one wave 16 MFMA, the other 48 v_fma_f32 + 16 v_exp_f32"),
    (8, "per SIMD: one wave 16 MFMA at s_setprio 3, the other 48 v_fma_f32 + 16 v_exp_f32"),
]
SPLIT = (4, 6, 7, 8)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=1000)
    args = ap.parse_args()
    lib = ctypes.CDLL(LIB)
    lib.miattn_probe_issue.argtypes = ([ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p] +
                                       [ctypes.c_int32] * 3 + [ctypes.c_void_p])
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, device="cuda")
    cyc = torch.zeros(blocks * 32, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    print("| pattern | waves per SIMD | cycles per round (workgroup span) | cycles per round, wave 0 "
          "| cycles per round, wave 4 |")
    print("|---|---|---|---|---|")
    for kind, name in PATTERNS:
        for wps in ((2,) if kind in SPLIT else (1, 2)):
            for _ in range(2):   # the second launch is the one read
                rc = lib.miattn_probe_issue(kind, out.data_ptr(), cyc.data_ptr(), blocks, wps, args.iters, stream)
                assert rc == 0, rc
            torch.cuda.synchronize()
            allc = cyc.view(blocks, 32).cpu().numpy()
            c = allc[:, :16].reshape(blocks, 8, 2)[:, :4 * wps]
            simd = allc[:, 16:16 + 4 * wps]
            span = (c[:, :, 1].max(1) - c[:, :, 0].min(1)).mean() / args.iters
            w0 = (c[:, 0, 1] - c[:, 0, 0]).mean() / args.iters
            w4 = f"{(c[:, 4, 1] - c[:, 4, 0]).mean() / args.iters:.1f}" if wps == 2 else "-"
            if kind in SPLIT:
                # every SIMD should hold one MFMA wave (0-3) and one vector wave (4-7)
                ok = all(sorted(r[:4]) == [0, 1, 2, 3] and sorted(r[4:]) == [0, 1, 2, 3] for r in simd)
                name += "" if ok else f" (SIMD ids of waves 0-7 in workgroup 0: {list(simd[0])})"
            print(f"| {name} | {wps} | {span:.1f} | {w0:.1f} | {w4} |", flush=True)


if __name__ == "__main__":
    main()
