#!/usr/bin/env python3
"""Benchmark of the MI355X attention forward (one JSON line on stdout).

A step is one attn_fwd_varlen call over the packed causal GQA workload: 16 sequences with
seed-0 lengths (T = 33,064 tokens, longest 3,977), Nq 32, Nkv 8, head_dim 128, bf16 inputs,
fp32 accumulation, causal per sequence, all inputs resident in HBM before timing.
The metric counts 4 * D * Nq * (visible (query, key) pairs) flops per step.

Also measured in the same run (reported under "secondary"):
  * the two small dense workloads: fp32 BNSD [1, 1, 128, 64] and bf16 BNSD [8, 8, 128, 64]
    (the SDPA blog's test shape), no mask; both are launch-latency bound;
  * the same forward with fp16 storage (same lengths and draws; 2.5 PFLOP/s fp16 peak);
  * the same forward with bottom-right causal plus a prefix of L/3 keys per sequence;
  * the same forward with dropout 0.1 on the probabilities;
  * an explicit mask tensor on dense bf16 [2, 32, 4096, 128], causal with 25% of keys
    masked out at random;
  * attn_lse_merge on the ring-merge workload (S 8192, N 32, D 128, SBH bf16), timed over
    rotating buffer sets (about 830 MB, larger than the 256 MB last-level cache);
  * causal attention over that workload's 4 key chunks of 2048 (a ring on one GPU): the
    fused attn_fwd_update chain vs attn_fwd + attn_lse_merge, and one full forward;
  * sparse_csr_attn on the CSR workload (B 2, N 8, S 4096, D 64, band 128 + 64 random), in
    fp32 and in fp64 (same pattern and draws);
  * head dim 256: dense causal bf16, S 8192, N 16 (4-wave workgroups, 32-key tiles);
  * head dim 768: dense causal bf16, S 4096, N 16 (the head-dim-general kernel);
  * fp32 inputs: dense causal, S 4096, N 16, D 128 (fp32 matrix-core products);
  * the multi-head self-attention module (mha_self_attn_fwd) at its defaults, embed 512 and
    8 heads, on B 8 x S 4096 bf16 in eval mode (projections + attention flops).

measured_peaks: the dense bf16 MFMA rate of the chip and the bandwidth of a plain 2-read /
1-write stream at the merge's size, from the peak probes (libmiattn_probes.so); each
roofline also states its fraction of the measured ceiling beside the datasheet one.

cpu_baseline: the CPU fp64 oracle (untuned) on a bounded sample of the same workload
(all sequences, the first --cpu-heads query heads), timed on this host's cores; under
"per_workload" the oracle timed on each of the other workloads (the small dense ones also
on one thread), with the CPU model.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (packed vector ALUs and matrix cores alike)
PEAK_F32_VALU_TFLOPS = 78.6  # fp32 vector ALUs without packed instructions (not built here)
PROBES_LIB = os.path.join(ROOT, "scaled_dot_product_02_amd", "libmiattn_probes.so")
PMC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_persist_varlen_causal_gqa_t33064_pmc.json")
# the kernel that serves the metric launch (bf16, D 128, 4 query heads per work item, packed)
METRIC_KERNEL = "fa_fwd_persist_kernel<128, __bf16, 4, true>"


def kernel_source_hash() -> str:
    """Hash of the metric kernel's code: its sources with comments and blank space
    removed, so that a comment edit does not retire the committed counter runs."""
    h = hashlib.sha256()
    for name in ("fa_fwd_persist.hip", "fa_mfma.h", "fa_params.h"):
        with open(os.path.join(ROOT, "scaled_dot_product_02_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        with open(PMC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def load_probes():
    """The peak probes (include/miattn_probes.h) through ctypes."""
    import ctypes
    if not os.path.exists(PROBES_LIB):
        raise SystemExit(f"{PROBES_LIB} is missing: build it with `python -m scaled_dot_product_02_amd.build`")
    lib = ctypes.CDLL(PROBES_LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.miattn_probe_mfma_bf16.argtypes = [P, I32, I32, P]
    lib.miattn_probe_mfma_bf16_flops.argtypes = [I32, I32]
    lib.miattn_probe_mfma_bf16_flops.restype = I64
    lib.miattn_probe_stream_r2w1.argtypes = [P, P, P, I64, P]
    lib.miattn_probe_l2_gather.argtypes = [P, I32, I32, I32, P, P]
    lib.miattn_probe_l2_gather_bytes.argtypes = [I32, I32]
    lib.miattn_probe_l2_gather_bytes.restype = I64
    return lib


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_launches(fn, steps: int, warmup: int, stream, warm_ms: float = 30.0):
    """Mean milliseconds per launch of fn over `steps` launches, after `warmup` launches and
    then more until at least warm_ms of warm-up work has run (the chip takes some
    milliseconds of load to reach its steady clock; the first launches of a large kernel
    run up to 20% slower)."""
    import time as _time
    import torch
    t0 = _time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while warm_ms > 0 and (_time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per launch


def cpu_baselines(oracle, synthetic, threads: int) -> dict:
    """The oracle (as it stands) timed on each workload other than the metric one: the two
    small dense ones whole (also on one thread), the ring merge whole plus its full causal
    forward on a sample of heads, and the CSR workload whole."""
    import numpy as np

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    res = {}
    for wname, dt_ in (("dense_f32_b1n1s128d64", "f32"), ("dense_bf16_b8n8s128d64", "bf16")):
        w = synthetic.make(wname)
        qv, kv, vv = (synthetic.storage_values(w[x], dt_) for x in ("q", "k", "v"))
        fl = 4.0 * w["B"] * w["Nq"] * w["Sq"] * w["Skv"] * w["D"]
        t1 = min(timed(lambda: oracle.attn(qv, kv, vv, 1 / math.sqrt(w["D"]), "none", threads=1))
                 for _ in range(3))
        tn = min(timed(lambda: oracle.attn(qv, kv, vv, 1 / math.sqrt(w["D"]), "none",
                                           threads=threads)) for _ in range(3))
        res[wname] = {"flop": fl, "seconds_1_thread": round(t1, 6),
                      f"seconds_{threads}_threads": round(tn, 6),
                      "tflops_1_thread": round(fl / t1 / 1e12, 6),
                      f"tflops_{threads}_threads": round(fl / tn / 1e12, 6)}
    # ring merge: the merge of two partials over all of S 8192, N 32, D 128 (random partials
    # of that shape), and the full causal forward over the first 4 of 32 heads
    rng = np.random.default_rng(0)
    S, N, Dm = 8192, 32, 128
    o1, o2 = (rng.standard_normal((1, N, S, Dm)) for _ in range(2))
    m1, m2 = (rng.standard_normal((1, N, S)) for _ in range(2))
    l1, l2 = (rng.uniform(1, 100, (1, N, S)) for _ in range(2))
    tm = timed(lambda: oracle.merge(o1, m1, l1, o2, m2, l2, threads=threads))
    mbytes = 3 * S * N * Dm * 2 + 6 * N * S * 4
    hs = 4
    qf, kf, vf = (rng.standard_normal((1, hs, S, Dm)) for _ in range(3))
    tf = timed(lambda: oracle.attn(qf, kf, vf, 1 / math.sqrt(Dm), "causal", threads=threads))
    ffl = 4.0 * Dm * hs * (S * (S + 1) // 2)
    res["ring_merge_sbh_bf16_s8192_n32_d128"] = {
        "merge_seconds": round(tm, 4), "merge_gbs_of_bf16_bytes": round(mbytes / tm / 1e9, 3),
        "causal_forward_sample": f"heads 0..{hs - 1} of {N}", "forward_flop": ffl,
        "forward_seconds": round(tf, 3), "forward_tflops": round(ffl / tf / 1e12, 5)}
    ws = synthetic.make("csr_sparse_f32_b2n8s4096d64")
    sfl = 4.0 * ws["B"] * ws["N"] * ws["nnz"] * ws["D"]
    ts = timed(lambda: oracle.sparse(ws["q"], ws["k"], ws["v"], ws["offset"], ws["columns"],
                                     1 / math.sqrt(ws["D"]), threads=threads))
    res["csr_sparse_f32_b2n8s4096d64"] = {"flop": sfl, "seconds": round(ts, 4),
                                          "tflops": round(sfl / ts / 1e12, 5)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="query heads in the oracle's CPU-baseline sample (0 = skip)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only the metric kernel (for profiler runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device-to-device copies of MIB MiB (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sharding across GPUs is design only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import scaled_dot_product_02_amd as mi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    def up(arr, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)

    # ---------------- metric: packed causal GQA forward ----------------
    name = synthetic.METRIC_WORKLOAD
    w = synthetic.make(name)
    Nq, Nkv, D, B, T = w["Nq"], w["Nkv"], w["D"], w["B"], w["Tq"]
    lengths = [int(x) for x in w["lengths_q"]]
    pairs = sum(L * (L + 1) // 2 for L in lengths)
    flops = 4.0 * D * Nq * pairs
    alg_bytes = 2 * (T * Nq * D * 2 + T * Nkv * D * 2) + 2 * 4 * Nq * T  # q,k,v,out + stats
    q, k, v = up(w["q"], "bf16"), up(w["k"], "bf16"), up(w["v"], "bf16")
    cu = torch.from_numpy(w["cu_q"]).to(dev)
    out = torch.empty_like(q)
    smax = torch.empty((Nq, T), dtype=torch.float32, device=dev)
    ssum = torch.empty((Nq, T), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)
    maxlen = max(lengths)

    def step():
        mi.attn_fwd_varlen(q, k, v, out, smax, ssum, cu, cu, B, T, T, maxlen, maxlen, Nq, Nkv, D,
                           "bf16", scale, "causal", 0, 0, stream.cuda_stream)

    ms = time_launches(step, args.steps, args.warmup, stream, warm_ms=0.0)   # exactly W warm-up steps
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic()

    result = {
        "metric": "attention fwd TFLOP/s (bf16 causal varlen GQA D=128) + % MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "batch_sequences": B, "total_tokens": T,
                   "max_seqlen": maxlen, "nq": Nq, "nkv": Nkv, "head_dim": D, "mask": "causal",
                   "layout": "TND", "visible_pairs_per_head": pairs, "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": alg_bytes,
                     "kernel": METRIC_KERNEL},
    }

    # ---------------- measured ceilings: dense bf16 MFMA rate of the chip ----------------
    probes = load_probes()
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count   # 8 waves per CU
    iters = 4096   # about a millisecond per launch: long enough for the clock to settle
    pout = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def mfma_probe():
        rc = probes.miattn_probe_mfma_bf16(pout.data_ptr(), blocks, iters, stream.cuda_stream)
        if rc:
            raise RuntimeError(f"mfma probe launch failed ({rc})")

    pms = time_launches(mfma_probe, 3, 1, stream)
    mfma_meas = probes.miattn_probe_mfma_bf16_flops(blocks, iters) / (pms * 1e-3) / 1e12
    result["measured_peaks"] = {
        "mfma_bf16_tflops": round(mfma_meas, 1),
        "mfma_method": f"{blocks} workgroups x 4 waves, back-to-back v_mfma_f32_32x32x16_bf16 "
                       "on 8 independent accumulators, random bf16 operands rotating per MFMA"}
    result["roofline"]["measured_peak"] = round(mfma_meas, 1)
    result["roofline"]["frac_of_measured_peak"] = round(tflops / mfma_meas, 4)
    del pout

    # ---------------- secondary: fp16 forward, merge and sparse ----------------
    if not args.no_secondary:
        sec = {}
        # the two small dense workloads (fp32 [1, 1, 128, 64] on the fp32 matrix-core path,
        # bf16 [8, 8, 128, 64] on the persistent kernel): far too small to fill the chip, so the
        # time per launch is launch latency; also timed as a captured graph of 100 launches
        for wname, dt_, peak in (("dense_f32_b1n1s128d64", "f32", PEAK_F32_TFLOPS),
                                 ("dense_bf16_b8n8s128d64", "bf16", PEAK_BF16_TFLOPS)):
            ws_ = synthetic.make(wname)
            sB, sN, sS, sD = ws_["B"], ws_["Nq"], ws_["Sq"], ws_["D"]
            tq, tk, tv = up(ws_["q"], dt_), up(ws_["k"], dt_), up(ws_["v"], dt_)
            to = torch.empty_like(tq)
            tm = torch.empty((sB, sN, sS), dtype=torch.float32, device=dev)
            tl = torch.empty_like(tm)
            sflop = 4.0 * sB * sN * sS * sS * sD

            def small_step(tq=tq, tk=tk, tv=tv, to=to, tm=tm, tl=tl, sB=sB, sN=sN, sS=sS, sD=sD,
                           dt_=dt_):
                mi.attn_fwd(tq, tk, tv, to, tm, tl, sB, sN, sN, sS, sS, sD, dt_, "BNSD",
                            1 / math.sqrt(sD), "none", 0, 0, stream.cuda_stream)

            sms_ = time_launches(small_step, 200, 20, stream)
            gstream = torch.cuda.Stream()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(gstream):
                small_step()   # settles the stream before capture
                gstream.synchronize()
                with torch.cuda.graph(graph, stream=gstream):
                    for _ in range(100):
                        mi.attn_fwd(tq, tk, tv, to, tm, tl, sB, sN, sN, sS, sS, sD, dt_, "BNSD",
                                    1 / math.sqrt(sD), "none", 0, 0, gstream.cuda_stream)
            gms_ = time_launches(graph.replay, 10, 2, stream) / 100
            stf_ = sflop / (gms_ * 1e-3) / 1e12
            sec[wname] = {
                "workload": wname, "flop_per_launch": sflop,
                "us_per_launch": round(sms_ * 1e3, 2),
                "us_per_launch_in_graph": round(gms_ * 1e3, 2),
                "roofline": {"bound": "latency", "achieved": round(stf_, 3), "peak": peak,
                             "unit": "TFLOP/s", "frac": round(stf_ / peak, 5)}}
            del graph, tq, tk, tv, to, tm, tl

        wh = synthetic.varlen_inputs(0, Nq, Nkv, D, "f16", B=B)   # same lengths, fp16 storage
        hq, hk, hv = (torch.from_numpy(np.ascontiguousarray(wh[x]).view(np.float16)).to(dev)
                      for x in ("q", "k", "v"))
        hout = torch.empty_like(hq)

        def step_f16():
            mi.attn_fwd_varlen(hq, hk, hv, hout, smax, ssum, cu, cu, B, T, T, maxlen, maxlen, Nq,
                               Nkv, D, "f16", scale, "causal", 0, 0, stream.cuda_stream)

        hms = time_launches(step_f16, args.steps, args.warmup, stream)
        htf = flops / (hms * 1e-3) / 1e12
        sec["attn_fwd_varlen_f16"] = {
            "workload": name.replace("bf16", "f16"), "ms_per_launch": round(hms, 4),
            "roofline": {"bound": "mfma", "achieved": round(htf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(htf / PEAK_BF16_TFLOPS, 4)}}
        del hq, hk, hv, hout

        # the same workload with bottom-right causal plus a per-sequence prefix of L/3 keys
        prefix = [L // 3 for L in lengths]
        pdev = torch.tensor(prefix, dtype=torch.int64, device=dev)
        ppairs = sum(sum(min(L, max(P, i + 1)) for i in range(L)) for L, P in zip(lengths, prefix))
        pflops = 4.0 * D * Nq * ppairs

        def step_prefix():
            mi.attn_fwd_varlen_ext(q, k, v, out, smax, ssum, cu, cu, B, T, T, maxlen, maxlen,
                                      Nq, Nkv, D, D, "bf16", scale, "causal_br", 0, 0, pdev, None,
                                      stream=stream.cuda_stream)

        pms = time_launches(step_prefix, args.steps, args.warmup, stream)
        ptf = pflops / (pms * 1e-3) / 1e12
        sec["attn_fwd_varlen_prefix"] = {
            "workload": name + "_prefix_len_div_3_causal_bottom_right",
            "ms_per_launch": round(pms, 4), "flop_per_launch": pflops,
            "roofline": {"bound": "mfma", "achieved": round(ptf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ptf / PEAK_BF16_TFLOPS, 4)}}

        # the same workload with dropout 0.1 on the probabilities (Philox4x32-10 bytes)
        def step_dropout():
            mi.attn_fwd_varlen_ext(q, k, v, out, smax, ssum, cu, cu, B, T, T, maxlen, maxlen,
                                   Nq, Nkv, D, D, "bf16", scale, "causal", 0, 0, None, None,
                                   0.1, 2026, 0, stream=stream.cuda_stream)

        dms_ = time_launches(step_dropout, args.steps, args.warmup, stream)
        dtf_ = flops / (dms_ * 1e-3) / 1e12
        sec["attn_fwd_varlen_dropout"] = {
            "workload": name + "_dropout_0.1", "ms_per_launch": round(dms_, 4),
            "roofline": {"bound": "mfma", "achieved": round(dtf_, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(dtf_ / PEAK_BF16_TFLOPS, 4)}}

        # explicit mask tensor: dense bf16 [2, 32, 4096, 128], causal plus a random 25% of
        # keys masked out (rows of whole 4-byte words: the MFMA path)
        Sx, Bx, Nx = 4096, 2, 32
        wx = synthetic.dense_inputs(0, Bx, Nx, Nx, Sx, Sx, D, "bf16", "BNSD")
        xq, xk, xv = up(wx["q"], "bf16"), up(wx["k"], "bf16"), up(wx["v"], "bf16")
        xo = torch.empty_like(xq)
        am_np = np.random.default_rng(0).random((Sx, Sx)) < 0.25
        xam = torch.from_numpy(am_np.astype(np.uint8)).to(dev)
        xpairs = int((np.tril(np.ones((Sx, Sx), dtype=bool)) & ~am_np).sum())
        xflops = 4.0 * D * Bx * Nx * xpairs

        def step_amask():
            mi.attn_fwd_ext(xq, xk, xv, xo, None, None, Bx, Nx, Nx, Sx, Sx, D, D, "bf16", "BNSD",
                               scale, "causal", 0, 0, None, xam, stream=stream.cuda_stream)

        xms = time_launches(step_amask, 5, 1, stream)
        xtf = xflops / (xms * 1e-3) / 1e12
        sec["attn_fwd_explicit_mask"] = {
            "workload": "dense_bf16_b2n32s4096d128_causal_random_mask_25pct",
            "ms_per_launch": round(xms, 3), "flop_per_launch": xflops,
            "roofline": {"bound": "mfma", "achieved": round(xtf, 3), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(xtf / PEAK_BF16_TFLOPS, 4)}}
        del xq, xk, xv, xo, xam
        S, N, Dm = 8192, 32, 128
        rng = np.random.default_rng(0)
        sets = []
        for _ in range(4):
            o1 = torch.randn((S, 1, N * Dm), device=dev).to(torch.bfloat16)
            o2 = torch.randn((S, 1, N * Dm), device=dev).to(torch.bfloat16)
            st = [torch.from_numpy(x).to(dev) for x in
                  (rng.standard_normal((1, N, S), dtype=np.float32),
                   rng.uniform(1, 100, (1, N, S)).astype(np.float32),
                   rng.standard_normal((1, N, S), dtype=np.float32),
                   rng.uniform(1, 100, (1, N, S)).astype(np.float32))]
            res = [torch.empty_like(o1), torch.empty((1, N, S), device=dev),
                   torch.empty((1, N, S), device=dev)]
            sets.append((o1, st[0], st[1], o2, st[2], st[3], *res))
        it = [0]

        def merge_step():
            s_ = sets[it[0] % len(sets)]
            it[0] += 1
            mi.attn_lse_merge(*s_, 1, N, S, Dm, "bf16", "SBH", stream.cuda_stream)

        mms = time_launches(merge_step, 4 * 25, 8, stream)

        # measured streaming ceiling at the same size: read two 64 MiB arrays, write one
        sbytes_stream = sets[0][0].numel() * 2

        def stream_step():
            s_ = sets[it[0] % len(sets)]
            it[0] += 1
            rc = probes.miattn_probe_stream_r2w1(s_[0].data_ptr(), s_[3].data_ptr(),
                                                 s_[6].data_ptr(), sbytes_stream, stream.cuda_stream)
            if rc:
                raise RuntimeError(f"stream probe launch failed ({rc})")

        stms = time_launches(stream_step, 4 * 25, 8, stream)
        stream_gbs = 3 * sbytes_stream / (stms * 1e-3) / 1e9
        result["measured_peaks"]["stream_2r1w_gbs"] = round(stream_gbs, 1)
        result["measured_peaks"]["stream_method"] = (
            "o[i] = a[i] ^ b[i] over 3 x 64 MiB, non-temporal 16-byte accesses, 4 rotating sets")

        # causal ring over 4 key chunks of the same workload: fused update vs
        # forward + merge kernel, and the single full forward for reference
        qr, kr, vr = sets[0][0], sets[1][0], sets[2][0]
        C, nch = S // 4, 4
        run_o, run_m, run_l = sets[3][6], sets[3][7], sets[3][8]
        part_o, part_m, part_l = sets[3][0], sets[3][1], sets[3][2]
        sc = 1.0 / math.sqrt(Dm)

        def ring_fused():
            for j in range(nch):
                kj, vj = kr[j * C:(j + 1) * C], vr[j * C:(j + 1) * C]
                if j == 0:
                    mi.attn_fwd(qr, kj, vj, run_o, run_m, run_l, 1, N, N, S, C, Dm, "bf16", "SBH",
                                sc, "causal", 0, 0, stream.cuda_stream)
                else:
                    mi.attn_fwd_update(qr, kj, vj, run_o, run_m, run_l, run_o, run_m, run_l, 1, N, N,
                                       S, C, Dm, "bf16", "SBH", sc, "band", 1 << 40, -j * C,
                                       stream.cuda_stream)

        def ring_unfused():
            for j in range(nch):
                kj, vj = kr[j * C:(j + 1) * C], vr[j * C:(j + 1) * C]
                if j == 0:
                    mi.attn_fwd(qr, kj, vj, run_o, run_m, run_l, 1, N, N, S, C, Dm, "bf16", "SBH",
                                sc, "causal", 0, 0, stream.cuda_stream)
                else:
                    mi.attn_fwd(qr, kj, vj, part_o, part_m, part_l, 1, N, N, S, C, Dm, "bf16",
                                "SBH", sc, "band", 1 << 40, -j * C, stream.cuda_stream)
                    mi.attn_lse_merge(run_o, run_m, run_l, part_o, part_m, part_l, run_o, run_m,
                                      run_l, 1, N, S, Dm, "bf16", "SBH", stream.cuda_stream)

        def full_causal():
            mi.attn_fwd(qr, kr, vr, run_o, run_m, run_l, 1, N, N, S, S, Dm, "bf16", "SBH", sc,
                        "causal", 0, 0, stream.cuda_stream)

        ring_flops = 4.0 * Dm * N * (S * (S + 1) // 2)
        ring = {"workload": "causal_ring_4chunks_sbh_bf16_s8192_n32_d128",
                "flop_per_pass": ring_flops}
        for key, fn in (("fused_update", ring_fused), ("forward_plus_merge", ring_unfused),
                        ("single_full_forward", full_causal)):
            rms = time_launches(fn, 20, 3, stream)
            ring[key] = {"ms_per_pass": round(rms, 4),
                         "tflops": round(ring_flops / (rms * 1e-3) / 1e12, 2)}
        sec["causal_ring_4_chunks"] = ring
        mbytes = 3 * S * N * Dm * 2 + 6 * N * S * 4
        mgbs = mbytes / (mms * 1e-3) / 1e9
        sec["attn_lse_merge"] = {
            "workload": "ring_merge_sbh_bf16_s8192_n32_d128", "us_per_launch": round(mms * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(mgbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(mgbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": mbytes, "rotating_sets": len(sets),
                         "measured_peak": round(stream_gbs, 1),
                         "frac_of_measured_peak": round(mgbs / stream_gbs, 4)}}
        del sets

        ws = synthetic.make("csr_sparse_f32_b2n8s4096d64")
        sq, sk, sv = (up(ws[x], "f32") for x in ("q", "k", "v"))
        so = torch.empty_like(sq)
        soff = torch.from_numpy(ws["offset"]).to(dev)
        scol = torch.from_numpy(ws["columns"]).to(dev)
        sB, sN, sS, sD, nnz = ws["B"], ws["N"], ws["S"], ws["D"], ws["nnz"]

        def sparse_step():
            mi.sparse_csr_attn(sq, sk, sv, so, soff, scol, nnz, sB, sN, sS, sD, "f32",
                               1 / math.sqrt(sD), stream.cuda_stream)

        sms = time_launches(sparse_step, 20, 3, stream)
        sflops = 4.0 * sB * sN * nnz * sD
        sbytes = 4 * 4 * sB * sN * sS * sD + 4 * sB * sN * (nnz + sS + 1)
        stf = sflops / (sms * 1e-3) / 1e12

        # measured ceiling of the sparse kernel's access: random 256-byte row gathers from a
        # 2 MiB region per XCD (the K and V of one (b, n) slice in fp32), held in L2
        rows_log2 = 13   # 8192 rows of 256 B = 2 MiB per region
        gtab = torch.randint(0, 1 << 30, (8 << rows_log2, 64), dtype=torch.int32, device=dev)
        gblocks, giters = 8 * torch.cuda.get_device_properties(0).multi_processor_count, 512
        gout = torch.empty(gblocks * 256, dtype=torch.int32, device=dev)

        def gather_probe():
            rc = probes.miattn_probe_l2_gather(gtab.data_ptr(), rows_log2, gblocks, giters,
                                               gout.data_ptr(), stream.cuda_stream)
            if rc:
                raise RuntimeError(f"gather probe launch failed ({rc})")

        gpms = time_launches(gather_probe, 10, 3, stream)
        gather_gbs = probes.miattn_probe_l2_gather_bytes(gblocks, giters) / (gpms * 1e-3) / 1e9
        result["measured_peaks"]["l2_gather_gbs"] = round(gather_gbs, 1)
        result["measured_peaks"]["l2_gather_method"] = (
            f"{gblocks} workgroups x 4 waves, random 256-byte rows (16 B a lane) from 2 MiB per "
            "XCD, 8 rows in flight per 16 lanes")
        del gtab, gout

        def sparse_split(dtype_):
            """Entries whose K / V rows the kernel reads from its LDS window (the keys before
            the end of each 64-row block, sparse_csr_window) and entries it gathers from
            global memory, and the rows the window copies take (coalesced)."""
            W = mi.sparse_csr_window(sD, dtype_)
            off_, col_ = ws["offset"].reshape(-1, sS + 1), ws["columns"].reshape(-1, nnz)
            in_w, copied = 0, 0
            r1_blocks = np.minimum(sS, np.arange(64, sS + 64, 64))
            copied = int(np.sum(r1_blocks - np.maximum(0, r1_blocks - W))) * off_.shape[0]
            for sl in range(off_.shape[0]):
                n_ = int(off_[sl, -1])
                rows_ = np.repeat(np.arange(sS), np.diff(off_[sl]))
                r1 = np.minimum(sS, (rows_ // 64 + 1) * 64)
                c_ = col_[sl, :n_]
                in_w += int(np.count_nonzero((c_ >= np.maximum(0, r1 - W)) & (c_ < r1)))
            return W, in_w, copied

        def sparse_roofline(seconds, elem, split):
            # every stored entry reads one K row and one V row of D elements: from the LDS
            # window or, for the rest, gathered from global memory (L2); the bound is the
            # latter against the measured random-row gather rate
            W, in_w, copied = split
            total = sB * sN * nnz
            gathered = 2.0 * (total - in_w) * sD * elem
            ach = gathered / seconds / 1e9
            return {"bound": "l2_gather", "achieved": round(ach, 1), "peak": round(gather_gbs, 1),
                    "unit": "GB/s", "frac": round(ach / gather_gbs, 4),
                    "gathered_bytes": gathered, "window_keys": W,
                    "entries_from_lds_window": in_w, "entries_total": total,
                    "window_copy_bytes": 2.0 * copied * sD * elem,
                    "row_bytes_all_entries": 2.0 * total * sD * elem}

        sec["sparse_csr_attn"] = {
            "workload": "csr_sparse_f32_b2n8s4096d64", "us_per_launch": round(sms * 1e3, 2),
            "tflops": round(stf, 3), "gbs_algorithmic": round(sbytes / (sms * 1e-3) / 1e9, 1),
            "roofline": sparse_roofline(sms * 1e-3, 4, sparse_split("f32")),
            "alu": {"achieved": round(stf, 3), "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(stf / PEAK_F32_VALU_TFLOPS, 4)}}
        # the same CSR workload with fp64 inputs and arithmetic
        wd = synthetic.sparse_inputs(0, sB, sN, sS, sD, band=128, n_random=64, dtype="f64")
        dq, dk, dv = (torch.from_numpy(np.ascontiguousarray(wd[x])).to(dev) for x in ("q", "k", "v"))
        do_ = torch.empty_like(dq)

        def sparse_step_f64():
            mi.sparse_csr_attn(dq, dk, dv, do_, soff, scol, nnz, sB, sN, sS, sD, "f64",
                               1 / math.sqrt(sD), stream.cuda_stream)

        dms = time_launches(sparse_step_f64, 10, 2, stream)
        dtf = sflops / (dms * 1e-3) / 1e12
        sec["sparse_csr_attn_f64"] = {
            "workload": "csr_sparse_f64_b2n8s4096d64", "us_per_launch": round(dms * 1e3, 2),
            "tflops": round(dtf, 3),
            "roofline": sparse_roofline(dms * 1e-3, 8, sparse_split("f64")),
            "alu": {"achieved": round(dtf, 3), "peak": 78.6, "unit": "TFLOP/s",
                    "frac": round(dtf / 78.6, 4)}}

        # head dim 256 (4-wave workgroups, 32-key tiles): dense causal bf16, S 8192, N 16
        Sd, Nd, Dd = 8192, 16, 256
        gd = torch.Generator(device=dev); gd.manual_seed(0)
        dq, dk, dv_ = (torch.randn((1, Nd, Sd, Dd), device=dev, generator=gd).to(torch.bfloat16)
                       for _ in range(3))
        do_ = torch.empty_like(dq)
        dflops = 4.0 * Dd * Nd * (Sd * (Sd + 1) // 2)

        def step_d256():
            mi.attn_fwd(dq, dk, dv_, do_, None, None, 1, Nd, Nd, Sd, Sd, Dd, "bf16", "BNSD",
                        1 / math.sqrt(Dd), "causal", stream=stream.cuda_stream)

        d2ms = time_launches(step_d256, 10, 2, stream)
        d2tf = dflops / (d2ms * 1e-3) / 1e12
        sec["attn_fwd_head_dim_256"] = {
            "workload": "dense_causal_bf16_b1n16s8192d256", "ms_per_launch": round(d2ms, 4),
            "flop_per_launch": dflops,
            "roofline": {"bound": "mfma", "achieved": round(d2tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(d2tf / PEAK_BF16_TFLOPS, 4)}}
        del dq, dk, dv_, do_

        # head dim 768, the operator's largest, on the head-dim-general kernel (head dims split
        # across the waves of a workgroup): dense causal bf16, S 4096, N 16
        Sw, Nw, Dw = 4096, 16, 768
        gw = torch.Generator(device=dev); gw.manual_seed(0)
        wq_, wk_, wv_ = (torch.randn((1, Nw, Sw, Dw), device=dev, generator=gw).to(torch.bfloat16)
                         for _ in range(3))
        wo_ = torch.empty_like(wq_)
        wflops = 4.0 * Dw * Nw * (Sw * (Sw + 1) // 2)

        def step_d768():
            mi.attn_fwd(wq_, wk_, wv_, wo_, None, None, 1, Nw, Nw, Sw, Sw, Dw, "bf16", "BNSD",
                        1 / math.sqrt(Dw), "causal", stream=stream.cuda_stream)

        wms = time_launches(step_d768, 10, 2, stream)
        wtf = wflops / (wms * 1e-3) / 1e12
        sec["attn_fwd_head_dim_768"] = {
            "workload": "dense_causal_bf16_b1n16s4096d768", "ms_per_launch": round(wms, 4),
            "flop_per_launch": wflops,
            "roofline": {"bound": "mfma", "achieved": round(wtf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(wtf / PEAK_BF16_TFLOPS, 4)}}
        del wq_, wk_, wv_, wo_

        # fp32 inputs (the general kernel's fp32 matrix-core path): dense causal, S 4096,
        # N 16, D 128
        Sf, Nf, Df = 4096, 16, 128
        gf = torch.Generator(device=dev); gf.manual_seed(0)
        fq, fk, fv = (torch.randn((1, Nf, Sf, Df), device=dev, generator=gf) for _ in range(3))
        fo = torch.empty_like(fq)
        fflops = 4.0 * Df * Nf * (Sf * (Sf + 1) // 2)

        def step_f32():
            mi.attn_fwd(fq, fk, fv, fo, None, None, 1, Nf, Nf, Sf, Sf, Df, "f32", "BNSD",
                        1 / math.sqrt(Df), "causal", stream=stream.cuda_stream)

        fms = time_launches(step_f32, 10, 2, stream)
        ftf = fflops / (fms * 1e-3) / 1e12
        sec["attn_fwd_fp32"] = {
            "workload": "dense_causal_f32_b1n16s4096d128", "ms_per_launch": round(fms, 4),
            "flop_per_launch": fflops,
            "roofline": {"bound": "mfma", "achieved": round(ftf, 2), "peak": PEAK_F32_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ftf / PEAK_F32_TFLOPS, 4)}}
        del fq, fk, fv, fo

        # the multi-head self-attention module at its defaults (embed 512, 8 heads), eval
        # mode: two rocBLAS projections around the attention kernel
        Bm, Sm, Em, Nm = 8, 4096, 512, 8
        gm = torch.Generator(device=dev); gm.manual_seed(0)
        mx = torch.randn((Bm, Sm, Em), device=dev, generator=gm).to(torch.bfloat16)
        a_ = 1.0 / math.sqrt(Em)
        mw = [(torch.rand(shape, device=dev, generator=gm) * 2 - 1).mul_(a_).to(torch.bfloat16)
              for shape in ((3 * Em, Em), (3 * Em,), (Em, Em), (Em,))]
        mo = torch.empty_like(mx)
        mws_bytes = mi.mha_workspace_bytes(Bm, Sm, Em, "bf16")
        mws = torch.empty(mws_bytes, dtype=torch.uint8, device=dev)
        mflops = 8.0 * Bm * Sm * Em * Em + 4.0 * Bm * Sm * Sm * Em   # projections + attention

        def step_mha():
            mi.mha_self_attn_fwd(mx, mw[0], mw[1], mw[2], mw[3], mo, mws, mws_bytes, Bm, Sm, Em, Nm,
                                 "bf16", stream=stream.cuda_stream)

        mms = time_launches(step_mha, 10, 2, stream)
        mtf = mflops / (mms * 1e-3) / 1e12
        sec["mha_self_attn"] = {
            "workload": "mha_self_attn_bf16_b8s4096_e512_h8", "ms_per_call": round(mms, 4),
            "flop_per_call": mflops,
            "roofline": {"bound": "mfma", "achieved": round(mtf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(mtf / PEAK_BF16_TFLOPS, 4)}}
        del mx, mw, mo, mws
        result["secondary"] = sec

    # ---------------- CPU baseline: the oracle on a bounded sample ----------------
    if args.cpu_heads > 0:
        import oracle
        hs = min(args.cpu_heads, Nq)
        G = Nq // Nkv
        kvh = (hs + G - 1) // G
        qs = synthetic.storage_values(w["q"][:, :hs], "bf16")
        ks = synthetic.storage_values(w["k"][:, :kvh], "bf16")
        vs = synthetic.storage_values(w["v"][:, :kvh], "bf16")
        # keep the head -> kv-head map: kv head of query head h is h // G
        if hs % G:
            raise SystemExit("--cpu-heads must be a multiple of the GQA group")
        threads = oracle.max_threads()
        t0 = time.perf_counter()
        oracle.attn_varlen(qs, ks, vs, w["cu_q"], w["cu_kv"], scale, "causal", threads=threads)
        dt = time.perf_counter() - t0
        sflops = 4.0 * D * hs * pairs
        result["cpu_baseline"] = {
            "value": round(sflops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"all {B} sequences x query heads 0..{hs - 1} of {Nq} "
                      f"({sflops / 1e9:.1f} GFLOP fp64, {dt:.1f} s wall)",
            "cpu_model": cpu_model(),
            "per_workload": cpu_baselines(oracle, synthetic, threads)}

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
