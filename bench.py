#!/usr/bin/env python3
"""Benchmark of non-causal DiT attention on one MI355X.

Metric: effective attention TFLOPS and fraction of MFMA peak at the Wan 2.2
shape B=1, H=40, S=75,600 (21 x 45 x 80 token grid), D=128.  Effective work
of one call is 4 * B * H * S^2 * D; skipped Skip-Softmax tiles count as done.

One step is one pass of the whole hot path over one batch of synthetic input
at that shape:
  1. dense BF16 attention (spatially peaked Q/K, the Skip-Softmax workload's
     inputs);
  2. SAGE attention, FP8 E4M3 Q/K + per-channel FP8 V, blocks (1, 4, 1), on
     Gaussian inputs with a per-channel K bias and outlier channels
     (quantization with K-smoothing included);
  3. Skip-Softmax attention on the same BF16 inputs as 1, threshold factor 1
     (lambda = 1 / S), with the host timestep gate evaluated (t = 0.5, D = 0.86).
Inputs are resident in HBM before the timed region.  The JSON line carries the
per-call breakdown, the MFMA roofline of the dominant kernel (timed with HIP
events on the launch stream), and the CPU oracle timed on a bounded sample on
this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense MFMA peaks (TFLOP/s; TOP/s for int8) and HBM bandwidth.
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "int8": 5000.0}
HBM_GBPS = 8000.0
WAN = dict(B=1, S=75600, H=40, D=128)
SKIP_FACTOR = 1.0
GATE_D, GATE_T = 0.86, 0.5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fmha_bf16_dense_wan_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "diffusion_transformer_attention_non_amd", "csrc", "fmha_bf16.hip")


PROFILE_CALLS = ("dense_bf16", "skip_bf16_factor1", "sage_fp8_141", "sage_int8_1161_s32768", "mxfp8_001",
                 "qk16pv8_000")


def eff_flops(B, S, H, D=128, Skv=None):
    return 4.0 * B * H * S * (S if Skv is None else Skv) * D


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads and the factor sweep")
    ap.add_argument("--profile-call", choices=PROFILE_CALLS, default=None,
                    help="run only this attention call (warmup + steps launches) for counter collection")
    return ap.parse_args()


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for_current_kernel():
    """HBM bytes per dense-kernel launch from committed rocprofv3 counter runs, or
    None when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != src_hash(KERNEL_SRC):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed_calls(fn, n, torch):
    """Average HIP-event time (ms) of fn() over n calls on the current stream."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return sum(ev[i].elapsed_time(ev[i + 1]) for i in range(n)) / n


def cpu_baseline(budget_s, S, H, step_flops):
    """The oracle as it stands, on sampled 64-row query tiles (full KV range) and
    one full head of SAGE quantization, extrapolated to one whole step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import diffusion_transformer_attention_non_amd as dit
    from diffusion_transformer_attention_non_amd.synth import generate
    from oracle import exact_attention, sage_attention, sage_quantize, skip_attention

    bm, bn = dit.tile_config()
    nqt = -(-S // bm)
    sc = 1 / math.sqrt(128)
    share = budget_s / 3.0
    # inputs of one head (the oracle works per head and per query tile)
    q5, k5, v5 = (t[:, :, :1].cpu() for t in generate("skip_wan_b1_h40_s75600", H=1, device="cuda"))
    q4, k4, v4 = (t.cpu() for t in generate("sage_fp8_wan_b1_h40_s75600", H=1, device="cuda"))
    rng = np.random.default_rng(0)

    def per_tile(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn(int(rng.integers(nqt)))
            n += 1
            el = time.perf_counter() - t0
            if el >= share or n >= 64:
                return el / n, n

    t_dense, n_dense = per_tile(lambda t: exact_attention(q5, k5, v5, sc, rows=np.arange(t * bm, min(S, t * bm + bm))))
    t_skip, n_skip = per_tile(lambda t: skip_attention(q5, k5, v5, sc, SKIP_FACTOR, bm, bn, qtiles=[t]))
    t0 = time.perf_counter()
    quant = sage_quantize(q4, k4, v4, "fp8", 1, 4)
    t_quant = time.perf_counter() - t0
    kv = dit.kv_tile()
    t_sage, n_sage = per_tile(lambda t: sage_attention(quant, sc, kv, rows=np.arange(t * bm, min(S, t * bm + bm))))
    step_s = (t_dense + t_skip + t_sage) * nqt * H + t_quant * H
    blas = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas")
    return {
        "value": step_flops / step_s / 1e12,
        "unit": "TFLOPS",
        "cores": int(blas or len(os.sched_getaffinity(0))),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on {n_dense} dense, {n_skip} skip and {n_sage} SAGE query tiles of "
                   f"{bm} rows x all {S} keys (head 0) plus SAGE quantization of one full head, extrapolated "
                   f"linearly to {nqt} tiles x {H} heads per call; oracle seconds per step {step_s:.4g}"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas_threads": blas,
    }


def profile_call(args, dit, generate, torch, dev):
    """One attention call kind only, for rocprofv3 counter passes: the same
    inputs and recipes as the bench step (the int8 SAGE one at S=32,768)."""
    name = args.profile_call
    if name in ("dense_bf16", "skip_bf16_factor1"):
        q, k, v = generate("skip_wan_b1_h40_s75600", device=dev)
    elif name == "sage_int8_1161_s32768":
        q, k, v = generate("sage_int8_b1_h40_s32768", device=dev)
    else:
        q, k, v = generate("sage_fp8_wan_b1_h40_s75600", device=dev)
    o = torch.empty_like(q)
    recipes = {"sage_fp8_141": ("fp8", 1, 4, 1), "sage_int8_1161_s32768": ("int8", 1, 16, 1),
               "mxfp8_001": ("mxfp8", 0, 0, 1), "qk16pv8_000": ("bf16", 0, 0, 0)}
    if name == "dense_bf16":
        fn = lambda: dit.attn_dense_bf16(q, k, v, out=o)
    elif name == "skip_bf16_factor1":
        fn = lambda: dit.attn_skip_softmax(q, k, v, SKIP_FACTOR, out=o)
    else:
        rt = recipes[name]
        rec = dit.SageRecipe(rt[0], "fp8", *rt[1:])
        ws = dit.sage_workspace(q, k, v, rec)
        fn = lambda: dit.attn_sage(q, k, v, rec, out=o, workspace=ws)
    for _ in range(args.warmup):
        fn()
    ms = timed_calls(fn, args.steps, torch)
    B, S, H = q.shape[0], q.shape[1], q.shape[2]
    print(json.dumps({"profile_call": name, "launches": args.warmup + args.steps, "ms": ms,
                      "effective_flops_per_call": eff_flops(B, S, H)}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import diffusion_transformer_attention_non_amd as dit
    from diffusion_transformer_attention_non_amd.synth import generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.profile_call:
        profile_call(args, dit, generate, torch, dev)
        return
    B, S, H, D = WAN["B"], WAN["S"], WAN["H"], WAN["D"]
    print(f"[bench] generating Wan-shaped inputs B={B} S={S} H={H} D={D}", file=sys.stderr, flush=True)
    q5, k5, v5 = generate("skip_wan_b1_h40_s75600", device=dev)
    q4, k4, v4 = generate("sage_fp8_wan_b1_h40_s75600", device=dev)
    rec = dit.SageRecipe("fp8", "fp8", 1, 4, 1)
    ws = dit.sage_workspace(q4, k4, v4, rec)
    o_dense = torch.empty_like(q5)
    o_sage = torch.empty_like(q4)
    o_skip = torch.empty_like(q5)
    gate = dit.SkipGate(GATE_D)
    torch.cuda.synchronize()

    skipped = [None]

    def call_dense():
        dit.attn_dense_bf16(q5, k5, v5, out=o_dense)

    def call_sage():
        dit.attn_sage(q4, k4, v4, rec, out=o_sage, workspace=ws)

    def call_skip():
        if gate.enabled(GATE_T):
            _, ex = dit.attn_skip_softmax(q5, k5, v5, SKIP_FACTOR, out=o_skip, return_count=True)
            skipped[0] = ex["skipped"]
        else:
            call_dense()

    calls = [("dense_bf16", call_dense), ("sage_fp8_141", call_sage), ("skip_bf16_factor1", call_skip)]
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        for i, (_, fn) in enumerate(calls):
            fn()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    per_call = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
                for i, (name, _) in enumerate(calls)}

    F = eff_flops(B, S, H, D)
    vote_m, vote_n = dit.tile_config()
    nqb, nkt = -(-S // vote_m), -(-S // vote_n)
    skip_frac = float(skipped[0][0]) / (B * H * nqb * nkt) if skipped[0] is not None else 0.0
    step_flops = F * len(calls)
    modes = {
        "dense_bf16": {"ms": per_call["dense_bf16"], "tflops": F / per_call["dense_bf16"] / 1e9,
                       "frac_of_peak": F / per_call["dense_bf16"] / 1e9 / PEAK_TFLOPS["bf16"], "peak": PEAK_TFLOPS["bf16"]},
        "sage_fp8_141": {"ms": per_call["sage_fp8_141"], "tflops": F / per_call["sage_fp8_141"] / 1e9,
                         "frac_of_peak": F / per_call["sage_fp8_141"] / 1e9 / PEAK_TFLOPS["fp8"],
                         "peak": PEAK_TFLOPS["fp8"], "includes": "quantization + attention"},
        "skip_bf16_factor1": {"ms": per_call["skip_bf16_factor1"], "tflops": F / per_call["skip_bf16_factor1"] / 1e9,
                              "frac_of_peak": F / per_call["skip_bf16_factor1"] / 1e9 / PEAK_TFLOPS["bf16"],
                              "peak": PEAK_TFLOPS["bf16"], "skip_fraction": skip_frac,
                              "algorithmic_tflops": (2 + 2 * (1 - skip_frac)) * B * H * S * S * D / per_call["skip_bf16_factor1"] / 1e9},
    }

    # Dominant kernel: the dense BF16 attention kernel (one launch per call).
    t_dense = timed_calls(call_dense, 3, torch)
    achieved = F / t_dense / 1e9
    traffic = traffic_for_current_kernel()
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": achieved / PEAK_TFLOPS["bf16"], "traffic": traffic,
                "kernel": "fmha_bf16_kernel", "avg_launch_ms": t_dense,
                "algorithmic_flops_per_launch": F, "algorithmic_hbm_bytes_per_launch": 4 * B * S * H * D * 2}

    # HBM calibration copy of a known size (also read by the counter runs).
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(buf)
    t_copy = timed_calls(lambda: dst.copy_(buf), 3, torch)
    copy_gbps = 2 * buf.numel() / t_copy / 1e6
    del buf, dst

    extra = {}
    if not args.no_extra:
        print("[bench] other workloads and the factor sweep", file=sys.stderr, flush=True)
        sweep = {}
        bitmap_total = B * H * nqb * nkt
        for f in (0.0, 1.0, 10.0, 100.0):
            cnt = {}

            def run_f(f=f, cnt=cnt):
                _, ex = dit.attn_skip_softmax(q5, k5, v5, f, out=o_skip, return_count=True)
                cnt["n"] = ex["skipped"]
            ms = timed_calls(run_f, 2, torch)
            frac = float(cnt["n"][0]) / bitmap_total
            sweep[str(f)] = {"ms": ms, "effective_tflops": F / ms / 1e9, "skip_fraction": frac,
                             "algorithmic_tflops": (2 + 2 * (1 - frac)) * B * H * S * S * D / ms / 1e9}
        extra["skip_factor_sweep_wan"] = sweep
        # SAGE FP8 (1,4,1) with Skip-Softmax on the same spatially peaked inputs
        # (quantization included); votes are 32 rows x one 64-key KV tile.
        sweep = {}
        sv_m, sv_n = dit.sage_skip_tile()
        sage_votes = B * H * -(-S // sv_m) * -(-S // sv_n)
        for f in (0.0, 1.0, 10.0, 100.0):
            cnt = {}

            def run_sf(f=f, cnt=cnt):
                _, ex = dit.attn_sage_skip_softmax(q5, k5, v5, rec, f, out=o_sage, workspace=ws, return_count=True)
                cnt["n"] = ex["skipped"]
            ms = timed_calls(run_sf, 2, torch)
            frac = float(cnt["n"][0]) / sage_votes
            sweep[str(f)] = {"ms": ms, "effective_tflops": F / ms / 1e9, "skip_fraction": frac,
                             "algorithmic_tflops": (2 + 2 * (1 - frac)) * B * H * S * S * D / ms / 1e9}
        extra["sage_fp8_skip_factor_sweep_wan"] = sweep
        # The other FP8-BMM2 recipes at the same shape, on the SAGE workload's
        # inputs (quantization included): QK16PV8 and MXFP8 Q/K.
        for name, r in (("qk16pv8_bf16_000", dit.SageRecipe("bf16", "fp8", 0, 0, 0)),
                        ("mxfp8_001", dit.SageRecipe("mxfp8", "fp8", 0, 0, 1))):
            wsr = dit.sage_workspace(q4, k4, v4, r)
            ms = timed_calls(lambda: dit.attn_sage(q4, k4, v4, r, out=o_sage, workspace=wsr), 3, torch)
            peak = PEAK_TFLOPS["fp8"] if r.qk_dtype == "mxfp8" else 1.0 / (0.5 / PEAK_TFLOPS["bf16"] + 0.5 / PEAK_TFLOPS["fp8"])
            extra[name + "_wan"] = {"ms": ms, "tflops": F / ms / 1e9, "frac_of_peak": F / ms / 1e9 / peak, "peak": peak,
                                    "includes": "quantization + attention"}
            del wsr
        # SAGE quantization alone (HBM-bound): algorithmic bytes = 2 B read + 1 B
        # written per element of Q, K and V, plus the statistics pass re-reading K and V.
        # Timed as a captured HIP graph, so the binding's host work between calls
        # (which exceeds these few kernels' device time) stays out of the figure.
        dit.sage_quantize(q4, k4, v4, rec, workspace=ws)
        torch.cuda.synchronize()
        gq = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gq):
            dit.sage_quantize(q4, k4, v4, rec, workspace=ws)
        ms_q = timed_calls(gq.replay, 5, torch)
        del gq
        qbytes = B * S * H * D * (3 + 5 + 5)
        extra["sage_quantize_fp8_141_wan"] = {"ms": ms_q, "algorithmic_bytes": qbytes, "gbps": qbytes / ms_q / 1e6,
                                              "frac_of_hbm_peak": qbytes / ms_q / 1e6 / HBM_GBPS}
        del q4, k4, v4, ws, o_sage
        q2, k2, v2 = generate("dense_gqa_b2_h24kv8_s8192", device=dev)
        ms = timed_calls(lambda: dit.attn_dense_bf16(q2, k2, v2), 5, torch)
        F2 = eff_flops(2, 8192, 24)
        extra["dense_gqa_b2_h24kv8_s8192"] = {"ms": ms, "tflops": F2 / ms / 1e9,
                                              "frac_of_peak": F2 / ms / 1e9 / PEAK_TFLOPS["bf16"]}
        del q2, k2, v2
        q3, k3, v3 = generate("sage_int8_b1_h40_s32768", device=dev)
        rec3 = dit.SageRecipe("int8", "fp8", 1, 16, 1)
        ws3 = dit.sage_workspace(q3, k3, v3, rec3)
        ms = timed_calls(lambda: dit.attn_sage(q3, k3, v3, rec3, workspace=ws3), 3, torch)
        ms_q = timed_calls(lambda: dit.sage_quantize(q3, k3, v3, rec3, workspace=ws3), 3, torch)
        F3 = eff_flops(1, 32768, 40)
        # respective peak for int8 BMM1 + fp8 BMM2: time = (F/2)/P_int8 + (F/2)/P_fp8
        extra["sage_int8_b1_h40_s32768"] = {"ms": ms, "quantize_ms": ms_q, "tflops": F3 / ms / 1e9,
                                            "frac_of_peak": F3 / ms / 1e9 / PEAK_TFLOPS["int8"]}
        del q3, k3, v3, ws3

    result = {
        "metric": "effective attention TFLOPS + % MFMA peak at S=75,600 H=40 D=128",
        "value": step_flops / (ms_step / 1e3) / 1e12,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp8",
        "data": "synthetic",
        "config": {"workload": "wan_b1_h40_s75600_d128: dense bf16 + sage fp8 (1,4,1) + skip-softmax bf16 factor 1",
                   "B": B, "S": S, "H": H, "D": D, "skip_factor": SKIP_FACTOR, "gate": {"D": GATE_D, "t": GATE_T}},
        "modes": modes,
        "roofline": roofline,
        "hbm_copy_gbps": copy_gbps,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, S, H, step_flops)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
