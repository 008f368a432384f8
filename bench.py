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
    ap.add_argument("--issue-probe", action="store_true",
                    help="print the VALU issue-rate and MFMA/VALU co-execution probes as one JSON line and exit")
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
    return timed_stats(fn, n, torch)["mean_ms"]


def timed_stats(fn, n, torch):
    """HIP-event times (ms) of n back-to-back calls of fn() on the current
    stream: mean, median and minimum."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ts = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
    return {"mean_ms": sum(ts) / n, "median_ms": med, "min_ms": ts[0], "launches": n}


EXTRA_LAUNCHES = 10


def mfma_peak_probe(torch):
    """Matrix-core peak of each dtype on this GPU: back-to-back MFMAs on every
    SIMD (two wavefronts each), timed with HIP events, with the shader clock the
    waves ran at (their cycle counter against the constant-rate wall clock)."""
    import ctypes
    import statistics
    path = os.path.join(ROOT, "diffusion_transformer_attention_non_amd", "libditattn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.mfma_probe_flops_per_mfma.restype = ctypes.c_double
    lib.mfma_probe_flops_per_mfma.argtypes = [ctypes.c_int]
    lib.mfma_probe_wall_rate_khz.restype = ctypes.c_int
    lib.mfma_probe_launch.restype = ctypes.c_int
    lib.mfma_probe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus                     # 4 wavefronts per workgroup: two per SIMD
    waves = 4 * wgs
    clocks = torch.zeros(4 * waves, dtype=torch.int64, device="cuda")
    sink = torch.zeros(waves * 64, dtype=torch.float32, device="cuda")
    wall_khz = lib.mfma_probe_wall_rate_khz()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {}
    for kind, name, iters, peak in ((0, "bf16", 200000, PEAK_TFLOPS["bf16"]), (1, "fp8", 100000, PEAK_TFLOPS["fp8"]),
                                    (2, "int8", 200000, PEAK_TFLOPS["int8"])):
        launch = lambda: lib.mfma_probe_launch(kind, wgs, iters, clocks.data_ptr(), sink.data_ptr(), stream)
        if launch() != 0:
            return None
        st = timed_stats(launch, 3, torch)
        c = clocks.view(waves, 4).cpu().numpy().astype("float64")
        ghz = statistics.median(((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * wall_khz / 1e6).tolist()) if wall_khz else None
        flops = waves * iters * 4 * lib.mfma_probe_flops_per_mfma(kind)
        tf = flops / st["min_ms"] / 1e9
        out[name] = {"tflops": tf, "shader_ghz": ghz, "published_peak": peak, "frac_of_published": tf / peak,
                     "tflops_at_2p4ghz": (tf * 2.4 / ghz) if ghz else None, "ms": st["min_ms"],
                     "mfma": {0: "v_mfma_f32_32x32x16_bf16", 1: "v_mfma_f32_32x32x64_f8f6f4",
                              2: "v_mfma_i32_32x32x32_i8"}[kind]}
    return out


ISSUE_VALU_KINDS = ("v_add_f32", "v_fma_f32", "v_max3_f32", "v_exp_f32", "v_cvt_pk_fp8_f32", "v_pk_fma_f16")
ISSUE_COEXEC_MODES = (
    ("mfma_only", "per wavefront one E4M3 32x32x64 MFMA (four independent accumulators)"),
    ("split", "half the wavefronts one MFMA, the other half 16 v_fma_f32 (2 wavefronts per SIMD)"),
    ("fma16_after_each_mfma", "one MFMA, then 16 independent v_fma_f32 of the same wavefront"),
    ("softmax_mix_after_each_mfma", "one MFMA, then four logits: fma -> exp2, sum, 2 max3, 2 E4M3 packs"),
    ("softmax_mix_burst", "the same work as four MFMAs followed by four logit groups"),
)


def issue_probe(torch):
    """Instruction-issue probes (csrc/issue_probe.hip), one workgroup per CU
    with 1-3 wavefronts per SIMD, each wavefront timing its loop with the
    shader cycle counter; reports the slowest wavefront's span per unit."""
    import ctypes
    path = os.path.join(ROOT, "diffusion_transformer_attention_non_amd", "libditattn_probe.so")
    lib = ctypes.CDLL(path)
    lib.issue_probe_launch.restype = ctypes.c_int
    lib.issue_probe_launch.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def span(probe, kind, wps, iters):
        waves = cus * 4 * wps
        cycles = torch.zeros(waves, dtype=torch.int64, device="cuda")
        sink = torch.zeros(waves * 64, dtype=torch.float32, device="cuda")
        for it in (8, iters):   # a short warm-up launch, then the timed one
            rc = lib.issue_probe_launch(probe, kind, wps, cus, it, cycles.data_ptr(), sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"issue_probe_launch({probe}, {kind}, {wps}) returned {rc}")
        torch.cuda.synchronize()
        return float(cycles.max().item())

    valu = {}
    for kind, name in enumerate(ISSUE_VALU_KINDS):
        iters = 4000
        valu[name] = {f"{w}_waves_per_simd": span(0, kind, w, iters) / (iters * lib.issue_probe_per_iter(0) * w)
                      for w in (1, 2, 3)}
    coexec = {}
    for mode, (name, what) in enumerate(ISSUE_COEXEC_MODES):
        iters = 2000
        rows, per_mfma = {}, {}
        for w in ((2,) if name == "split" else (1, 2, 3)):
            rows[f"{w}_waves_per_simd"] = span(1, mode, w, iters) / (iters * lib.issue_probe_per_iter(1))
            if name != "split":   # every wavefront issues one MFMA per step
                per_mfma[f"{w}_waves_per_simd"] = rows[f"{w}_waves_per_simd"] / w
        coexec[name] = {"step": what, "simd_cycles_per_step": rows}
        if per_mfma:
            coexec[name]["simd_cycles_per_mfma"] = per_mfma
    return {"probe": "instruction issue (csrc/issue_probe.hip)", "cus": cus,
            "valu_simd_cycles_per_wavefront_instruction": valu,
            "mfma_valu_coexecution": coexec,
            "note": "a step is per wavefront; with w wavefronts per SIMD the SIMD runs w steps in the span, "
                    "so an E4M3 MFMA alone costs 64 * w cycles per step at the full rate"}


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


def cpu_baseline_configs(gpu_ms):
    """The oracle timed per workload beside its GPU figure, on this host's
    cores (one BLAS thread per worker, workers over heads): the small dense
    case and the GQA case in full; the SAGE and Skip-Softmax cases on sampled
    64-row query tiles (first and last included) of 4 heads over the full key
    range, extrapolated linearly to every tile of every head, plus the SAGE
    quantizer on the full tensors."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    import diffusion_transformer_attention_non_amd as dit
    from diffusion_transformer_attention_non_amd.synth import WORKLOADS, generate
    from oracle import exact_attention, sage_attention, sage_quantize, skip_attention

    sc = 1 / math.sqrt(128)
    workers = min(16, len(os.sched_getaffinity(0)))
    heads_sample = [0, 13, 26, 39]
    out = {}

    def pmap(fn, items):
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, items))

    def tiles(S, n):
        nqt = -(-S // 64)
        inner = np.linspace(1, nqt - 2, n - 2).round().astype(int)
        return nqt, np.unique(np.concatenate([[0, nqt - 1], inner]))

    def report(name, seconds, extrapolated, sample, flops):
        e = {"oracle_s": seconds, "oracle_s_full_call": extrapolated, "sample": sample,
             "oracle_gflops": flops / extrapolated / 1e9, "threads": workers}
        if gpu_ms.get(name):
            e["gpu_ms"] = gpu_ms[name]
            e["gpu_speedup_over_oracle"] = extrapolated * 1e3 / gpu_ms[name]
        out[name] = e

    for name in ("dense_b1_h2_s256", "dense_gqa_b2_h24kv8_s8192"):
        w = WORKLOADS[name]
        q, k, v = (t.cpu() for t in generate(name, device="cuda"))
        G = w.Hq // w.Hkv
        jobs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
        t0 = time.perf_counter()
        pmap(lambda bh: exact_attention(q[bh[0]:bh[0] + 1, :, bh[1]:bh[1] + 1],
                                        k[bh[0]:bh[0] + 1, :, bh[1] // G:bh[1] // G + 1],
                                        v[bh[0]:bh[0] + 1, :, bh[1] // G:bh[1] // G + 1], sc), jobs)
        el = time.perf_counter() - t0
        report(name, el, el, "every row of every head", eff_flops(w.B, w.S, w.Hq))

    for name, n_tiles in (("sage_int8_b1_h40_s32768", 16), ("sage_fp8_wan_b1_h40_s75600", 8)):
        w = WORKLOADS[name]
        dt, _, (qb, kb, vb) = w.recipe
        q, k, v = (t.cpu() for t in generate(name, device="cuda"))
        t0 = time.perf_counter()
        quants = pmap(lambda h: sage_quantize(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], dt, qb, kb, vb),
                      range(w.Hq))
        t_quant = time.perf_counter() - t0
        nqt, sel = tiles(w.S, n_tiles)
        rows = np.concatenate([np.arange(t * 64, min(w.S, t * 64 + 64)) for t in sel])
        t0 = time.perf_counter()
        pmap(lambda h: sage_attention(quants[h], sc, dit.kv_tile(), rows=rows), heads_sample)
        t_att = time.perf_counter() - t0
        scale = (nqt * w.Hq) / (len(sel) * len(heads_sample))
        report(name, t_quant + t_att, t_quant + t_att * scale,
               f"quantizer on all {w.Hq} heads ({t_quant:.3g} s); attention on {len(sel)} query tiles x "
               f"{len(heads_sample)} heads ({t_att:.3g} s), x{scale:.4g} for the whole call",
               eff_flops(w.B, w.S, w.Hq))
        del quants

    name = "skip_wan_b1_h40_s75600"
    w = WORKLOADS[name]
    q, k, v = (t.cpu() for t in generate(name, device="cuda"))
    bm, bn = dit.tile_config()
    nqt = -(-w.S // bm)
    _, sel = tiles(w.S, 8)
    t0 = time.perf_counter()
    pmap(lambda h: skip_attention(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], sc, SKIP_FACTOR, bm, bn,
                                  qtiles=sel), heads_sample)
    el = time.perf_counter() - t0
    scale = (nqt * w.Hq) / (len(sel) * len(heads_sample))
    report(name + "_factor1", el, el * scale,
           f"{len(sel)} query tiles x {len(heads_sample)} heads ({el:.3g} s), x{scale:.4g} for the whole call",
           eff_flops(w.B, w.S, w.Hq))
    return out


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
    if args.issue_probe:
        print(json.dumps(issue_probe(torch)), flush=True)
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
    # The low-precision path at the same shape: one attn_sage call (the
    # quantization launches, 2 % of it, included) against the FP8 peak.
    t_sage = timed_calls(call_sage, 3, torch)
    roofline_sage = {"bound": "mfma", "achieved": F / t_sage / 1e9, "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                     "frac": F / t_sage / 1e9 / PEAK_TFLOPS["fp8"], "traffic": None,
                     "kernel": "fmha_sage_kernel<E4M3, k_block 4> + SAGE quantization", "avg_call_ms": t_sage,
                     "algorithmic_flops_per_call": F}

    # HBM calibration copy of a known size (also read by the counter runs).
    buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(buf)
    t_copy = timed_calls(lambda: dst.copy_(buf), 3, torch)
    copy_gbps = 2 * buf.numel() / t_copy / 1e6
    del buf, dst

    print("[bench] matrix-core peak probe", file=sys.stderr, flush=True)
    probe = mfma_peak_probe(torch)

    def entry(fn, flops, peak, **kw):
        st = timed_stats(fn, EXTRA_LAUNCHES, torch)
        e = {"ms": st["median_ms"], "min_ms": st["min_ms"], "mean_ms": st["mean_ms"], "launches": st["launches"]}
        if flops is not None:
            e.update(tflops=flops / st["median_ms"] / 1e9, frac_of_peak=flops / st["median_ms"] / 1e9 / peak,
                     peak=peak)
        e.update(kw)
        return e

    extra = {}
    c1_ms = None
    if not args.no_extra:
        print("[bench] other workloads and the factor sweep", file=sys.stderr, flush=True)
        sweep = {}
        bitmap_total = B * H * nqb * nkt
        for f in (0.0, 1.0, 10.0, 100.0):
            cnt = {}

            def run_f(f=f, cnt=cnt):
                _, ex = dit.attn_skip_softmax(q5, k5, v5, f, out=o_skip, return_count=True)
                cnt["n"] = ex["skipped"]
            e = entry(run_f, None, None)
            frac = float(cnt["n"][0]) / bitmap_total
            e.update(effective_tflops=F / e["ms"] / 1e9, skip_fraction=frac,
                     algorithmic_tflops=(2 + 2 * (1 - frac)) * B * H * S * S * D / e["ms"] / 1e9)
            sweep[str(f)] = e
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
            e = entry(run_sf, None, None)
            frac = float(cnt["n"][0]) / sage_votes
            e.update(effective_tflops=F / e["ms"] / 1e9, skip_fraction=frac,
                     algorithmic_tflops=(2 + 2 * (1 - frac)) * B * H * S * S * D / e["ms"] / 1e9)
            sweep[str(f)] = e
        extra["sage_fp8_skip_factor_sweep_wan"] = sweep
        # The other FP8-BMM2 recipes at the same shape, on the SAGE workload's
        # inputs (quantization included): QK16PV8 and MXFP8 Q/K.
        for name, r in (("qk16pv8_bf16_000", dit.SageRecipe("bf16", "fp8", 0, 0, 0)),
                        ("mxfp8_001", dit.SageRecipe("mxfp8", "fp8", 0, 0, 1))):
            wsr = dit.sage_workspace(q4, k4, v4, r)
            peak = PEAK_TFLOPS["fp8"] if r.qk_dtype == "mxfp8" else 1.0 / (0.5 / PEAK_TFLOPS["bf16"] + 0.5 / PEAK_TFLOPS["fp8"])
            extra[name + "_wan"] = entry(lambda: dit.attn_sage(q4, k4, v4, r, out=o_sage, workspace=wsr), F, peak,
                                         includes="quantization + attention")
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
        qbytes = B * S * H * D * (3 + 5 + 5)
        e = entry(gq.replay, None, None)
        e.update(algorithmic_bytes=qbytes, gbps=qbytes / e["ms"] / 1e6, frac_of_hbm_peak=qbytes / e["ms"] / 1e6 / HBM_GBPS)
        extra["sage_quantize_fp8_141_wan"] = e
        del gq
        del q4, k4, v4, ws, o_sage
        q1, k1, v1 = generate("dense_b1_h2_s256", device=dev)
        o1 = torch.empty(q1.shape, dtype=torch.float32, device=dev)
        extra["dense_b1_h2_s256_fp32out"] = entry(lambda: dit.attn_dense_bf16(q1, k1, v1, out=o1), eff_flops(1, 256, 2),
                                                  PEAK_TFLOPS["bf16"])
        c1_ms = extra["dense_b1_h2_s256_fp32out"]["ms"]
        del q1, k1, v1, o1
        q2, k2, v2 = generate("dense_gqa_b2_h24kv8_s8192", device=dev)
        extra["dense_gqa_b2_h24kv8_s8192"] = entry(lambda: dit.attn_dense_bf16(q2, k2, v2), eff_flops(2, 8192, 24),
                                                   PEAK_TFLOPS["bf16"])
        del q2, k2, v2
        q3, k3, v3 = generate("sage_int8_b1_h40_s32768", device=dev)
        rec3 = dit.SageRecipe("int8", "fp8", 1, 16, 1)
        ws3 = dit.sage_workspace(q3, k3, v3, rec3)
        F3 = eff_flops(1, 32768, 40)
        # respective peak for int8 BMM1 + fp8 BMM2: time = (F/2)/P_int8 + (F/2)/P_fp8 (both 5.0 P)
        e = entry(lambda: dit.attn_sage(q3, k3, v3, rec3, workspace=ws3), F3, PEAK_TFLOPS["int8"],
                  includes="quantization + attention")
        e["quantize_ms"] = timed_stats(lambda: dit.sage_quantize(q3, k3, v3, rec3, workspace=ws3), 3, torch)["median_ms"]
        extra["sage_int8_b1_h40_s32768"] = e
        del q3, k3, v3, ws3

    # The step mixes bf16 and fp8 calls: its share of the blended peak is the
    # time the three calls would take at their own peaks over the step time.
    ideal_ms = (F / PEAK_TFLOPS["bf16"] + F / PEAK_TFLOPS["fp8"] + F / PEAK_TFLOPS["bf16"]) / 1e9
    sweep_bf16 = extra.get("skip_factor_sweep_wan", {})
    sweep_sage = extra.get("sage_fp8_skip_factor_sweep_wan", {})
    targets = {
        "dense_bf16_60pct_of_peak": {"measured": modes["dense_bf16"]["frac_of_peak"], "met": modes["dense_bf16"]["frac_of_peak"] >= 0.6},
        "sage_fp8_50pct_of_peak": {"measured": modes["sage_fp8_141"]["frac_of_peak"], "met": modes["sage_fp8_141"]["frac_of_peak"] >= 0.5},
    }
    if sweep_bf16:
        sp = sweep_bf16["0.0"]["ms"] / sweep_bf16["100.0"]["ms"]
        targets["skip_bf16_factor100_faster_than_dense"] = {"measured_speedup": sp, "met": sp > 1.0}
    if sweep_sage:
        sp = sweep_sage["0.0"]["ms"] / sweep_sage["100.0"]["ms"]
        targets["sage_skip_factor100_faster_than_sage"] = {"measured_speedup": sp, "met": sp > 1.0}
    if "sage_int8_b1_h40_s32768" in extra:
        fr = extra["sage_int8_b1_h40_s32768"]["frac_of_peak"]
        targets["sage_int8_50pct_of_peak"] = {"measured": fr, "met": fr >= 0.5}

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
        "frac_of_blended_peak": ideal_ms / ms_step,
        "targets": targets,
        "modes": modes,
        "roofline": roofline,
        "roofline_sage_fp8": roofline_sage,
        "mfma_peak_probe": probe,
        "hbm_copy_gbps": copy_gbps,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, S, H, step_flops)
        if not args.no_extra:
            print("[bench] CPU oracle per workload", file=sys.stderr, flush=True)
            gpu_ms = {"dense_b1_h2_s256": c1_ms, "dense_gqa_b2_h24kv8_s8192": extra["dense_gqa_b2_h24kv8_s8192"]["ms"],
                      "sage_int8_b1_h40_s32768": extra["sage_int8_b1_h40_s32768"]["ms"],
                      "sage_fp8_wan_b1_h40_s75600": per_call["sage_fp8_141"],
                      "skip_wan_b1_h40_s75600_factor1": per_call["skip_bf16_factor1"]}
            result["cpu_baseline_per_workload"] = cpu_baseline_configs(gpu_ms)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
