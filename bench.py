#!/usr/bin/env python3
"""Benchmark: achieved HBM GB/s of the q4f16_1 decode-step weight sweep on one GPU.

Workload (one "step"): the full Phi-3-mini-shaped decode step at M = 1 --
32 layers x {qkv 3072->9216, o 3072->3072, gate_up 3072->16384, down 8192->3072}
plus lm_head 3072->32064, 129 GEMVs over 2,093,838,336 bytes of q4f16_1 words and
scales (Zero TVM documentation, "The memory-bandwidth ceiling": ~2.09 GB per
token), seeded synthetic codes and scales, x reused by every layer.  One step is
one q4_decode_step call over the 129 descriptors, inputs resident in HBM.

Prints ONE JSON line (rank 0):
  value = algorithmic bytes per step / time per step, in GB/s;
  roofline = the dominant kernel's algorithmic bytes per launch / its average
             launch duration (HIP events on the stream it runs on) vs 8 TB/s;
  cpu_baseline = the CPU oracle on this host over one full step (on every usable core up
                 to the 16-thread share, plus a single-thread figure beside it).

Profiling aids (see profiles/):
  --copy-probe BYTES        run only a plain device copy of BYTES (counter calibration)
  --summarize-profiles DIR  turn the rocprofv3 CSV output under DIR (stats/, fetch/,
                            write/, copy_fetch/, copy_write/, commands.txt) into the
                            summaries profiles/k_step_phi3_decode_sweep.{md,json}
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, published
# the dominant kernel and the sources it is built from: traffic figures measured
# with hardware counters are reported only while these are unchanged
KERNEL = "k_step"
KERNEL_SOURCES = ["bit_weight_streaming_q4f16_amd/csrc/q4_step.hip",
                  "bit_weight_streaming_q4f16_amd/csrc/q4_step.h",
                  "bit_weight_streaming_q4f16_amd/csrc/q4_device.h",
                  "bit_weight_streaming_q4f16_amd/csrc/q4_internal.h"]
PROFILE = os.path.join(ROOT, "profiles", "k_step_phi3_decode_sweep")
# the kernels with committed counter summaries: the headline step, and the small-M
# step on the 2B-class sweep at M = 8
PROFILED = {
    "k_step": dict(profile=PROFILE, sources=KERNEL_SOURCES, model="phi3", M=1,
                   title="Phi-3-mini decode-step weight sweep, M=1 (129 GEMVs, one launch)"),
    "k_step_mfma": dict(
        profile=os.path.join(ROOT, "profiles", "k_step_mfma_2b_decode_sweep_m8"),
        sources=["bit_weight_streaming_q4f16_amd/csrc/q4_step_mfma.hip",
                 "bit_weight_streaming_q4f16_amd/csrc/q4_step_mfma.h",
                 "bit_weight_streaming_q4f16_amd/csrc/q4_device.h",
                 "bit_weight_streaming_q4f16_amd/csrc/q4_internal.h"],
        model="2b", M=8,
        title="2B-class decode-step weight sweep, M=8 (113 GEMVs, one launch)"),
}
METRIC = "achieved HBM GB/s (% of peak) and projected decode tok/s, q4 GEMV sweep"


# ordered: every GEMV waits for its predecessor, kept in the persistent kernel
# (0x10) where the driver would otherwise launch one kernel per GEMV
MODES = {"ordered": 0x2 | 0x10, "hazards": 0x0, "launch_each": 0x1, "persistent": 0x10}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--mode", choices=["ordered", "hazards", "launch_each"], default="hazards",
                    help="ordered: every GEMV waits for its predecessor (a decode step's "
                         "dependency chain); hazards: waits only on shared memory; "
                         "launch_each: one kernel per GEMV")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config figures (single GEMV, one MLP, the M=8 sweep)")
    ap.add_argument("--only-step", action="store_true",
                    help="time only the decode step (for profiler runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="run only a plain device copy of BYTES, 3 times (counter calibration)")
    ap.add_argument("--only-m8", action="store_true",
                    help="time only the 2B-class sweep at M=8 (for profiler runs)")
    ap.add_argument("--only-mlp", action="store_true",
                    help="time only one Phi-3 MLP as two q4_gemv calls (for counter runs)")
    ap.add_argument("--only-affine", action="store_true",
                    help="time only the affine-format Phi-3 sweeps")
    ap.add_argument("--only-q3", action="store_true",
                    help="time only the q3f16_1 and mixed-format Phi-3 sweeps")
    ap.add_argument("--only-tokens", action="store_true",
                    help="time only the Phi-3-shaped decode-token loop (for profiler runs)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 CSV output under DIR")
    ap.add_argument("--kernel", choices=sorted(PROFILED), default="k_step",
                    help="the kernel --summarize-profiles summarizes")
    return ap.parse_args()


def build_sweep(torch, q4, synth, np, model="phi3", M=1):
    shapes = synth.sweep_shapes(model)
    xs = {}
    for K in sorted({K for _, _, K in shapes}):
        h = synth.activations(f"{model}/x{K}", 0, M * K)
        xs[K] = torch.from_numpy(h.view(np.int16)).cuda().view(torch.float16)
    descs, meta = [], []
    for label, N, K in shapes:
        m = synth.Matrix(label, N, K)
        W = m.words_torch("cuda")
        S = torch.from_numpy(m.scales().view(np.int16)).cuda().view(torch.float16)
        Y = torch.empty(N * M, dtype=torch.float16, device="cuda")
        descs.append((W, S, xs[K], Y))
        meta.append((label, N, K))
    return descs, meta


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.kernel)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import bit_weight_streaming_q4f16_amd as q4

    torch.cuda.set_device(0)
    q4.load()
    stream = torch.cuda.Stream()          # default priority
    if args.copy_probe:
        copy_probe(torch, q4, stream, args.copy_probe)
        return
    if args.only_mlp:
        print(json.dumps({"mlp_gate_up_down_m1": mlp_only(torch, q4, synth, np, stream)}),
              flush=True)
        return
    if args.only_q3:
        print(json.dumps({"phi3_sweep_q3f16_1": q3_sweep(torch, q4, synth, np, stream)}),
              flush=True)
        return
    if args.only_affine:
        print(json.dumps({"phi3_sweep_af4g64": affine_sweep(torch, q4, synth, np, stream)}),
              flush=True)
        return
    if args.only_tokens:
        descs, meta = build_sweep(torch, q4, synth, np)
        print(json.dumps({"decode_tokens": token_figures(torch, q4, synth, np, stream, descs,
                                                         meta)}), flush=True)
        return
    if args.only_m8:
        print(json.dumps({"twob_sweep_m8": m8_sweep(torch, q4, synth, np, stream, args.steps,
                                                    args.warmup)}), flush=True)
        return
    t0 = time.time()
    descs, meta = build_sweep(torch, q4, synth, np)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    layers = q4.make_layers(descs)
    step_bytes = sum(synth.algorithmic_bytes(1, N, K) for _, N, K in meta)
    weight_bytes = sum(synth.Matrix(l, N, K).weight_bytes for l, N, K in meta)

    # the same GEMVs with each x a prefix of the previous GEMV's y: a decode
    # step's dependency chain with the operations between the GEMVs left out
    chain_layers = q4.make_layers(
        [descs[0]] + [(W, S, descs[i - 1][3][:x.numel()], y)
                      for i, (W, S, x, y) in enumerate(descs) if i > 0])

    def time_mode(mode, steps, warmup, lay=None):
        """One planned list run `steps` times after `warmup` runs, each step between
        its own pair of HIP events on the stream the kernel runs on; the median,
        p10, p90 and the mean over the whole bracket, and the host's time per
        q4_step_run call."""
        flags = MODES[mode]
        plan = q4.StepPlan(layers if lay is None else lay, 1, flags, stream=stream)
        sp = q4.C.c_void_p(stream.cuda_stream)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                plan.run_raw(sp)
            plan.status(stream)                       # waits; the error word must be 0
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            host = 0.0
            w0.record(stream)
            for a, b in ev:
                a.record(stream)
                h0 = time.perf_counter()
                rc = plan.run_raw(sp)
                host += time.perf_counter() - h0
                b.record(stream)
                if rc:
                    raise SystemExit(f"q4_step_run failed: {rc}")
            w1.record(stream)
            torch.cuda.synchronize()
            plan.status(stream)
        per = np.sort(np.array([a.elapsed_time(b) for a, b in ev]))
        return {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
                "p90": float(np.percentile(per, 90)), "mean": w0.elapsed_time(w1) / steps,
                "host_us": host / steps * 1e6}

    t = time_mode(args.mode, args.steps, args.warmup)
    ms = t["median"]
    gbs = step_bytes / (ms * 1e-3) / 1e9
    if gbs > PEAK_GBS * 1.02:
        raise SystemExit(f"measured {gbs:.0f} GB/s is above the HBM peak: measurement error")
    probe = None if args.no_probe else probe_read(torch, q4, stream)

    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "q4f16/f32acc",
        "data": "synthetic (seeded SplitMix64 codes/scales, N(0,1) x)",
        "config": {"workload": "phi3-mini decode-step weight sweep, M=1: 32 x {qkv 3072->9216, "
                               "o 3072->3072, gate_up 3072->16384, down 8192->3072} + lm_head "
                               "3072->32064, q4f16_1 group 32",
                   "gemvs_per_step": len(meta), "algorithmic_bytes_per_step": step_bytes,
                   "weight_bytes_per_step": weight_bytes, "mode": args.mode},
        "timing": {"statistic": "median of per-step HIP event pairs",
                   "ms_p10": round(t["p10"], 5), "ms_p90": round(t["p90"], 5),
                   "ms_mean_over_bracket": round(t["mean"], 5),
                   "host_enqueue_us_per_step": round(t["host_us"], 2)},
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "projected_tok_s": round(1e3 / ms, 1),
        "setup_s": round(setup_s, 1),
    }
    if probe is not None:
        result["probe_read_gbs"] = probe
        result["pct_of_probe_ceiling"] = round(100 * gbs / probe["best_gbs"], 2)
    # dominant kernel: the persistent step kernel, one launch per step (nothing
    # else is launched); its algorithmic bytes per launch are the step's, its
    # duration the event time per step
    result["us_per_gemv"] = round(ms * 1e3 / len(meta), 3)
    result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS,
                          "unit": "GB/s", "frac": round(gbs / PEAK_GBS, 4),
                          "traffic": measured_traffic() if args.mode == "hazards" else None,
                          "kernel": KERNEL if args.mode != "launch_each" else "k_gemv_m1 (all)",
                          "algorithmic_bytes_per_launch": step_bytes}
    if not args.only_step:
        other = {}
        for mode in MODES:
            if mode in (args.mode, "persistent"):
                continue
            m = time_mode(mode, max(5, args.steps // 5), max(3, args.warmup // 4))
            other[mode] = {"ms_per_step": round(m["median"], 5),
                           "gbs": round(step_bytes / (m["median"] * 1e-3) / 1e9, 1)}
        for mode in ("persistent", "launch_each", "hazards"):
            m = time_mode(mode, max(5, args.steps // 5), max(3, args.warmup // 4), chain_layers)
            key = "chain_default_choice" if mode == "hazards" else f"chain_{mode}"
            other[key] = {"ms_per_step": round(m["median"], 5),
                          "gbs": round(step_bytes / (m["median"] * 1e-3) / 1e9, 1)}
        # the one-call entry point (plans and writes the tables every call)
        m = one_call_timing(torch, q4, stream, layers, max(5, args.steps // 10))
        other["one_call_q4_decode_step"] = {"ms_per_step": round(m, 5),
                                            "gbs": round(step_bytes / (m * 1e-3) / 1e9, 1)}
        result["other_modes"] = other
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline(np, torch, descs, meta)
        if not args.no_configs:
            result["per_config"] = per_config(torch, q4, synth, np, stream,
                                              cpu=not args.no_cpu_baseline)
            result["decode_tokens"] = token_figures(torch, q4, synth, np, stream, descs, meta)
    print(json.dumps(result), flush=True)


def _timed(torch, stream, fn, calls, warm=3):
    with torch.cuda.stream(stream):
        for _ in range(warm):
            fn(0)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(calls):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def _fig(nbytes, ms, **kw):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(us=round(ms * 1e3, 2), gbs=round(gbs, 1), pct_of_peak=round(100 * gbs / PEAK_GBS, 2),
                **kw)


def per_config(torch, q4, synth, np, stream, cpu=False):
    """The other workloads: a single qkv GEMV and one MLP (gate_up then down), each
    over distinct weight copies totalling > 512 MB so every call streams from HBM,
    timed as back-to-back calls and as one decode-step list; and the 2B-class
    sweep at M = 8."""
    import synth as S
    out = {}

    def mats(prefix, shapes, copies, M=1):
        xs = {}
        descs = []
        for c in range(copies):
            for role, N, K in shapes:
                if K not in xs:
                    h = S.activations(f"{prefix}/x{K}", 0, M * K)
                    xs[K] = torch.from_numpy(h.view(np.int16)).cuda().view(torch.float16)
                m = S.Matrix(f"{prefix}/c{c}/{role}", N, K)
                sc = torch.from_numpy(m.scales().view(np.int16)).cuda().view(torch.float16)
                y = torch.empty(M * N, dtype=torch.float16, device="cuda")
                descs.append((m.words_torch("cuda"), sc, xs[K], y, N, K))
        return descs

    def gemv_calls(descs):
        ws = {}
        for (W, Sc, x, y, N, K) in descs:
            nb = q4.q4_workspace_bytes(1, N, K)
            if nb and nb > ws.get("n", 0):
                ws["n"] = nb
        wsb = torch.empty(max(ws.get("n", 0), 16), dtype=torch.uint8, device="cuda")

        def fn(i):
            W, Sc, x, y, N, K = descs[i % len(descs)]
            q4.q4_gemv(W, Sc, x, y, ws=wsb, stream=stream)
        return fn

    def step_call(descs, M=1):
        plan = q4.StepPlan(q4.make_layers([d[:4] for d in descs]), M, 0, stream=stream)

        def fn(i):
            plan.run(stream)
        return fn

    # single qkv GEMV 3072 -> 9216
    qkv = [("qkv", 9216, 3072)]
    d = mats("bench/qkv", qkv, 34)
    b1 = synth.algorithmic_bytes(1, 9216, 3072)
    ms_launch = _timed(torch, stream, gemv_calls(d), 4 * len(d))
    ms_step = _timed(torch, stream, step_call(d), 5) / len(d)
    out["qkv_3072x9216_m1"] = {"q4_gemv": _fig(b1, ms_launch, copies=len(d)),
                               "in_decode_step": _fig(b1, ms_step, copies=len(d))}
    del d
    # one MLP: gate_up 3072 -> 16384, then down 8192 -> 3072
    mlp = [("gate_up", 16384, 3072), ("down", 3072, 8192)]
    d = mats("bench/mlp", mlp, 13)
    b2 = synth.algorithmic_bytes(1, 16384, 3072) + synth.algorithmic_bytes(1, 3072, 8192)
    ms_launch = _timed(torch, stream, gemv_calls(d), 4 * len(d)) * 2
    ms_step = _timed(torch, stream, step_call(d), 5) / (len(d) // 2)
    out["mlp_gate_up_down_m1"] = {"q4_gemv": _fig(b2, ms_launch, copies=len(d) // 2),
                                  "in_decode_step": _fig(b2, ms_step, copies=len(d) // 2)}
    del d
    # the MLP with its glue: gate_up 3072 -> 16384, then down over fp16(silu(gate)
    # * up): fused (the glue formed while down's input is staged, one decode-step
    # list), as three calls per MLP (q4_gemv, q4_silu_mul, q4_gemv), and one
    # kernel per GEMV (glue kernel, then each GEMV)
    copies = 13
    pairs = []
    for c in range(copies):
        mg = S.Matrix(f"bench/mlpg/c{c}/gate_up", 16384, 3072)
        md = S.Matrix(f"bench/mlpg/c{c}/down", 3072, 8192)
        to_t = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
        pairs.append((mg.words_torch("cuda"), to_t(mg.scales()), md.words_torch("cuda"),
                      to_t(md.scales()), torch.empty(16384, dtype=torch.float16, device="cuda"),
                      torch.empty(3072, dtype=torch.float16, device="cuda")))
    xg = torch.from_numpy(S.activations("bench/mlpg/x", 0, 3072).view(np.int16)).cuda().view(
        torch.float16)
    hbuf = torch.empty(8192, dtype=torch.float16, device="cuda")
    b3 = (synth.algorithmic_bytes(1, 16384, 3072) + synth.algorithmic_bytes(1, 3072, 8192) +
          2 * 8192)                                  # down reads gate | up
    glue_layers = q4.make_layers(
        [t for (Wg, Sg, Wd, Sd, gu, y) in pairs
         for t in ((Wg, Sg, xg, gu), (Wd, Sd, gu, y, q4.X_SILU_MUL))])

    def glue_step(flags):
        plan = q4.StepPlan(glue_layers, 1, flags, stream=stream)

        def fn(i):
            plan.run(stream)
        return fn
    wsg = torch.empty(max(q4.q4_workspace_bytes(1, 16384, 3072),
                          q4.q4_workspace_bytes(1, 3072, 8192), 16), dtype=torch.uint8,
                      device="cuda")

    def unfused(i):
        Wg, Sg, Wd, Sd, gu, y = pairs[i % copies]
        q4.q4_gemv(Wg, Sg, xg, gu, ws=wsg, stream=stream)
        q4.q4_silu_mul(gu, hbuf, stream=stream)
        q4.q4_gemv(Wd, Sd, hbuf, y, ws=wsg, stream=stream)
    out["mlp_silu_gate_up_down_m1"] = {
        "fused_decode_step": _fig(b3, _timed(torch, stream, glue_step(q4.STEP_PERSISTENT), 5) /
                                  copies, copies=copies),
        "three_calls": _fig(b3, _timed(torch, stream, unfused, 4 * copies), copies=copies),
        "decode_step_one_kernel_per_gemv": _fig(
            b3, _timed(torch, stream, glue_step(q4.STEP_LAUNCH_EACH), 5) / copies,
            copies=copies)}
    del pairs, glue_layers
    # the format variants: the qkv-shaped GEMV 3072 -> 9216 in each format, over
    # distinct copies (> 512 MB) so every call streams from HBM; bytes counted in
    # each format's own size (words + scales + biases + x + y)
    fmts = {}
    N, K = 9216, 3072
    for name, f in (("q4f16_1", 0), ("q3f16_1", q4.FMT_Q3F16_1), ("q4f32_1", q4.FMT_Q4F32_1),
                    ("af4g64", q4.FMT_AF4_G64)):
        wb = q4.q4_format_weight_bytes(f, N, K)
        copies = max(8, (600 << 20) // wb)
        es = 4 if f == q4.FMT_Q4F32_1 else 2
        nwords = N * K // 32 * (3 if f == q4.FMT_Q3F16_1 else 4)
        per_group = 64 if f == q4.FMT_AF4_G64 else 32
        mk = []
        for c in range(copies):
            lab = f"bench/fmt/{name}/c{c}"
            W = S.words_torch(lab + "/w", 0, nwords).reshape(N, -1)
            sc = (torch.rand(N, K // per_group, device="cuda") * 0.01 + 1e-3).to(
                torch.float32 if es == 4 else torch.float16)
            bi = ((torch.rand(N, K // per_group, device="cuda") - 0.5) * 0.1).half() \
                if f == q4.FMT_AF4_G64 else None
            mk.append((W, sc, bi))
        xdt = torch.float32 if es == 4 else torch.float16
        xf = torch.randn(K, device="cuda").to(xdt)
        yf = torch.empty(N, device="cuda", dtype=xdt)
        wsf = torch.empty(max(q4.q4_workspace_bytes(1, N, K), 16), dtype=torch.uint8,
                          device="cuda")

        def fn(i, mk=mk, f=f, xf=xf, yf=yf, wsf=wsf):
            W, sc, bi = mk[i % len(mk)]
            if f == 0:
                q4.q4_gemv(W, sc, xf, yf, ws=wsf, stream=stream)
            else:
                q4.q4_gemv_format(f, W, sc, xf, K, biases=bi, y=yf, stream=stream)
        nb = wb + es * (N + K)
        fmts[name] = _fig(nb, _timed(torch, stream, fn, 4 * copies), copies=copies,
                          weight_bytes=wb)
        del mk
    out["formats_qkv_3072x9216_m1"] = fmts
    out["formats_large_m1"] = formats_large(torch, q4, S, stream)
    out["twob_sweep_m8"] = m8_sweep(torch, q4, synth, np, stream, cpu=cpu)
    out["phi3_sweep_q3f16_1"] = q3_sweep(torch, q4, synth, np, stream)
    out["phi3_sweep_af4g64"] = affine_sweep(torch, q4, synth, np, stream)
    return out


def formats_large(torch, q4, S, stream, N=262144, K=3072, calls=20):
    """Each format on one GEMV of 262144 x 3072 (350-500 MB: larger than the 256 MB
    last-level cache, and long enough that the fixed cost of a launch is a few per
    cent): what each format's decode streams at, and its time per weight -- whether
    fewer bytes per weight buy time here.  q4f16_1 also in the persistent
    decode-step kernel, one descriptor."""
    out = {}
    for name, f in (("q4f16_1", 0), ("q3f16_1", q4.FMT_Q3F16_1), ("q4f32_1", q4.FMT_Q4F32_1),
                    ("af4g64", q4.FMT_AF4_G64)):
        wb = q4.q4_format_weight_bytes(f, N, K)
        es = 4 if f == q4.FMT_Q4F32_1 else 2
        nwords = N * K // 32 * (3 if f == q4.FMT_Q3F16_1 else 4)
        per_group = 64 if f == q4.FMT_AF4_G64 else 32
        W = S.words_torch(f"bench/fmtL/{name}/w", 0, nwords).reshape(N, -1)
        sc = (torch.rand(N, K // per_group, device="cuda") * 0.01 + 1e-3).to(
            torch.float32 if es == 4 else torch.float16)
        bi = ((torch.rand(N, K // per_group, device="cuda") - 0.5) * 0.1).half() \
            if f == q4.FMT_AF4_G64 else None
        xdt = torch.float32 if es == 4 else torch.float16
        xf = torch.randn(K, device="cuda").to(xdt)
        yf = torch.empty(N, device="cuda", dtype=xdt)
        wsf = torch.empty(max(q4.q4_workspace_bytes(1, N, K), 16), dtype=torch.uint8,
                          device="cuda")

        def fn(i, W=W, sc=sc, bi=bi, f=f, xf=xf, yf=yf, wsf=wsf):
            if f == 0:
                q4.q4_gemv(W, sc, xf, yf, ws=wsf, stream=stream)
            else:
                q4.q4_gemv_format(f, W, sc, xf, K, biases=bi, y=yf, stream=stream)
        nb = wb + es * (N + K)
        ms = _timed(torch, stream, fn, calls, warm=5)
        out[name] = _fig(nb, ms, weight_bytes=wb, ns_per_kweight=round(ms * 1e6 / (N * K / 1e3), 4))
        if f == 0:
            # the persistent kernel on this one GEMV (the driver alone would run a
            # one-descriptor list as one GEMV kernel)
            plan = q4.StepPlan(q4.make_layers([(W, sc, xf, yf)]), 1, q4.STEP_PERSISTENT,
                               stream=stream)

            def fs(i):
                plan.run(stream)
            ms = _timed(torch, stream, fs, calls, warm=5)
            out["q4f16_1_decode_step"] = _fig(nb, ms, weight_bytes=wb,
                                              ns_per_kweight=round(ms * 1e6 / (N * K / 1e3), 4))
        del W, sc, bi
        torch.cuda.empty_cache()
    return out


def m8_sweep(torch, q4, synth, np, stream, steps=300, warmup=50, cpu=False):
    """The 2B-class sweep at M = 8 (113 GEMVs, eight rows of X each) as one
    q4_decode_step call per step; with the small-M kernel's HBM traffic from its
    committed counter summary while that kernel is unchanged.  cpu: also the CPU
    oracle over the whole sweep on every usable core (capped at 16), which checks
    every output of the last step (the GEMV tolerance per row of X)."""
    S = synth
    shapes = synth.sweep_shapes("2b")
    descs = []
    xs = {}
    for label, N, K in shapes:
        if K not in xs:
            h = S.activations(f"2b/X{K}", 0, 8 * K)
            xs[K] = torch.from_numpy(h.view(np.int16)).cuda().view(torch.float16)
        m = S.Matrix(label, N, K)
        sc = torch.from_numpy(m.scales().view(np.int16)).cuda().view(torch.float16)
        descs.append((m.words_torch("cuda"), sc, xs[K], torch.empty(8 * N, dtype=torch.float16,
                                                                       device="cuda"), N, K))
    b5 = sum(synth.algorithmic_bytes(8, N, K) for _, N, K in shapes)
    plan = q4.StepPlan(q4.make_layers([d[:4] for d in descs]), 8, 0, stream=stream)
    sp = q4.C.c_void_p(stream.cuda_stream)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            plan.run_raw(sp)
        plan.status(stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            plan.run_raw(sp)
            b.record(stream)
        torch.cuda.synchronize()
        plan.status(stream)
    per = np.array([a.elapsed_time(b) for a, b in ev])
    ms = float(np.median(per))
    flops = sum(2 * 8 * N * K for _, N, K in shapes)
    tr = measured_traffic("k_step_mfma")
    fig = _fig(b5, ms, gemvs=len(shapes), steps_per_s=round(1e3 / ms, 1),
               tok_per_s=round(8e3 / ms, 1), tflops=round(flops / (ms * 1e-3) / 1e12, 2),
               us_p10=round(float(np.percentile(per, 10)) * 1e3, 2),
               us_p90=round(float(np.percentile(per, 90)) * 1e3, 2), statistic="median",
               kernel="k_step_mfma", traffic=tr,
               traffic_over_algorithmic=None if tr is None else round(tr / b5, 4))
    if cpu:
        fig["cpu_oracle"] = cpu_sweep_m8(np, torch, descs, b5)
    del descs
    torch.cuda.empty_cache()
    return fig


def cpu_sweep_m8(np, torch, descs, nbytes, max_threads=16):
    """The fp64 oracle over the M = 8 sweep with its OpenMP row loops, once, and the
    parity of all its outputs against the GPU's last step."""
    import oracle
    model, nproc, usable = host_cpu()
    threads = max(1, min(usable, max_threads))
    old = oracle.get_threads()
    worst, checked, tn = 0.0, 0, 0.0
    try:
        oracle.set_threads(threads)
        for W, Sc, X, Y, N, K in descs:
            w = W.cpu().numpy().view(np.uint32)
            s = Sc.view(torch.int16).cpu().numpy().view(np.uint16)
            x = X.view(torch.int16).cpu().numpy().view(np.uint16).reshape(8, K)
            y = Y.view(torch.int16).cpu().numpy().view(np.float16).astype(np.float64).reshape(8, N)
            t0 = time.perf_counter()
            ref = oracle.gemv_f64(w, s, x)
            tn += time.perf_counter() - t0
            rn = oracle.row_norms(w, s).max()
            for m in range(8):
                tol = 2e-3 * oracle.vec_norm(x[m]) * rn
                worst = max(worst, float(np.abs(y[m] - ref[m]).max() / tol))
            checked += 8 * N
    finally:
        oracle.set_threads(old)
    return {"value": round(nbytes / tn / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_step": round(tn, 3), "host_cpu": model,
            "sample": "the whole M = 8 sweep (113 GEMVs x 8 rows of X), fp64 plain C oracle "
                      f"with OpenMP row loops on {threads} threads, once",
            "parity_all_outputs": {"outputs": checked, "max_error_over_tolerance": round(worst, 4),
                                   "ok": worst <= 1.0}}


def mlp_only(torch, q4, synth, np, stream, rounds=4):
    """One Phi-3-mini MLP at M = 1 (gate_up 3072 -> 16384, then down 8192 -> 3072)
    as two q4_gemv calls, over 13 weight copies (> 512 MB, so every call streams
    from HBM), `rounds` passes back to back: the workload of the per-GEMV counter
    profile.  Returns the mean time per MLP."""
    S = synth
    shapes = [("gate_up", 16384, 3072), ("down", 3072, 8192)]
    xs, descs = {}, []
    for c in range(13):
        for role, N, K in shapes:
            if K not in xs:
                h = S.activations(f"bench/mlp/x{K}", 0, K)
                xs[K] = torch.from_numpy(h.view(np.int16)).cuda().view(torch.float16)
            m = S.Matrix(f"bench/mlp/c{c}/{role}", N, K)
            sc = torch.from_numpy(m.scales().view(np.int16)).cuda().view(torch.float16)
            descs.append((m.words_torch("cuda"), sc, xs[K],
                          torch.empty(N, dtype=torch.float16, device="cuda"), N, K))
    nb = max(q4.q4_workspace_bytes(1, N, K) for _, N, K in shapes)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    b2 = sum(S.algorithmic_bytes(1, N, K) for _, N, K in shapes)

    def fn(i):
        W, Sc, x, y, N, K = descs[i % len(descs)]
        q4.q4_gemv(W, Sc, x, y, ws=ws, stream=stream)
    ms = _timed(torch, stream, fn, rounds * len(descs)) * 2
    return _fig(b2, ms, copies=len(descs) // 2, calls=rounds * len(descs))


def q3_sweep(torch, q4, synth, np, stream, steps=300, warmup=100):
    """The Phi-3-shaped sweep with q3f16_1 weights (14 bytes per 32 weights) in the
    persistent decode-step kernel, and the same list with q3f16_1 and q4f16_1
    layers alternating: one event pair per step on the kernel's stream, median."""
    S = synth
    shapes = S.sweep_shapes("phi3")
    xs = {}
    out = {}
    for name, pick in (("q3f16_1", lambda i: True), ("mixed", lambda i: i % 2 == 0)):
        descs, nbytes = [], 0
        for i, (label, N, K) in enumerate(shapes):
            if K not in xs:
                h = S.activations(f"phi3/x{K}", 0, K)
                xs[K] = torch.from_numpy(h.view(np.int16)).cuda().view(torch.float16)
            q3 = pick(i)
            y = torch.empty(N, dtype=torch.float16, device="cuda")
            if q3:
                words = S.words_torch(label + "/q3words", 0, N * K // 32 * 3).view(N, -1)
                sc = S.scales_halfnormal(label + "/scales", 0, 0, N * K // 32, 0.01, 1e-3)
                sc = torch.from_numpy(sc.view(np.int16)).cuda().view(torch.float16)
                descs.append((words, sc, xs[K], y, 0, q4.FMT_Q3F16_1))
                nbytes += N * K // 32 * 14 + 2 * K + 2 * N
            else:
                m = S.Matrix(label, N, K)
                sc = torch.from_numpy(m.scales().view(np.int16)).cuda().view(torch.float16)
                descs.append((m.words_torch("cuda"), sc, xs[K], y, 0, 0))
                nbytes += S.algorithmic_bytes(1, N, K)
        plan = q4.StepPlan(q4.make_layers(descs), 1, 0, stream=stream)
        sp = q4.C.c_void_p(stream.cuda_stream)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                plan.run_raw(sp)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record(stream)
                plan.run_raw(sp)
                b.record(stream)
            torch.cuda.synchronize()
            plan.status(stream)
        per = np.array([a.elapsed_time(b) for a, b in ev])
        ms = float(np.median(per))
        out[name] = _fig(nbytes, ms, gemvs=len(shapes),
                         q3_layers=sum(1 for i in range(len(shapes)) if pick(i)),
                         tok_per_s=round(1e3 / ms, 1),
                         us_p10=round(float(np.percentile(per, 10)) * 1e3, 2),
                         us_p90=round(float(np.percentile(per, 90)) * 1e3, 2),
                         statistic="median", kernel="k_step")
        del descs, plan
        torch.cuda.empty_cache()
    return out


def affine_sweep(torch, q4, synth, np, stream, steps=300, warmup=100):
    """The Phi-3-shaped sweep with MLX affine weights (Q4_FMT_AF4_G64: bf16 scale and
    bias per 64 weights, 18 bytes per 32 like q4f16_1; centred groups, b = -7.5 s +
    0.1 s N(0, 1)) in the persistent decode-step kernel, and the same list with
    affine and q4f16_1 layers alternating: one event pair per step, median."""
    S = synth
    shapes = S.sweep_shapes("phi3")
    xs = {}
    out = {}
    for name, pick in (("af4g64", lambda i: True), ("mixed", lambda i: i % 2 == 0)):
        descs, nbytes = [], 0
        for i, (label, N, K) in enumerate(shapes):
            if K not in xs:
                h = S.activations(f"phi3/x{K}", 0, K)
                xs[K] = torch.from_numpy(h.view(np.int16)).cuda().view(torch.float16)
            y = torch.empty(N, dtype=torch.float16, device="cuda")
            if pick(i):
                words = S.words_torch(label + "/afwords", 0, N * K // 8).view(N, -1)
                sv = np.abs(0.01 * S.normal(label + "/afs", 0, 0, N * K // 64)) + 1e-3
                bv = -7.5 * sv + 0.1 * sv * S.normal(label + "/afb", 0, 0, N * K // 64)
                dev = lambda v: torch.from_numpy(S.to_bf16_bits(v).view(np.int16)).cuda()
                descs.append((words, dev(sv), xs[K], y, 0, q4.FMT_AF4_G64, dev(bv)))
            else:
                m = S.Matrix(label, N, K)
                sc = torch.from_numpy(m.scales().view(np.int16)).cuda().view(torch.float16)
                descs.append((m.words_torch("cuda"), sc, xs[K], y, 0, 0))
            nbytes += S.algorithmic_bytes(1, N, K)      # 18 bytes per 32 weights either way
        plan = q4.StepPlan(q4.make_layers(descs), 1, 0, stream=stream)
        sp = q4.C.c_void_p(stream.cuda_stream)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                plan.run_raw(sp)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record(stream)
                plan.run_raw(sp)
                b.record(stream)
            torch.cuda.synchronize()
            plan.status(stream)
        per = np.array([a.elapsed_time(b) for a, b in ev])
        ms = float(np.median(per))
        out[name] = _fig(nbytes, ms, gemvs=len(shapes),
                         affine_layers=sum(1 for i in range(len(shapes)) if pick(i)),
                         tok_per_s=round(1e3 / ms, 1),
                         us_p10=round(float(np.percentile(per, 10)) * 1e3, 2),
                         us_p90=round(float(np.percentile(per, 90)) * 1e3, 2),
                         statistic="median", kernel="k_step")
        del descs, plan
        torch.cuda.empty_cache()
    return out


def token_figures(torch, q4, synth, np, stream, descs, meta, steps=32):
    """The whole weights-only decode step of a Phi-3-mini-shaped model (32 blocks,
    the sweep's weights, a seeded q4 embedding table),
    attention at a single position (timing does not depend on the values; norm
    weights near 0.1 keep them finite): one q4_decode_token per token with a host
    synchronisation after each (one token per host call), and q4_decode_tokens
    with `steps` tokens per host call, kernels enqueued per step or one captured
    step replayed as a graph (every residual add + RMSNorm inside the GEMV it feeds,
    bitwise the separate kernels); and the graph replay with the norms in factored
    form (Q4_MODEL_FACTORED_NORM)."""
    D, F, V = 3072, 8192, 32064
    labels = [l for l, _, _ in meta]
    assert len(descs) == 129 and labels[-1].endswith("lm_head"), labels[-1]
    emb = synth.Matrix("tokens/embed", V, D, sigma=0.05, floor=0.0125)
    embed = (emb.words_torch("cuda"),
             torch.from_numpy(emb.scales().view(np.int16)).cuda().view(torch.float16))
    # norm weights near 0.1 keep the residual stream of these (uncalibrated) weights
    # within fp16 over 32 blocks
    gamma = torch.from_numpy((0.1 + 0.01 * synth.normal("tokens/gamma", 0, 0, D)).astype(
        np.float16).view(np.int16)).cuda().view(torch.float16)
    blocks = [dict(qkv=descs[4 * b][:2], o=descs[4 * b + 1][:2], gate_up=descs[4 * b + 2][:2],
                   down=descs[4 * b + 3][:2], attn_norm=gamma, ffn_norm=gamma) for b in range(32)]
    model = q4.Model(embed, blocks, gamma, descs[128][:2], 1e-5)
    ws = torch.empty(q4.q4_decode_token_workspace_bytes(model), dtype=torch.uint8, device="cuda")
    weight_bytes = sum(synth.Matrix(l, N, K).weight_bytes for l, N, K in meta) + D // 2 + D // 16
    tok_in = torch.tensor([1], dtype=torch.int32, device="cuda")
    tok_out = torch.empty(1, dtype=torch.int32, device="cuda")
    tokens = torch.zeros(steps + 1, dtype=torch.int32, device="cuda")
    out = {"model": "phi3-mini-shaped, 32 blocks, vocabulary 32064, attention at one position",
           "weight_bytes_per_token": weight_bytes, "tokens_per_call": steps,
           "norms": "each residual add + RMSNorm inside the GEMV it feeds, bitwise the "
                    "separate kernels (factored: the scalar after the product)"}
    with torch.cuda.stream(stream):
        for _ in range(3):
            q4.q4_decode_token(model, tok_in, tok_out, ws=ws, stream=stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 50
        for _ in range(n):
            q4.q4_decode_token(model, tok_in, tok_out, ws=ws, stream=stream)
            stream.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / n
        out["one_token_per_call"] = {"ms_per_token": round(ms, 4), "tok_s": round(1e3 / ms, 1),
                                     "gbs": round(weight_bytes / (ms * 1e-3) / 1e9, 1)}
        graph = q4.TokensGraph(model, tokens, ws=ws, stream=stream)
        for name, graphed in (("tokens_per_call_eager", False), ("tokens_per_call_graph", True)):
            def call():
                if graphed:
                    graph.run(steps, stream=stream)
                else:
                    q4.q4_decode_tokens(model, tokens, steps, ws=ws, stream=stream)
            call()
            torch.cuda.synchronize()
            reps = 5
            t0 = time.perf_counter()
            for _ in range(reps):
                call()
            stream.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / (reps * steps)
            out[name] = {"ms_per_token": round(ms, 4), "tok_s": round(1e3 / ms, 1),
                         "gbs": round(weight_bytes / (ms * 1e-3) / 1e9, 1)}
        torch.cuda.synchronize()
        graph.close()
    out["tokens"] = tokens[: min(steps + 1, 9)].cpu().tolist()
    # the same loop with the norms in factored form
    folded = q4.Model(embed, blocks, gamma, descs[128][:2], 1e-5,
                      options=q4.MODEL_FACTORED_NORM)
    wsf = torch.empty(q4.q4_decode_token_workspace_bytes(folded), dtype=torch.uint8,
                      device="cuda")
    with torch.cuda.stream(stream):
        graph = q4.TokensGraph(folded, tokens, ws=wsf, stream=stream)
        graph.run(steps, stream=stream)
        torch.cuda.synchronize()
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.run(steps, stream=stream)
        stream.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / (reps * steps)
        graph.close()
    out["tokens_per_call_graph_factored_norms"] = {
        "ms_per_token": round(ms, 4), "tok_s": round(1e3 / ms, 1),
        "gbs": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
        "tokens": tokens[: min(steps + 1, 9)].cpu().tolist()}
    del ws, wsf
    out["whole_token_kernel"] = whole_token_figures(torch, q4, np, stream, folded, tokens,
                                                    weight_bytes, steps)
    del model, folded
    return out


def whole_token_figures(torch, q4, np, stream, model, tokens, weight_bytes, steps, reps=10):
    """The whole-token persistent kernel (q4_tokens_run) on the same model: `steps`
    tokens per launch, one event pair per launch on the kernel's stream (median,
    p10, p90 over `reps` launches after warm-up), and one token per launch with a
    host synchronisation after each.  The error word is checked afterwards."""
    import ctypes
    plan = q4.TokensPlan(model, stream=stream)
    sp = ctypes.c_void_p(stream.cuda_stream)
    tp = ctypes.c_void_p(tokens.data_ptr())
    with torch.cuda.stream(stream):
        for _ in range(3):
            assert plan.run_raw(tp, steps, sp) == 0
        stream.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            assert plan.run_raw(tp, steps, sp) == 0
            b.record(stream)
        stream.synchronize()
        per = np.array([a.elapsed_time(b) / steps for a, b in ev])
        t0 = time.perf_counter()
        n1 = 50
        for _ in range(n1):
            assert plan.run_raw(tp, 1, sp) == 0
            stream.synchronize()
        ms1 = (time.perf_counter() - t0) * 1e3 / n1
    plan.status(stream)
    ms = float(np.median(per))
    out = {"ms_per_token": round(ms, 4), "p10": round(float(np.percentile(per, 10)), 4),
           "p90": round(float(np.percentile(per, 90)), 4), "tok_s": round(1e3 / ms, 1),
           "gbs": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
           "pct_of_8tbs": round(100 * weight_bytes / (ms * 1e-3) / 8e12, 1),
           "tokens_per_launch": steps,
           "one_token_per_launch_ms": round(ms1, 4),
           "tokens": tokens[: min(steps + 1, 9)].cpu().tolist()}
    del plan
    return out


def source_hash(kernel=KERNEL):
    h = hashlib.sha256()
    for f in PROFILED[kernel]["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel=KERNEL):
    """HBM bytes per launch of a profiled kernel from its committed counter
    summary, or None when there is none or the kernel has changed since."""
    try:
        with open(PROFILED[kernel]["profile"] + ".json") as fh:
            prof = json.load(fh)
    except (OSError, ValueError):
        return None
    if prof.get("source_sha256") != source_hash(kernel):
        return None
    return prof.get("traffic_bytes_per_launch")


def copy_probe(torch, q4, stream, nbytes, reps=3):
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            q4.q4_probe_copy(src, dst, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ok = bool(torch.equal(src[:1 << 20], dst[:1 << 20]))
    print(json.dumps({"copy_bytes": nbytes, "launches": reps, "ms_per_launch": round(ms, 4),
                      "gbs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                      "copied": ok}), flush=True)


def _csv_rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _is_kernel(name, kernel):
    return re.search(r"(^|[\s:])" + re.escape(kernel) + r"(\(|<|$|\s)", name or "") is not None


def _counter_per_dispatch(d, kernel, counter):
    """Mean over the kernel's dispatches of the counter summed over its instances."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if not _is_kernel(r.get("Kernel_Name", ""), kernel) or r.get("Counter_Name") != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{counter} of {kernel}: no rows under {d}")
    return sum(per.values()) / len(per), len(per)


def summarize_profiles(d, kernel=KERNEL):
    """Write the kernel's profiles/ summary (.md, .json) from rocprofv3 output."""
    import synth
    P = PROFILED[kernel]
    KERNEL_, PROFILE_ = kernel, P["profile"]
    shapes = synth.sweep_shapes(P["model"])
    step_bytes = sum(synth.algorithmic_bytes(P["M"], N, K) for _, N, K in shapes)
    stats = {}
    for r in _csv_rows(os.path.join(d, "stats"), "kernel_stats.csv"):
        for k in (KERNEL_, "k_zero", "k_put"):
            if _is_kernel(r["Name"], k):
                stats[k] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                            "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                            "percentage": float(r["Percentage"])}
    fetch, nf = _counter_per_dispatch(os.path.join(d, "fetch"), KERNEL_, "FETCH_SIZE")
    write, nw = _counter_per_dispatch(os.path.join(d, "write"), KERNEL_, "WRITE_SIZE")
    cfetch, _ = _counter_per_dispatch(os.path.join(d, "copy_fetch"), "k_probe_copy", "FETCH_SIZE")
    cwrite, _ = _counter_per_dispatch(os.path.join(d, "copy_write"), "k_probe_copy", "WRITE_SIZE")
    copy_bytes = None
    for f in glob.glob(os.path.join(d, "copy_*", "*.out")):
        for line in open(f):
            if line.startswith("{") and "copy_bytes" in line:
                copy_bytes = json.loads(line)["copy_bytes"]
    if copy_bytes is None:
        raise SystemExit("copy probe output (copy_*/*.out) not found")
    ff = copy_bytes / (cfetch * 1024)
    fw = copy_bytes / (cwrite * 1024)
    traffic = fetch * 1024 * ff + write * 1024 * fw
    commands = open(os.path.join(d, "commands.txt")).read().strip()
    avg = stats[KERNEL_]["avg_us"]
    out = {
        "kernel": KERNEL_, "workload": P["title"],
        "source_sha256": source_hash(kernel), "sources": P["sources"],
        "kernel_stats": stats,
        "algorithmic_bytes_per_launch": step_bytes,
        "achieved_gbs_from_avg_duration": round(step_bytes / (avg * 1e-6) / 1e9, 1),
        "FETCH_SIZE_KiB_per_dispatch": fetch, "WRITE_SIZE_KiB_per_dispatch": write,
        "dispatches_counted": {"FETCH_SIZE": nf, "WRITE_SIZE": nw},
        "copy_calibration": {"bytes_read_and_written": copy_bytes, "FETCH_SIZE_KiB": cfetch,
                             "WRITE_SIZE_KiB": cwrite, "fetch_factor": ff, "write_factor": fw},
        "traffic_bytes_per_launch": round(traffic),
        "traffic_over_algorithmic": round(traffic / step_bytes, 4),
        "commands": commands.splitlines(),
    }
    with open(PROFILE_ + ".json", "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    lines = [
        f"# {KERNEL_}: {P['title']}", "",
        "Commands ($REPO: the repository root; run from /tmp with TMPDIR=/tmp):", "",
        *["    " + c for c in commands.splitlines()], "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
        "| kernel | calls | avg us | min us | max us | % of GPU time |",
        "|---|---|---|---|---|---|",
        *[f"| {k} | {v['calls']} | {v['avg_us']:.2f} | {v['min_us']:.2f} | {v['max_us']:.2f} | "
          f"{v['percentage']:.2f} |" for k, v in stats.items()], "",
        f"Algorithmic bytes per launch: {step_bytes:,} -> {out['achieved_gbs_from_avg_duration']}"
        f" GB/s at the average duration ({100 * out['achieved_gbs_from_avg_duration'] / PEAK_GBS:.1f}"
        " % of 8 TB/s).", "",
        "## HBM traffic (rocprofv3 --pmc, one counter per run)", "",
        f"- {KERNEL_}: FETCH_SIZE {fetch:,.0f} KiB, WRITE_SIZE {write:,.0f} KiB per dispatch "
        f"(mean of {nf} / {nw} dispatches)",
        f"- calibration, k_probe_copy of {copy_bytes:,} bytes: FETCH_SIZE {cfetch:,.0f} KiB, "
        f"WRITE_SIZE {cwrite:,.0f} KiB -> factors {ff:.4f} (fetch), {fw:.4f} (write)",
        f"- traffic per launch = FETCH x 1024 x {ff:.4f} + WRITE x 1024 x {fw:.4f} = "
        f"{traffic:,.0f} bytes = {traffic / step_bytes:.4f} x algorithmic", "",
        f"Kernel sources (sha256 {out['source_sha256'][:16]}...): " + ", ".join(P["sources"]),
    ]
    with open(PROFILE_ + ".md", "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def probe_read(torch, q4, stream, nbytes=4 << 30, reps=10):
    """Streaming-read ceiling: best over grid sizes of reading a 4 GiB buffer."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = {}
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    with torch.cuda.stream(stream):
        for mult in (2, 4, 8, 16, 32):
            blocks = cus * mult
            q4.q4_probe_read(buf, sink, blocks, stream=stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                q4.q4_probe_read(buf, sink, blocks, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            best[blocks] = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    b = max(best, key=best.get)
    return {"best_gbs": round(best[b], 1), "blocks": b,
            "sweep": {str(k): round(v, 1) for k, v in best.items()}}


def host_cpu():
    """Host CPU model (lscpu, else /proc/cpuinfo), logical CPUs, and the CPUs this
    process may run on."""
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return model, os.cpu_count(), usable


def cpu_baseline(np, torch, descs, meta, max_threads=16):
    """The CPU oracle on this host over the full step (129 GEMVs, all rows):
    plain C in fp64, once on one thread and three times on every usable core
    (its OpenMP row loops, capped at max_threads, the machine's CPU share); the
    all-cores output is also checked against every GPU output of the last step
    (the GEMV tolerance)."""
    import oracle
    import synth
    model, nproc, usable = host_cpu()
    threads = max(1, min(usable, max_threads))
    host = []
    for (W, S, X, Y), (label, N, K) in zip(descs, meta):
        host.append((W.cpu().numpy().view(np.uint32), S.view(torch.int16).cpu().numpy().view(
            np.uint16), X.view(torch.int16).cpu().numpy().view(np.uint16),
            Y.view(torch.int16).cpu().numpy().view(np.uint16), N, K))
    step_bytes = sum(synth.algorithmic_bytes(1, N, K) for _, N, K in meta)
    old = oracle.get_threads()
    try:
        oracle.set_threads(1)
        t0 = time.perf_counter()
        for w, s, x, _, _, _ in host:
            oracle.gemv_f64(w, s, x)
        t1 = time.perf_counter() - t0
        oracle.set_threads(threads)
        reps, tn, worst, checked = 3, 0.0, 0.0, 0
        for r in range(reps):
            t0 = time.perf_counter()
            ys = [oracle.gemv_f64(w, s, x) for w, s, x, _, _, _ in host]
            tn += time.perf_counter() - t0
        for (w, s, x, y, N, K), ref in zip(host, ys):
            tol = 2e-3 * oracle.vec_norm(x) * oracle.row_norms(w, s).max()
            err = np.abs(y.view(np.float16).astype(np.float64) - ref)
            worst = max(worst, float(err.max() / tol))
            checked += N
    finally:
        oracle.set_threads(old)
    tn /= reps
    return {"value": round(step_bytes / tn / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full step ({len(meta)} GEMVs, all rows, {step_bytes:,} algorithmic "
                      f"bytes), fp64 plain C oracle with OpenMP row loops on {threads} threads, "
                      f"{reps} times",
            "seconds_per_step": round(tn, 3), "host_cpu": model, "nproc": nproc,
            "usable_cpus": usable,
            "single_thread": {"value": round(step_bytes / t1 / 1e9, 4), "unit": "GB/s",
                              "seconds_per_step": round(t1, 2)},
            "parity_all_outputs": {"outputs": checked, "max_error_over_tolerance": round(worst, 4),
                                   "ok": worst <= 1.0}}


def one_call_timing(torch, q4, stream, layers, calls):
    """ms per q4_decode_step call (planning and table writes on every call)."""
    ws = torch.empty(max(q4.q4_decode_step_workspace_bytes(layers, 1, 0), 16), dtype=torch.uint8,
                     device="cuda")
    with torch.cuda.stream(stream):
        q4.q4_decode_step(layers, 1, 0, ws=ws, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(calls):
            q4.q4_decode_step(layers, 1, 0, ws=ws, stream=stream, check=False)
        e1.record(stream)
        torch.cuda.synchronize()
        q4.q4_step_status(ws, stream)
    return e0.elapsed_time(e1) / calls


if __name__ == "__main__":
    main()
