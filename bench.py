"""Throughput of the sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1] [--y-dtype bf16]

One step = one moe_layer_forward over the whole workload (router, selection, dispatch
indices, row gather, grouped gate/up + SwiGLU GEMM, grouped down GEMM, weighted
combine), inputs resident in HBM. Prints ONE JSON line. `value` and `ms_per_step` come from
K back-to-back moe_layer_forward calls between two events. The per-stage durations come
from a second timed pass of K moe_layer_forward_traced calls (the same kernels, plus HIP
events that the library records on its own stream at each stage boundary), so the dominant
kernel's time is measured live on its launch stream; those events cost about 4 us each, which
is why the headline pass runs without them. After the timed steps: the same steps with the
last-level cache flushed before each ("cold"), and measured ceilings on this GPU
("achievable": the vendor GEMM library on the dense-equivalent gate/up GEMM, and this
repository's microbenchmarks of the matrix cores, the LDS and an HBM stream copy). The
cpu_baseline leg times the CPU oracle on a bounded token sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + grouped-GEMM MFMA util %, Mixtral-shaped layer bf16"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3        # MI355X float32 vector: 256 CUs x 128 FMA lanes x 2 flop x 2.4 GHz

# The pages' own figures, reported beside the measurements as context (they are whole-model
# figures on hardware the pages do not state, so no vs_baseline is derived from them):
# hrletsgo page "MoE vs MoT routing inference cost", basic-structure and measured-figures
# sections (Mixtral 8x7B sizes and FP16 serving memory); gist.science summary of
# "Capacity-Aware Inference", Results section (speed-ups of the two drop variants).
PAGES_CONTEXT = {
    "mixtral_8x7b_params_total_billion": 46.7,
    "mixtral_8x7b_params_active_billion": 12.9,
    "mixtral_8x7b_fp16_serving_gb": 90,
    "capacity_aware_token_drop_speedup": 1.3,
    "capacity_aware_expanded_drop_speedup_max": 1.85,
    "note": "whole-model figures from the pages, hardware not stated: context, not targets",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=0, help="override T (decode-shaped runs)")
    ap.add_argument("--y-dtype", default="", choices=["", "bf16", "f32"])
    ap.add_argument("--gamma", type=float, default=None, help="override the capacity factor")
    ap.add_argument("--expand-m", type=int, default=0, help="Expanded Drop: extra candidates")
    ap.add_argument("--cap-groups", type=int, default=0, help="capacity per group of E/D experts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="tokens in the oracle sample (default: about 15 s of oracle work)")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="after timing, run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch.matmul (the vendor GEMM library) on the same expert "
                         "GEMM shapes, as a reference point for the grouped GEMM")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache steps (last-level cache flushed before each)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured ceilings (library GEMM, device copy)")
    return ap.parse_args()


def algorithmic(cfg, n_kept):
    """Algorithmic work per layer: flops of the two grouped GEMMs (kept rows only, no
    padding) and bytes each memory-bound stage must move."""
    d, f, fs, T, E, k = cfg.d_model, cfg.d_ff, cfg.d_ff_shared, cfg.T, cfg.E, cfg.k
    elt = 2 if cfg.dtype == "bf16" else 4
    yel = 2 if (cfg.y_dtype or cfg.dtype) == "bf16" else 4
    gate_up = 4.0 * d * f * n_kept + 4.0 * d * fs * T
    down = 2.0 * d * f * n_kept + 2.0 * d * fs * T
    route = T * d * elt + d * E * 4 + T * E * 4 + T * k * 8
    dispatch = 0.0                                     # folded into the gate/up GEMM
    combine = n_kept * d * 4 + n_kept * 8 + T * d * yel + (T * d * 4 if fs else 0)
    return dict(gate_up=gate_up, down=down, route=route, dispatch=dispatch, combine=combine)


def gemm_hbm_bytes(cfg, counts):
    """Bytes each grouped GEMM must move at least: the weights of every expert with rows
    (and the shared expert), the rows it reads and the rows it writes, each once."""
    import numpy as np
    d, f, fs, T = cfg.d_model, cfg.d_ff, cfg.d_ff_shared, cfg.T
    elt = 2 if cfg.dtype == "bf16" else 4
    used = int(np.count_nonzero(counts))
    rows = int(np.sum(counts))
    gate_up = (used * 2 * f * d + 2 * fs * d) * elt + (rows + (T if fs else 0)) * d * elt \
        + (rows * f + T * fs) * elt
    down = (used * f * d + fs * d) * elt + (rows * f + T * fs) * elt + (rows + (T if fs else 0)) * d * 4
    return dict(gate_up=float(gate_up), down=float(down))


def cpu_baseline(inp, sample_tokens=0, target_s=20.0):
    """Time the CPU oracle (float64 numpy) on the first N tokens of the workload; routing is
    always computed over all T tokens, as the method requires. Unless N is given, a 256-token
    run is timed first; if it took less than half of target_s, N is scaled up from it, and
    once more from a fixed-plus-per-token fit if that run still took under 10 s (the oracle
    widens every expert's weights once per call). The last sample is the one reported."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    T = inp.cfg.T

    def timed(n):
        t0 = time.perf_counter()
        oracle.layer_forward(inp, tokens=np.arange(n))
        return time.perf_counter() - t0

    if sample_tokens:
        dt = timed(sample_tokens)
    else:
        n1 = min(T, 256)
        t1 = timed(n1)
        sample_tokens, dt = n1, t1
        if t1 < target_s / 2 and n1 < T:
            sample_tokens = int(min(T, n1 * target_s / t1))
            dt = timed(sample_tokens)
            if dt < 10.0 and sample_tokens < T and dt > t1:
                # the oracle has a fixed cost (widening the weights); fit a + b N and aim again
                b = (dt - t1) / (sample_tokens - n1)
                sample_tokens = int(min(T, sample_tokens + (target_s - dt) / b))
                dt = timed(sample_tokens)
    reps = 1
    if sample_tokens == T and dt < 10.0:
        # the whole workload is quicker than the bound: repeat it until ~10 s of work is timed
        reps, dt = 0, 0.0
        while dt < 10.0 and reps < 100000:
            dt += timed(T)
            reps += 1
    what = (f"all {T} tokens, {reps} runs" if reps > 1 else
            f"first {sample_tokens} of {T} tokens (routing over all {T})")
    return {"value": round(reps * sample_tokens / dt, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{what}, float64 numpy oracle, {dt:.1f} s on {threads} BLAS threads"}


def recorded_traffic(workload):
    """HBM bytes per launch of the gate/up GEMM kernel from the committed counter summary,
    if it was measured on the current kernel source (else None)."""
    import hashlib
    import re
    src = os.path.join(ROOT, "mixture_experts_layer_42_amd", "csrc", "gemm.hip")
    summ = os.path.join(ROOT, "profiles", "hbm_traffic_gemm.md")
    if not (os.path.exists(src) and os.path.exists(summ)):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    m = re.search(r"```json\n(.*?)\n```", open(summ).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("gemm_hip_sha256") != sha:
        return None
    ent = rec.get("gate_up", {}).get(workload)
    return None if ent is None else float(ent["hbm_bytes_per_launch"])


def library_gemm(cfg, counts, dev, reps=10):
    """Reference throughput of the vendor GEMM library (torch.matmul) on the routed expert
    GEMMs: one call per expert with that expert's row count (contiguous rows, no gather, no
    SwiGLU), and the same kept rows through a single expert's weights as one dense call
    (the weights then stay in cache across row tiles). Flops count kept rows only."""
    import torch
    d, f = cfg.d_model, cfg.d_ff
    rows = [int(c) for c in counts]
    n = sum(rows)
    torch.manual_seed(0)
    xs = torch.randn(max(n, 1), d, device="cuda", dtype=torch.bfloat16)
    hs = torch.randn(max(n, 1), f, device="cuda", dtype=torch.bfloat16)
    wgu = [torch.cat([dev["w_gate"][e], dev["w_up"][e]], 0) if r else None
           for e, r in enumerate(rows)]
    wdn = dev["w_down"]

    def timed(fn):
        for _ in range(2):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps * 1e-3

    def per_expert(kind):
        def run():
            o = 0
            for e, r in enumerate(rows):
                if r:
                    if kind == "gate_up":
                        torch.matmul(xs[o:o + r], wgu[e].t())
                    else:
                        torch.matmul(hs[o:o + r], wdn[e].t())
                    o += r
        return run

    e0 = next(e for e, r in enumerate(rows) if r)
    out = {}
    for kind, fl in (("gate_up", 4.0 * d * f * n), ("down", 2.0 * d * f * n)):
        t_pe = timed(per_expert(kind))
        if kind == "gate_up":
            t_dn = timed(lambda: torch.matmul(xs[:n], wgu[e0].t()))
        else:
            t_dn = timed(lambda: torch.matmul(hs[:n], wdn[e0].t()))
        out[kind] = {"per_expert_tflops": round(fl / t_pe / 1e12, 1),
                     "per_expert_frac": round(fl / t_pe / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "dense_tflops": round(fl / t_dn / 1e12, 1),
                     "dense_frac": round(fl / t_dn / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


def achievable(cfg, n_kept, dev):
    """Measured ceilings on this GPU for the two rooflines: the vendor GEMM library
    (torch.matmul) on the dense-equivalent of the gate/up GEMM (the kept rows through one
    expert's gate and up weights, so the weights are reused by every row tile), and a plain
    device copy of 1 GiB (read + write bytes / time)."""
    import torch
    out = {}

    def timed(fn, reps):
        for _ in range(2):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps * 1e-3

    if cfg.dtype == "bf16" and n_kept >= 256:
        torch.manual_seed(0)
        a = torch.randn(n_kept, cfg.d_model, device="cuda", dtype=torch.bfloat16)
        w = torch.cat([dev["w_gate"][0], dev["w_up"][0]], 0)
        t = timed(lambda: torch.matmul(a, w.t()), 10)
        tf = 4.0 * cfg.d_model * cfg.d_ff * n_kept / t / 1e12
        out["gemm_tflops"] = round(tf, 1)
        out["gemm_frac_of_peak"] = round(tf / PEAK_BF16_TFLOPS, 4)
        out["gemm_how"] = "torch.matmul bf16, kept rows x one expert's gate+up weights (dense)"
        del a, w
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 10)
    gbs = 2.0 * src.numel() / t / 1e9
    out["hbm_copy_gbs"] = round(gbs, 1)
    out["hbm_copy_frac_of_peak"] = round(gbs / PEAK_HBM_GBS, 4)
    del src, dst
    # this repository's microbenchmarks (libmoe_peak.so): matrix-core loop with its clock,
    # LDS read loop, hand-written stream copy
    from mixture_experts_layer_42_amd import peak
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    mf = peak.mfma(ncu)
    out["mfma_loop_tflops"] = mf["tflops"]
    out["mfma_loop_frac_of_peak"] = round(mf["tflops"] / PEAK_BF16_TFLOPS, 4)
    out["mfma_loop_clock_ghz"] = mf["clock_ghz"]
    out["mfma_loop_how"] = mf["how"]
    ld = peak.lds(ncu)
    out["lds_read_tb_s"] = ld["tb_s"]
    out["lds_read_per_cu_gb_s"] = ld["per_cu_gb_s"]
    cp = peak.copy(ncu)
    out["stream_copy_gbs"] = cp["gb_s"]
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs the layer on one GPU only; "
                                   "--gpus must be 1 (multi-GPU expert sharding is not built)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import mixture_experts_layer_42_amd as moe
    import moe_inputs as mi

    cfg = mi.CONFIGS[args.config]
    if args.tokens:
        cfg = cfg.with_(T=args.tokens)
    if args.y_dtype:
        cfg = cfg.with_(y_dtype=args.y_dtype)
    if args.gamma is not None:
        cfg = cfg.with_(gamma=args.gamma)
    if args.expand_m or args.cap_groups:
        cfg = cfg.with_(expand_m=args.expand_m, cap_groups=args.cap_groups)
    print(f"[bench] generating {cfg.name} T={cfg.T}", file=sys.stderr, flush=True)
    inp = mi.make_inputs(cfg, threads=16)
    dev = {n: moe.device_tensor(getattr(inp, n)) for n in
           ("x", "w_router", "bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    prob = moe.problem_of(cfg)
    nbytes = moe.moe_workspace_bytes(prob)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ydt = torch.bfloat16 if (cfg.y_dtype or cfg.dtype) == "bf16" else torch.float32
    y = torch.empty(cfg.T, cfg.d_model, dtype=ydt, device="cuda")
    rb = moe.RoutingBuffers(prob)
    stream = torch.cuda.current_stream()
    nev = moe.MOE_STAGE_COUNT + 1

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
        for e in evs:
            e.record(stream)           # creates the underlying HIP event
        return evs

    def step(evs):
        moe.moe_layer_forward_traced(prob, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"],
                                     dev["w_up"], dev["w_down"], dev["ws_gate"], dev["ws_up"],
                                     dev["ws_down"], y, rb.struct, ws, nbytes, stream, evs)

    def step_plain():
        moe.moe_layer_forward(prob, dev["x"], dev["w_router"], dev["bias"], dev["w_gate"],
                              dev["w_up"], dev["w_down"], dev["ws_gate"], dev["ws_up"],
                              dev["ws_down"], y, rb.struct, ws, nbytes, stream)

    warm = new_events()
    for _ in range(args.warmup):
        step_plain()
    step(warm)
    step_events = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step_plain()
    t_end.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    total_ms = t_start.elapsed_time(t_end)
    # second pass: the same steps with the stage events, for the per-kernel durations
    for i in range(args.steps):
        step(step_events[i])
    torch.cuda.synchronize()
    traced_ms = float(np.mean([step_events[i][0].elapsed_time(step_events[i][moe.MOE_STAGE_COUNT])
                               for i in range(args.steps)]))
    stage_ms = np.array([[step_events[i][s].elapsed_time(step_events[i][s + 1])
                          for s in range(moe.MOE_STAGE_COUNT)] for i in range(args.steps)])
    stage_avg = stage_ms.mean(axis=0)
    n_kept = int(rb.offsets[-1].item())
    work = algorithmic(cfg, n_kept)
    gemm_bytes = gemm_hbm_bytes(cfg, rb.counts.cpu().numpy())
    ms_per_step = total_ms / args.steps
    value = cfg.T / (ms_per_step * 1e-3)

    cold = None
    if not args.no_cold:
        # the same steps with the 256 MB last-level cache flushed (a 512 MB write) before
        # each; per-step time between the layer's first and last stage events
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold_ms = []
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            step(step_events[i])
        torch.cuda.synchronize()
        cold_ms = [step_events[i][0].elapsed_time(step_events[i][moe.MOE_STAGE_COUNT])
                   for i in range(args.steps)]
        cold = float(np.median(cold_ms))
        del flush

    if args.pmc_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    gu_ms, dn_ms = stage_avg[moe.STAGE_NAMES.index("gate_up")], stage_avg[moe.STAGE_NAMES.index("down")]
    gu_tf = work["gate_up"] / (gu_ms * 1e-3) / 1e12
    gemm_tf = (work["gate_up"] + work["down"]) / ((gu_ms + dn_ms) * 1e-3) / 1e12
    # the dominant kernel and its roofline: the gate/up GEMM on the matrix cores (bf16), its
    # weight stream when every expert holds at most 64 rows (the skinny path, HBM-bound), or
    # the float32 SIMT GEMM (vector ALU) for float32 problems
    skinny = cfg.dtype == "bf16" and cfg.T <= 64
    if cfg.dtype != "bf16":
        roofline = {"kernel": "grouped gate/up GEMM + SwiGLU, float32 SIMT (gemm_f32_kernel<true>)",
                    "bound": "alu", "achieved": round(gu_tf, 3), "peak": PEAK_F32_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(gu_tf / PEAK_F32_TFLOPS, 6), "traffic": None}
    elif skinny:
        gbs = gemm_bytes["gate_up"] / (gu_ms * 1e-3) / 1e9
        roofline = {"kernel": "grouped gate/up GEMM + SwiGLU, skinny path (gemm_skinny_kernel<true, *>)",
                    "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roofline = {"kernel": "grouped gate/up GEMM + SwiGLU (gemm_bf16_kernel<true, 8>)",
                    "bound": "mfma", "achieved": round(gu_tf, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(gu_tf / PEAK_BF16_TFLOPS, 4),
                    "traffic": None if (args.tokens or args.gamma is not None or args.expand_m
                                        or args.cap_groups) else recorded_traffic(cfg.name)}
        if roofline["traffic"] is not None:
            roofline["traffic_note"] = ("bytes between the L2 caches and the fabric (FETCH_SIZE x2 + "
                                        "WRITE_SIZE per launch); they include hits in the "
                                        "last-level cache, so they bound HBM traffic from above")
    stages = {}
    for i, name in enumerate(moe.STAGE_NAMES):
        ent = {"us": round(float(stage_avg[i]) * 1e3, 2)}
        if name == "dispatch":
            ent["note"] = "row gather folded into the gate/up GEMM operand loads"
        elif name in ("gate_up", "down"):
            tf = work[name] / (stage_avg[i] * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), mfma_frac=round(tf / PEAK_BF16_TFLOPS, 4))
            # the HBM view (the bound when few rows reach each expert): weights of the
            # experts that received rows, plus the activations read and written once
            gbs = gemm_bytes[name] / (stage_avg[i] * 1e-3) / 1e9
            ent.update(gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        else:
            gbs = work[name] / (stage_avg[i] * 1e-3) / 1e9
            ent.update(gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
        stages[name] = ent
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random inputs and random-init weights of the stated shape)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d_model={cfg.d_model} E={cfg.E} k={cfg.k} "
                               f"d_ff={cfg.d_ff} d_ff_shared={cfg.d_ff_shared} routing={cfg.routing} "
                               f"gamma={cfg.gamma}"
                               + (f" expand_m={cfg.expand_m}" if cfg.expand_m else "")
                               + (f" cap_groups={cfg.cap_groups}" if cfg.cap_groups else "")
                               + f" {cfg.dtype} weights/activations, fp32 router, "
                               f"y {cfg.y_dtype or cfg.dtype}",
                   "tokens": cfg.T, "rows_kept": n_kept, "parallelism": "single GPU"},
        "roofline": roofline,
        "grouped_gemm_mfma_util": round(gemm_tf / PEAK_BF16_TFLOPS, 4),
        "traced_ms_per_step": round(traced_ms, 4),
        "cold": None if cold is None else {
            "ms_per_step": round(cold, 4), "tokens_per_s": round(cfg.T / (cold * 1e-3), 1),
            "how": "median over the steps, 512 MB write before each (flushes the last-level cache)"},
        "stages": stages,
        "host_s": round(host_s, 4),
    }
    if not args.no_achievable:
        print("[bench] measured ceilings", file=sys.stderr, flush=True)
        ach = achievable(cfg, n_kept, dev)
        out["achievable"] = ach
        if "gemm_tflops" in ach and out["roofline"]["bound"] == "mfma":
            out["roofline"]["frac_of_achievable"] = round(gu_tf / ach["gemm_tflops"], 4)
            out["roofline"]["frac_of_mfma_loop"] = round(gu_tf / ach["mfma_loop_tflops"], 4)
    if args.library_gemm and cfg.dtype == "bf16":
        print("[bench] library GEMM reference", file=sys.stderr, flush=True)
        out["library_gemm"] = library_gemm(cfg, rb.counts.cpu().numpy(), dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: oracle on a token sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample)
    out["pages_context"] = PAGES_CONTEXT
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
