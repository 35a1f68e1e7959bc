#!/usr/bin/env python3
"""Benchmark of the MoE FFN forward on one MI355X.

One step = one full forward of the layer (routing, permutation, grouped
gate||up GEMM with the fused activation, grouped down GEMM, combine) over one
batch of synthetic, seeded inputs already resident in HBM.  The default
workload is the Mixtral-8x7B-shaped prefill layer (T=4096, H=4096, I=14336,
E=8, top-2, bf16, split gate||up, softmax renormalised, SiLU-gated).

Prints ONE JSON line (the last line of stdout).  The dominant kernel's
duration is measured live with HIP events recorded by the library around
each stage on the launch stream (moe_forward_timed).  The CPU baseline is the
fp64 oracle timed on a bounded token sample of the same workload.
"""
import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer active TFLOP/s + tokens/s (prefill); weight-stream HBM GB/s "
          "(decode)")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
STAGES = ["route", "permute", "gemm_gate_up", "gemm_down", "combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """Raw HIP events through libamdhip64 (recorded by the library itself)."""

    def __init__(self):
        self.L = C.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]

    def event(self):
        e = C.c_void_p()
        assert self.L.hipEventCreate(C.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        rc = self.L.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b))
        assert rc == 0, rc
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(C.c_void_p(e))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_kernels.h", "gemm_prefill.hip", "gemm_prefill_mx.hip",
              "gemm_mid.hip", "gemm_decode.hip", "gemm_common.h", "moe_kernels.h"):
        with open(os.path.join(ROOT, "mixture_experts_ffn_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch of the gate||up GEMM from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"gemm_gate_up_{workload}_traffic.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, inp, budget_s: float, stream_bytes=None):
    """The oracle on the host cores over a bounded token sample.  With
    stream_bytes (a decode step) and the whole step in the sample, the rate is
    those weight bytes over the oracle's time, as for the GPU line."""
    import numpy as np
    import oracle
    oracle.build()
    threads = min(os.cpu_count() or 1, 16)
    host = {k: v.cpu() for k, v in inp.items()}
    p = oracle.params_of(cfg)
    rng = np.random.default_rng(1)
    t0 = time.perf_counter()
    oracle.forward(p, host, tokens=np.arange(min(threads, cfg.T)), threads=threads,
                   use_router=cfg.router)
    per_tok = (time.perf_counter() - t0) / min(threads, cfg.T)
    n = int(max(threads, min(cfg.T, budget_s / max(per_tok, 1e-6))))
    n = (n // threads) * threads or threads
    toks = np.sort(rng.choice(cfg.T, size=min(n, cfg.T), replace=False))
    t0 = time.perf_counter()
    oracle.forward(p, host, tokens=toks, threads=threads, use_router=cfg.router)
    dt = time.perf_counter() - t0
    if stream_bytes is not None and len(toks) == cfg.T:
        value, unit = stream_bytes / dt / 1e9, "GB/s"
    else:
        value, unit = cfg.flops / cfg.T * len(toks) / dt / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{len(toks)} of {cfg.T} tokens of {cfg.name} (full weights), "
                      f"{dt:.3g} s on {threads} threads; {len(toks) / dt:.2f} tokens/s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--activation", default=None,
                    help="override the workload's activation (e.g. relu, gelu, identity)")
    ap.add_argument("--weigh-inputs", action="store_true",
                    help="weigh-inputs routing (weights scale the experts' inputs)")
    ap.add_argument("--router", action="store_true",
                    help="the layer's own router computes the logits (x.Wr+Br) in the step")
    ap.add_argument("--gemm-variant", type=int, default=0,
                    help="grouped-GEMM tiles: 0 auto, 1 256-row, 2 32-row, 3 128-row")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain device copy of known size (HBM counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no collectives or sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_ffn_03_amd import from_config, synth

    cfg = synth.CONFIGS[args.workload]
    over = {}
    if args.activation:
        over["activation"] = args.activation
    if args.weigh_inputs:
        over["weigh_inputs"] = True
    if args.router:
        over["router"] = True
    if over:
        cfg = cfg.replace(**over)
    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name} inputs on {dev}")
    inp = synth.make_inputs(cfg, device=dev)
    layer = from_config(cfg, gemm_variant=args.gemm_variant)
    layer.set_weights_from(inp)
    x, lg = inp["x"], inp["logits"]
    out = torch.empty_like(x)
    ws = layer.workspace(cfg.T, dev)
    # with the layer's own router the step computes the logits itself
    step_logits = None if cfg.router else lg
    if cfg.router:
        lg = layer.router_logits(x)
    # experts that receive tokens (their weights are the ones a step streams)
    touched = int((layer.route(lg)["expert_counts"] > 0).sum().item())
    wb = 0.5 + 1.0 / 32.0 if cfg.w_dtype == "mxfp4" else (4.0 if cfg.w_dtype == "f32" else 2.0)
    gu_bytes = (2.0 if cfg.gated else 1.0) * cfg.I * cfg.H * wb
    dn_bytes = 1.0 * cfg.H * cfg.I * wb
    # few rows per expert: the step streams weights (same threshold the library
    # uses to pick its small-M tiles)
    decode = cfg.T * cfg.K < 96 * cfg.E
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 268435456 bytes read + written")

    hip = Hip()
    evs = [[hip.event() for _ in range(6)] for _ in range(args.steps)]
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        layer(x, step_logits, out=out, workspace=ws)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    start.record()
    for k in range(args.steps):
        layer(x, step_logits, out=out, workspace=ws, events=evs[k])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    stage_ms = {}
    for i, name in enumerate(STAGES):
        stage_ms[name] = sum(hip.elapsed_ms(evs[k][i], evs[k][i + 1])
                             for k in range(args.steps)) / args.steps
    for row in evs:
        for e in row:
            hip.destroy(e)

    flops = float(cfg.flops)
    gemm1_flops = (4.0 if cfg.gated else 2.0) * cfg.T * cfg.K * cfg.H * cfg.I
    g1 = stage_ms["gemm_gate_up"]
    traffic = load_traffic(cfg.name)
    if decode:
        # weight-stream rate: each touched expert's weights are read once per step
        stream = touched * (gu_bytes + dn_bytes)
        value, unit = stream / (ms * 1e-3) / 1e9, "GB/s"
        g1_bytes = touched * gu_bytes + cfg.T * cfg.H * 2 + cfg.T * cfg.K * cfg.I * 2
        roof = {"bound": "hbm", "kernel": "gate||up grouped GEMM (decode tiles)",
                "achieved": g1_bytes / (g1 * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        value, unit = flops / (ms * 1e-3) / 1e12, "TFLOP/s"
        roof = {"bound": "mfma", "kernel": "gate||up grouped GEMM",
                "achieved": gemm1_flops / (g1 * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    res = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "tokens_per_s": cfg.T / (ms * 1e-3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.x_dtype if cfg.w_dtype != "mxfp4" else "bf16 (mxfp4 weights)",
        "data": "synthetic (seeded, random-init weights of the workload's shape)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "K": cfg.K, "layout": cfg.layout, "weights": cfg.w_dtype,
                   "scoring": cfg.scoring, "activation": cfg.activation,
                   "weigh_inputs": cfg.weigh_inputs, "router_in_step": cfg.router,
                   "parallelism": "none (1 GPU)"},
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "active_tflops": flops / (ms * 1e-3) / 1e12,
        "weight_stream_gbs": touched * (gu_bytes + dn_bytes) / (ms * 1e-3) / 1e9,
        "experts_touched": touched,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(
            cfg, inp, args.cpu_seconds,
            stream_bytes=touched * (gu_bytes + dn_bytes) if decode else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
