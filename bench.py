#!/usr/bin/env python3
"""Benchmark of the MoE FFN forward on one MI355X.

One step = one full forward of the layer (routing, permutation, grouped
gate||up GEMM with the fused activation, grouped down GEMM, combine) over one
batch of synthetic, seeded inputs already resident in HBM.  The headline
workload is the Mixtral-8x7B-shaped prefill layer (T=4096, H=4096, I=14336,
E=8, top-2, bf16, split gate||up, softmax renormalised, SiLU-gated): its K
back-to-back steps are the timed region, bracketed by device synchronisation.

Prints ONE JSON line (the last line of stdout).  Besides the headline figures
it carries:
  - "decode": the Qwen3-30B-A3B-shaped decode step (T=32), whose metric is
    the weight-stream rate (touched experts' weight bytes per step);
  - "workloads": the gpt-oss-20b-shaped MXFP4 layer and the DeepSeek-V3-shaped
    layer (and the decode step again), each with its own roofline object.
  - "decode.graph_replay": the same decode step captured once into a HIP graph
    and replayed (no host launch gaps between its kernels), timed the same way.
Each of these is timed step by step with HIP events on the launch stream
(the step time from plain steps between two events, the stage times from a
second pass with the library's stage events),
with a 1 GiB scratch buffer read between steps (outside the events) so that
a step never finds the previous step's weights in the 256 MiB Infinity
Cache.  The flush reads rather than writes: a write would leave the caches
full of dirty lines whose write-back then competes with the measured step's
weight stream (a serving step follows layers that read their weights).  The
headline's timed loop has no flush: its 2.8 GB of weights cycle the cache by
themselves; its per-step flushed time is reported next to it.

The dominant kernel's duration is measured live with HIP events recorded by
the library around each stage on the launch stream (moe_forward_timed).  The
CPU baseline is the fp64 oracle timed on a bounded token sample of the
headline workload.
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
FLUSH_BYTES = 1 << 30       # scratch read between flushed steps (4x the MALL)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Hip:
    """Raw HIP events through libamdhip64 (recorded by the library itself, or
    on torch's current stream, which is the stream the layer launches on)."""

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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Threads the CPU baseline may use: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when the host sets it (a shared GPU host gives
    each GPU's jobs a fixed CPU share and says so there)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    n = min(avail, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else avail
    return n, avail


def cpu_baseline(cfg, inp, budget_s: float, stream_bytes=None):
    """The oracle on the host cores over a bounded token sample.  With
    stream_bytes (a decode step) and the whole step in the sample, the rate is
    those weight bytes over the oracle's time, as for the GPU line."""
    import numpy as np
    import oracle
    oracle.build()
    threads, avail = host_threads()
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
    cap = os.environ.get("OMP_NUM_THREADS")
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "cpus_available": avail,
            "cores_note": (f"capped at OMP_NUM_THREADS={cap}, the host's CPU share per GPU"
                           if cap and threads < avail else "all CPUs available to the process"),
            "sample": f"{len(toks)} of {cfg.T} tokens of {cfg.name} (full weights), "
                      f"{dt:.3g} s on {threads} threads; {len(toks) / dt:.2f} tokens/s"}


class Workload:
    """One workload's inputs, layer and per-step accounting."""

    def __init__(self, cfg, dev, gemm_variant=0):
        from mixture_experts_ffn_03_amd import from_config, synth
        import torch
        self.cfg = cfg
        log(f"[bench] generating {cfg.name} inputs on {dev}")
        self.inp = synth.make_inputs(cfg, device=dev)
        self.layer = from_config(cfg, gemm_variant=gemm_variant)
        self.layer.set_weights_from(self.inp)
        self.layer.initialize()
        self.x, lg = self.inp["x"], self.inp["logits"]
        self.out = torch.empty_like(self.x)
        self.ws = self.layer.workspace(cfg.T, dev)
        # with the layer's own router the step computes the logits itself
        self.step_logits = None if cfg.router else lg
        if cfg.router:
            lg = self.layer.router_logits(self.x)
        # experts that receive tokens (their weights are the ones a step streams)
        self.touched = int((self.layer.route(lg)["expert_counts"] > 0).sum().item())
        wb = 0.5 + 1.0 / 32.0 if cfg.w_dtype == "mxfp4" else (4.0 if cfg.w_dtype == "f32" else 2.0)
        self.gu_bytes = (2.0 if cfg.gated else 1.0) * cfg.I * cfg.H * wb
        self.dn_bytes = 1.0 * cfg.H * cfg.I * wb
        # few rows per expert: the step streams weights (the threshold the
        # library uses to pick its small-M tiles)
        self.decode = cfg.T * cfg.K < 96 * cfg.E
        torch.cuda.synchronize()

    def step(self, events=None):
        self.layer(self.x, self.step_logits, out=self.out, workspace=self.ws, events=events)

    def stream_bytes(self) -> float:
        return self.touched * (self.gu_bytes + self.dn_bytes)

    def summary(self, ms: float, stage_ms: dict, flushed: bool) -> dict:
        """Rates of one workload from its step time and stage times, with the
        roofline object of its gate||up GEMM (the dominant kernel)."""
        cfg = self.cfg
        g1 = stage_ms["gemm_gate_up"]
        gemm1_flops = (4.0 if cfg.gated else 2.0) * cfg.T * cfg.K * cfg.H * cfg.I
        d = {
            "workload": cfg.name, "ms_per_step": ms,
            "active_tflops": cfg.flops / (ms * 1e-3) / 1e12,
            "tokens_per_s": cfg.T / (ms * 1e-3),
            "weight_stream_gbs": self.stream_bytes() / (ms * 1e-3) / 1e9,
            "experts_touched": self.touched,
            "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
            "mall_flushed_between_steps": flushed,
            "gemm_ms": round(g1 + stage_ms["gemm_down"], 4),
        }
        if self.decode:
            g1_bytes = (self.touched * self.gu_bytes + cfg.T * cfg.H * 2
                        + cfg.T * cfg.K * cfg.I * 2)
            roof = {"bound": "hbm", "kernel": "gate||up grouped GEMM (decode tiles)",
                    "achieved": g1_bytes / (g1 * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s"}
            d["gemms_weight_stream_gbs"] = self.stream_bytes() / (d["gemm_ms"] * 1e-3) / 1e9
            d["gemms_hbm_frac"] = d["gemms_weight_stream_gbs"] / PEAK_HBM_GBS
        else:
            # the bound is whichever floor is the longer: the MFMA work at the
            # dense bf16 peak, or the touched weights plus x and h at HBM peak
            # (the skewed DeepSeek-V3 shape streams 13 GB of gate||up weights)
            g1_bytes = (self.touched * self.gu_bytes + cfg.T * cfg.H * 2
                        + cfg.T * cfg.K * cfg.I * 2)
            floor_mfma = gemm1_flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
            floor_hbm = g1_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
            if floor_hbm > floor_mfma:
                roof = {"bound": "hbm", "kernel": "gate||up grouped GEMM",
                        "achieved": g1_bytes / (g1 * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s"}
            else:
                roof = {"bound": "mfma", "kernel": "gate||up grouped GEMM",
                        "achieved": gemm1_flops / (g1 * 1e-3) / 1e12,
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
            roof["floors_ms"] = {"mfma": round(floor_mfma, 4), "hbm": round(floor_hbm, 4)}
            roof["mfma_frac"] = gemm1_flops / (g1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
            gemm2_flops = 2.0 * cfg.T * cfg.K * cfg.H * cfg.I
            d["gemm_down_frac"] = gemm2_flops / (stage_ms["gemm_down"] * 1e-3) / 1e12 \
                / PEAK_BF16_TFLOPS
            d["gemms_frac"] = cfg.flops / (d["gemm_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = load_traffic(cfg.name)
        d["roofline"] = roof
        return d


def stage_times(hip, evs):
    out = {}
    for i, name in enumerate(STAGES):
        out[name] = sum(hip.elapsed_ms(row[i], row[i + 1]) for row in evs) / len(evs)
    return out


def timed_flushed(wl, hip, steps: int, warmup: int, scratch):
    """Step by step with a read of the FLUSH_BYTES scratch before each step,
    outside the step's timing.  Two passes: plain steps, each between two
    events on the launch stream (the step time), then steps with the
    library's stage events (stage times; on a step of a few tenths of a
    millisecond the six extra event packets add about 3 us each).
    Returns (mean ms, stage ms, min ms, mean ms of the staged pass)."""
    import torch
    words = scratch.view(torch.int32)
    for _ in range(warmup):
        words.max()
        wl.step()
    torch.cuda.synchronize()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for k in range(steps):
        words.max()
        pairs[k][0].record()
        wl.step()
        pairs[k][1].record()
    torch.cuda.synchronize()
    plain = [a.elapsed_time(b) for a, b in pairs]
    evs = [[hip.event() for _ in range(6)] for _ in range(steps)]
    for k in range(steps):
        words.max()
        wl.step(events=evs[k])
    torch.cuda.synchronize()
    staged = [hip.elapsed_ms(row[0], row[5]) for row in evs]
    st = stage_times(hip, evs)
    for row in evs:
        for e in row:
            hip.destroy(e)
    return sum(plain) / len(plain), st, min(plain), sum(staged) / len(staged)


def timed_graph(wl, steps: int, scratch):
    """The step captured once into a HIP graph and replayed: a prepared
    layer's forward on a caller workspace and output is kernel launches only,
    so torch.cuda.graph can capture it (as a serving loop would) and a replay
    drops the host launch gaps between the step's kernels.  Each replay is
    timed between two events after the same 1 GiB scratch read as the eager
    steps.  Returns (mean ms, min ms)."""
    import torch
    words = scratch.view(torch.int32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wl.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.step()
    torch.cuda.synchronize()
    words.max()
    g.replay()
    torch.cuda.synchronize()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for k in range(steps):
        words.max()
        pairs[k][0].record()
        g.replay()
        pairs[k][1].record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in pairs]
    del g
    return sum(t) / len(t), min(t)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="headline workload only (no decode / gpt-oss / DeepSeek sub-results)")
    ap.add_argument("--sub-steps", type=int, default=10,
                    help="flushed steps timed per sub-result workload")
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
    from mixture_experts_ffn_03_amd import synth

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
    wl = Workload(cfg, dev, args.gemm_variant)

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 268435456 bytes read + written")
        del a, b

    hip = Hip()
    evs = [[hip.event() for _ in range(6)] for _ in range(args.steps)]
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        wl.step(events=evs[k])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    stage_ms = stage_times(hip, evs)
    for row in evs:
        for e in row:
            hip.destroy(e)
    head = wl.summary(ms, stage_ms, flushed=False)

    scratch = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    fl_ms, fl_st, fl_min, fl_staged = timed_flushed(wl, hip, min(args.steps, 10), 1, scratch)
    log(f"[bench] {cfg.name}: {ms:.4f} ms/step back to back, {fl_ms:.4f} flushed")

    if wl.decode:
        value, unit = wl.stream_bytes() / (ms * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = cfg.flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    res = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "tokens_per_s": head["tokens_per_s"],
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
        "stages_ms": head["stages_ms"],
        "active_tflops": head["active_tflops"],
        "weight_stream_gbs": head["weight_stream_gbs"],
        "experts_touched": wl.touched,
        "gemms_frac": head.get("gemms_frac"),
        "flushed": {"ms_per_step": fl_ms, "min_ms": fl_min,
                    "ms_per_step_with_stage_events": fl_staged,
                    "stages_ms": {k: round(v, 4) for k, v in fl_st.items()},
                    "scratch_read_bytes": FLUSH_BYTES},
        "roofline": head["roofline"],
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(cfg, wl.inp, args.cpu_seconds,
                                           stream_bytes=wl.stream_bytes() if wl.decode else None)

    if not args.no_sub and not over and args.gemm_variant == 0:
        subs = {}
        headline = cfg.name
        del wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        for name in ("qwen3_decode", "gptoss_mxfp4", "deepseek_v3"):
            if name == headline:
                continue
            sw = Workload(synth.CONFIGS[name], dev)
            s_ms, s_st, s_min, s_staged = timed_flushed(sw, hip, args.sub_steps, 2, scratch)
            d = sw.summary(s_ms, s_st, flushed=True)
            d["min_ms"] = s_min
            d["ms_per_step_with_stage_events"] = s_staged
            if sw.decode:
                g_ms, g_min = timed_graph(sw, args.sub_steps, scratch)
                d["graph_ms_per_step"] = g_ms
                d["graph_min_ms"] = g_min
                d["graph_weight_stream_gbs"] = sw.stream_bytes() / (g_ms * 1e-3) / 1e9
            log(f"[bench] {name}: {s_ms:.4f} ms/step (flushed), gate||up "
                f"{d['roofline']['frac']:.3f} of {d['roofline']['bound']} peak")
            subs[name] = d
            del sw
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        res["workloads"] = subs
        if "qwen3_decode" in subs:
            q = subs["qwen3_decode"]
            res["decode"] = {
                "workload": "qwen3_decode", "metric": "weight-stream HBM GB/s (decode)",
                "value": q["weight_stream_gbs"], "unit": "GB/s",
                "hbm_frac_step": q["weight_stream_gbs"] / PEAK_HBM_GBS,
                "gemms_weight_stream_gbs": q["gemms_weight_stream_gbs"],
                "gemms_hbm_frac": q["gemms_hbm_frac"],
                "ms_per_step": q["ms_per_step"], "mall_flushed_between_steps": True,
                "roofline": q["roofline"]}
            if "graph_ms_per_step" in q:
                res["decode"]["graph_replay"] = {
                    "ms_per_step": q["graph_ms_per_step"], "min_ms": q["graph_min_ms"],
                    "weight_stream_gbs": q["graph_weight_stream_gbs"],
                    "hbm_frac_step": q["graph_weight_stream_gbs"] / PEAK_HBM_GBS}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
