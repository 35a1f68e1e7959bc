"""Seeded synthetic inputs for the mixture-of-experts FFN forward.

This module is the single source of inputs for both the HIP path and the CPU
oracle.  It draws random numbers and converts storage types; it holds none of
the layer's arithmetic (no routing, no activation, no contraction).

Workloads are model-shaped (Mixtral-8x7B, Qwen3-30B-A3B, gpt-oss-20b,
DeepSeek-V3 expert layers).  No dataset or trained checkpoint is involved:
every tensor is drawn here from a counter-style seed derived from
(workload id, tensor id, expert index), so any expert's slab can be
regenerated on its own and on any device.

Distribution reading: ``N(0, s)`` means mean 0 and standard deviation ``s``;
expert weights use ``s = 1/sqrt(fan_in)`` (fan_in = H for gate/up rows, I for
down rows).  MXFP4 stacks draw each 4-bit e2m1 code uniformly over all 16
codes and each e8m0 block scale uniformly over the exponents -8..-4
(biased bytes 119..123); codes are packed two per byte, element 2i in the low
nibble of byte i, one scale byte per 32 consecutive elements along the
reduction dimension.
"""
from __future__ import annotations

import dataclasses
import math
import hashlib
from typing import Dict, Optional

import torch

# tensor ids used in seeds
T_X, T_LOGITS, T_GATE_UP, T_UP, T_DOWN, T_GU_BIAS, T_DOWN_BIAS, T_SEL_BIAS, \
    T_GATE_BIAS, T_SHARED, T_ROUTER_W, T_ROUTER_B, T_SHARED_GATE = range(13)

# activations that read a gate and an up projection (the others read one)
GATED_ACTS = ("silu", "swiglu_clamped")


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    cid: int                      # workload id (seed domain)
    T: int                        # tokens
    H: int                        # hidden size
    I: int                        # expert intermediate size
    E: int                        # experts
    K: int                        # experts kept per token
    x_dtype: str = "bf16"         # "f32" | "bf16"
    w_dtype: str = "bf16"         # "f32" | "bf16" | "mxfp4"
    layout: str = "split"         # "unfused" | "interleaved" | "split"
    scoring: str = "softmax"      # "softmax" | "sigmoid"
    renormalize: bool = True
    n_group: int = 0
    topk_group: int = 0
    routed_scaling_factor: float = 1.0
    activation: str = "silu"      # "silu" (SiLU-gated) | "swiglu_clamped"
    swiglu_alpha: float = 1.0
    swiglu_beta: float = 0.0
    swiglu_limit: float = 0.0
    expert_biases: bool = False   # gate/up and down biases
    bias_std: float = 0.02
    selection_bias_std: Optional[float] = None   # e_score_correction_bias [E]
    logit_std: float = 1.0
    shared_output: bool = False   # draw a [T,H] shared-expert output
    shared_gate: bool = False     # draw a shared-expert gate g [H] (x . g ~ N(0, 1))
    gelu_mode: str = "erf"        # "erf" | "tanh" (activation "gelu")
    weigh_inputs: bool = False    # kept weight scales the expert's input
    router: bool = False          # draw router_weight [H,E] and router_bias [E]

    def replace(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)

    @property
    def gated(self) -> bool:
        return self.activation in GATED_ACTS

    @property
    def flops(self) -> int:
        """Active multiply-add flops of the expert FFNs: 6*T*K*H*I gated,
        4*T*K*H*I with one fc1 projection (router not counted)."""
        return (6 if self.gated else 4) * self.T * self.K * self.H * self.I


# The five workloads.  Full sizes are the measured shapes; the "_small"
# variants keep every structural feature (layout, dtypes, routing mode,
# skew, biases) at sizes the CPU oracle finishes in seconds while still
# spanning several GEMM tiles and ragged tails.
CONFIGS: Dict[str, MoeConfig] = {}


def _reg(c: MoeConfig) -> MoeConfig:
    CONFIGS[c.name] = c
    return c


TINY_FP32 = _reg(MoeConfig(
    name="tiny_fp32", cid=0, T=16, H=64, I=128, E=4, K=2,
    x_dtype="f32", w_dtype="f32", layout="unfused"))
MIXTRAL_PREFILL = _reg(MoeConfig(
    name="mixtral_prefill", cid=1, T=4096, H=4096, I=14336, E=8, K=2))
QWEN3_DECODE = _reg(MoeConfig(
    name="qwen3_decode", cid=2, T=32, H=2048, I=768, E=128, K=8,
    logit_std=2.0))
GPTOSS_MXFP4 = _reg(MoeConfig(
    name="gptoss_mxfp4", cid=3, T=2048, H=2880, I=2880, E=32, K=4,
    w_dtype="mxfp4", layout="interleaved", expert_biases=True,
    activation="swiglu_clamped", swiglu_alpha=1.702, swiglu_beta=1.0,
    swiglu_limit=7.0))
DEEPSEEK_V3 = _reg(MoeConfig(
    name="deepseek_v3", cid=4, T=8192, H=7168, I=2048, E=256, K=8,
    scoring="sigmoid", selection_bias_std=0.1, n_group=8, topk_group=4,
    routed_scaling_factor=2.5))

MIXTRAL_SMALL = _reg(MIXTRAL_PREFILL.replace(
    name="mixtral_small", cid=11, T=1200, H=576, I=448))
QWEN3_SMALL = _reg(QWEN3_DECODE.replace(
    name="qwen3_small", cid=12, T=32, H=512, I=192))
GPTOSS_SMALL = _reg(GPTOSS_MXFP4.replace(
    name="gptoss_small", cid=13, T=300, H=320, I=288))
DEEPSEEK_SMALL = _reg(DEEPSEEK_V3.replace(
    name="deepseek_small", cid=14, T=512, H=512, I=256))

FULL_CONFIGS = ["tiny_fp32", "mixtral_prefill", "qwen3_decode",
                "gptoss_mxfp4", "deepseek_v3"]
SMALL_CONFIGS = ["tiny_fp32", "mixtral_small", "qwen3_small",
                 "gptoss_small", "deepseek_small"]


def seed_of(cid: int, tensor: int, expert: int = -1) -> int:
    """Deterministic 63-bit seed for one tensor (or one expert's slab)."""
    h = hashlib.sha256(f"moe-ffn/{cid}/{tensor}/{expert}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal(shape, std: float, dtype: torch.dtype, device, seed: int) -> torch.Tensor:
    """N(0, std) drawn in fp32 and stored in `dtype` (bf16 by round-to-nearest-even)."""
    t = torch.randn(shape, generator=_gen(device, seed), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def mxfp4_stack(E: int, N: int, Kdim: int, cid: int, tensor: int, device):
    """Packed MXFP4 stack: codes uint8 [E, N, Kdim/2], scales uint8 [E, N, Kdim/32]."""
    assert Kdim % 32 == 0
    codes = torch.empty((E, N, Kdim // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((E, N, Kdim // 32), dtype=torch.uint8, device=device)
    for e in range(E):
        g = _gen(device, seed_of(cid, tensor, e))
        # a uniform byte is two independent uniform 4-bit codes
        codes[e] = torch.randint(0, 256, (N, Kdim // 2), generator=g,
                                 device=device, dtype=torch.int32).to(torch.uint8)
        scales[e] = torch.randint(119, 124, (N, Kdim // 32), generator=g,
                                  device=device, dtype=torch.int32).to(torch.uint8)
    return codes, scales


def dense_stack(E: int, N: int, Kdim: int, dtype: torch.dtype, cid: int,
                tensor: int, device) -> torch.Tensor:
    """Dense stack [E, N, Kdim] with N(0, 1/sqrt(Kdim)) entries, drawn per expert."""
    out = torch.empty((E, N, Kdim), dtype=dtype, device=device)
    std = 1.0 / (Kdim ** 0.5)
    for e in range(E):
        out[e] = normal((N, Kdim), std, dtype, device, seed_of(cid, tensor, e))
    return out


def make_inputs(cfg: MoeConfig, device="cpu", T: Optional[int] = None) -> dict:
    """All tensors of one workload, on `device`.

    Keys: x [T,H], logits [T,E] f32, and the weight slots named as the layer
    binds them: gate_up_experts, gate_experts (unfused only), down_experts,
    their ``*_scales`` for MXFP4, gate_up_bias / gate_bias / down_bias (when
    the workload has expert biases), e_score_correction_bias [E] f32 (when it
    has a selection bias), shared_output [T,H] and shared_gate [H] (when
    requested).

    Fused layouts put 2*I rows in gate_up_experts; for the unfused layout
    gate_up_experts holds the *up* rows [E,I,H] and gate_experts the gate rows.
    ``T`` overrides the token count.
    """
    T = cfg.T if T is None else T
    dev = torch.device(device)
    xd = _torch_dtype(cfg.x_dtype)
    E, H, I, cid = cfg.E, cfg.H, cfg.I, cfg.cid
    out = {}
    out["x"] = normal((T, H), 1.0, xd, dev, seed_of(cid, T_X))
    out["logits"] = normal((T, E), cfg.logit_std, torch.float32, dev,
                           seed_of(cid, T_LOGITS))
    # non-gated activations: one fc1 stack [E, I, H] in gate_up_experts
    fused = cfg.gated and cfg.layout in ("split", "interleaved")
    two = cfg.gated and not fused
    n_gu = 2 * I if fused else I
    if cfg.w_dtype == "mxfp4":
        out["gate_up_experts"], out["gate_up_scales"] = mxfp4_stack(
            E, n_gu, H, cid, T_GATE_UP, dev)
        out["down_experts"], out["down_scales"] = mxfp4_stack(
            E, H, I, cid, T_DOWN, dev)
        if two:
            out["gate_experts"], out["gate_scales"] = mxfp4_stack(
                E, I, H, cid, T_UP, dev)
    else:
        wd = _torch_dtype(cfg.w_dtype)
        out["gate_up_experts"] = dense_stack(E, n_gu, H, wd, cid, T_GATE_UP, dev)
        out["down_experts"] = dense_stack(E, H, I, wd, cid, T_DOWN, dev)
        if two:
            out["gate_experts"] = dense_stack(E, I, H, wd, cid, T_UP, dev)
    if cfg.expert_biases:
        out["gate_up_bias"] = normal((E, n_gu), cfg.bias_std, xd, dev,
                                     seed_of(cid, T_GU_BIAS))
        out["down_bias"] = normal((E, H), cfg.bias_std, xd, dev,
                                  seed_of(cid, T_DOWN_BIAS))
        if two:
            out["gate_bias"] = normal((E, I), cfg.bias_std, xd, dev,
                                      seed_of(cid, T_GATE_BIAS))
    if cfg.selection_bias_std is not None:
        out["e_score_correction_bias"] = normal(
            (E,), cfg.selection_bias_std, torch.float32, dev,
            seed_of(cid, T_SEL_BIAS))
    if cfg.shared_output:
        out["shared_output"] = normal((T, H), 1.0, xd, dev, seed_of(cid, T_SHARED))
    if cfg.shared_gate:
        out["shared_gate"] = normal((H,), 1.0 / math.sqrt(H), xd, dev,
                                    seed_of(cid, T_SHARED_GATE))
    if cfg.router:
        # router Wr [H, E] (the layout of the MoeSpec router index arithmetic)
        out["router_weight"] = normal((H, E), 1.0 / math.sqrt(H), xd, dev,
                                      seed_of(cid, T_ROUTER_W))
        out["router_bias"] = normal((E,), cfg.bias_std, xd, dev, seed_of(cid, T_ROUTER_B))
    return out
