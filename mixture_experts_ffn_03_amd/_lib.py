"""ctypes binding of ``libmoe_mi355x.so`` (the C ABI of include/moe_mi355x.h).

Argument marshalling only: torch tensors become ``moe_tensor`` views (device
pointer, dtype, shape); every step of the layer runs in the HIP kernels.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

# enums (include/moe_mi355x.h)
MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_SHAPE_MISMATCH",
                3: "MOE_ERR_NOT_DECLARED", 4: "MOE_ERR_UNBOUND",
                5: "MOE_ERR_UNSUPPORTED", 6: "MOE_ERR_WORKSPACE", 7: "MOE_ERR_HIP"}
MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_MXFP4, MOE_DTYPE_I32 = 0, 1, 2, 3
SCORING = {"softmax": 0, "sigmoid": 1}
ACTIVATION = {"silu": 0, "swiglu_clamped": 1, "relu": 2, "gelu": 3, "silu_plain": 4,
              "identity": 5}
GELU_MODE = {"erf": 0, "tanh": 1}
FUSION = {"unfused": 0, "interleaved": 1, "split": 2}
WDTYPE = {"f32": MOE_DTYPE_F32, "bf16": MOE_DTYPE_BF16, "mxfp4": MOE_DTYPE_MXFP4}

EXPORTS = ["moe_options_default", "moe_create", "moe_set_weights", "moe_prepare",
           "moe_workspace_size", "moe_forward", "moe_forward_timed", "moe_route",
           "moe_router_logits", "moe_borrowed_slots", "moe_forward_noalloc", "moe_destroy",
           "moe_last_error", "moe_status_string"]
NOALLOC_SCRATCH_BYTES = 32 << 20
# moe_borrowed_slots bits, one per moe_weights member in field order
SLOT_BITS = {"gate_up_experts": 0x001, "down_experts": 0x002, "gate_experts": 0x004,
             "gate_up_bias": 0x008, "down_bias": 0x010, "gate_bias": 0x020,
             "e_score_correction_bias": 0x040, "router_weight": 0x080, "router_bias": 0x100,
             "shared_gate": 0x200}
MOE_STAGE_EVENTS = 6


class moe_options(C.Structure):
    _fields_ = [("scoring", C.c_int32), ("renormalize", C.c_int32),
                ("n_group", C.c_int32), ("topk_group", C.c_int32),
                ("routed_scaling_factor", C.c_float), ("activation", C.c_int32),
                ("swiglu_fusion", C.c_int32), ("swiglu_alpha", C.c_float),
                ("swiglu_beta", C.c_float), ("swiglu_limit", C.c_float),
                ("gemm_variant", C.c_int32), ("gelu_mode", C.c_int32),
                ("weigh_inputs", C.c_int32), ("down_fp16_copy", C.c_int32),
                ("pack_weights", C.c_int32)]


class moe_tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scales", C.c_void_p), ("dtype", C.c_int32),
                ("ndim", C.c_int32), ("shape", C.c_int64 * 4)]


class moe_weights(C.Structure):
    _fields_ = [(n, moe_tensor) for n in (
        "gate_up_experts", "down_experts", "gate_experts", "gate_up_bias",
        "down_bias", "gate_bias", "e_score_correction_bias", "router_weight",
        "router_bias", "shared_gate")]


class moe_routing_out(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "topk_ids", "topk_weights", "expert_counts", "expert_offsets",
        "row_token", "slot_row")]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP extension first "
                "(python -m mixture_experts_ffn_03_amd.build)")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        sig = {
            "moe_options_default": ([C.POINTER(moe_options)], C.c_int),
            "moe_create": ([C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int,
                            C.c_int, C.POINTER(moe_options), C.POINTER(P)], C.c_int),
            "moe_set_weights": ([P, C.POINTER(moe_weights)], C.c_int),
            "moe_prepare": ([P, P], C.c_int),
            "moe_workspace_size": ([P, C.c_int64, C.POINTER(C.c_size_t)], C.c_int),
            "moe_forward": ([P, C.POINTER(moe_tensor), C.POINTER(moe_tensor),
                             C.POINTER(moe_tensor), C.POINTER(moe_tensor), P, C.c_size_t,
                             C.POINTER(moe_routing_out), P], C.c_int),
            "moe_forward_timed": ([P, C.POINTER(moe_tensor), C.POINTER(moe_tensor),
                                   C.POINTER(moe_tensor), C.POINTER(moe_tensor), P,
                                   C.c_size_t, C.POINTER(moe_routing_out), P,
                                   C.POINTER(P)], C.c_int),
            "moe_route": ([P, C.POINTER(moe_tensor), C.POINTER(moe_routing_out), P,
                           C.c_size_t, P], C.c_int),
            "moe_router_logits": ([P, C.POINTER(moe_tensor), C.POINTER(moe_tensor), P,
                                   C.c_size_t, P], C.c_int),
            "moe_borrowed_slots": ([P, C.POINTER(C.c_uint32)], C.c_int),
            "moe_forward_noalloc": ([P, C.POINTER(moe_tensor), C.POINTER(moe_tensor),
                                     C.POINTER(moe_tensor), C.POINTER(moe_tensor),
                                     C.POINTER(moe_routing_out), P], C.c_int),
            "moe_destroy": ([P], C.c_int),
            "moe_last_error": ([], C.c_char_p),
            "moe_status_string": ([C.c_int], C.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def options(**kw) -> moe_options:
    """moe_options from the defaults, overridden by clika-style kwargs
    (scoring/routing_mode, renormalize, n_group, topk_group,
    routed_scaling_factor, activation, swiglu_fusion, swiglu_alpha,
    swiglu_beta, swiglu_limit, gemm_variant, gelu_mode,
    weigh_inputs / apply_router_weight_on_input, down_fp16_copy, pack_weights)."""
    o = moe_options()
    check(lib().moe_options_default(C.byref(o)))
    for k, v in kw.items():
        if k in ("scoring", "routing_mode") and isinstance(v, str):
            v = SCORING[{"softmax_topk": "softmax"}.get(v, v)]
            k = "scoring"
        elif k == "activation" and isinstance(v, str):
            v = ACTIVATION[v]
        elif k == "swiglu_fusion" and isinstance(v, str):
            v = FUSION[v]
        elif k == "gelu_mode" and isinstance(v, str):
            v = GELU_MODE[v]
        elif k == "apply_router_weight_on_input":
            k = "weigh_inputs"
        setattr(o, k, int(v) if isinstance(v, bool) else v)
    return o


_TORCH_DT = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16,
             torch.int32: MOE_DTYPE_I32}


def tensor(t, scales: Optional[torch.Tensor] = None) -> moe_tensor:
    """moe_tensor view of a contiguous device tensor (None -> absent slot).
    An MXFP4 stack is passed as codes (uint8 [..., K/2]) with its scales."""
    m = moe_tensor()
    if t is None:
        return m
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if scales is not None:
        if not scales.is_contiguous():
            raise ValueError("tensors must be contiguous")
        m.dtype = MOE_DTYPE_MXFP4
        shape = list(t.shape[:-1]) + [t.shape[-1] * 2]
        m.scales = scales.data_ptr()
    else:
        if t.dtype not in _TORCH_DT:
            raise ValueError(f"unsupported dtype {t.dtype}")
        m.dtype = _TORCH_DT[t.dtype]
        shape = list(t.shape)
    if len(shape) > 4:
        raise ValueError("at most 4 dims")
    m.data = t.data_ptr()
    m.ndim = len(shape)
    for i, d in enumerate(shape):
        m.shape[i] = d
    return m


def stream_ptr(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream
