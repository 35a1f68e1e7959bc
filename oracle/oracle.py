"""ctypes wrapper of the C oracle (``moe_oracle.c``) -- TEST INFRASTRUCTURE.

Accepts numpy arrays or CPU torch tensors.  bf16 tensors are passed as their
raw 16-bit patterns; the oracle widens them exactly to fp64.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

ORC_F32, ORC_BF16, ORC_MXFP4 = 0, 1, 2
LAYOUTS = {"unfused": 0, "interleaved": 1, "split": 2}
SCORING = {"softmax": 0, "sigmoid": 1}
ACTS = {"silu": 0, "swiglu_clamped": 1, "relu": 2, "gelu": 3, "silu_plain": 4,
        "identity": 5}
GELU_MODES = {"erf": 0, "tanh": 1}
KINDS = {"f32": ORC_F32, "bf16": ORC_BF16, "mxfp4": ORC_MXFP4}


class OrcParams(C.Structure):
    _fields_ = [("T", C.c_int64), ("H", C.c_int64), ("I", C.c_int64),
                ("E", C.c_int64), ("K", C.c_int64),
                ("x_kind", C.c_int32), ("w_kind", C.c_int32),
                ("layout", C.c_int32), ("scoring", C.c_int32),
                ("renormalize", C.c_int32), ("n_group", C.c_int32),
                ("topk_group", C.c_int32), ("activation", C.c_int32),
                ("routed_scaling_factor", C.c_double),
                ("alpha", C.c_double), ("beta", C.c_double), ("limit", C.c_double),
                ("gelu_mode", C.c_int32), ("weigh_inputs", C.c_int32)]


class OrcInputs(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "x", "logits", "w_gu", "w_gu_scales", "w_gate", "w_gate_scales",
        "w_down", "w_down_scales", "b_gu", "b_gate", "b_down", "sel_bias",
        "shared_output", "router_w", "router_b", "shared_gate")]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        lib.orc_route.argtypes = [C.POINTER(OrcParams)] + [C.c_void_p] * 6
        lib.orc_route.restype = C.c_int
        lib.orc_permute.argtypes = [C.POINTER(OrcParams)] + [C.c_void_p] * 5
        lib.orc_permute.restype = None
        lib.orc_forward.argtypes = [C.POINTER(OrcParams), C.POINTER(OrcInputs),
                                    C.c_int64, C.c_void_p, C.c_int] + [C.c_void_p] * 5
        lib.orc_forward.restype = C.c_int
        lib.orc_mxfp4_value.argtypes = [C.c_uint8, C.c_uint8]
        lib.orc_mxfp4_value.restype = C.c_double
        lib.orc_activation.argtypes = [C.POINTER(OrcParams), C.c_double, C.c_double]
        lib.orc_activation.restype = C.c_double
        lib.orc_activation1.argtypes = [C.POINTER(OrcParams), C.c_double]
        lib.orc_activation1.restype = C.c_double
        lib.orc_router_logits.argtypes = [C.POINTER(OrcParams), C.POINTER(OrcInputs),
                                          C.c_void_p]
        lib.orc_router_logits.restype = C.c_int
        lib.orc_bf16_to_double.argtypes = [C.c_uint16]
        lib.orc_bf16_to_double.restype = C.c_double
        _lib = lib
    return _lib


def params_of(cfg, T: Optional[int] = None, **over) -> OrcParams:
    """OrcParams from a ``synth.MoeConfig`` (fields may be overridden)."""
    d = dict(T=cfg.T if T is None else T, H=cfg.H, I=cfg.I, E=cfg.E, K=cfg.K,
             x_kind=KINDS[cfg.x_dtype], w_kind=KINDS[cfg.w_dtype],
             layout=LAYOUTS[cfg.layout], scoring=SCORING[cfg.scoring],
             renormalize=int(cfg.renormalize), n_group=cfg.n_group,
             topk_group=cfg.topk_group, activation=ACTS[cfg.activation],
             routed_scaling_factor=cfg.routed_scaling_factor,
             alpha=cfg.swiglu_alpha, beta=cfg.swiglu_beta, limit=cfg.swiglu_limit,
             gelu_mode=GELU_MODES[cfg.gelu_mode], weigh_inputs=int(cfg.weigh_inputs))
    d.update(over)
    return OrcParams(**d)


def _np(a, dtype=None) -> Optional[np.ndarray]:
    """Contiguous host numpy view; bf16 torch tensors become uint16 bit patterns."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach()
            if a.device.type != "cpu":
                a = a.cpu()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16)
            a = a.contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def route(p: OrcParams, logits, sel_bias=None):
    """Routing of every token: dict(ids [T,K] i32, weights [T,K] f64,
    scores [T,E] f64, keys [T,E] f64)."""
    lib = load()
    lg = _np(logits, np.float32)
    sb = _np(sel_bias, np.float32)
    T, E, K = p.T, p.E, p.K
    assert lg.shape == (T, E)
    ids = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    sc = np.zeros((T, E), np.float64)
    ky = np.zeros((T, E), np.float64)
    rc = lib.orc_route(C.byref(p), _ptr(lg), _ptr(sb), _ptr(ids), _ptr(w),
                       _ptr(sc), _ptr(ky))
    if rc != 0:
        raise ValueError("oracle rejected the routing options")
    return dict(ids=ids, weights=w, scores=sc, keys=ky)


def permute(p: OrcParams, ids):
    """dict(counts [E], offsets [E+1], row_token [T*K], slot_row [T,K])."""
    lib = load()
    ids = _np(ids, np.int32)
    T, E, K = p.T, p.E, p.K
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    row_token = np.zeros(T * K, np.int32)
    slot_row = np.zeros((T, K), np.int32)
    lib.orc_permute(C.byref(p), _ptr(ids), _ptr(counts), _ptr(offsets),
                    _ptr(row_token), _ptr(slot_row))
    return dict(counts=counts, offsets=offsets, row_token=row_token,
                slot_row=slot_row)


def _inputs(inp: dict, keep: dict, use_router: bool) -> OrcInputs:
    def arr(name, dtype=None):
        a = _np(inp.get(name), dtype)
        keep[name] = a
        return _ptr(a)

    return OrcInputs(
        x=arr("x"), logits=None if use_router else arr("logits", np.float32),
        w_gu=arr("gate_up_experts"), w_gu_scales=arr("gate_up_scales", np.uint8),
        w_gate=arr("gate_experts"), w_gate_scales=arr("gate_scales", np.uint8),
        w_down=arr("down_experts"), w_down_scales=arr("down_scales", np.uint8),
        b_gu=arr("gate_up_bias"), b_gate=arr("gate_bias"), b_down=arr("down_bias"),
        sel_bias=arr("e_score_correction_bias", np.float32),
        shared_output=arr("shared_output"),
        router_w=arr("router_weight") if use_router else None,
        router_b=arr("router_bias") if use_router else None,
        shared_gate=arr("shared_gate"))


def router_logits(p: OrcParams, inp: dict) -> np.ndarray:
    """fp64 router logits [T,E] = x . Wr + Br from inp's router_weight [H,E]
    and optional router_bias [E]."""
    keep = {}
    ins = _inputs(inp, keep, True)
    out = np.zeros((p.T, p.E), np.float64)
    if load().orc_router_logits(C.byref(p), C.byref(ins), _ptr(out)) != 0:
        raise ValueError("oracle rejected the router inputs")
    return out


def forward(p: OrcParams, inp: dict, tokens=None, threads: Optional[int] = None,
            stages: bool = False, use_router: bool = False):
    """Forward of the layer on `tokens` (None: all).  `inp` uses the slot
    names of ``synth.make_inputs``; with use_router the logits come from its
    router_weight / router_bias instead of its logits.  Returns dict(out [n,H]
    f64, ids, weights, and with stages=True h [n,K,I], y [n,K,H])."""
    lib = load()
    keep = {}
    ins = _inputs(inp, keep, use_router)
    x = keep["x"]
    assert x.shape == (p.T, p.H), (x.shape, p.T, p.H)
    if tokens is None:
        n, tk = p.T, None
    else:
        tk = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        n = len(tk)
    out = np.zeros((n, p.H), np.float64)
    ids = np.zeros((n, p.K), np.int32)
    w = np.zeros((n, p.K), np.float64)
    h = np.zeros((n, p.K, p.I), np.float64) if stages else None
    y = np.zeros((n, p.K, p.H), np.float64) if stages else None
    if threads is None:
        threads = min(os.cpu_count() or 1, 16)
    rc = lib.orc_forward(C.byref(p), C.byref(ins), n, _ptr(tk), threads,
                         _ptr(out), _ptr(ids), _ptr(w), _ptr(h), _ptr(y))
    if rc != 0:
        raise ValueError("oracle rejected the inputs")
    res = dict(out=out, ids=ids, weights=w)
    if stages:
        res.update(h=h, y=y)
    return res


def mxfp4_value(code4: int, scale_byte: int) -> float:
    return load().orc_mxfp4_value(code4, scale_byte)


def activation(p: OrcParams, g: float, u: float) -> float:
    return load().orc_activation(C.byref(p), g, u)


def activation1(p: OrcParams, v: float) -> float:
    return load().orc_activation1(C.byref(p), v)
