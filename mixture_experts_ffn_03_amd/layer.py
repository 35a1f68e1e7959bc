"""Python surface of the layer, shaped like the clika "MoE" module page:
``MoE(num_experts, hidden_size, intermediate_size, top_k, *, gate_up_bias,
down_bias, dtype, **options)``, ``set_weights(...)`` with the same slot names,
and ``forward(x, router_logits, shared_output=None)``.

Marshalling only: torch allocates the output and the workspace and supplies
the stream; all computation happens in the HIP library behind the C ABI.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _lib


class MoE:
    def __init__(self, num_experts: int, hidden_size: int, intermediate_size: int,
                 top_k: int, *, gate_up_bias: bool = False, down_bias: bool = False,
                 dtype: str = "bf16", **options):
        self.E, self.H, self.I, self.K = num_experts, hidden_size, intermediate_size, top_k
        self.dtype = dtype
        self.opts = _lib.options(**options)
        h = C.c_void_p()
        _lib.check(_lib.lib().moe_create(num_experts, hidden_size, intermediate_size, top_k,
                                         _lib.WDTYPE[dtype], int(gate_up_bias),
                                         int(down_bias), C.byref(self.opts), C.byref(h)))
        self._h = h
        self._bound = {}
        self._ws = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib._lib is not None:
            _lib.lib().moe_destroy(h)
            self._h = None

    # -- binding -------------------------------------------------------------
    def set_weights(self, gate_up_experts, down_experts, *, gate_up_bias=None,
                    down_bias=None, gate_experts=None, gate_bias=None,
                    e_score_correction_bias=None, gate_up_scales=None,
                    down_scales=None, gate_scales=None, router_weight=None,
                    router_bias=None, shared_gate=None):
        """Bind the slots (device tensors, borrowed).  MXFP4 stacks are given as
        codes with their ``*_scales``.  router_weight [H, E] / router_bias [E]
        (optional) let forward compute the router logits itself; shared_gate
        [H] (optional) scales a given shared output by sigmoid(x . g)."""
        w = _lib.moe_weights()
        w.gate_up_experts = _lib.tensor(gate_up_experts, gate_up_scales)
        w.down_experts = _lib.tensor(down_experts, down_scales)
        w.gate_experts = _lib.tensor(gate_experts, gate_scales)
        w.gate_up_bias = _lib.tensor(gate_up_bias)
        w.down_bias = _lib.tensor(down_bias)
        w.gate_bias = _lib.tensor(gate_bias)
        w.e_score_correction_bias = _lib.tensor(e_score_correction_bias)
        w.router_weight = _lib.tensor(router_weight)
        w.router_bias = _lib.tensor(router_bias)
        w.shared_gate = _lib.tensor(shared_gate)
        _lib.check(_lib.lib().moe_set_weights(self._h, C.byref(w)))
        # the library borrows these buffers: keep them alive while bound
        self._bound = dict(gate_up_experts=gate_up_experts, down_experts=down_experts,
                           gate_experts=gate_experts, gate_up_bias=gate_up_bias,
                           down_bias=down_bias, gate_bias=gate_bias,
                           e_score_correction_bias=e_score_correction_bias,
                           gate_up_scales=gate_up_scales, down_scales=down_scales,
                           gate_scales=gate_scales, router_weight=router_weight,
                           router_bias=router_bias, shared_gate=shared_gate)

    def set_weights_from(self, inp: dict):
        """Bind from a dict keyed by slot name (as ``synth.make_inputs`` returns)."""
        keys = ("gate_up_experts", "down_experts", "gate_experts", "gate_up_bias",
                "down_bias", "gate_bias", "e_score_correction_bias", "gate_up_scales",
                "down_scales", "gate_scales", "router_weight", "router_bias", "shared_gate")
        kw = {k: inp.get(k) for k in keys}
        self.set_weights(kw.pop("gate_up_experts"), kw.pop("down_experts"), **kw)

    def initialize(self, stream=None):
        _lib.check(_lib.lib().moe_prepare(self._h, C.c_void_p(_lib.stream_ptr(stream))))

    def borrowed_slots(self) -> set:
        """Names of the bound slots whose caller tensors a forward still reads
        (moe_borrowed_slots); after initialize() the others may be released."""
        m = C.c_uint32()
        _lib.check(_lib.lib().moe_borrowed_slots(self._h, C.byref(m)))
        return {k for k, bit in _lib.SLOT_BITS.items() if m.value & bit}

    # -- running ---------------------------------------------------------------
    def workspace_size(self, T: int) -> int:
        n = C.c_size_t()
        _lib.check(_lib.lib().moe_workspace_size(self._h, T, C.byref(n)))
        return n.value

    def workspace(self, T: int, device, stream=None) -> torch.Tensor:
        """A cached byte workspace big enough for T tokens, one per (device,
        stream): allocated on the stream the library launches on, so the
        caching allocator orders its reuse after that stream's kernels, and
        calls on two streams never share one."""
        n = self.workspace_size(T)
        dev = torch.device(device)
        s = torch.cuda.current_stream(dev) if stream is None else stream
        key = (str(dev), s.cuda_stream)
        if self._ws is None:
            self._ws = {}
        ws = self._ws.get(key)
        if ws is None or ws.numel() < n:
            with torch.cuda.stream(s):
                ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
            self._ws[key] = ws
        return ws

    @staticmethod
    def routing_buffers(T: int, E: int, K: int, device) -> dict:
        i32 = dict(dtype=torch.int32, device=device)
        return dict(topk_ids=torch.empty((T, K), **i32),
                    topk_weights=torch.empty((T, K), dtype=torch.float32, device=device),
                    expert_counts=torch.empty((E,), **i32),
                    expert_offsets=torch.empty((E + 1,), **i32),
                    row_token=torch.empty((T * K,), **i32),
                    slot_row=torch.empty((T, K), **i32))

    @staticmethod
    def _routing_struct(bufs: Optional[dict]):
        if bufs is None:
            return None
        r = _lib.moe_routing_out()
        for k, v in bufs.items():
            setattr(r, k, v.data_ptr() if v is not None else None)
        return r

    def forward(self, x: torch.Tensor, router_logits: Optional[torch.Tensor],
                shared_output: Optional[torch.Tensor] = None, *, out=None,
                routing: Optional[dict] = None, workspace=None, stream=None,
                events=None):
        """One MoE step.  router_logits None: the bound router computes them.
        `events` (optional): MOE_STAGE_EVENTS raw hipEvent_t handles recorded
        at the stage boundaries (moe_forward_timed)."""
        T = x.numel() // x.shape[-1]
        if out is None:
            with torch.cuda.stream(torch.cuda.current_stream(x.device) if stream is None
                                   else stream):
                out = torch.empty_like(x)
        ws = self.workspace(T, x.device, stream) if workspace is None else workspace
        xt, lt, ot = _lib.tensor(x), _lib.tensor(router_logits), _lib.tensor(out)
        st = _lib.tensor(shared_output)
        r = self._routing_struct(routing)
        args = (self._h, C.byref(xt), C.byref(lt), C.byref(st), C.byref(ot),
                C.c_void_p(ws.data_ptr()), ws.numel(), C.byref(r) if r is not None else None,
                C.c_void_p(_lib.stream_ptr(stream)))
        if events is None:
            _lib.check(_lib.lib().moe_forward(*args))
        else:
            arr = (C.c_void_p * _lib.MOE_STAGE_EVENTS)(*events)
            _lib.check(_lib.lib().moe_forward_timed(*args, arr))
        return out

    __call__ = forward

    def forward_noalloc(self, x: torch.Tensor, router_logits: Optional[torch.Tensor],
                        shared_output: Optional[torch.Tensor] = None, *, out: torch.Tensor,
                        routing: Optional[dict] = None, stream=None):
        """moe_forward_noalloc: the same step with the library's static per-GPU
        workspace and no device allocation (the layer must be initialized and
        `out` given)."""
        xt, lt, ot = _lib.tensor(x), _lib.tensor(router_logits), _lib.tensor(out)
        st = _lib.tensor(shared_output)
        r = self._routing_struct(routing)
        _lib.check(_lib.lib().moe_forward_noalloc(
            self._h, C.byref(xt), C.byref(lt), C.byref(st), C.byref(ot),
            C.byref(r) if r is not None else None, C.c_void_p(_lib.stream_ptr(stream))))
        return out

    def router_logits(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        """x . Wr + Br (f32 [T, E]) from the bound router."""
        T = x.numel() // x.shape[-1]
        if out is None:
            with torch.cuda.stream(torch.cuda.current_stream(x.device) if stream is None
                                   else stream):
                out = torch.empty((T, self.E), dtype=torch.float32, device=x.device)
        ws = self.workspace(T, x.device, stream)
        xt, lt = _lib.tensor(x), _lib.tensor(out)
        _lib.check(_lib.lib().moe_router_logits(self._h, C.byref(xt), C.byref(lt),
                                                C.c_void_p(ws.data_ptr()), ws.numel(),
                                                C.c_void_p(_lib.stream_ptr(stream))))
        return out

    def route(self, router_logits: torch.Tensor, routing: Optional[dict] = None,
              stream=None) -> dict:
        T = router_logits.numel() // router_logits.shape[-1]
        if routing is None:
            with torch.cuda.stream(torch.cuda.current_stream(router_logits.device)
                                   if stream is None else stream):
                routing = self.routing_buffers(T, self.E, self.K, router_logits.device)
        ws = self.workspace(T, router_logits.device, stream)
        lt = _lib.tensor(router_logits)
        r = self._routing_struct(routing)
        _lib.check(_lib.lib().moe_route(self._h, C.byref(lt), C.byref(r),
                                        C.c_void_p(ws.data_ptr()), ws.numel(),
                                        C.c_void_p(_lib.stream_ptr(stream))))
        return routing


def from_config(cfg, **over) -> MoE:
    """A layer declared from a ``synth.MoeConfig``."""
    kw = dict(scoring=cfg.scoring, renormalize=cfg.renormalize, n_group=cfg.n_group,
              topk_group=cfg.topk_group, routed_scaling_factor=cfg.routed_scaling_factor,
              activation=cfg.activation, swiglu_fusion=cfg.layout,
              swiglu_alpha=cfg.swiglu_alpha, swiglu_beta=cfg.swiglu_beta,
              swiglu_limit=cfg.swiglu_limit, gelu_mode=cfg.gelu_mode,
              weigh_inputs=cfg.weigh_inputs)
    kw.update(over)
    return MoE(cfg.E, cfg.H, cfg.I, cfg.K, gate_up_bias=cfg.expert_biases,
               down_bias=cfg.expert_biases, dtype=cfg.w_dtype, **kw)
