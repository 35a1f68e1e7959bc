"""The allocation-free forward (moe_forward_noalloc, static per-GPU scratch)
against moe_forward with a caller workspace, through the C ABI: the same
kernels on the same inputs, so outputs and routing must agree bit for bit
(a stronger bar than the oracle's tolerance, which moe_forward meets in the
parity tests).  Two calls in a row, the second with fewer tokens, so the
second runs on a scratch still holding the first call's contents; then a
different layer on the same scratch."""
import pytest
import torch

from mixture_experts_ffn_03_amd import _lib, from_config, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_both(layer, inp, T):
    x, lg = inp["x"][:T].contiguous(), inp["logits"][:T].contiguous()
    ref_r = layer.routing_buffers(T, layer.E, layer.K, DEV)
    ref = layer(x, lg, routing=ref_r)
    out = torch.full_like(x, float("nan"))
    r = layer.routing_buffers(T, layer.E, layer.K, DEV)
    layer.forward_noalloc(x, lg, out=out, routing=r)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), (T, (out.float() - ref.float()).abs().max().item())
    for k in ref_r:
        assert torch.equal(r[k], ref_r[k]), k


@pytest.mark.parametrize("name,T1,T2", [("qwen3_small", 32, 5), ("mixtral_small", 300, 41),
                                        ("gptoss_small", 300, 17)])
def test_noalloc_matches_forward(name, T1, T2):
    cfg = synth.CONFIGS[name].replace(T=T1)
    inp = synth.make_inputs(cfg, device=DEV)
    layer = from_config(cfg)
    layer.set_weights_from(inp)
    layer.initialize()
    assert layer.workspace_size(T1) <= _lib.NOALLOC_SCRATCH_BYTES
    _run_both(layer, inp, T1)
    _run_both(layer, inp, T2)


def test_noalloc_errors():
    cfg = synth.MIXTRAL_SMALL.replace(T=64)
    inp = synth.make_inputs(cfg, device=DEV)
    layer = from_config(cfg)
    layer.set_weights_from(inp)
    out = torch.empty_like(inp["x"])
    with pytest.raises(_lib.MoeError) as ei:          # not prepared: preparing allocates
        layer.forward_noalloc(inp["x"], inp["logits"], out=out)
    assert ei.value.status == 1
    layer.initialize()
    big = next(T for T in (1 << k for k in range(6, 20))
               if layer.workspace_size(T) > _lib.NOALLOC_SCRATCH_BYTES)
    xb = torch.zeros((big, cfg.H), dtype=torch.bfloat16, device=DEV)
    lb = torch.zeros((big, cfg.E), dtype=torch.float32, device=DEV)
    ob = torch.empty_like(xb)
    with pytest.raises(_lib.MoeError) as ei:          # beyond the static scratch
        layer.forward_noalloc(xb, lb, out=ob)
    assert ei.value.status == 6
    layer.forward_noalloc(inp["x"], inp["logits"], out=out)
    ref = layer(inp["x"], inp["logits"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
