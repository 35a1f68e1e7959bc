"""moe_forward captured into a HIP graph (torch.cuda.graph) after moe_prepare.

With a caller workspace and output, a prepared layer's forward is a fixed
sequence of kernel launches on the caller's stream (no allocation, memset or
host synchronisation), so a serving loop can capture it once and replay it.
Each replay runs on new contents of the captured x and logits buffers,
written eagerly between replays, and must equal an eager forward of the same
inputs bit for bit (the kernels are deterministic).  Replays are separated by
eager library work and a device synchronisation."""
import pytest
import torch

from mixture_experts_ffn_03_amd import from_config, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("name", ["qwen3_small", "mixtral_small", "gptoss_small",
                                  "deepseek_small"])
def test_graph_replays_match_eager(name):
    cfg = synth.CONFIGS[name]
    inp = synth.make_inputs(cfg, device=DEV)
    layer = from_config(cfg)
    layer.set_weights_from(inp)
    layer.initialize()
    x, lg = inp["x"].clone(), inp["logits"].clone()
    out = torch.empty_like(x)
    ws = torch.empty(layer.workspace_size(cfg.T), dtype=torch.uint8, device=DEV)
    # warm-up on a side stream, then capture on torch's capture stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(x, lg, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, lg, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i in range(3):
        x.copy_(synth.normal(tuple(x.shape), 1.0, x.dtype, DEV, 9001 + i))
        lg.copy_(synth.normal(tuple(lg.shape), cfg.logit_std, torch.float32, DEV, 9101 + i))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = layer(x.clone(), lg.clone())
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, i, (out.float() - ref.float()).abs().max().item())
