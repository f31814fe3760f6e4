"""HIP graph capture of the fused layer call: the library only enqueues
kernels on the caller's stream (no allocation, no memset, no host sync), so
moe_layer_forward can be captured once and replayed. Every replay must give
the bits of the eager call, also after the input buffer's contents change
between replays (with eager work and synchronizations in between)."""
from dataclasses import replace

import pytest
import torch

import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_layer, make_stack_layer, make_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits16(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("name,T", [("a3b_pp8192", 4), ("skew_shared", 16), ("tiny", 37)])
def test_layer_graph_replay(name, T):
    cfg = replace(CONFIGS[name], T=T)
    li = make_layer(cfg, device=DEV)
    x = make_tokens(cfg, device=DEV)
    x2 = make_tokens(replace(cfg, seed=cfg.seed + 1), device=DEV)
    layer = qm.MoELayer(cfg, li, DEV, T)
    ref1 = layer.forward(x).clone()
    ref2 = layer.forward(x2).clone()
    torch.cuda.synchronize()
    assert not torch.equal(bits16(ref1), bits16(ref2))

    xin = x.clone()
    out = torch.empty_like(ref1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(xin, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(xin, out=out)
    torch.cuda.synchronize()

    for i in range(4):
        src, ref = (x, ref1) if i % 2 == 0 else (x2, ref2)
        xin.copy_(src)
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits16(out), bits16(ref)), f"replay {i} differs from the eager call"


def test_stack_graph_replay():
    """Eight layers of the stack40 shape (256 experts, asymmetric G = 32,
    shared expert, RMSNorm + residual) on 16 tokens, captured once with
    MoEStack.capture: every replay, on fresh input contents with eager work
    in between, gives the bits of the eager stack."""
    cfg = replace(CONFIGS["stack40"], T=16, n_layers=8)
    layers = [make_stack_layer(cfg, l, device=DEV) for l in range(cfg.n_layers)]
    stack = qm.MoEStack(cfg, layers, DEV, eps=cfg.rms_eps, chunk=16)
    x = make_tokens(cfg, device=DEV, rows=16)
    x2 = make_tokens(replace(cfg, seed=cfg.seed + 1), device=DEV, rows=16)
    ref1 = stack.forward(x.clone())
    ref2 = stack.forward(x2.clone())
    torch.cuda.synchronize()
    assert not torch.equal(bits16(ref1), bits16(ref2))
    buf = x.clone()
    graph = stack.capture(buf)
    for i in range(4):
        src, ref = (x, ref1) if i % 2 == 0 else (x2, ref2)
        buf.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits16(buf), bits16(ref)), f"replay {i} differs from the eager stack"
        # eager work on the same layers between replays
        stack.forward(x2.clone())
        torch.cuda.synchronize()
