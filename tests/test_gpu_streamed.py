"""GPU checks of moe_layer_forward_streamed: cold experts in pinned host
memory copied over PCIe into a staging buffer chunk by chunk, hot experts on
the device. Where moe_layer_forward runs the same tiled kernels (above 16
tokens, and below the wide-tile kernel's average of 256 rows per expert)
the output must equal its output bit for bit; elsewhere (at most 16 tokens:
the weight-streaming kernels; the a3b_pp8192 batch: the wide-tile kernels)
both are gated against the oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_layer, make_tokens
from tests.gpu_util import bits, f64_of_bf16, gate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(cfg, hot, stage_experts, T=None, copy_stream=None):
    li = make_layer(cfg, device=DEV)
    x = make_tokens(cfg, device=DEV, rows=T)
    shape = qm.shape_of(cfg)
    ex = qm.StreamedExperts(li, hot, DEV)
    stage = torch.empty(qm.moe_stream_stage_bytes(shape, stage_experts), dtype=torch.uint8, device=DEV)
    out = qm.moe_layer_forward_streamed(shape, x, li.w_router, li.router_bias, ex, stage,
                                        copy_stream=copy_stream)
    ref = qm.MoELayer(cfg, li, DEV, x.shape[0]).forward(x)
    torch.cuda.synchronize()
    return li, x, out, ref


@pytest.mark.parametrize("name,hot,stage_experts", [
    ("tiny", [], 2),                 # every expert cold, one expert per chunk
    ("tiny", [0, 3, 5], 4),          # hot set + two cold chunks
    ("tiny", list(range(8)), 2),     # every expert hot
    ("a3b_pp512", list(range(0, 128, 4)), 16),
])
def test_streamed_equals_resident_bitwise(name, hot, stage_experts):
    cfg = CONFIGS[name]
    _, _, out, ref = run(cfg, hot, stage_experts)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_streamed_full_size_a3b_pp8192():
    """The bench batch with 32 hot experts: every output row against the
    oracle (teacher-forced on the GPU logits), as is the resident layer's."""
    cfg = CONFIGS["a3b_pp8192"]
    li, x, out, res = run(cfg, list(range(32)), 24)
    shape = qm.shape_of(cfg)
    logits, _, _, _ = qm.moe_route(shape, x, li.w_router, li.router_bias, None, want_logits=True)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(bits(x), li.to("cpu"), cfg.k, cfg.G, cfg.quant,
                           logits32=logits.cpu().numpy())
    gate(f64_of_bf16(out), ref["out"], "out (streamed, T=8192)")
    gate(f64_of_bf16(res), ref["out"], "out (resident, T=8192)")


@pytest.mark.parametrize("T", [1, 16])
def test_streamed_small_T_against_oracle(T):
    cfg = CONFIGS["a3b_pp512"]
    li, x, out, _ = run(cfg, [1, 2, 3], 8, T=T)
    shape = qm.shape_of(cfg)
    logits, _, _, _ = qm.moe_route(shape, x, li.w_router, li.router_bias, None, want_logits=True)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(bits(x), li.to("cpu"), cfg.k, cfg.G, cfg.quant,
                           logits32=logits.cpu().numpy())
    gate(f64_of_bf16(out), ref["out"], f"out (streamed, T={T})")


@pytest.mark.parametrize("name,hot,stage_experts", [
    ("tiny", [], 2),
    ("a3b_pp512", list(range(0, 128, 4)), 16),
])
def test_streamed_copy_stream_bitwise(name, hot, stage_experts):
    """Copies on a second stream, three calls back to back into the same
    staging buffer (a later call's first copies must wait for the earlier
    call's last kernels), each bit-identical to the resident layer."""
    cfg = CONFIGS[name]
    cs = torch.cuda.Stream(device=DEV)
    li = make_layer(cfg, device=DEV)
    shape = qm.shape_of(cfg)
    ex = qm.StreamedExperts(li, hot, DEV)
    stage = torch.empty(qm.moe_stream_stage_bytes(shape, stage_experts), dtype=torch.uint8, device=DEV)
    outs, refs = [], []
    for i in range(3):
        x = make_tokens(replace(cfg, seed=cfg.seed + i), device=DEV)
        outs.append(qm.moe_layer_forward_streamed(shape, x, li.w_router, li.router_bias, ex, stage,
                                                  copy_stream=cs))
        refs.append(x)
    torch.cuda.synchronize()
    layer = qm.MoELayer(cfg, li, DEV, refs[0].shape[0])
    for i, (out, x) in enumerate(zip(outs, refs)):
        ref = layer.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {i}"
