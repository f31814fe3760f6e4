"""GPU parity of mixed-width layers (4-bit experts beside 3- and 2-bit ones,
moe_expert_ffn_mixed / moe_layer_forward_mixed) against the oracle on the
same seeded inputs: the grouping bit for bit, the expert outputs and the
layer output within the floating-point gates of tests/gpu_util.py, routing
teacher-forced on the GPU logits."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_tokens
from synth.mixed import make_mixed_layer
from tests.gpu_util import bits, f64_of_bf16, f64_of_f16, gate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def width_map(E, pattern, seed=0):
    """Per-expert widths: `pattern` repeated over a seeded permutation of the experts."""
    perm = np.random.default_rng(seed).permutation(E)
    out = [4] * E
    for i, e in enumerate(perm):
        out[e] = pattern[i % len(pattern)]
    return out


def mixed_check(cfg, widths, x=None, randomize=False):
    ml = make_mixed_layer(cfg, widths, device=DEV)
    if randomize:
        g = torch.Generator(device=DEV).manual_seed(3)
        for b, (w13, s13, w2, s2) in ml.tiers.items():
            for t in (w13, w2):
                t.copy_(torch.randint(0, 256, t.shape, generator=g, device=DEV, dtype=torch.int32)
                        .to(torch.uint8))
            for t in (s13, s2):
                t.copy_((1e-3 + 2e-2 * torch.rand(t.shape, generator=g, device=DEV)).to(torch.float16))
    if x is None:
        x = make_tokens(cfg, device=DEV)
    shape = qm.shape_of(cfg)
    ex = qm.MixedExperts(ml, DEV)
    logits, ids, tw, _ = qm.moe_route(shape, x, ml.w_router, ml.router_bias, None, want_logits=True)
    counts, offsets, sp, inv = qm.moe_permute(shape, ids)
    y_perm = qm.moe_expert_ffn_mixed(shape, x, ex, counts, offsets, sp)
    out = qm.moe_combine(shape, y_perm, inv, tw)
    out2 = qm.moe_layer_forward_mixed(shape, x, ml.w_router, ml.router_bias, ex)
    torch.cuda.synchronize()
    ref = oracle.moe_layer_mixed(bits(x), ml.to("cpu"), cfg.k, cfg.G, logits32=logits.cpu().numpy())
    assert np.array_equal(sp.cpu().numpy(), ref["sorted_pairs"])
    gate(f64_of_f16(y_perm), ref["y_perm"], "y_perm (mixed widths)", fmt="fp16")
    gate(f64_of_bf16(out), ref["out"], "out (mixed widths)")
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    return ref


@pytest.mark.parametrize("G", [32, 64, 128])
def test_mixed_tiny_all_widths(G):
    cfg = replace(CONFIGS["tiny"], G=G)
    mixed_check(cfg, width_map(cfg.E, [4, 3, 2]))


@pytest.mark.parametrize("only", [3, 2])
def test_single_lower_width(only):
    cfg = replace(CONFIGS["a3b_pp512"], T=200, E=16, I=256)
    mixed_check(cfg, [only] * cfg.E)


def test_mixed_random_bytes_all_codes():
    cfg = replace(CONFIGS["tiny"], T=77, E=6, k=2, G=64)
    mixed_check(cfg, [4, 3, 2, 2, 3, 4], randomize=True)


def test_mixed_a3b_shape_hot_and_cold():
    """The a3b layer at T=512: a quarter of the experts at 4 bits, the rest
    at 3 and 2 bits (several K stages, every expert active)."""
    cfg = CONFIGS["a3b_pp512"]
    mixed_check(cfg, width_map(cfg.E, [4, 3, 3, 2, 2, 2, 3, 2]))


def test_mixed_full_size_a3b_pp8192():
    """The bench workload at full size with mixed widths, whole-layer oracle."""
    cfg = CONFIGS["a3b_pp8192"]
    mixed_check(cfg, width_map(cfg.E, [4, 3, 2, 3]))


def test_mixed_small_T_and_empty_tier():
    # 3 tokens of a 16-expert layer: most experts (and maybe a whole width) get no rows
    cfg = replace(CONFIGS["a3b_pp512"], T=3, E=16, I=256)
    mixed_check(cfg, width_map(cfg.E, [2, 3, 4, 2]))
