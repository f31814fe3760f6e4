"""GPU parity of the integer route (8-bit activations x symmetric 4-bit
experts) against the oracle's integer route on the same seeded inputs: the
activation codes and scales bit for bit (the quantization decisions are
taken in fp32 on both sides), the expert outputs and the layer output
within the floating-point gates of tests/gpu_util.py. The int8 h is
teacher-forced: its codes are decided on the GPU's fp16 h (itself gated
against the oracle's), as the top-k choice is taken on the GPU's logits,
because an h computed in another summation order can round to a different
fp16 value and move a code by one step. The forcing is bounded, not
assumed: the codes of the GPU's h and of the oracle's own h are compared,
every difference must be one step and at most a 5e-3 fraction may differ.
Without the forcing the relative L2 gate still applies (its max-abs is
printed). The route's own distance from the exact layer (the
8-bit rounding of x and h) is checked against the floating-point oracle
with its own, looser bound."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_layer, make_tokens
from synth.gen import f32_to_bf16_bits, randomize_packed
from tests.gpu_util import bits, f64_of_bf16, f64_of_f16, gate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# Distance of the integer route from the exact layer: the activations'
# 8-bit rounding error is about max/(127 sqrt 12) of each row's RMS (1 % for
# Gaussian x, a few % for the heavier-tailed h); the oracle measures 1.5-2.5 %
# relative L2 on these layers.
ROUTE_REL_L2 = 5e-2

# The GPU's fp16 h comes from fp32 sums in another order than the oracle's
# float64 ones (and from the offset-float group sums, about 1e-4 relative),
# so about one h value in six rounds to the neighbouring fp16 number. One
# fp16 ulp of h moves its code by 127 * 2^-11 * |h| / max|h| < 0.07 of a
# step, so a code changes only where the value sat within that distance of
# a rounding boundary, and then by one step: a few codes in a thousand at
# most (1e-3 measured on these layers). Bound on the fraction of h codes that
# differ between the GPU's h and the oracle's own:
H_CODE_FRAC = 5e-3

_CACHE = {}


def setup(cfg, rows=None, random_bytes=False):
    key = (cfg, random_bytes)
    if key not in _CACHE:
        _CACHE.clear()
        li = make_layer(cfg, device=DEV)
        if random_bytes:
            li = randomize_packed(li, seed=7)
        _CACHE[key] = (li, li.to("cpu"))
    li, cpu = _CACHE[key]
    x = make_tokens(cfg, device=DEV, rows=rows)
    return li, cpu, x


def i8_check(cfg, li, cpu, x, route_err=True):
    shape = qm.shape_of(cfg)
    logits, ids, tw, _ = qm.moe_route(shape, x, li.w_router, li.router_bias, None, want_logits=True)
    counts, offsets, sp, inv = qm.moe_permute(shape, ids)
    ex = qm.Experts(li)
    y_perm, h = qm.moe_expert_ffn_i8(shape, x, ex, counts, offsets, sp, want_h=True)
    out = qm.moe_combine(shape, y_perm, inv, tw)
    out2 = qm.moe_layer_forward_i8(shape, x, li.w_router, li.router_bias, ex)
    torch.cuda.synchronize()
    L = logits.cpu().numpy()
    own = oracle.moe_layer_i8(bits(x), cpu, cfg.k, cfg.G, logits32=L)
    assert np.array_equal(ids.cpu().numpy(), own["ids"])
    assert np.array_equal(sp.cpu().numpy(), own["sorted_pairs"])
    h_gpu = f64_of_f16(h)
    gate(h_gpu, own["h16"], "h (int8 route)", fmt="fp16")
    check_h_codes(h_gpu, own)
    ref = oracle.moe_layer_i8(bits(x), cpu, cfg.k, cfg.G, logits32=L, h16_forced=h_gpu)
    gate(f64_of_f16(y_perm), ref["y_perm"], "y_perm (int8 route, h forced)", fmt="fp16")
    gate(f64_of_bf16(out), ref["out"], "out (int8 route, h forced)")
    gate(f64_of_bf16(out), own["out"], "out (int8 route, relL2 only)", mx=np.inf)
    # the layer call gives the same bits as the entry points in turn
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    if route_err:
        fp = oracle.moe_layer(bits(x), cpu, cfg.k, cfg.G, cfg.quant, logits32=L)
        rel = np.linalg.norm(f64_of_bf16(out) - fp["out"]) / np.linalg.norm(fp["out"])
        print(f"[route] int8 route vs exact layer: relL2 {rel:.3e} (<= {ROUTE_REL_L2:.0e})")
        assert rel <= ROUTE_REL_L2
    return out


def check_h_codes(h_gpu, own):
    """The codes of the GPU's h (quantized as the GPU does, which
    test_quantize_rows_bit_exact pins bit for bit) against the codes of the
    oracle's own h: every difference is one step, and few differ."""
    q_gpu, s_gpu = oracle.quantize_rows_i8(np.asarray(h_gpu, np.float64).astype(np.float32))
    dq = np.abs(q_gpu.astype(np.int32) - own["hq"].astype(np.int32))
    n_codes = int(np.count_nonzero(dq))
    n_h = int(np.count_nonzero(np.asarray(h_gpu) != own["h16"]))
    n_rows = int(np.count_nonzero(s_gpu.view(np.uint32) != own["sh"].view(np.uint32)))
    print(f"[h codes] {n_codes} of {dq.size} codes differ (max step {int(dq.max()) if dq.size else 0}); "
          f"{n_h} fp16 h values differ; {n_rows} of {len(s_gpu)} row scales differ")
    if dq.size:
        assert dq.max() <= 1, "an h code differs by more than one step"
    assert n_codes <= H_CODE_FRAC * dq.size, f"{n_codes} h codes differ (> {H_CODE_FRAC:.0e})"


def test_quantize_rows_bit_exact():
    g = torch.Generator().manual_seed(21)
    rows = []
    for scale in (1.0, 1e-3, 3e4, 1e-30, 1e30):
        rows.append(torch.randn(24, 520, generator=g) * scale)
    x = torch.cat(rows)
    x[0] = 0.0                       # all zero
    x[1] = 0.0
    x[1, 17] = -3.0                  # a single nonzero
    x[2] = 0.0
    x[2, :8] = torch.tensor([2.0, 1.0, 0.5, -0.25, -2.0, 1.5, 0.75, 0.0])  # r = 63.5: 1 * r ties
    x[3] = 1e-36                     # below the 2^-100 floor: zeros
    xb = f32_to_bf16_bits(x.numpy())
    xd = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    q, s = qm.moe_quantize_rows_i8(xd)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows_i8(oracle.bf16_to_f64(xb).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert q_ref[2, :8].tolist() == [127, 64, 32, -16, -127, 95, 48, 0]


@pytest.mark.parametrize("name,over", [
    ("tiny", dict(G=128)),
    ("tiny", dict(G=128, T=77, E=5, k=1)),       # ragged rows, k = 1, odd expert count
    ("tiny", dict(G=128, T=50, E=4, k=4)),       # k = E
    ("a3b_pp512", {}),
    ("a3b_pp512", dict(T=300, H=1024, I=384, E=16)),  # three K stages in the down GEMM
])
def test_i8_layer_parity(name, over):
    cfg = replace(CONFIGS[name], **over)
    li, cpu, x = setup(cfg)
    i8_check(cfg, li, cpu, x)


def test_i8_random_bytes_all_nibbles():
    cfg = replace(CONFIGS["tiny"], G=128)
    li, cpu, x = setup(cfg, random_bytes=True)
    i8_check(cfg, li, cpu, x, route_err=False)


@pytest.mark.parametrize("T", [1, 5, 16])
def test_i8_small_T(T):
    cfg = replace(CONFIGS["a3b_pp8192"], T=T)
    li, cpu, x = setup(CONFIGS["a3b_pp8192"], rows=T)
    i8_check(cfg, li, cpu, x)


def test_i8_skewed_routing_empty_experts():
    """A router bias that sends most pairs to a few experts: long row runs
    of one expert (several 128-row tiles) next to empty experts."""
    cfg = replace(CONFIGS["a3b_pp512"], T=700, H=512, E=32, I=256, zipf_bias=True)
    li, cpu, x = setup(cfg)
    li.router_bias = li.router_bias * 4
    cpu.router_bias = cpu.router_bias * 4
    try:
        out = i8_check(cfg, li, cpu, x)
    finally:
        _CACHE.clear()  # the cached layer's bias was changed
    assert out.shape == (cfg.T, cfg.H)


def test_i8_full_size_a3b_pp8192():
    """The bench workload at full size through the integer route: every row
    of h, y_perm and out against the oracle's integer route (teacher-forced
    on the GPU logits), the h codes bounded, the layer call bit-equal to the
    entry points, and the route's distance from the exact layer."""
    cfg = CONFIGS["a3b_pp8192"]
    li, cpu, x = setup(cfg)
    i8_check(cfg, li, cpu, x)


def test_i8_determinism_bitwise():
    cfg = CONFIGS["a3b_pp512"]
    li, cpu, x = setup(cfg)
    shape = qm.shape_of(cfg)
    ex = qm.Experts(li)
    a = qm.moe_layer_forward_i8(shape, x, li.w_router, li.router_bias, ex).clone()
    b = qm.moe_layer_forward_i8(shape, x, li.w_router, li.router_bias, ex).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
