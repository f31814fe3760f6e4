"""GPU parity of the stacked configuration: pre-norm MoE layers with a bf16
residual stream, run chunk by chunk (MoEStack). Each layer is checked
teacher-forced: the oracle gets the GPU's bf16 layer input and the GPU's
fp32 router logits, so a rare near-tie routing flip in an earlier layer
cannot fail a later one; the end-to-end error against the oracle's own
stack is reported (not gated) for the shrunken case."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_stack_layer, make_tokens
from tests.gpu_util import bits, f64_of_bf16, gate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_traced(stack, x):
    """The stack's own sequence of calls, layer by layer, keeping each
    layer's input and the router logits it was routed on."""
    cfg = stack.cfg
    shape = qm.shape_of(cfg)
    trace = []
    for r0 in range(0, x.shape[0], stack.chunk):
        xc = x[r0:r0 + stack.chunk]
        for li_idx, layer in enumerate(stack.layers):
            x_in = xc.clone()
            xn = qm.moe_rmsnorm(xc, layer.li.norm_weight, stack.eps)
            logits, _, _, _ = qm.moe_route(shape, xn, layer.li.w_router, layer.li.router_bias,
                                           layer.li.shared_gate, want_logits=True)
            stack.layer_step(layer, xc)
            trace.append((r0, li_idx, x_in, xn, logits, xc.clone()))
    torch.cuda.synchronize()
    return trace


def check_layer(cfg, li_cpu, x_in, xn, logits, x_out, rows=None):
    """One traced layer against the oracle (all rows, or the listed ones)."""
    xb = bits(x_in)
    # RMSNorm: fp32 math, one bf16 rounding
    ref_n = oracle.rmsnorm(xb if rows is None else xb[rows], li_cpu.norm_weight.numpy(), cfg.rms_eps)
    got_n = f64_of_bf16(xn) if rows is None else f64_of_bf16(xn)[rows]
    assert np.all(np.abs(got_n - ref_n) <= 2.0 ** -8 * np.abs(ref_n) * 1.01 + 1e-30)
    xnb = bits(xn)
    L = logits.cpu().numpy()
    if rows is None:
        ref = oracle.moe_layer(xnb, li_cpu, cfg.k, cfg.G, cfg.quant, logits32=L,
                               residual_bits=xb)["out"]
        got = f64_of_bf16(x_out)
    else:
        ref = oracle.moe_layer_rows(xnb, rows, li_cpu, cfg.k, cfg.G, cfg.quant,
                                    logits32_rows=L[rows], residual_bits=xb)["out"]
        got = f64_of_bf16(x_out)[rows]
    return gate(got, ref, "layer out")


def test_stack_shrunken_per_layer_and_driver():
    """Six stacked layers, three chunks with a ragged last one."""
    cfg = replace(CONFIGS["stack40"], T=300, H=256, E=16, k=4, I=128, shared_I=128, G=32,
                  n_layers=6, chunk=128)
    layers = [make_stack_layer(cfg, l, device=DEV) for l in range(cfg.n_layers)]
    x0 = make_tokens(cfg, device=DEV)
    stack = qm.MoEStack(cfg, layers, DEV, eps=cfg.rms_eps, chunk=cfg.chunk)

    xt = x0.clone()
    trace = run_traced(stack, xt)
    cpu_layers = [li.to("cpu") for li in layers]
    for r0, l, x_in, xn, logits, x_out in trace:
        check_layer(cfg, cpu_layers[l], x_in, xn, logits, x_out)

    # the driver itself gives the same bits as the traced sequence
    xd = stack.forward(x0.clone())
    torch.cuda.synchronize()
    assert torch.equal(xd.view(torch.int16), xt.view(torch.int16))

    # end to end against the oracle's own stack: reported, plus a loose check
    ref = oracle.moe_stack(bits(x0), cpu_layers, cfg.k, cfg.G, cfg.quant, cfg.rms_eps,
                           chunk=cfg.chunk)
    got = f64_of_bf16(xd)
    r = oracle.bf16_to_f64(ref)
    rel = np.linalg.norm(got - r) / np.linalg.norm(r)
    print(f"[stack end-to-end] relL2={rel:.3e} maxabs={np.max(np.abs(got - r)):.3e}")
    assert rel <= 5e-3


def test_stack_full_size_two_layers_sampled():
    """The stacked configuration's own shapes (H=2048, 256 experts, top-8,
    I=512 + shared 512, asymmetric G=32, 16384 rows in two 8192-row chunks)
    for two layers; sampled rows of every (chunk, layer) teacher-forced."""
    cfg = replace(CONFIGS["stack40"], n_layers=2)
    layers = [make_stack_layer(cfg, l, device=DEV) for l in range(cfg.n_layers)]
    x0 = make_tokens(cfg, device=DEV)
    stack = qm.MoEStack(cfg, layers, DEV, eps=cfg.rms_eps, chunk=cfg.chunk)
    trace = run_traced(stack, x0.clone())
    cpu_layers = [li.to("cpu") for li in layers]
    rng = np.random.default_rng(1)
    for r0, l, x_in, xn, logits, x_out in trace:
        n = x_in.shape[0]
        rows = np.concatenate([rng.choice(n, 24, replace=False), [0, n - 1]])
        check_layer(cfg, cpu_layers[l], x_in, xn, logits, x_out, rows=rows)
