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


def progress(capfd, msg):
    """A progress line straight to the terminal, past pytest's output
    capture: a test that runs for minutes keeps showing that it is alive."""
    with capfd.disabled():
        print(msg, flush=True)


@pytest.mark.timeout(1200)
def test_stack40_full_depth(capfd):
    """The stacked configuration at full size and depth: 40 layers (H=2048,
    256 experts, top-8, I=512 + shared 512, asymmetric G=32, Zipf-biased
    routing), 16,384 rows in two chunks of 8192, chunk-major on the GPU.

    Every (chunk, layer) is checked on all its rows, teacher-forced (the
    oracle takes the GPU's bf16 layer input, its normed input and its fp32
    logits): RMSNorm within one bf16 ulp; the layer's MoE part alone (the
    same layer call without the residual, bf16) and the layer output
    x + MoE(RMSNorm(x)) through the floating-point gates. End to end, the
    GPU stack is compared with the oracle's own stack, which routes on its
    own logits at every layer: relative L2, max-abs and the number of
    (token, slot) selections that differ are reported (a near-tie in one
    layer legitimately changes a token's later path), with loose bounds: none
    may differ in the first layer, whose input is the same on both sides."""
    cfg = CONFIGS["stack40"]
    shape = qm.shape_of(cfg)
    nl, ch = cfg.n_layers, cfg.chunk
    layers = [make_stack_layer(cfg, l, device=DEV) for l in range(nl)]
    x0 = make_tokens(cfg, device=DEV)
    stack = qm.MoEStack(cfg, layers, DEV, eps=cfg.rms_eps, chunk=ch)
    moe_only = torch.empty((ch, cfg.H), dtype=torch.bfloat16, device=DEV)

    # GPU, chunk-major; each layer's input, normed input, logits, ids and
    # MoE-only output kept on the host
    x = x0.clone()
    rec = {}
    n_chunks = cfg.T // ch
    for ci in range(n_chunks):
        xc = x[ci * ch:(ci + 1) * ch]
        for l, layer in enumerate(stack.layers):
            x_in = bits(xc)
            xn = qm.moe_rmsnorm(xc, layer.li.norm_weight, stack.eps)
            logits, ids, _, _ = qm.moe_route(shape, xn, layer.li.w_router, layer.li.router_bias,
                                             layer.li.shared_gate, want_logits=True)
            layer.forward(xn, out=moe_only)
            stack.layer_step(layer, xc)
            rec[(ci, l)] = (x_in, bits(xn), logits.cpu().numpy(), ids.cpu().numpy(),
                            bits(moe_only))
        progress(capfd, f"[stack40] GPU chunk {ci} done")
    torch.cuda.synchronize()
    x_final = bits(x)
    # the stack's own driver gives the same bits as the recorded sequence
    xd = stack.forward(x0.clone())
    torch.cuda.synchronize()
    assert np.array_equal(bits(xd), x_final)
    del xd

    # oracle, layer by layer: teacher-forced checks of both chunks, then one
    # step of the oracle's own chain over all rows (rows do not interact)
    xo = bits(x0)
    slot_flips = set_flips = 0
    flips_by_layer = []
    worst_moe = worst_out = 0.0
    for l in range(nl):
        cpu = layers[l].to("cpu")
        cache = {}
        for ci in range(n_chunks):
            x_in, xn, L, ids, moe = rec[(ci, l)]
            x_out = rec[(ci, l + 1)][0] if l + 1 < nl else x_final[ci * ch:(ci + 1) * ch]
            ref_n = oracle.rmsnorm(x_in, cpu.norm_weight.numpy(), cfg.rms_eps)
            got_n = oracle.bf16_to_f64(xn)
            assert np.all(np.abs(got_n - ref_n) <= 2.0 ** -8 * np.abs(ref_n) * 1.01 + 1e-30), (l, ci)
            r = oracle.moe_layer(xn, cpu, cfg.k, cfg.G, cfg.quant, logits32=L, cache=cache)
            assert np.array_equal(ids, r["ids"]), (l, ci)
            _, m = gate(oracle.bf16_to_f64(moe), r["out"], f"layer {l} chunk {ci} MoE part")
            _, o = gate(oracle.bf16_to_f64(x_out), r["out"] + oracle.bf16_to_f64(x_in),
                        f"layer {l} chunk {ci} output")
            worst_moe, worst_out = max(worst_moe, m), max(worst_out, o)
            del r
        xo, r = oracle.stack_layer(xo, cpu, cfg.k, cfg.G, cfg.quant, cfg.rms_eps, cache=cache)
        gpu_ids = np.concatenate([rec[(ci, l)][3] for ci in range(n_chunks)])
        f = int(np.count_nonzero(gpu_ids != r["ids"]))
        flips_by_layer.append(f)
        slot_flips += f
        set_flips += int(np.count_nonzero(np.sort(gpu_ids, axis=1) != np.sort(r["ids"], axis=1)))
        del r, cache, cpu
        for ci in range(n_chunks):
            rec[(ci, l)] = None
        progress(capfd, f"[stack40] layer {l} checked; selections differing so far: "
                        f"{slot_flips} (token, slot), {set_flips} by set")

    got = oracle.bf16_to_f64(x_final)
    ref = oracle.bf16_to_f64(xo)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    mx = np.max(np.abs(got - ref)) / rms
    n_sel = cfg.T * cfg.k * nl
    print(f"[stack40 end-to-end] relL2={rel:.3e} maxabs/rms={mx:.3e}; per-layer worst "
          f"max-abs beyond rounding/rms: MoE part {worst_moe:.3e}, output {worst_out:.3e}; "
          f"(token, slot) selections differing from the oracle's own routing: {slot_flips} of "
          f"{n_sel} ({set_flips} by set)")
    print(f"[stack40] (token, slot) selections differing per layer: {flips_by_layer}")
    # Both chains start from the same bits: the first layer routes identically.
    # Later layers drift apart through bf16 rounding decisions of the residual
    # stream (the GPU's fp16 intermediates move its pre-rounding sums by about
    # 1e-4 of x, so a few per cent of the elements round to the neighbouring
    # bf16 number in each layer) and the near-tie routing flips they cause; the
    # bounds below are far above that drift (measured: relL2 1.5e-2, 1.6 % of
    # the selections) and far below what one wrong layer would cause.
    assert flips_by_layer[0] == 0
    assert rel <= 5e-2
    assert slot_flips <= 5e-2 * n_sel
