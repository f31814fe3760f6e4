"""The fp16 range of the layer's intermediates.

The GPU carries x (converted from bf16), h, y_perm and y_shared as fp16
(binary16: largest finite value 65504). Inside that range the conversion of
x is exact and h, y are rounded once; beyond it every fp16 store saturates
to +-65504 instead of producing an infinity, so the layer output stays
finite (and is then not the layer's value for the tokens concerned; tokens
do not interact, so every other token is unaffected).

These tests scale the activations and the down-projection scales by powers
of two (exact in bf16 and fp16), so that the oracle sees exactly the inputs
the GPU sees."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_layer, make_tokens
from tests.gpu_util import bits, f64_of_bf16, f64_of_f16, gate

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F16_MAX = 65504.0

CASES = {
    "sym": replace(CONFIGS["a3b_pp512"], T=256, H=512, E=16, k=4, I=256, G=64),
    "asym_shared": replace(CONFIGS["skew_shared"], T=256, H=512, E=16, k=4, I=256, G=32,
                           shared_I=256),
}


def scaled(li, xb, a_exp, b_exp, one=None):
    """x times 2^a_exp (bf16 bits), and the down projection's scales (and
    mins) times 2^b_exp (fp16 bits), exactly; with one = (e, c), routed
    expert e's down scales (and mins) by a further 2^c. Returns (x bits,
    CPU layer)."""
    x = oracle.bf16_to_f64(xb) * 2.0 ** a_exp
    xs = oracle.round_to_bf16(x)
    assert np.array_equal(oracle.bf16_to_f64(xs), x)
    cpu = li.to("cpu")
    for name in ("w2_scale", "w2_min", "s2_scale", "s2_min"):
        t = getattr(cpu, name, None)
        if t is None:
            continue
        f = np.full(t.shape[0] if name.startswith("w") else 1, 2.0 ** b_exp)
        if one is not None and name.startswith("w"):
            f[one[0]] *= 2.0 ** one[1]
        v = t.numpy().astype(np.float64) * f.reshape((-1,) + (1,) * (t.dim() - 1))
        v16 = v.astype(np.float16)
        assert np.array_equal(v16.astype(np.float64), v) and np.all(np.isfinite(v16))
        setattr(cpu, name, torch.from_numpy(v16))
    return xs, cpu


def oracle_layer(xs, cpu, cfg, L=None):
    return oracle.moe_layer(xs, cpu, cfg.k, cfg.G, cfg.quant, logits32=L)


def peak(r):
    hm = max(np.abs(r["h_perm"]).max(), np.abs(r["h_shared"]).max() if r["h_shared"] is not None else 0)
    ym = max(np.abs(r["y_perm"]).max(), np.abs(r["y_shared"]).max() if r["y_shared"] is not None else 0)
    return hm, ym


def find_scales(li, xb, cfg, lo=16384.0, hi=0.92 * F16_MAX):
    """Powers of two for x and for the down scales that put the largest |h|
    and then the largest |y| in [lo, hi] on the oracle."""
    a = 0
    for _ in range(40):
        hm, _ = peak(oracle_layer(*scaled(li, xb, a, 0), cfg))
        if hm > hi:
            a -= 1
        elif hm < lo:
            a += 1
        else:
            break
    b = 0
    for _ in range(40):
        hm, ym = peak(oracle_layer(*scaled(li, xb, a, b), cfg))
        if ym > hi:
            b -= 1
        elif ym < lo:
            b += 1
        else:
            break
    return a, b


def run_gpu(cfg, li, xs, cpu):
    """The entry points in turn on the scaled inputs (the device copy of
    the layer takes the CPU layer's scaled down scales)."""
    shape = qm.shape_of(cfg)
    dl = cpu.to(DEV)
    x = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).to(DEV)
    logits, ids, tw, sw = qm.moe_route(shape, x, dl.w_router, dl.router_bias, dl.shared_gate,
                                       want_logits=True)
    counts, offsets, sp, inv = qm.moe_permute(shape, ids)
    y_perm, y_sh = qm.moe_expert_ffn(shape, x, qm.Experts(dl), counts, offsets, sp)
    out = qm.moe_combine(shape, y_perm, inv, tw, y_sh, sw)
    out2 = qm.MoELayer(cfg, dl, DEV, cfg.T).forward(x)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    return logits.cpu().numpy(), y_perm, y_sh, out


@pytest.mark.parametrize("case", sorted(CASES))
def test_large_magnitudes_in_range(case):
    """h and y_perm (and the shared expert's) up to between 2^14 and 92 % of
    the fp16 limit: every intermediate and the output within the gates."""
    cfg = CASES[case]
    li = make_layer(cfg, device="cpu")
    xb = bits(make_tokens(cfg, device="cpu"))
    a, b = find_scales(li, xb, cfg)
    xs, cpu = scaled(li, xb, a, b)
    L, y_perm, y_sh, out = run_gpu(cfg, li, xs, cpu)
    ref = oracle_layer(xs, cpu, cfg, L)
    hm, ym = peak(ref)
    print(f"[range] {case}: x * 2^{a}, down scales * 2^{b}: max |h| {hm:.0f}, max |y| {ym:.0f}, "
          f"max |x| {np.abs(oracle.bf16_to_f64(xs)).max():.0f}")
    assert 16384 <= max(hm, ym) <= 0.92 * F16_MAX and ym >= 16384
    gate(f64_of_f16(y_perm), ref["y_perm"], "y_perm (large)", fmt="fp16")
    if cfg.shared_I:
        gate(f64_of_f16(y_sh), ref["y_shared"], "y_shared (large)", fmt="fp16")
    gate(f64_of_bf16(out), ref["out"], "out (large)")


@pytest.mark.parametrize("case", sorted(CASES))
def test_beyond_range_saturates(case):
    """Past the fp16 range: a few activations beyond 65504 (their fp16 copy
    saturates, and so do their h and y), and one expert whose outputs exceed
    the range. The output is finite everywhere, and every token whose x, h
    and y all stay inside the range matches the oracle."""
    cfg = CASES[case]
    li = make_layer(cfg, device="cpu")
    xb = bits(make_tokens(cfg, device="cpu"))
    a, b = find_scales(li, xb, cfg)
    # (1) activations beyond the range on two tokens
    xs, cpu = scaled(li, xb, a, b)
    xs = xs.copy()
    big = {5: [(0, 1.0e5), (1, -2.5e5), (7, 7.0e4)], 9: [(100, -3.0e6)]}
    for t, items in big.items():
        for c, v in items:
            xs[t, c] = oracle.round_to_bf16(np.array([v]))[0]
    # (2) the same batch with one routed expert's down scales 2^6 larger:
    # the outputs of that expert's rows beyond the range
    e_hot = 3
    for tag, (xin, cpu_in) in {"x beyond": (xs, cpu),
                               "y beyond": scaled(li, xb, a, b, one=(e_hot, 6))}.items():
        L, y_perm, y_sh, out = run_gpu(cfg, li, xin, cpu_in)
        got = f64_of_bf16(out)
        assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
        assert np.all(np.isfinite(f64_of_f16(y_perm))), f"{tag}: non-finite y_perm"
        ref = oracle_layer(xin, cpu_in, cfg, L)
        # tokens that leave the fp16 range anywhere: x, h or y of any of its pairs
        xin_f = oracle.bf16_to_f64(xin)
        bad = np.abs(xin_f).max(axis=1) > F16_MAX
        P = cfg.T * cfg.k
        pair_bad = (np.abs(ref["h_perm"]).max(axis=1) > F16_MAX) | \
                   (np.abs(ref["y_perm"]).max(axis=1) > F16_MAX)
        tok_of_row = ref["sorted_pairs"] // cfg.k
        bad[np.unique(tok_of_row[pair_bad])] = True
        if ref["h_shared"] is not None:
            bad |= (np.abs(ref["h_shared"]).max(axis=1) > F16_MAX) | \
                   (np.abs(ref["y_shared"]).max(axis=1) > F16_MAX)
        n_bad = int(bad.sum())
        print(f"[range] {case} {tag}: {n_bad} of {cfg.T} tokens leave the fp16 range; "
              f"max |y_perm| on the GPU {np.abs(f64_of_f16(y_perm)).max():.0f}")
        assert 0 < n_bad < cfg.T // 2, n_bad
        assert P == len(tok_of_row)
        gate(got[~bad], ref["out"][~bad], f"out, tokens inside the range ({tag})")
