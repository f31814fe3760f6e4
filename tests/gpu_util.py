"""Helpers shared by the GPU parity tests: input setup on the device, copies
back to numpy, and the floating-point gates."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Floating-point parity gate: relative L2 error <= 5e-3, and max-abs error
# <= 2e-2 x RMS of the reference on top of each element's own rounding to the
# result's storage format (half an ulp of bf16 for the layer output, of fp16
# for the expert outputs). The format term is there because a correctly
# rounded bf16 value already differs from the exact one by up to 2^-8 of its
# magnitude, about 2% of the RMS for the largest (5-6 RMS) elements of a
# large output; the stated 2% is a budget for the computation itself.
REL_L2 = 5e-3
MAX_ABS_RMS = 2e-2
U = 2.0 ** -24  # unit roundoff of fp32


def half_ulp(ref: np.ndarray, fmt: str) -> np.ndarray:
    """Half the spacing of `fmt` numbers at each |ref| (the largest error of
    a correctly rounded value)."""
    sig, tiny = {"bf16": (8, -133), "fp16": (11, -24), None: (None, None)}[fmt]
    if sig is None:
        return np.zeros_like(ref)
    r = np.abs(np.asarray(ref, np.float64))
    _, e = np.frexp(np.where(r > 0, r, 1.0))     # r = m 2^e, 0.5 <= m < 1
    return np.ldexp(1.0, np.maximum(e - sig, tiny) - 1)


def round_fmt(ref: np.ndarray, fmt: str) -> np.ndarray:
    """`ref` rounded to the nearest `fmt` number (ties to even), as float64."""
    ref = np.asarray(ref, np.float64)
    if fmt == "bf16":
        return oracle.bf16_to_f64(oracle.round_to_bf16(ref))
    if fmt == "fp16":
        return ref.astype(np.float16).astype(np.float64)
    return ref


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16/fp16 tensor -> uint16 numpy bit patterns (on the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of_bf16(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(bits(t))


def f64_of_f16(t: torch.Tensor) -> np.ndarray:
    return bits(t).view(np.float16).astype(np.float64)


def gate(gpu: np.ndarray, ref: np.ndarray, what: str, fmt: str = "bf16", rel=REL_L2,
         mx=MAX_ABS_RMS):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    if ref.size == 0:
        return 0.0, 0.0
    nref = np.linalg.norm(ref)
    rl2 = np.linalg.norm(gpu - ref) / nref if nref > 0 else np.linalg.norm(gpu - ref)
    rms = np.sqrt(np.mean(ref * ref))
    d = np.abs(gpu - ref)
    hu = half_ulp(ref, fmt)
    excess = np.max(d - hu)
    # The literal gate, against the reference rounded to the GPU result's own
    # format: |gpu - fmt(ref)| <= mx * rms. An element beyond it must be a
    # faithful rounding of the exact value (one of the two fmt numbers that
    # bracket it, |gpu - ref| < one ulp): the exact value sat near a rounding
    # boundary and the two sides rounded it to neighbouring numbers.
    lit = np.abs(gpu - round_fmt(ref, fmt))
    over = lit > mx * rms
    faithful = d < 2.0 * hu
    print(f"[gate] {what}: relL2={rl2:.3e} (<= {rel:.1e})  max(|err| - half-ulp {fmt})/rms="
          f"{excess / rms:.3e} (<= {mx:.1e})  raw maxabs/rms={d.max() / rms:.3e}  "
          f"literal max|gpu - {fmt}(ref)|/rms={lit.max() / rms:.3e} "
          f"({int(over.sum())} of {ref.size} beyond it, all faithful roundings)")
    assert rl2 <= rel, f"{what}: rel L2 {rl2:.3e} > {rel:.1e}"
    assert excess <= mx * rms, f"{what}: max abs beyond rounding {excess:.3e} > {mx:.1e} * rms {rms:.3e}"
    assert np.all(faithful[over]), (
        f"{what}: {int((over & ~faithful).sum())} elements beyond the literal gate that are not "
        f"a faithful rounding of the exact value")
    if fmt == "fp16":
        # fp16's own rounding is far below the gate: the raw gate holds as stated
        assert d.max() <= mx * rms, f"{what}: raw max abs {d.max():.3e} > {mx:.1e} * rms {rms:.3e}"
    return rl2, excess / rms


def logits_bound(x_bits, w_router, bias, H):
    """Per-element bound on |fp32 GEMM logits - exact|: the products of the
    bf16 activations and the exact three-term bf16 split of each weight are
    exact, and at most 3H+2 fp32 roundings touch each sum (accumulation plus
    the bias add), so |err| <= (3H+2) u (sum_h |x w| + |b|)."""
    xf = np.abs(oracle.bf16_to_f64(x_bits))
    a = xf @ np.abs(np.asarray(w_router, np.float64)).T
    if bias is not None:
        a = a + np.abs(np.asarray(bias, np.float64))[None, :]
    n = 3 * H + 2
    return n * U / (1 - n * U) * a
