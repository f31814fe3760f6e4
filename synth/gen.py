"""Seeded synthetic tensors for the 4-bit MoE prefill layer.

Recipe (every tensor has its own torch.Generator, seeded from the config seed
and a fixed tag, so any tensor can be regenerated on its own):

* activations x[T][H]: N(0, 1) in fp32, rounded to bf16 (round to nearest even);
* router Wr[E][H]: N(0, 0.02) fp32 (0.02 is a standard deviation);
* router bias (skewed configs): b[e] = 2*ln(1/(e+1)), a Zipf-like load;
* shared-expert gate w_s[H]: N(0, 0.02) fp32;
* expert weights gate/up [2I][H] and down [H][I]: N(0, 0.02) fp32, then
  quantized per group of G consecutive K (input) elements of a row:
    - symmetric:  s = max|w|/7 -> fp16; q = clamp(rint(w/s), -8, 7); stored
      nibble = q + 8 (an all-zero group stores s = 0, q = 0);
    - asymmetric: m = min w, s = (max w - m)/15 -> fp16 (m, s);
      q = clamp(rint((w - m)/s), 0, 15); stored nibble = q;
  and packed two per byte, the even K index in the low nibble;
* RMSNorm weight (stacked layers): 1 + N(0, 0.02) fp32.

The quantizer is the offline weight-conversion step that produces the packed
layer; the prefill path only ever reads the packed bytes.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, fields
from typing import Optional

import numpy as np
import torch

from .configs import MoEConfig

WEIGHT_STD = 0.02
ROUTER_STD = 0.02
NORM_STD = 0.02


def _generator(seed: int, tag: str, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed((int(seed) * 1_000_003 + zlib.crc32(tag.encode())) % (2**62))
    return g


def _randn(shape, seed, tag, device, std=1.0):
    g = _generator(seed, tag, device)
    out = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        out.mul_(std)
    return out


# ---------------------------------------------------------------------------
# dtype plumbing (bit patterns), used by tests to move data across numpy
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# weight preparation: quantize + pack
# ---------------------------------------------------------------------------

def pack_nibbles(q: torch.Tensor) -> torch.Tensor:
    """[R][K] integer nibbles (0..15) -> [R][K/2] uint8; even K in bits 0-3."""
    q = q.to(torch.uint8)
    lo = q[:, 0::2]
    hi = q[:, 1::2]
    return (lo | (hi << 4)).contiguous()


def quantize_sym(w: torch.Tensor, G: int):
    """Symmetric int4 per group of G along the last dim: returns
    (packed uint8 [R][K/2], scale fp16 [R][K/G])."""
    R, K = w.shape
    wg = w.reshape(R, K // G, G)
    s16 = (wg.abs().amax(dim=-1) / 7.0).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.round(wg / safe).clamp_(-8, 7)
    q = torch.where(s > 0, q, torch.zeros_like(q))
    nib = (q + 8).to(torch.uint8).reshape(R, K)
    return pack_nibbles(nib), s16.contiguous()


def quantize_asym(w: torch.Tensor, G: int):
    """Asymmetric int4 per group of G along the last dim: returns
    (packed uint8 [R][K/2], scale fp16 [R][K/G], min fp16 [R][K/G])."""
    R, K = w.shape
    wg = w.reshape(R, K // G, G)
    mn = wg.amin(dim=-1)
    mx = wg.amax(dim=-1)
    s16 = ((mx - mn) / 15.0).to(torch.float16)
    m16 = mn.to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(-1)
    m = m16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.round((wg - m) / safe).clamp_(0, 15)
    q = torch.where(s > 0, q, torch.zeros_like(q))
    nib = q.to(torch.uint8).reshape(R, K)
    return pack_nibbles(nib), s16.contiguous(), m16.contiguous()


def _quantize(w, G, quant):
    if quant == "sym":
        p, s = quantize_sym(w, G)
        return p, s, None
    if quant == "asym":
        return quantize_asym(w, G)
    raise ValueError(quant)


# ---------------------------------------------------------------------------
# layer inputs
# ---------------------------------------------------------------------------

@dataclass
class LayerInputs:
    """All tensors of one MoE layer (torch tensors on one device).

    Shapes: x [T][H] bf16; w_router [E][H] f32; router_bias [E] f32 or None;
    shared_gate [H] f32 or None; w13 [E][2I][H/2] u8 (rows 0..I-1 gate,
    I..2I-1 up); w13_scale/w13_min [E][2I][H/G] f16; w2 [E][H][I/2] u8;
    w2_scale/w2_min [E][H][I/G] f16; s13/s2 and their scales: the shared
    expert with E = 1 and I = shared_I (None if absent); norm_weight [H] f32
    (stacked layers only). *_min tensors are None for symmetric weights.
    """
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    shared_gate: Optional[torch.Tensor]
    w13: torch.Tensor
    w13_scale: torch.Tensor
    w13_min: Optional[torch.Tensor]
    w2: torch.Tensor
    w2_scale: torch.Tensor
    w2_min: Optional[torch.Tensor]
    s13: Optional[torch.Tensor] = None
    s13_scale: Optional[torch.Tensor] = None
    s13_min: Optional[torch.Tensor] = None
    s2: Optional[torch.Tensor] = None
    s2_scale: Optional[torch.Tensor] = None
    s2_min: Optional[torch.Tensor] = None
    norm_weight: Optional[torch.Tensor] = None

    def to(self, device) -> "LayerInputs":
        kw = {}
        for f in fields(self):
            v = getattr(self, f.name)
            kw[f.name] = None if v is None else v.to(device)
        return LayerInputs(**kw)

    def nbytes(self) -> int:
        n = 0
        for f in fields(self):
            v = getattr(self, f.name)
            if v is not None:
                n += v.numel() * v.element_size()
        return n


def make_tokens(cfg: MoEConfig, device="cpu", rows: Optional[int] = None) -> torch.Tensor:
    """Activations [rows][H] bf16: the first `rows` rows of the config's
    full T-row token tensor (so a short sweep reuses the long batch's rows)."""
    if rows is not None and rows > cfg.T:
        raise ValueError(f"{cfg.name} holds {cfg.T} token rows; asked for {rows}")
    x = _randn((cfg.T, cfg.H), cfg.seed, "x", device).to(torch.bfloat16)
    if rows is not None:
        x = x[:rows].contiguous()
    return x


def _expert_tensors(cfg, seed, tag, I, n_exp, device):
    E = n_exp
    H, G = cfg.H, cfg.G
    w13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
    w13s = torch.empty((E, 2 * I, H // G), dtype=torch.float16, device=device)
    w2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
    w2s = torch.empty((E, H, I // G), dtype=torch.float16, device=device)
    asym = cfg.quant == "asym"
    w13m = torch.empty_like(w13s) if asym else None
    w2m = torch.empty_like(w2s) if asym else None
    for e in range(E):
        wa = _randn((2 * I, H), seed, f"{tag}.{e}.w13", device, WEIGHT_STD)
        p, s, m = _quantize(wa, G, cfg.quant)
        w13[e].copy_(p)
        w13s[e].copy_(s)
        if asym:
            w13m[e].copy_(m)
        wb = _randn((H, I), seed, f"{tag}.{e}.w2", device, WEIGHT_STD)
        p, s, m = _quantize(wb, G, cfg.quant)
        w2[e].copy_(p)
        w2s[e].copy_(s)
        if asym:
            w2m[e].copy_(m)
    return w13, w13s, w13m, w2, w2s, w2m


def zipf_bias(E: int) -> torch.Tensor:
    """b[e] = 2*ln(1/rank), rank = e + 1 (natural log), fp32."""
    return torch.tensor([2.0 * math.log(1.0 / (e + 1)) for e in range(E)], dtype=torch.float32)


def make_layer(cfg: MoEConfig, device="cpu", seed: Optional[int] = None) -> LayerInputs:
    """Weights of one layer. `seed` overrides the config seed (stacked layers
    use one seed per layer)."""
    seed = cfg.seed if seed is None else seed
    H, E = cfg.H, cfg.E
    wr = _randn((E, H), seed, "w_router", device, ROUTER_STD)
    bias = zipf_bias(E).to(device) if cfg.zipf_bias else None
    w13, w13s, w13m, w2, w2s, w2m = _expert_tensors(cfg, seed, "expert", cfg.I, E, device)
    li = LayerInputs(w_router=wr, router_bias=bias, shared_gate=None,
                     w13=w13, w13_scale=w13s, w13_min=w13m,
                     w2=w2, w2_scale=w2s, w2_min=w2m)
    if cfg.shared_I:
        li.shared_gate = _randn((H,), seed, "shared_gate", device, ROUTER_STD)
        s13, s13s, s13m, s2, s2s, s2m = _expert_tensors(cfg, seed, "shared", cfg.shared_I, 1, device)
        li.s13, li.s13_scale, li.s13_min = s13[0], s13s[0], (s13m[0] if s13m is not None else None)
        li.s2, li.s2_scale, li.s2_min = s2[0], s2s[0], (s2m[0] if s2m is not None else None)
    return li


def stack_layer_seed(cfg: MoEConfig, layer: int) -> int:
    return cfg.seed + 1000 + layer


def make_stack_layer(cfg: MoEConfig, layer: int, device="cpu") -> LayerInputs:
    """Layer `layer` of a stacked config: its own seed, plus the RMSNorm
    weight 1 + N(0, 0.02)."""
    seed = stack_layer_seed(cfg, layer)
    li = make_layer(cfg, device=device, seed=seed)
    li.norm_weight = 1.0 + _randn((cfg.H,), seed, "norm", device, NORM_STD)
    return li


def randomize_packed(li: LayerInputs, seed: int, scale_lo=1e-3, scale_hi=2e-2) -> LayerInputs:
    """Replace every packed byte with a uniform random byte (all 16 nibble
    values occur) and every scale/min with random fp16 values; used to test
    that decoding covers the whole code space, not only quantizer output."""
    out = LayerInputs(**{f.name: getattr(li, f.name) for f in fields(li)})
    for i, name in enumerate(["w13", "w2", "s13", "s2"]):
        v = getattr(li, name)
        if v is None:
            continue
        g = _generator(seed, "rb." + name, v.device)
        setattr(out, name, torch.randint(0, 256, v.shape, generator=g, device=v.device,
                                         dtype=torch.int32).to(torch.uint8))
        for suf, lo, hi in (("_scale", scale_lo, scale_hi), ("_min", -scale_hi * 8, 0.0)):
            t = getattr(li, name + suf)
            if t is None:
                continue
            g2 = _generator(seed, "rb." + name + suf, t.device)
            r = torch.rand(t.shape, generator=g2, device=t.device, dtype=torch.float32)
            setattr(out, name + suf, (lo + (hi - lo) * r).to(torch.float16))
    return out
