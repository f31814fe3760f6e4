"""Inputs of a layer whose routed experts come in several bit widths: 4-bit
on some experts, 3- or 2-bit on the others (the mixed-precision expert
tiers of the hipfire 0.4.3 benchmarks page, "New Flash-Next tiers": lower-bit
experts on most of the routed experts, the rest kept at 4 bits).

Packing follows the library's lower-bit row layouts (include/moe.h):
  4-bit: byte j = element 2j (bits 0-3) | element 2j+1 (bits 4-7);
  2-bit: each little-endian 32-bit word m holds elements 16m .. 16m+15:
         byte 0 = elements 0-3, byte 1 = 8-11, byte 2 = 4-7, byte 3 = 12-15
         (of the word's 16), element i of a byte's four at bits 2i, 2i+1;
  3-bit: each 32-element block takes 12 bytes: the low two bits of its 32
         elements in the 2-bit layout (8 bytes), then one 32-bit word whose
         bit 4c+i is the third bit of element 8c+i and bit 16+4c+i that of
         element 8c+i+4 (c = 0..3, i = 0..3).
Symmetric codes only: w = (q - 2^(b-1)) * scale, one fp16 scale per group
of G along K.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import torch

from .configs import MoEConfig
from .gen import ROUTER_STD, WEIGHT_STD, _randn, pack_nibbles, zipf_bias

__all__ = ["pack_codes", "quantize_sym_bits", "MixedLayer", "make_mixed_layer", "row_bytes"]


def row_bytes(K: int, bits: int) -> int:
    return K * bits // 8


def _pack2(q: torch.Tensor) -> torch.Tensor:
    """[R][K] codes 0..3 (K % 16 == 0) -> [R][K/4] bytes in the 2-bit layout."""
    R, K = q.shape
    g = q.reshape(R, K // 16, 16).to(torch.int32)

    def byte(e0):
        return g[..., e0] | (g[..., e0 + 1] << 2) | (g[..., e0 + 2] << 4) | (g[..., e0 + 3] << 6)

    out = torch.stack([byte(0), byte(8), byte(4), byte(12)], dim=-1)
    return out.reshape(R, K // 4).to(torch.uint8)


def pack_codes(q: torch.Tensor, bits: int) -> torch.Tensor:
    """[R][K] integer codes 0 .. 2^bits - 1 -> packed uint8 rows."""
    q = q.to(torch.int32)
    if bits == 4:
        return pack_nibbles(q)
    if bits == 2:
        return _pack2(q)
    if bits != 3:
        raise ValueError(f"unsupported width {bits}")
    R, K = q.shape
    blk = q.reshape(R * (K // 32), 32)
    lo = _pack2(blk & 3)                                  # [R*K/32][8]
    hi = (blk >> 2) & 1
    h = torch.zeros(blk.shape[0], dtype=torch.int64, device=q.device)
    for c in range(4):
        for i in range(4):
            h |= hi[:, 8 * c + i].to(torch.int64) << (4 * c + i)
            h |= hi[:, 8 * c + i + 4].to(torch.int64) << (16 + 4 * c + i)
    hb = torch.stack([(h >> (8 * b)) & 0xFF for b in range(4)], dim=-1).to(torch.uint8)
    return torch.cat([lo, hb], dim=-1).reshape(R, K // 32 * 12).contiguous()


def quantize_sym_bits(w: torch.Tensor, G: int, bits: int):
    """Symmetric b-bit codes per group of G along the last dim: scale =
    fp16(max |w| / (2^(b-1) - 1)), q = clamp(rint(w / scale)) + 2^(b-1).
    Returns (packed uint8 [R][K*b/8], scale fp16 [R][K/G])."""
    R, K = w.shape
    half = 1 << (bits - 1)
    wg = w.reshape(R, K // G, G)
    s16 = (wg.abs().amax(dim=-1) / (half - 1)).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.round(wg / safe).clamp_(-half, half - 1)
    q = torch.where(s > 0, q, torch.zeros_like(q))
    codes = (q + half).to(torch.int32).reshape(R, K)
    return pack_codes(codes, bits), s16.contiguous()


@dataclass
class MixedLayer:
    """One layer with per-expert bit widths. bits[e] is expert e's width;
    tiers[b] = (w13 [E_b][2I][H*b/8], w13_scale [E_b][2I][H/G], w2
    [E_b][H][I*b/8], w2_scale [E_b][H][I/G]) for each width b present, the
    experts of width b in ascending order; slot[e] is expert e's index in its
    width's tensors."""
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    bits: List[int]
    slot: List[int]
    tiers: Dict[int, Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]]

    def to(self, device) -> "MixedLayer":
        return MixedLayer(self.w_router.to(device),
                          None if self.router_bias is None else self.router_bias.to(device),
                          list(self.bits), list(self.slot),
                          {b: tuple(t.to(device) for t in v) for b, v in self.tiers.items()})

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for v in self.tiers.values() for t in v)


def make_mixed_layer(cfg: MoEConfig, bits: List[int], device="cpu",
                     seed: Optional[int] = None) -> MixedLayer:
    """The float weights of make_layer(cfg) (same seeds), each expert
    quantized symmetrically to its own width bits[e] in {4, 3, 2}."""
    seed = cfg.seed if seed is None else seed
    H, E, I, G = cfg.H, cfg.E, cfg.I, cfg.G
    assert len(bits) == E and all(b in (2, 3, 4) for b in bits)
    wr = _randn((E, H), seed, "w_router", device, ROUTER_STD)
    bias = zipf_bias(E).to(device) if cfg.zipf_bias else None
    lists: Dict[int, List[List[torch.Tensor]]] = {}
    slot = []
    for e in range(E):
        b = bits[e]
        wa = _randn((2 * I, H), seed, f"expert.{e}.w13", device, WEIGHT_STD)
        wb = _randn((H, I), seed, f"expert.{e}.w2", device, WEIGHT_STD)
        p13, s13 = quantize_sym_bits(wa, G, b)
        p2, s2 = quantize_sym_bits(wb, G, b)
        lst = lists.setdefault(b, [[], [], [], []])
        slot.append(len(lst[0]))
        for acc, t in zip(lst, (p13, s13, p2, s2)):
            acc.append(t)
    tiers = {b: tuple(torch.stack(v).contiguous() for v in lst) for b, lst in lists.items()}
    return MixedLayer(wr, bias, list(bits), slot, tiers)
