"""The tiled 4-bit weight layout (include/moe.h, moe_w_layout_t and
moe_pack_w4): the pack kernel against the layout's definition written out in
numpy, and every path that reads tiled weights against the same call on the
row-major weights, bit for bit (the same products in the same order: only
the addresses of the weight loads differ). The row-major calls are checked
against the oracle elsewhere."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_layer, make_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def tiled_ref(src: np.ndarray, rows: int, K: int) -> np.ndarray:
    """dst[((r/16)(K/128) + k/128) 1024 + (((k%128)/32) 16 + r%16) 16 + (k%32)/2]
    = src[r (K/2) + k/2]: split rows into (group, r16) and each row's bytes
    into (stage, lg, 16 bytes), then order (group, stage, lg, r16, bytes)."""
    a = src.reshape(rows // 16, 16, K // 128, 4, 16)
    return a.transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("rows,K", [(16, 128), (48, 384), (256, 2048), (1536, 768)])
def test_pack_w4_layout(rows, K):
    g = torch.Generator(device="cpu").manual_seed(rows * 7 + K)
    src = torch.randint(0, 256, (rows, K // 2), dtype=torch.uint8, generator=g)
    dst = qm.moe_pack_w4(src.to(DEV), rows, K).cpu().numpy().reshape(-1)
    ref = tiled_ref(src.numpy(), rows, K)
    assert np.array_equal(dst, ref)
    # a permutation of the bytes: nothing lost or duplicated
    assert np.array_equal(np.sort(dst), np.sort(src.numpy().reshape(-1)))


def bits16(t):
    return t.view(torch.int16)


# (workload, tokens): the 128-row tiles with the cross-tile pipeline, the
# 64-row tiles, the skewed asymmetric G = 32 layer with a shared expert
# (scale windows, the shared expert folded into the tiled launches), and
# the few-token paths (the four-launch small layer, the streaming kernels)
CASES = [("a3b_pp8192", 8192), ("a3b_pp512", 512), ("skew_shared", 600), ("skew_shared", 4096),
         ("tiny", 64), ("a3b_pp8192", 1), ("a3b_pp8192", 16), ("skew_shared", 16), ("tiny", 5)]


@pytest.mark.parametrize("name,T", CASES)
def test_tiled_layer_bitwise(name, T):
    cfg = replace(CONFIGS[name], T=T)
    li = make_layer(cfg, device=DEV)
    x = make_tokens(cfg, device=DEV)
    rows = qm.MoELayer(cfg, li, DEV, T)
    tiled = qm.MoELayer(cfg, li, DEV, T, tiled=True)
    assert tiled.shape.w_layout == qm.MOE_W_TILED
    assert not torch.equal(tiled.li.w13, li.w13)
    ref = rows.forward(x).clone()
    got = tiled.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(bits16(got), bits16(ref)), f"{name} T={T}: tiled layer differs"
    if T <= 2400:
        st = qm.moe_layer_forward_static(tiled.shape, x, li.w_router, li.router_bias,
                                         li.shared_gate, tiled.experts)
        torch.cuda.synchronize()
        assert torch.equal(bits16(st), bits16(ref)), f"{name} T={T}: static tiled call differs"


@pytest.mark.parametrize("name,T", [("a3b_pp512", 512), ("skew_shared", 16), ("a3b_pp8192", 3)])
def test_tiled_expert_ffn_bitwise(name, T):
    """moe_expert_ffn on tiled weights: y_perm (and y_shared) bit-equal."""
    cfg = replace(CONFIGS[name], T=T)
    li = make_layer(cfg, device=DEV)
    x = make_tokens(cfg, device=DEV)
    shape = qm.shape_of(cfg)
    _, ids, _, _ = qm.moe_route(shape, x, li.w_router, li.router_bias, li.shared_gate)
    counts, offsets, sp, _ = qm.moe_permute(shape, ids)
    ref = qm.moe_expert_ffn(shape, x, qm.Experts(li), counts, offsets, sp)
    lt = qm.pack_layer(cfg, li)
    got = qm.moe_expert_ffn(qm.shape_of(cfg, qm.MOE_W_TILED), x, qm.Experts(lt), counts, offsets, sp)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        if b is None:
            assert a is None
            continue
        assert torch.equal(bits16(a), bits16(b))


def tier_tiled_ref(src: np.ndarray, rows: int, K: int, bits: int, gate_up: bool) -> np.ndarray:
    """moe_pack_tier written out from its definition: rows reordered by sigma
    (the 3- and 2-bit gate/up matrices: within each 32-row group, row
    16 p + i takes row 2 p + 8 (i // 4) + (0, 4, 1, 5)[i % 4]), then each
    row's 4 bits-byte blocks of 32 elements ordered (stripe, stage, lg, r16)."""
    a = src.reshape(rows, K * bits // 8)
    if gate_up and bits < 4:
        sigma = np.empty(rows, dtype=np.int64)
        for r in range(rows):
            g, q = divmod(r, 32)
            p, i = divmod(q, 16)
            sigma[r] = 32 * g + 2 * p + 8 * (i // 4) + (0, 4, 1, 5)[i % 4]
        assert np.array_equal(np.sort(sigma), np.arange(rows))
        a = a[sigma]
    a = a.reshape(rows // 16, 16, K // 128, 4, 4 * bits)
    out = a.transpose(0, 2, 3, 1, 4).reshape(-1)
    if bits == 3:
        # the third word of every 12-byte block: bit 4c + i + 16h moves to
        # bit (2 + 2i + 16h + (0, 1, 8, 9)[c]) mod 32
        words = out.view("<u4").reshape(-1, 3).copy()
        hb = words[:, 2]
        new = np.zeros_like(hb)
        for c in range(4):
            for i in range(4):
                for h in range(2):
                    bit = (hb >> np.uint32(4 * c + i + 16 * h)) & np.uint32(1)
                    new |= bit << np.uint32((2 + 2 * i + 16 * h + (0, 1, 8, 9)[c]) % 32)
        words[:, 2] = new
        out = words.reshape(-1).view(np.uint8)
    return out


@pytest.mark.parametrize("bits", [4, 3, 2])
@pytest.mark.parametrize("gate_up", [False, True])
@pytest.mark.parametrize("rows,K", [(32, 128), (96, 384), (1536, 2048)])
def test_pack_tier_layout(bits, gate_up, rows, K):
    g = torch.Generator(device="cpu").manual_seed(rows * 11 + K + bits)
    src = torch.randint(0, 256, (rows, K * bits // 8), dtype=torch.uint8, generator=g)
    dst = qm.moe_pack_tier(src.to(DEV), rows, K, bits, gate_up).cpu().numpy().reshape(-1)
    assert np.array_equal(dst, tier_tiled_ref(src.numpy(), rows, K, bits, gate_up))
    if bits < 4:
        # every bit kept: the same number of ones per matrix
        assert (np.unpackbits(dst).sum() == np.unpackbits(src.numpy().reshape(-1)).sum())
    if bits == 4:
        assert np.array_equal(dst, qm.moe_pack_w4(src.to(DEV), rows, K).cpu().numpy().reshape(-1))


# mixed-width layers: (workload, tokens, width pattern); the patterns of
# tests/test_gpu_mixed.py, whose row-major calls are checked against the oracle
MIXED_CASES = [("tiny", 64, [4, 3, 2]), ("a3b_pp512", 512, [4, 3, 3, 2, 2, 2, 3, 2]),
               ("a3b_pp8192", 8192, [4, 3, 2, 3]), ("a3b_pp8192", 8192, [3]),
               ("a3b_pp8192", 8192, [2]), ("a3b_pp512", 3, [2, 3, 4, 2])]


@pytest.mark.parametrize("name,T,pattern", MIXED_CASES)
def test_tiled_mixed_bitwise(name, T, pattern):
    """Mixed-width layers on tiers regrouped by moe_pack_tier: y_perm and the
    layer output bit-equal to the same calls on row-major tiers."""
    from synth.mixed import make_mixed_layer
    cfg = replace(CONFIGS[name], T=T)
    perm = np.random.default_rng(0).permutation(cfg.E)
    widths = [4] * cfg.E
    for i, e in enumerate(perm):
        widths[e] = pattern[i % len(pattern)]
    ml = make_mixed_layer(cfg, widths, device=DEV)
    x = make_tokens(cfg, device=DEV)
    shape = qm.shape_of(cfg)
    tshape = qm.shape_of(cfg, qm.MOE_W_TILED)
    ex = qm.MixedExperts(ml, DEV)
    mt = qm.pack_mixed(cfg, ml)
    ext = qm.MixedExperts(mt, DEV)
    for b in ml.tiers:
        assert not torch.equal(mt.tiers[b][0], ml.tiers[b][0])
    _, ids, _, _ = qm.moe_route(shape, x, ml.w_router, ml.router_bias, None)
    counts, offsets, sp, _ = qm.moe_permute(shape, ids)
    y_ref = qm.moe_expert_ffn_mixed(shape, x, ex, counts, offsets, sp).clone()
    y_got = qm.moe_expert_ffn_mixed(tshape, x, ext, counts, offsets, sp)
    out_ref = qm.moe_layer_forward_mixed(shape, x, ml.w_router, ml.router_bias, ex).clone()
    out_got = qm.moe_layer_forward_mixed(tshape, x, ml.w_router, ml.router_bias, ext)
    torch.cuda.synchronize()
    assert torch.equal(bits16(y_got), bits16(y_ref)), f"{name} T={T} {pattern}: tiled y_perm differs"
    assert torch.equal(bits16(out_got), bits16(out_ref)), f"{name} T={T} {pattern}: tiled out differs"
