"""GPU parity: every entry point of the C ABI against the CPU oracle on the
same seeded inputs. Integer results (top-k ids given the GPU's logits, the
permutation) must match bit for bit; floating-point results must meet the
relative-L2 / max-abs gates of tests/gpu_util.py."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import quantized_moe_prefill_amd as qm
from synth import CONFIGS, make_layer, make_tokens
from synth.gen import randomize_packed
from tests.gpu_util import bits, f64_of_bf16, f64_of_f16, gate, logits_bound

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


_CACHE = {}


def setup(cfg, rows=None, random_bytes=False):
    """Device weights (cached per config) and tokens for a config."""
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


def run_pipeline(cfg, li, x):
    """Each entry point in turn; returns every intermediate on the device."""
    shape = qm.shape_of(cfg)
    logits, ids, tw, sw = qm.moe_route(shape, x, li.w_router, li.router_bias, li.shared_gate,
                                       want_logits=True)
    counts, offsets, sp, inv = qm.moe_permute(shape, ids)
    ex = qm.Experts(li)
    y_perm, y_sh = qm.moe_expert_ffn(shape, x, ex, counts, offsets, sp)
    out = qm.moe_combine(shape, y_perm, inv, tw, y_sh, sw)
    torch.cuda.synchronize()
    return dict(logits=logits, ids=ids, tw=tw, sw=sw, counts=counts, offsets=offsets, sp=sp,
                inv=inv, y_perm=y_perm, y_sh=y_sh, out=out)


def check_route(cfg, cpu, x, g):
    xb = bits(x)
    L = g["logits"].cpu().numpy()
    ref = oracle.router_logits(oracle.bf16_to_f64(xb), cpu.w_router.numpy(),
                               None if cpu.router_bias is None else cpu.router_bias.numpy())
    bound = logits_bound(xb, cpu.w_router.numpy(),
                         None if cpu.router_bias is None else cpu.router_bias.numpy(), cfg.H)
    assert np.all(np.abs(L - ref) <= bound), "router logits outside the fp32 GEMM error bound"
    ids_ref, w_ref = oracle.select_topk(L, cfg.k)
    assert np.array_equal(g["ids"].cpu().numpy(), ids_ref), "top-k ids differ (same logits)"
    assert np.allclose(g["tw"].cpu().numpy(), w_ref, rtol=0, atol=2e-6)
    if cfg.shared_I:
        s_ref = oracle.shared_gate(oracle.bf16_to_f64(xb), cpu.shared_gate.numpy())
        assert np.allclose(g["sw"].cpu().numpy(), s_ref, rtol=0, atol=2e-6)
    return L, ids_ref


def check_permute(cfg, ids_np, g):
    c, o, s, i = oracle.permute(ids_np, cfg.E)
    assert np.array_equal(g["counts"].cpu().numpy(), c)
    assert np.array_equal(g["offsets"].cpu().numpy(), o)
    assert np.array_equal(g["sp"].cpu().numpy(), s)
    assert np.array_equal(g["inv"].cpu().numpy(), i)


def full_check(cfg, li, cpu, x):
    g = run_pipeline(cfg, li, x)
    L, ids = check_route(cfg, cpu, x, g)
    check_permute(cfg, ids, g)
    ref = oracle.moe_layer(bits(x), cpu, cfg.k, cfg.G, cfg.quant, logits32=L)
    gate(f64_of_f16(g["y_perm"]), ref["y_perm"], "y_perm", fmt="fp16")
    if cfg.shared_I:
        gate(f64_of_f16(g["y_sh"]), ref["y_shared"], "y_shared", fmt="fp16")
    gate(f64_of_bf16(g["out"]), ref["out"], "out (entry points)")
    # the fused layer call must give the same bits as the four calls
    out2 = qm.MoELayer(cfg, li, DEV, x.shape[0]).forward(x)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), g["out"].view(torch.int16))
    return g, ref


@pytest.mark.parametrize("name", ["tiny", "a3b_pp512", "skew_shared"])
def test_layer_parity(name):
    cfg = CONFIGS[name]
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


def test_layer_parity_mixed_tile_heights():
    """T = 1536 on the A3B shape: 96 rows per expert on average, so gate/up
    runs on 64-row tiles and down on 128-row tiles."""
    cfg = replace(CONFIGS["a3b_pp512"], T=1536)
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


def test_layer_parity_T4096():
    """T = 4096 on the A3B shape (256 rows per expert on average, 128-row
    tiles, each expert's last tile partly filled): every intermediate
    against the oracle, and the fused call bit-equal to the entry points."""
    cfg = replace(CONFIGS["a3b_pp512"], T=4096)
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


def test_tiny_random_bytes_all_nibbles():
    cfg = CONFIGS["tiny"]
    li, cpu, x = setup(cfg, random_bytes=True)
    full_check(cfg, li, cpu, x)


def test_asym_random_bytes_with_shared():
    cfg = replace(CONFIGS["skew_shared"], T=256, E=32, I=256, shared_I=128)
    li, cpu, x = setup(cfg, random_bytes=True)
    full_check(cfg, li, cpu, x)


@pytest.mark.parametrize("G,quant", [(64, "sym"), (32, "sym"), (128, "asym"), (64, "asym")])
def test_group_sizes(G, quant):
    cfg = replace(CONFIGS["a3b_pp512"], T=200, E=16, I=256, G=G, quant=quant)
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_weight_streaming_sweep(T):
    cfg = CONFIGS["a3b_pp8192"]
    li, cpu, x = setup(cfg, rows=T)
    full_check(replace(cfg, T=T), li, cpu, x)


@pytest.mark.parametrize("name,T,over", [
    ("skew_shared", 1, {}),
    ("skew_shared", 5, {}),
    ("skew_shared", 16, {}),
    ("tiny", 1, {}),
    ("tiny", 3, {}),
    # gate/up K = 768: six 128-wide stages over four waves (two waves repeat
    # a stage whose products are skipped); down K = 384: three stages, one
    # wave without work
    ("a3b_pp512", 7, dict(H=768, I=384, E=16, G=64)),
    # every expert takes every token: exactly one full 16-row block each
    ("a3b_pp512", 16, dict(H=1024, I=256, E=8, G=32, quant="asym")),
])
def test_small_T_weight_streaming(name, T, over):
    """At most 16 tokens: the expert GEMMs run as the weight-streaming
    kernel (asymmetric and symmetric, shared expert, 1/2/4 stages per wave)."""
    cfg = replace(CONFIGS[name], T=T, **over)
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


def test_streaming_more_rows_than_a_block():
    """Few tokens, but each sends three of its four rows to expert 0 (the
    entry points accept repeated ids): 36 rows of one expert, walked by the
    weight-streaming kernel in 16-row blocks with its weights held."""
    cfg = replace(CONFIGS["skew_shared"], T=12, E=16, k=4, I=256, shared_I=128, G=32)
    li, cpu, x = setup(cfg)
    rng = np.random.default_rng(5)
    ids = np.array([[0, 0, 0, rng.integers(1, 16)] for _ in range(cfg.T)], np.int32)
    shape = qm.shape_of(cfg)
    counts, offsets, sp, inv = qm.moe_permute(shape, torch.from_numpy(ids).to(DEV))
    y_perm, y_sh = qm.moe_expert_ffn(shape, x, qm.Experts(li), counts, offsets, sp)
    torch.cuda.synchronize()
    c, o, s, _ = oracle.permute(ids, cfg.E)
    assert c[0] == 36
    w = oracle.moe_oracle._weights_dict(cpu)
    xf = f64_of_bf16(x)
    _, y_ref = oracle.expert_ffn(xf, s, o, cfg.k, w, cfg.G, cfg.quant)
    gate(f64_of_f16(y_perm), y_ref, "y_perm", fmt="fp16")
    _, ys_ref = oracle.moe_oracle.shared_expert(xf, w, cfg.G, cfg.quant)
    gate(f64_of_f16(y_sh), ys_ref, "y_shared", fmt="fp16")


def test_ragged_and_k1():
    # T not a multiple of any tile, k = 1, odd expert count
    cfg = replace(CONFIGS["tiny"], T=37, E=5, k=1)
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


def test_k_equals_E():
    cfg = replace(CONFIGS["tiny"], T=50, E=4, k=4)
    li, cpu, x = setup(cfg)
    full_check(cfg, li, cpu, x)


def test_full_size_a3b_pp8192():
    """The bench workload at full size (8192 tokens, 65,536 pairs): routing
    and the permutation bit-exact, every row of y_perm and of out against the
    oracle (teacher-forced on the GPU logits), the fused layer call bit-equal
    to the separate entry points (its router GEMM writes the fp16 copy of x,
    moe_expert_ffn converts x itself) and to a second fused call. Gate/up
    runs 128-row tiles with 16 K stages (16 % 3 == 1: the last stage's
    repeated activation load targets the ring slot that the epilogue reuses
    for its output sub-tiles)."""
    cfg = CONFIGS["a3b_pp8192"]
    li, cpu, x = setup(cfg)
    g, _ = full_check(cfg, li, cpu, x)
    layer = qm.MoELayer(cfg, li, DEV, cfg.T)
    a = layer.forward(x).clone()
    b = layer.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), g["out"].view(torch.int16))


def test_max_T_sampled():
    """The largest call the size limits allow at the a3b_pp8192 shape:
    174,762 tokens, whose h (T*k*I*2 bytes) is just below 2^31, so the
    GEMMs' 32-bit buffer offsets run up to their limit. Routing and the
    permutation bit-exact, sampled output rows (the first, the last, and
    rows near the end) against the oracle, teacher-forced on the GPU logits."""
    T = ((1 << 31) - 1) // (8 * 768 * 2)
    cfg = replace(CONFIGS["a3b_pp8192"], T=T)
    li = make_layer(cfg, device=DEV)
    x = make_tokens(cfg, device=DEV)
    shape = qm.shape_of(cfg)
    out = qm.MoELayer(cfg, li, DEV, T).forward(x)
    logits, ids, _, _ = qm.moe_route(shape, x, li.w_router, li.router_bias, None, want_logits=True)
    counts, offsets, sp, inv = qm.moe_permute(shape, ids)
    torch.cuda.synchronize()
    L = logits.cpu().numpy()
    ids_ref, _ = oracle.select_topk(L, cfg.k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    c, o, s, i = oracle.permute(ids_ref, cfg.E)
    assert np.array_equal(counts.cpu().numpy(), c) and np.array_equal(sp.cpu().numpy(), s)
    assert np.array_equal(inv.cpu().numpy(), i) and np.array_equal(offsets.cpu().numpy(), o)
    rows = np.random.default_rng(1).choice(T, 24, replace=False)
    rows = np.concatenate([rows, [0, T - 2, T - 1]])
    cpu = li.to("cpu")
    ref = oracle.moe_layer_rows(bits(x), rows, cpu, cfg.k, cfg.G, cfg.quant, logits32_rows=L[rows])
    gate(f64_of_bf16(out)[rows], ref["out"], "out rows (max T)")


@pytest.mark.parametrize("name", ["a3b_pp512", "skew_shared"])
def test_determinism_bitwise(name):
    """Repeated layer calls give identical bits: the 64-row tile instance
    (a3b_pp512), and the 128-row one with the shared expert folded in
    (skew_shared: gate/up 16 K stages, down 4; in both the last stage's
    repeated activation load targets the ring slot of the epilogue's output
    sub-tiles). y_perm and y_shared are compared too."""
    cfg = CONFIGS[name]
    li, cpu, x = setup(cfg)
    outs = [run_pipeline(cfg, li, x) for _ in range(3)]
    for key in ("y_perm", "y_sh", "out"):
        if outs[0][key] is None:
            continue
        for o in outs[1:]:
            assert torch.equal(outs[0][key].view(torch.int16), o[key].view(torch.int16)), key
    layer = qm.MoELayer(cfg, li, DEV, cfg.T)
    a = layer.forward(x).clone()
    b = layer.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), outs[0]["out"].view(torch.int16))


def test_token_permutation_equivariance():
    cfg = CONFIGS["tiny"]
    li, cpu, x = setup(cfg)
    layer = qm.MoELayer(cfg, li, DEV, cfg.T)
    perm = torch.randperm(cfg.T, generator=torch.Generator().manual_seed(3)).to(DEV)
    a = layer.forward(x)
    b = layer.forward(x[perm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a[perm].view(torch.int16), b.view(torch.int16))


def test_permute_edge_cases():
    cfg = replace(CONFIGS["tiny"], E=16, k=4)
    shape = qm.shape_of(cfg)
    rng = np.random.default_rng(4)
    cases = [
        np.zeros((0, 4), np.int32),                                     # T = 0
        np.array([[3, 1, 2, 0]], np.int32),                             # T = 1
        np.tile(np.array([[5, 6, 7, 8]], np.int32), (1000, 1)),        # 4 experts, 12 empty
        np.stack([rng.choice(16, 4, replace=False) for _ in range(777)]).astype(np.int32),
    ]
    for ids in cases:
        g = dict(zip(["counts", "offsets", "sp", "inv"],
                     qm.moe_permute(shape, torch.from_numpy(ids).to(DEV))))
        torch.cuda.synchronize()
        if ids.shape[0] == 0:
            assert g["counts"].cpu().numpy().tolist() == [0] * 16
            assert g["offsets"].cpu().numpy().tolist() == [0] * 17
            continue
        check_permute(cfg, ids, g)


@pytest.mark.parametrize("E,k,shared,bias", [
    (1, 1, False, False), (3, 2, True, True), (64, 6, True, False), (100, 8, True, True),
    (128, 4, True, True), (200, 8, False, True), (256, 8, True, False)])
def test_route_expert_counts(E, k, shared, bias):
    """Router alone over expert counts that exercise every per-lane width of
    the selection and both places of the shared-gate column."""
    cfg = replace(CONFIGS["a3b_pp512"], T=333, H=512, E=E, k=k, I=128,
                  shared_I=128 if shared else 0, zipf_bias=bias)
    li, cpu, x = setup(cfg)
    shape = qm.shape_of(cfg)
    logits, ids, tw, sw = qm.moe_route(shape, x, li.w_router, li.router_bias, li.shared_gate,
                                       want_logits=True)
    torch.cuda.synchronize()
    check_route(cfg, cpu, x, dict(logits=logits, ids=ids, tw=tw, sw=sw))


def test_permute_large_and_duplicates():
    """Several 2048-pair chunks with a ragged tail, all 256 experts, skewed
    and repeated ids (moe_permute does not need distinct ids per token)."""
    rng = np.random.default_rng(11)
    # (8192 pairs: four whole chunks; 8200: a tail chunk of eight)
    for E, k, T, kind in [(256, 8, 1000, "zipf"), (200, 7, 3001, "uniform"), (1, 1, 4097, "one"),
                          (32, 8, 513, "dup"), (64, 8, 1024, "uniform"),
                          (64, 8, 1025, "uniform")]:
        cfg = replace(CONFIGS["tiny"], E=E, k=k)
        if kind == "zipf":
            p = 1.0 / np.arange(1, E + 1)
            ids = rng.choice(E, size=(T, k), p=p / p.sum())
        elif kind == "uniform":
            ids = rng.integers(0, E, size=(T, k))
        elif kind == "one":
            ids = np.zeros((T, k))
        else:
            ids = np.repeat(rng.integers(0, 3, size=(T, 1)), k, axis=1)
        ids = ids.astype(np.int32)
        g = dict(zip(["counts", "offsets", "sp", "inv"],
                     qm.moe_permute(qm.shape_of(cfg), torch.from_numpy(ids).to(DEV))))
        torch.cuda.synchronize()
        check_permute(cfg, ids, g)


def test_combine_with_residual_in_place():
    cfg = CONFIGS["skew_shared"]
    T, k, H = 300, cfg.k, cfg.H
    g = torch.Generator(device=DEV).manual_seed(5)
    y = torch.randn((T * k, H), device=DEV, generator=g).to(torch.float16)
    ysh = torch.randn((T, H), device=DEV, generator=g).to(torch.float16)
    res = torch.randn((T, H), device=DEV, generator=g).to(torch.bfloat16)
    inv = torch.randperm(T * k, device=DEV, generator=g).to(torch.int32)
    tw = torch.rand((T, k), device=DEV, generator=g)
    sw = torch.rand((T,), device=DEV, generator=g)
    shape = qm.shape_of(cfg)
    res_np = f64_of_bf16(res)
    out = res.clone()
    qm.moe_combine(shape, y, inv, tw, ysh, sw, residual=out, out=out)  # out aliases residual
    torch.cuda.synchronize()
    ref = oracle.combine(f64_of_f16(y), inv.cpu().numpy(), tw.cpu().numpy().astype(np.float64),
                         f64_of_f16(ysh), sw.cpu().numpy().astype(np.float64), res_np)
    got = f64_of_bf16(out)
    # fp32 sums of k + 2 terms, then one bf16 rounding
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * (np.abs(ref) + 1))


def test_rmsnorm_parity():
    cfg = CONFIGS["stack40"]
    g = torch.Generator(device=DEV).manual_seed(9)
    x = (torch.randn((333, cfg.H), device=DEV, generator=g) * 3).to(torch.bfloat16)
    w = 1 + 0.02 * torch.randn((cfg.H,), device=DEV, generator=g)
    out = qm.moe_rmsnorm(x, w, cfg.rms_eps)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(bits(x), w.cpu().numpy(), cfg.rms_eps)
    got = f64_of_bf16(out)
    # fp32 math then one bf16 rounding: within one bf16 ulp
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) * 1.01 + 1e-30)
