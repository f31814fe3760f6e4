"""Plain, slow, obviously-correct CPU oracle for 4-bit MoE prefill.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.

What it follows. The pages describe the prefill route of an A3B-class MoE
model whose experts are stored as 4-bit integers with a per-block scale:
the hipfire 0.4.3 benchmarks page, section "Read this before comparing
columns" (defaults table: the MoE prefill route is either "per-expert
buffers" or "symmetric IU4 MoE") and section "Known limits" (the fast route
needs the symmetric expert recipe; the older asymmetric file prefills
slower and its numerics differ slightly), and the prefill-chunk row of the
same table (prompts are processed in chunks of 8192 rows). hipEngine's
announcement ("hipEngine: Fast Native Qwen 3.6 Inference for RDNA3",
section "Implementation Notes") keeps a CPU-reference oracle for each
kernel; this module is that practice for this layer. The pages fix neither
the router, the expert FFN form, the group size nor the nibble layout; the
readings used here (all listed with the workload recipe) are:

* the router is an fp32 linear map over bf16 activations, optionally with a
  per-expert bias; the k largest biased logits are selected (ties go to the
  lower expert index, in descending logit order) and their weights are the
  softmax over the k selected logits;
* each expert is a SwiGLU MLP: h = silu(x Wg^T) * (x Wu^T), y = h Wd^T with
  silu(z) = z / (1 + exp(-z)); gate rows come first in the packed gate/up
  matrix;
* 4-bit weights, two per byte, even K index in the low nibble; a group of G
  consecutive K elements of a row shares an fp16 scale (and, for the
  asymmetric format, an fp16 minimum): symmetric w = (nibble - 8) * scale,
  asymmetric w = nibble * scale + min;
* an optional shared expert runs on every token and is added with weight
  sigmoid(x . w_s);
* stacked layers are pre-norm: x <- bf16(x + MoE(bf16(RMSNorm(x)))).

Precision: float64 throughout, except where a floating-point value decides
an integer: the top-k choice is made on fp32 logits, the precision of the
GPU router's output. Layer inputs and outputs are bf16 by definition of the
interface, so the stack rounds to bf16 at those boundaries only.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64",
    "round_to_bf16",
    "unpack_nibbles",
    "dequant",
    "router_logits",
    "shared_gate",
    "select_topk",
    "permute",
    "unpermute",
    "swiglu_expert",
    "expert_ffn",
    "combine",
    "moe_layer",
    "moe_layer_rows",
    "rmsnorm",
    "stack_layer",
    "moe_stack",
    "silu",
    "sigmoid",
    "quantize_rows_i8",
    "dequant_rows_i8",
    "expert_ffn_i8",
    "moe_layer_i8",
    "moe_layer_rows_i8",
    "unpack_codes",
    "dequant_bits",
    "moe_layer_mixed",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact: bf16 is the top half
    of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(bits_or_half) -> np.ndarray:
    a = np.asarray(bits_or_half)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as
    uint16 bit patterns. bf16 keeps 8 significant bits and the binary32
    exponent range; below 2^-126 the spacing is fixed at 2^-133."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    finite = np.isfinite(v) & (v != 0)
    _, e = np.frexp(np.where(finite, v, 1.0))          # v = m * 2^e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))   # spacing of 8-bit significands
    r = np.rint(v / quantum) * quantum                  # rint: ties to even
    out[...] = np.where(finite, r, v)
    big = np.abs(out) > 3.3895313892515355e38            # largest finite bf16
    out = np.where(big & finite, np.copysign(np.inf, out), out)
    bits32 = out.astype(np.float32).view(np.uint32)     # exact: value has 8 bits
    return (bits32 >> 16).astype(np.uint16)


def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# 4-bit block dequantization
# ---------------------------------------------------------------------------

def unpack_nibbles(packed) -> np.ndarray:
    """[R][K/2] bytes -> [R][K] nibble values 0..15. Byte j of a row holds
    element 2j in bits 0-3 and element 2j+1 in bits 4-7."""
    p = np.asarray(packed, dtype=np.uint8)
    R, half = p.shape
    out = np.empty((R, 2 * half), dtype=np.int64)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def dequant(packed, scale, minv, G: int, quant: str) -> np.ndarray:
    """Dequantize one weight matrix [R][K] to float64.

    symmetric (quant == "sym"):  w[r,k] = (nib[r,k] - 8) * scale[r, k//G]
    asymmetric (quant == "asym"): w[r,k] = nib[r,k] * scale[r, k//G] + min[r, k//G]
    """
    nib = unpack_nibbles(packed).astype(np.float64)
    R, K = nib.shape
    if K % G:
        raise ValueError("K must be a multiple of the group size")
    s = np.repeat(f16_to_f64(scale).reshape(R, K // G), G, axis=1)
    if quant == "sym":
        return (nib - 8.0) * s
    if quant == "asym":
        m = np.repeat(f16_to_f64(minv).reshape(R, K // G), G, axis=1)
        return nib * s + m
    raise ValueError(quant)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def router_logits(xf, w_router, bias=None) -> np.ndarray:
    """L[t,e] = sum_h x[t,h] * Wr[e,h] (+ b[e]), float64."""
    L = np.asarray(xf, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def shared_gate(xf, w_s) -> np.ndarray:
    """sigmoid(x . w_s) per token, float64."""
    return sigmoid(np.asarray(xf, np.float64) @ np.asarray(w_s, np.float64))


def select_topk(logits32, k: int):
    """Top-k selection on fp32 logits.

    ids[t] lists the k experts with the largest logit, largest first; equal
    logits are ordered by ascending expert index (-0.0 equals +0.0, since the
    comparison is numeric). weights[t,j] = exp(L_j - L_max) / sum over the k
    selected of exp(L_i - L_max), computed in float64.
    """
    L = np.asarray(logits32, dtype=np.float32)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # lexsort: last key is primary. Primary: -logit (numeric, so -0.0 == +0.0),
    # secondary: expert index ascending.
    Ld = L.astype(np.float64)
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.empty((T, E), dtype=np.int64)
    for t in range(T):
        order[t] = np.lexsort((idx[t], -Ld[t]))
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(Ld, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


def permute(ids, E: int):
    """Group the T*k (token, slot) pairs by expert.

    Pair p = t*k + j. counts[e] = number of pairs routed to e; offsets is the
    exclusive prefix sum (E+1 entries); sorted_pairs lists, expert by expert,
    the pairs of that expert in ascending p; inv[p] is the position of p in
    sorted_pairs.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    if counts.size != E:
        raise ValueError("expert id out of range")
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int64)
    inv = np.empty(P, dtype=np.int64)
    inv[sorted_pairs] = np.arange(P)
    return counts, offsets, sorted_pairs, inv


def unpermute(rows_sorted, inv):
    """Back to pair order: out[p] = rows_sorted[inv[p]]."""
    return np.asarray(rows_sorted)[np.asarray(inv)]


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------

def swiglu_expert(X, W13, W2):
    """One SwiGLU expert on rows X [n][H]: W13 [2I][H] (gate rows first),
    W2 [H][I]. Returns (h [n][I], y [n][H])."""
    I = W13.shape[0] // 2
    g = X @ W13[:I].T
    u = X @ W13[I:].T
    h = silu(g) * u
    return h, h @ W2.T


def _expert_mats(w, e, G, quant, prefix="w"):
    def m(name):
        t = w.get(f"{prefix}{name}")
        if t is None:
            return None
        return t[e] if e is not None else t
    W13 = dequant(m("13"), m("13_scale"), m("13_min"), G, quant)
    W2 = dequant(m("2"), m("2_scale"), m("2_min"), G, quant)
    return W13, W2


def expert_ffn(xf, sorted_pairs, offsets, k: int, w: dict, G: int, quant: str, cache=None):
    """Run every routed expert on its rows, in expert-sorted order.

    Row r of expert e (offsets[e] <= r < offsets[e+1]) is the token
    sorted_pairs[r] // k. Returns (h_perm [P][I], y_perm [P][H]) float64,
    unweighted. `cache` (a dict) keeps dequantized experts between calls on
    the same weights.
    """
    xf = np.asarray(xf, np.float64)
    E = len(offsets) - 1
    P = int(offsets[-1])
    I = w["w13"].shape[1] // 2
    H = xf.shape[1]
    h_perm = np.zeros((P, I))
    y_perm = np.zeros((P, H))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        if cache is None:
            W13, W2 = _expert_mats(w, e, G, quant)
        else:
            if e not in cache:
                cache[e] = _expert_mats(w, e, G, quant)
            W13, W2 = cache[e]
        X = xf[np.asarray(sorted_pairs[a:b]) // k]
        h, y = swiglu_expert(X, W13, W2)
        h_perm[a:b] = h
        y_perm[a:b] = y
    return h_perm, y_perm


def shared_expert(xf, w: dict, G: int, quant: str, cache=None):
    if cache is None:
        W13, W2 = _expert_mats(w, None, G, quant, prefix="s")
    else:
        if "shared" not in cache:
            cache["shared"] = _expert_mats(w, None, G, quant, prefix="s")
        W13, W2 = cache["shared"]
    return swiglu_expert(np.asarray(xf, np.float64), W13, W2)


def combine(y_perm, inv, topk_w, y_shared=None, shared_w=None, residual=None):
    """out[t] = sum_j w[t,j] * y_perm[inv[t*k+j]] (+ sigma[t] * y_shared[t])
    (+ residual[t]), float64."""
    T, k = np.asarray(topk_w).shape
    yp = np.asarray(y_perm, np.float64)[np.asarray(inv).reshape(T, k)]   # [T][k][H]
    out = np.einsum("tk,tkh->th", np.asarray(topk_w, np.float64), yp)
    if y_shared is not None:
        out = out + np.asarray(shared_w, np.float64)[:, None] * np.asarray(y_shared, np.float64)
    if residual is not None:
        out = out + np.asarray(residual, np.float64)
    return out


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def _weights_dict(li) -> dict:
    """Accept either a dict of numpy arrays or an object with attributes
    (numpy or CPU torch tensors)."""
    names = ["w_router", "router_bias", "shared_gate", "w13", "w13_scale", "w13_min",
             "w2", "w2_scale", "w2_min", "s13", "s13_scale", "s13_min",
             "s2", "s2_scale", "s2_min", "norm_weight"]
    d = {}
    for n in names:
        v = li.get(n) if isinstance(li, dict) else getattr(li, n, None)
        if v is None:
            d[n] = None
            continue
        if hasattr(v, "detach"):
            v = v.detach().cpu()
            if str(v.dtype) == "torch.float16":
                v = v.view(dtype=__import__("torch").int16).numpy().view(np.uint16)
            else:
                v = v.numpy()
        d[n] = np.asarray(v)
    return d


def moe_layer(x_bits, li, k: int, G: int, quant: str, logits32=None, residual_bits=None,
              cache=None):
    """One MoE layer on bf16 activations x_bits [T][H] (uint16 bit patterns).

    If logits32 is given (fp32 [T][E]) the top-k decision is taken on those
    logits instead of the oracle's own (teacher forcing for parity checks);
    everything after the decision is recomputed here. Returns a dict with
    every intermediate: logits (float64), logits32, ids, weights, counts,
    offsets, sorted_pairs, inv, h_perm, y_perm, shared_w, y_shared, out
    (float64, before the final bf16 rounding). `cache` (a dict) keeps the
    dequantized experts of these weights between calls.
    """
    w = _weights_dict(li)
    xf = bf16_to_f64(x_bits)
    E = w["w_router"].shape[0]
    L = router_logits(xf, w["w_router"], w["router_bias"])
    L32 = L.astype(np.float32) if logits32 is None else np.asarray(logits32, np.float32)
    ids, tw = select_topk(L32, k)
    counts, offsets, sorted_pairs, inv = permute(ids, E)
    h_perm, y_perm = expert_ffn(xf, sorted_pairs, offsets, k, w, G, quant, cache=cache)
    sw = ys = hs = None
    if w["s13"] is not None:
        sw = shared_gate(xf, w["shared_gate"])
        hs, ys = shared_expert(xf, w, G, quant, cache=cache)
    res = bf16_to_f64(residual_bits) if residual_bits is not None else None
    out = combine(y_perm, inv, tw, ys, sw, res)
    return dict(logits=L, logits32=L32, ids=ids, weights=tw, counts=counts, offsets=offsets,
                sorted_pairs=sorted_pairs, inv=inv, h_perm=h_perm, y_perm=y_perm,
                shared_w=sw, h_shared=hs, y_shared=ys, out=out)


def moe_layer_rows(x_bits, rows, li, k: int, G: int, quant: str, logits32_rows=None,
                   residual_bits=None, cache=None):
    """Layer output for a subset of tokens only (tokens do not interact in
    an MoE FFN, so each token's output depends on its own row alone).

    rows: token indices; x_bits: the full [T][H] activation tensor (only the
    listed rows are read); logits32_rows: fp32 logits of those rows for
    teacher forcing. `cache` (a dict) keeps dequantized experts between calls.
    Returns dict(ids, weights, logits, out) for the listed rows.
    """
    w = _weights_dict(li)
    rows = np.asarray(rows, dtype=np.int64)
    xf = bf16_to_f64(np.asarray(x_bits)[rows])
    L = router_logits(xf, w["w_router"], w["router_bias"])
    L32 = L.astype(np.float32) if logits32_rows is None else np.asarray(logits32_rows, np.float32)
    ids, tw = select_topk(L32, k)
    cache = {} if cache is None else cache
    out = np.zeros_like(xf)
    for i in range(len(rows)):
        for j in range(k):
            e = int(ids[i, j])
            if e not in cache:
                cache[e] = _expert_mats(w, e, G, quant)
            W13, W2 = cache[e]
            _, y = swiglu_expert(xf[i:i + 1], W13, W2)
            out[i] += tw[i, j] * y[0]
    if w["s13"] is not None:
        if "shared" not in cache:
            cache["shared"] = _expert_mats(w, None, G, quant, prefix="s")
        W13, W2 = cache["shared"]
        _, ys = swiglu_expert(xf, W13, W2)
        out += shared_gate(xf, w["shared_gate"])[:, None] * ys
    if residual_bits is not None:
        out += bf16_to_f64(np.asarray(residual_bits)[rows])
    return dict(ids=ids, weights=tw, logits=L, out=out)


def rmsnorm(x_bits, weight, eps: float) -> np.ndarray:
    """RMSNorm: x * (mean_h x^2 + eps)^(-1/2) * g, float64 (eps inside the
    square root)."""
    xf = bf16_to_f64(x_bits)
    r = 1.0 / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + eps)
    return xf * r * np.asarray(weight, np.float64)[None, :]


def stack_layer(x_bits, li, k: int, G: int, quant: str, eps: float, cache=None):
    """One pre-norm layer of the stack on bf16 rows x_bits:
    x <- bf16(x + MoE(bf16(RMSNorm(x)))). Returns (new x bits, the layer's
    moe_layer dict, which holds its routing decisions)."""
    w = _weights_dict(li)
    xn = round_to_bf16(rmsnorm(x_bits, w["norm_weight"], eps))
    res = moe_layer(xn, li, k, G, quant, residual_bits=x_bits, cache=cache)
    return round_to_bf16(res["out"]), res


def moe_stack(x_bits, layers, k: int, G: int, quant: str, eps: float, chunk: int = 0):
    """Pre-norm stack: for each chunk of rows, for each layer l,
    x <- bf16(x + MoE_l(bf16(RMSNorm_l(x)))). Returns bf16 bits [T][H]."""
    x = np.array(x_bits, dtype=np.uint16, copy=True)
    T = x.shape[0]
    chunk = T if chunk <= 0 else chunk
    for r0 in range(0, T, chunk):
        xc = x[r0:r0 + chunk]
        for li in layers:
            xc, _ = stack_layer(xc, li, k, G, quant, eps)
        x[r0:r0 + chunk] = xc
    return x


# ---------------------------------------------------------------------------
# integer route: 8-bit activations x symmetric 4-bit experts
# ---------------------------------------------------------------------------
#
# The pages name an integer MoE prefill route for the symmetric expert file
# (hipfire 0.4.3 benchmarks page, "Read this before comparing columns": the
# "symmetric IU4 MoE" route, admitted only on the symmetric file) and an INT8
# prefill route that replaced an F16 one within a stated quality budget
# (same page, "Qwen3.8-Flash (Flash-Next)" table, first row). They fix no
# activation format. The reading used here: each activation row (a token's
# x, and each (token, expert) row of h) is quantized to 8-bit integers with
# one scale per row; the products with the 4-bit weights are then exact
# integer dot products, and the layer is the exact layer evaluated on the
# 8-bit-rounded activations. So the oracle below is the plain layer on
# dequantized activations: x^ = q_x * s_x, h^ = q_h * s_h. h is rounded to
# fp16 before its quantization (the GPU route stores h as fp16 between its
# two products, and a quantized code is decided on the value actually
# quantized).

_I8_TINY = 2.0 ** -100


def quantize_rows_i8(v32):
    """Per-row symmetric 8-bit quantization of float32 rows [R][C].

    The decisions are taken in binary32 (the precision of the GPU route):
    a = max |v| of the row; r = 127 / a and s = a / 127, each a correctly
    rounded binary32 division; q = rint(v * r), the product rounded to
    binary32 and then to the nearest integer (ties to even), which lies in
    [-127, 127] because v * r <= 127 (1 + 2^-24). A row with a < 2^-100
    (in particular an all-zero row) gets q = 0 and s = 0.
    Returns (q int8 [R][C], s float32 [R]).
    """
    v = np.asarray(v32, dtype=np.float32)
    a = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    ok = a >= np.float32(_I8_TINY)
    a_safe = np.where(ok, a, np.float32(1.0)).astype(np.float32)
    r = (np.float32(127.0) / a_safe).astype(np.float32)
    s = np.where(ok, (a_safe / np.float32(127.0)).astype(np.float32), np.float32(0.0))
    prod = (v * r[:, None]).astype(np.float32)
    q = np.clip(np.rint(prod), -127, 127)
    q = np.where(ok[:, None], q, 0.0).astype(np.int8)
    return q, s.astype(np.float32)


def dequant_rows_i8(q, s) -> np.ndarray:
    """q [R][C] int8, s [R] -> float64 q * s (exact)."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[:, None]


def _f16_round(v) -> np.ndarray:
    """float64 -> nearest fp16 (ties to even), as float64."""
    return np.asarray(v, np.float64).astype(np.float16).astype(np.float64)


def _i8_gateup(Xhat, W13):
    """Gate/up of one expert on the integer route: Xhat [n][H] are
    dequantized 8-bit activations. Returns h [n][I] rounded to fp16."""
    I = W13.shape[0] // 2
    return _f16_round(silu(Xhat @ W13[:I].T) * (Xhat @ W13[I:].T))


def _i8_down(h16, W2):
    """Down projection of fp16 h rows on the integer route: returns
    (hq, sh, y)."""
    hq, sh = quantize_rows_i8(np.asarray(h16, np.float64).astype(np.float32))
    return hq, sh, dequant_rows_i8(hq, sh) @ W2.T


def expert_ffn_i8(x_bits, sorted_pairs, offsets, k: int, w: dict, G: int, h16_forced=None):
    """The routed experts on the integer route (symmetric weights only).

    1. x (bf16) -> q_x, s_x per token (quantize_rows_i8);
    2. row r of expert e (offsets[e] <= r < offsets[e+1]) is token
       t = sorted_pairs[r] // k: h = silu(x^_t Wg^T) * (x^_t Wu^T),
       x^ = q_x s_x, rounded to fp16;
    3. h -> q_h, s_h per row (quantize_rows_i8 on the fp16 values);
    4. y_perm[r] = h^_r Wd^T, h^ = q_h s_h.
    Products in float64 on the dequantized weights. Returns a dict with xq,
    sx, h16 [P][I], hq, sh [P], y_perm [P][H] (float64, unweighted).

    h16_forced [P][I] (teacher forcing): steps 3-4 take these fp16 values
    instead of the oracle's own h. A quantized code is decided on the value
    actually quantized; h computed in another order rounds to fp16
    differently in rare cases, and then a code can differ by one step.
    """
    xq, sx = quantize_rows_i8(bf16_to_f64(x_bits).astype(np.float32))
    xhat = dequant_rows_i8(xq, sx)
    E = len(offsets) - 1
    P = int(offsets[-1])
    I = w["w13"].shape[1] // 2
    H = xhat.shape[1]
    h16 = np.zeros((P, I))
    hq = np.zeros((P, I), np.int8)
    sh = np.zeros(P, np.float32)
    y = np.zeros((P, H))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        W13, W2 = _expert_mats(w, e, G, "sym")
        X = xhat[np.asarray(sorted_pairs[a:b]) // k]
        h16[a:b] = _i8_gateup(X, W13)
        hin = h16[a:b] if h16_forced is None else np.asarray(h16_forced, np.float64)[a:b]
        hq[a:b], sh[a:b], y[a:b] = _i8_down(hin, W2)
    return dict(xq=xq, sx=sx, h16=h16, hq=hq, sh=sh, y_perm=y)


def moe_layer_i8(x_bits, li, k: int, G: int, logits32=None, residual_bits=None,
                 h16_forced=None):
    """One MoE layer on the integer route: routing exactly as moe_layer (on
    the bf16 activations, fp32 logits, optional teacher forcing), experts by
    expert_ffn_i8 (h16_forced as there), combine as moe_layer. No shared
    expert."""
    w = _weights_dict(li)
    if w["s13"] is not None:
        raise ValueError("the integer route has no shared expert")
    xf = bf16_to_f64(x_bits)
    E = w["w_router"].shape[0]
    L = router_logits(xf, w["w_router"], w["router_bias"])
    L32 = L.astype(np.float32) if logits32 is None else np.asarray(logits32, np.float32)
    ids, tw = select_topk(L32, k)
    counts, offsets, sorted_pairs, inv = permute(ids, E)
    f = expert_ffn_i8(x_bits, sorted_pairs, offsets, k, w, G, h16_forced=h16_forced)
    res = bf16_to_f64(residual_bits) if residual_bits is not None else None
    out = combine(f["y_perm"], inv, tw, None, None, res)
    f.update(logits=L, logits32=L32, ids=ids, weights=tw, counts=counts, offsets=offsets,
             sorted_pairs=sorted_pairs, inv=inv, out=out)
    return f


def moe_layer_rows_i8(x_bits, rows, li, k: int, G: int, logits32_rows=None, cache=None,
                      h16_rows=None):
    """moe_layer_i8's output for a subset of tokens (each token's output,
    its activation scale and its k rows of h depend on its own x row only).
    h16_rows [len(rows)][k][I]: teacher forcing of the fp16 h of each
    (token, slot), as in expert_ffn_i8. Returns dict(ids, weights, out, h16)
    for the listed rows."""
    w = _weights_dict(li)
    rows = np.asarray(rows, dtype=np.int64)
    xb = np.asarray(x_bits)[rows]
    xf = bf16_to_f64(xb)
    L = router_logits(xf, w["w_router"], w["router_bias"])
    L32 = L.astype(np.float32) if logits32_rows is None else np.asarray(logits32_rows, np.float32)
    ids, tw = select_topk(L32, k)
    xq, sx = quantize_rows_i8(xf.astype(np.float32))
    xhat = dequant_rows_i8(xq, sx)
    cache = {} if cache is None else cache
    out = np.zeros_like(xf)
    I = w["w13"].shape[1] // 2
    h16 = np.zeros((len(rows), k, I))
    for i in range(len(rows)):
        for j in range(k):
            e = int(ids[i, j])
            if e not in cache:
                cache[e] = _expert_mats(w, e, G, "sym")
            W13, W2 = cache[e]
            h16[i, j] = _i8_gateup(xhat[i:i + 1], W13)[0]
            hin = h16[i, j] if h16_rows is None else np.asarray(h16_rows, np.float64)[i, j]
            out[i] += tw[i, j] * _i8_down(hin[None, :], W2)[2][0]
    return dict(ids=ids, weights=tw, logits=L, out=out, h16=h16)


# ---------------------------------------------------------------------------
# lower-bit expert tiers (3 and 2 bits) beside 4-bit experts
# ---------------------------------------------------------------------------
#
# The pages ship expert files where most routed experts are stored below
# 4 bits and the rest stay at 4 bits (hipfire 0.4.3 benchmarks page, "New
# Flash-Next tiers": 3-bit experts on part of the routed experts; 2-bit
# experts, there with an E8P codebook, on others). They define neither
# format. The reading used here: plain symmetric scalar codes of b bits per
# weight, w = (q - 2^(b-1)) * scale with one fp16 scale per group of G along
# K, in this library's row layouts (stated in unpack_codes). E8P's lattice
# codebook is not defined on the pages and is not reproduced.

def unpack_codes(packed, bits: int) -> np.ndarray:
    """Packed rows [R][K*bits/8] -> codes [R][K] (0 .. 2^bits - 1).

    4 bits: byte j holds element 2j in bits 0-3 and 2j+1 in bits 4-7.
    2 bits: little-endian 32-bit word m holds elements 16m .. 16m+15; its
            bytes 0, 1, 2, 3 hold the word's elements 0-3, 8-11, 4-7, 12-15,
            element i of a byte's four in bits 2i and 2i+1.
    3 bits: 12 bytes per 32-element block: 8 bytes of the elements' low two
            bits in the 2-bit layout, then a 32-bit word whose bit 4c+i is the
            high bit of element 8c+i and bit 16+4c+i that of element 8c+i+4
            (c, i in 0..3).
    """
    p = np.asarray(packed, dtype=np.uint8)
    if bits == 4:
        return unpack_nibbles(p)
    R = p.shape[0]
    if bits == 2:
        words = p.reshape(R, -1, 4).astype(np.int64)
        out = np.empty((R, words.shape[1], 16), dtype=np.int64)
        for b, first in enumerate((0, 8, 4, 12)):     # byte b of a word -> its four elements
            for i in range(4):
                out[:, :, first + i] = (words[:, :, b] >> (2 * i)) & 3
        return out.reshape(R, -1)
    if bits == 3:
        blocks = p.reshape(R, -1, 12)
        low = unpack_codes(blocks[:, :, :8].reshape(R, -1), 2).reshape(R, -1, 32)
        hw = blocks[:, :, 8:12].astype(np.int64)
        h = hw[:, :, 0] | (hw[:, :, 1] << 8) | (hw[:, :, 2] << 16) | (hw[:, :, 3] << 24)
        high = np.zeros_like(low)
        for c in range(4):
            for i in range(4):
                high[:, :, 8 * c + i] = (h >> (4 * c + i)) & 1
                high[:, :, 8 * c + i + 4] = (h >> (16 + 4 * c + i)) & 1
        return (low + 4 * high).reshape(R, -1)
    raise ValueError(f"unsupported width {bits}")


def dequant_bits(packed, scale, G: int, bits: int) -> np.ndarray:
    """Symmetric b-bit weights [R][K]: w = (q - 2^(b-1)) * scale[r, k // G]."""
    q = unpack_codes(packed, bits).astype(np.float64) - float(1 << (bits - 1))
    s = f16_to_f64(scale)
    return q * np.repeat(s, G, axis=1)


def _mixed_mats(ml, e, G):
    b = int(ml.bits[e])
    j = int(ml.slot[e])
    w13, s13, w2, s2 = (np.asarray(t.detach().cpu().numpy() if hasattr(t, "detach") else t)
                        for t in ml.tiers[b])
    if s13.dtype == np.float16:
        s13, s2 = s13.view(np.uint16), s2.view(np.uint16)
    return dequant_bits(w13[j], s13[j], G, b), dequant_bits(w2[j], s2[j], G, b)


def moe_layer_mixed(x_bits, ml, k: int, G: int, logits32=None):
    """One layer whose expert e is stored with ml.bits[e] bits per weight:
    routing as moe_layer (fp32 logits, optional teacher forcing), each
    expert's SwiGLU FFN on its dequantized weights, combine. Returns the
    routing arrays, y_perm and out (float64)."""
    w_router = ml.w_router.detach().cpu().numpy() if hasattr(ml.w_router, "detach") else ml.w_router
    bias = ml.router_bias
    if bias is not None and hasattr(bias, "detach"):
        bias = bias.detach().cpu().numpy()
    xf = bf16_to_f64(x_bits)
    E = w_router.shape[0]
    L = router_logits(xf, w_router, bias)
    L32 = L.astype(np.float32) if logits32 is None else np.asarray(logits32, np.float32)
    ids, tw = select_topk(L32, k)
    counts, offsets, sorted_pairs, inv = permute(ids, E)
    P = int(offsets[-1])
    y = np.zeros((P, xf.shape[1]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        W13, W2 = _mixed_mats(ml, e, G)
        _, y[a:b] = swiglu_expert(xf[np.asarray(sorted_pairs[a:b]) // k], W13, W2)
    out = combine(y, inv, tw)
    return dict(logits=L, logits32=L32, ids=ids, weights=tw, counts=counts, offsets=offsets,
                sorted_pairs=sorted_pairs, inv=inv, y_perm=y, out=out)
