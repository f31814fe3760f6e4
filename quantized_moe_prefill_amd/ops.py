"""Python binding of the C ABI (include/moe.h), one function per entry point.

Argument marshalling only: each function checks dtypes, devices and
contiguity, allocates outputs and the workspace with torch (device memory is
the only thing torch provides here), and passes raw device pointers and
torch's current HIP stream to the library. Every step of the computation
runs in the library's kernels.
"""
from __future__ import annotations

import copy
import ctypes
import dataclasses
from typing import Optional

import torch

from . import _native as N

_U16 = (torch.bfloat16, torch.float16, torch.int16, torch.uint16)


def make_shape(H: int, E: int, k: int, I: int, G: int, quant: str, shared_I: int = 0,
               w_layout: int = N.MOE_W_ROWS) -> N.MoeShape:
    q = {"sym": N.MOE_Q4_SYM, "asym": N.MOE_Q4_ASYM}[quant]
    return N.MoeShape(H, E, k, I, G, q, w_layout, shared_I)


def shape_of(cfg, w_layout: int = N.MOE_W_ROWS) -> N.MoeShape:
    """Shape struct of a synth.MoEConfig (expert weights in `w_layout`)."""
    return make_shape(cfg.H, cfg.E, cfg.k, cfg.I, cfg.G, cfg.quant, cfg.shared_I, w_layout)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes=None, device=None) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Experts:
    """Packed expert weights of one layer as the C struct (keeps the tensors
    alive). Accepts any object with the attribute names of synth.LayerInputs."""

    def __init__(self, li):
        u8 = (torch.uint8,)
        names = ["w13", "w13_scale", "w13_min", "w2", "w2_scale", "w2_min",
                 "s13", "s13_scale", "s13_min", "s2", "s2_scale", "s2_min"]
        self.tensors = {n: getattr(li, n, None) for n in names}
        vals = []
        for n in names:
            t = self.tensors[n]
            dt = u8 if n in ("w13", "w2", "s13", "s2") else _U16
            vals.append(_ptr(t, n, dt))
        self.struct = N.MoeExperts(*vals)
        self.device = self.tensors["w13"].device

    def ref(self):
        return ctypes.byref(self.struct)


def moe_pack_w4(src: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    """The MOE_W_TILED copy of one packed 4-bit matrix src [rows][K/2] (u8,
    any leading shape with that many bytes)."""
    dev = src.device
    if src.numel() != rows * K // 2:
        raise ValueError(f"src holds {src.numel()} bytes, expected rows * K / 2 = {rows * K // 2}")
    dst = torch.empty_like(src)
    N.check(N.lib().moe_pack_w4(_ptr(src, "src", (torch.uint8,), dev), _ptr(dst, "dst", (torch.uint8,), dev),
                                int(rows), int(K), _stream(dev)))
    return dst


def moe_pack_tier(src: torch.Tensor, rows: int, K: int, bits: int, gate_up: bool) -> torch.Tensor:
    """The MOE_W_TILED copy of one packed matrix of a mixed-width tier,
    src [rows][K * bits / 8] (u8, any leading shape with that many bytes);
    gate_up: a w13 matrix (its 3- and 2-bit rows are also put in the order
    the gate/up kernel reads them)."""
    dev = src.device
    if src.numel() != rows * K * bits // 8:
        raise ValueError(f"src holds {src.numel()} bytes, expected rows * K * bits / 8 = "
                         f"{rows * K * bits // 8}")
    dst = torch.empty_like(src)
    N.check(N.lib().moe_pack_tier(_ptr(src, "src", (torch.uint8,), dev),
                                  _ptr(dst, "dst", (torch.uint8,), dev), int(rows), int(K),
                                  int(bits), 1 if gate_up else 0, _stream(dev)))
    return dst


def pack_mixed(cfg, ml):
    """A copy of a mixed-width layer (synth.MixedLayer or alike) whose tiers'
    w13 and w2 are in the MOE_W_TILED layout (moe_pack_tier), for the
    mixed-width calls with shape_of(cfg, N.MOE_W_TILED). Scales are shared."""
    out = dataclasses.replace(ml) if dataclasses.is_dataclass(ml) else copy.copy(ml)
    H, I = cfg.H, cfg.I
    tiers = {}
    for b, (w13, s13, w2, s2) in ml.tiers.items():
        n = int(w13.shape[0])
        tiers[b] = (moe_pack_tier(w13, n * 2 * I, H, int(b), True), s13,
                    moe_pack_tier(w2, n * H, I, int(b), False), s2)
    out.tiers = tiers
    return out


def pack_layer(cfg, li):
    """A copy of a layer's tensors (synth.LayerInputs or alike) whose four
    4-bit matrices (w13, w2 and the shared expert's s13, s2) are in the
    MOE_W_TILED layout, for calls with shape_of(cfg, N.MOE_W_TILED). The
    other tensors are shared with li."""
    out = dataclasses.replace(li) if dataclasses.is_dataclass(li) else copy.copy(li)
    E, H, I, Is = cfg.E, cfg.H, cfg.I, cfg.shared_I
    out.w13 = moe_pack_w4(li.w13, E * 2 * I, H)
    out.w2 = moe_pack_w4(li.w2, E * H, I)
    if Is > 0 and getattr(li, "s13", None) is not None:
        out.s13 = moe_pack_w4(li.s13, 2 * Is, H)
        out.s2 = moe_pack_w4(li.s2, H, Is)
    return out


def moe_workspace_size(shape: N.MoeShape, T: int, kind: int = N.MOE_WS_LAYER) -> int:
    n = ctypes.c_size_t(0)
    N.check(N.lib().moe_workspace_size(ctypes.byref(shape), int(T), int(kind), ctypes.byref(n)))
    return n.value


def workspace(shape: N.MoeShape, T: int, device, kind: int = N.MOE_WS_LAYER) -> torch.Tensor:
    n = moe_workspace_size(shape, T, kind)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(shape, x, w_router, router_bias=None, shared_gate=None, want_logits=False,
              ws=None):
    T = x.shape[0]
    dev = x.device
    E, k = shape.num_experts, shape.top_k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    sw = torch.empty((T,), dtype=torch.float32, device=dev) if shared_gate is not None else None
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_ROUTE)
    N.check(N.lib().moe_route(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), _ptr(w_router, "w_router", (torch.float32,), dev),
        _ptr(router_bias, "router_bias", (torch.float32,), dev),
        _ptr(shared_gate, "shared_gate", (torch.float32,), dev), _ptr(logits, "logits"),
        _ptr(ids, "ids"), _ptr(tw, "tw"), _ptr(sw, "sw"), _ptr(ws, "ws"), ws.numel(), _stream(dev)))
    return logits, ids, tw, sw


def moe_permute(shape, topk_ids, ws=None):
    T = topk_ids.shape[0]
    dev = topk_ids.device
    E, k = shape.num_experts, shape.top_k
    P = T * k
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sp = torch.empty((max(P, 1),), dtype=torch.int32, device=dev)
    inv = torch.empty((max(P, 1),), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_PERMUTE)
    N.check(N.lib().moe_permute(
        ctypes.byref(shape), T, _ptr(topk_ids, "topk_ids", (torch.int32,), dev), _ptr(counts, "counts"),
        _ptr(offsets, "offsets"), _ptr(sp, "sorted_pairs"), _ptr(inv, "inv"), _ptr(ws, "ws"),
        ws.numel(), _stream(dev)))
    return counts, offsets, sp[:P], inv[:P]


def moe_expert_ffn(shape, x, experts: Experts, counts, offsets, sorted_pairs, ws=None):
    T = x.shape[0]
    dev = x.device
    P = T * shape.top_k
    y_perm = torch.empty((max(P, 1), shape.hidden), dtype=torch.float16, device=dev)
    y_sh = (torch.empty((T, shape.hidden), dtype=torch.float16, device=dev)
            if shape.shared_inter else None)
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_EXPERT_FFN)
    N.check(N.lib().moe_expert_ffn(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), experts.ref(),
        _ptr(counts, "counts", (torch.int32,), dev), _ptr(offsets, "offsets", (torch.int32,), dev),
        _ptr(sorted_pairs, "sorted_pairs", (torch.int32,), dev), _ptr(y_perm, "y_perm"),
        _ptr(y_sh, "y_shared"), _ptr(ws, "ws"), ws.numel(), _stream(dev)))
    return y_perm[:P], y_sh


def moe_combine(shape, y_perm, inv, topk_w, y_shared=None, shared_w=None, residual=None,
                out=None):
    T = topk_w.shape[0]
    dev = topk_w.device
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device=dev)
    N.check(N.lib().moe_combine(
        ctypes.byref(shape), T, _ptr(y_perm, "y_perm", _U16, dev), _ptr(inv, "inv", (torch.int32,), dev),
        _ptr(topk_w, "topk_w", (torch.float32,), dev), _ptr(y_shared, "y_shared", _U16, dev),
        _ptr(shared_w, "shared_w", (torch.float32,), dev), _ptr(residual, "residual", _U16, dev),
        _ptr(out, "out", _U16, dev), _stream(dev)))
    return out


def moe_layer_forward(shape, x, w_router, router_bias, shared_gate, experts: Experts,
                      residual=None, out=None, ws=None):
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_LAYER)
    N.check(N.lib().moe_layer_forward(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), _ptr(w_router, "w_router", (torch.float32,), dev),
        _ptr(router_bias, "router_bias", (torch.float32,), dev),
        _ptr(shared_gate, "shared_gate", (torch.float32,), dev), experts.ref(),
        _ptr(residual, "residual", _U16, dev), _ptr(out, "out", _U16, dev), _ptr(ws, "ws"),
        ws.numel(), _stream(dev)))
    return out


def moe_layer_forward_static(shape, x, w_router, router_bias, shared_gate, experts: Experts,
                             residual=None, out=None):
    """moe_layer_forward with its intermediates in the library's static
    per-GPU workspace (no workspace argument; the call allocates nothing
    besides `out` when it is not given)."""
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device=dev)
    N.check(N.lib().moe_layer_forward_static(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), _ptr(w_router, "w_router", (torch.float32,), dev),
        _ptr(router_bias, "router_bias", (torch.float32,), dev),
        _ptr(shared_gate, "shared_gate", (torch.float32,), dev), experts.ref(),
        _ptr(residual, "residual", _U16, dev), _ptr(out, "out", _U16, dev), _stream(dev)))
    return out


def moe_quantize_rows_i8(x):
    """bf16 rows [R][C] -> (int8 codes [R][C], fp32 scales [R])."""
    R, C = x.shape
    dev = x.device
    q = torch.empty((R, C), dtype=torch.int8, device=dev)
    sc = torch.empty((max(R, 1),), dtype=torch.float32, device=dev)
    N.check(N.lib().moe_quantize_rows_i8(R, C, _ptr(x, "x", _U16, dev), _ptr(q, "q"),
                                         _ptr(sc, "scale"), _stream(dev)))
    return q, sc[:R]


def moe_expert_ffn_i8(shape, x, experts: Experts, counts, offsets, sorted_pairs, ws=None,
                      want_h=False):
    """Returns y_perm, or (y_perm, h_perm) with want_h (the fp16 h rows the
    int8 h was quantized from)."""
    T = x.shape[0]
    dev = x.device
    P = T * shape.top_k
    y_perm = torch.empty((max(P, 1), shape.hidden), dtype=torch.float16, device=dev)
    h = torch.empty((max(P, 1), shape.inter), dtype=torch.float16, device=dev) if want_h else None
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_EXPERT_FFN_I8)
    N.check(N.lib().moe_expert_ffn_i8(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), experts.ref(),
        _ptr(counts, "counts", (torch.int32,), dev), _ptr(offsets, "offsets", (torch.int32,), dev),
        _ptr(sorted_pairs, "sorted_pairs", (torch.int32,), dev), _ptr(y_perm, "y_perm"),
        _ptr(h, "h_perm"), _ptr(ws, "ws"), ws.numel(), _stream(dev)))
    return (y_perm[:P], h[:P]) if want_h else y_perm[:P]


def moe_layer_forward_i8(shape, x, w_router, router_bias, experts: Experts, residual=None,
                         out=None, ws=None):
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_LAYER_I8)
    N.check(N.lib().moe_layer_forward_i8(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), _ptr(w_router, "w_router", (torch.float32,), dev),
        _ptr(router_bias, "router_bias", (torch.float32,), dev), experts.ref(),
        _ptr(residual, "residual", _U16, dev), _ptr(out, "out", _U16, dev), _ptr(ws, "ws"),
        ws.numel(), _stream(dev)))
    return out


class MixedExperts:
    """Mixed-width expert weights of one layer as the C tier array plus the
    per-expert width and slot arrays on the device (keeps the tensors
    alive). Accepts a synth.MixedLayer (or any object with `bits`, `slot`
    and `tiers` = {bits: (w13, w13_scale, w2, w2_scale)})."""

    def __init__(self, ml, device):
        self.keep = []
        tiers = []
        for b, (w13, s13, w2, s2) in sorted(ml.tiers.items(), reverse=True):
            self.keep += [w13, s13, w2, s2]
            tiers.append(N.MoeTier(int(b), int(w13.shape[0]), _ptr(w13, "w13", (torch.uint8,)),
                                   _ptr(s13, "w13_scale", _U16), _ptr(w2, "w2", (torch.uint8,)),
                                   _ptr(s2, "w2_scale", _U16)))
        self.n = len(tiers)
        self.array = (N.MoeTier * self.n)(*tiers)
        self.bits = torch.tensor(list(ml.bits), dtype=torch.int32, device=device)
        self.slot = torch.tensor(list(ml.slot), dtype=torch.int32, device=device)


def moe_expert_ffn_mixed(shape, x, experts: MixedExperts, counts, offsets, sorted_pairs, ws=None):
    T = x.shape[0]
    dev = x.device
    P = T * shape.top_k
    y_perm = torch.empty((max(P, 1), shape.hidden), dtype=torch.float16, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_EXPERT_FFN)
    N.check(N.lib().moe_expert_ffn_mixed(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), experts.array, experts.n,
        _ptr(experts.bits, "expert_bits"), _ptr(experts.slot, "expert_slot"),
        _ptr(counts, "counts", (torch.int32,), dev), _ptr(offsets, "offsets", (torch.int32,), dev),
        _ptr(sorted_pairs, "sorted_pairs", (torch.int32,), dev), _ptr(y_perm, "y_perm"),
        _ptr(ws, "ws"), ws.numel(), _stream(dev)))
    return y_perm[:P]


def moe_layer_forward_mixed(shape, x, w_router, router_bias, experts: MixedExperts, residual=None,
                            out=None, ws=None):
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = workspace(shape, T, dev, N.MOE_WS_LAYER)
    N.check(N.lib().moe_layer_forward_mixed(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), _ptr(w_router, "w_router", (torch.float32,), dev),
        _ptr(router_bias, "router_bias", (torch.float32,), dev), experts.array, experts.n,
        _ptr(experts.bits, "expert_bits"), _ptr(experts.slot, "expert_slot"),
        _ptr(residual, "residual", _U16, dev), _ptr(out, "out", _U16, dev), _ptr(ws, "ws"),
        ws.numel(), _stream(dev)))
    return out


def _host_ptr(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu":
        raise ValueError(f"{name} must be a host (CPU) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class StreamedExperts:
    """A layer's experts split into a device-resident hot set and host-
    resident (pinned) cold experts, for moe_layer_forward_streamed. `li` has
    the attribute names of synth.LayerInputs (symmetric, no shared expert);
    `hot` lists the expert indices kept on `device`."""

    def __init__(self, li, hot, device, pin=True):
        E = li.w13.shape[0]
        hot = sorted(set(int(e) for e in hot))
        cold = [e for e in range(E) if e not in set(hot)]
        self.hot_slot = (ctypes.c_int32 * E)(*[-1] * E)
        for j, e in enumerate(hot):
            self.hot_slot[e] = j
        names = ("w13", "w13_scale", "w2", "w2_scale")
        self.hot_t = {n: getattr(li, n)[hot].to(device).contiguous() for n in names} if hot else {}
        self.cold_t = {}
        for n in names:
            t = getattr(li, n)[cold].to("cpu").contiguous() if cold else None
            self.cold_t[n] = t.pin_memory() if (t is not None and pin) else t
        self.n_hot = len(hot)
        self.n_cold = len(cold)
        h = self.hot_t
        self.hot = N.MoeExperts(*(_ptr(h.get("w13"), "w13"), _ptr(h.get("w13_scale"), "w13_scale"), None,
                                  _ptr(h.get("w2"), "w2"), _ptr(h.get("w2_scale"), "w2_scale"), None,
                                  None, None, None, None, None, None)) if hot else None
        c = self.cold_t
        self.cold = N.MoeExperts(_host_ptr(c["w13"], "w13"), _host_ptr(c["w13_scale"], "w13_scale"),
                                 None, _host_ptr(c["w2"], "w2"), _host_ptr(c["w2_scale"], "w2_scale"),
                                 None, None, None, None, None, None, None) if cold else None

    def cold_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.cold_t.values() if t is not None)


def moe_stream_stage_bytes(shape, experts: int) -> int:
    n = ctypes.c_size_t(0)
    N.check(N.lib().moe_stream_stage_bytes(ctypes.byref(shape), int(experts), ctypes.byref(n)))
    return n.value


def moe_layer_forward_streamed(shape, x, w_router, router_bias, experts: StreamedExperts, stage,
                               residual=None, out=None, ws=None, copy_stream=None):
    """copy_stream: a torch.cuda.Stream for the host->device copies (they then
    overlap the kernels), or None to order them on the current stream.

    The copies read `experts`' pinned host tensors asynchronously, outside
    torch's pinned-memory bookkeeping: keep `experts` and `stage` alive until
    the current stream has finished this call."""
    T = x.shape[0]
    dev = x.device
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device=dev)
    if ws is None:
        n = moe_workspace_size(shape, T, N.MOE_WS_LAYER) + 8 * shape.num_experts + 512
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    N.check(N.lib().moe_layer_forward_streamed(
        ctypes.byref(shape), T, _ptr(x, "x", _U16, dev), _ptr(w_router, "w_router", (torch.float32,), dev),
        _ptr(router_bias, "router_bias", (torch.float32,), dev),
        ctypes.byref(experts.hot) if experts.hot is not None else None, experts.n_hot,
        ctypes.byref(experts.cold) if experts.cold is not None else None, experts.hot_slot,
        _ptr(stage, "stage"), stage.numel() if stage is not None else 0,
        _ptr(residual, "residual", _U16, dev), _ptr(out, "out", _U16, dev), _ptr(ws, "ws"),
        ws.numel(), _stream(dev), copy_stream.cuda_stream if copy_stream is not None else None))
    return out


def moe_rmsnorm(x, weight, eps: float, out=None):
    T, H = x.shape
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    N.check(N.lib().moe_rmsnorm(T, H, _ptr(x, "x", _U16, dev), _ptr(weight, "weight", (torch.float32,), dev),
                                ctypes.c_float(eps), _ptr(out, "out", _U16, dev), _stream(dev)))
    return out


# ---- profiling ------------------------------------------------------------

def profile_enable(max_launches: int):
    N.check(N.lib().moe_profile_enable(int(max_launches)))


def profile_reset():
    N.check(N.lib().moe_profile_reset())


def profile_read(kernel: str):
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    N.check(N.lib().moe_profile_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


class MoELayer:
    """One layer's weights resident on the device, with a reusable
    workspace (its own, or one shared with other layers of the same shape),
    for repeated moe_layer_forward calls."""

    def __init__(self, cfg, li, device, T_max: int, ws=None, tiled: bool = False):
        # tiled: the 4-bit matrices are regrouped once into MOE_W_TILED (a
        # packed copy; li itself is left as it is)
        self.cfg = cfg
        self.shape = shape_of(cfg, N.MOE_W_TILED if tiled else N.MOE_W_ROWS)
        self.li = pack_layer(cfg, li) if tiled else li
        self.experts = Experts(self.li)
        self.ws = ws if ws is not None else workspace(self.shape, T_max, device)

    def forward(self, x, residual=None, out=None):
        return moe_layer_forward(self.shape, x, self.li.w_router, self.li.router_bias,
                                 self.li.shared_gate, self.experts, residual=residual, out=out,
                                 ws=self.ws)


class MoEStack:
    """A pre-norm stack of MoE FFN layers resident on the device (the
    attention blocks of the model are not part of it):

        for each chunk of `chunk` rows, for each layer l:
            xn = moe_rmsnorm(x, g_l)
            x  = moe_layer_forward(xn, ..., residual=x, out=x)

    i.e. x <- x + MoE_l(RMSNorm_l(x)) with a bf16 residual stream, chunk by
    chunk as a prefill engine processes a long prompt. Orchestration only:
    every step runs in the library's kernels; the layers share one
    workspace."""

    def __init__(self, cfg, layers, device, eps: float = 1e-6, chunk: int = 0,
                 tiled: bool = False):
        self.cfg = cfg
        self.eps = eps
        self.chunk = chunk if chunk > 0 else cfg.T
        shape = shape_of(cfg)
        self.ws = workspace(shape, self.chunk, device)
        self.layers = [MoELayer(cfg, li, device, self.chunk, ws=self.ws, tiled=tiled)
                       for li in layers]
        self.xn = torch.empty((self.chunk, cfg.H), dtype=torch.bfloat16, device=device)

    def layer_step(self, layer: "MoELayer", xc: torch.Tensor) -> torch.Tensor:
        """One layer on one chunk, in place: xc <- xc + MoE(RMSNorm(xc))."""
        xn = self.xn[: xc.shape[0]]
        moe_rmsnorm(xc, layer.li.norm_weight, self.eps, out=xn)
        layer.forward(xn, residual=xc, out=xc)
        return xc

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """x [T][H] bf16, updated in place and returned."""
        for r0 in range(0, x.shape[0], self.chunk):
            xc = x[r0:r0 + self.chunk]
            for layer in self.layers:
                self.layer_step(layer, xc)
        return x

    def capture(self, x: torch.Tensor) -> "torch.cuda.CUDAGraph":
        """The whole stack on the buffer x, captured once as a HIP graph:
        graph.replay() then applies all the layers to x's current contents in
        place, without a launch per kernel (every step only enqueues kernels
        on the current stream: no allocation, memset or host sync). x must
        stay allocated, and its contents are consumed by the warm-up run."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.forward(x)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x)
        torch.cuda.synchronize()
        return graph
