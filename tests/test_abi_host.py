"""Host-side checks of the C ABI: the built library loads, exports every
symbol include/moe.h declares, sizes workspaces, and rejects bad arguments
with the documented status codes before launching anything (no GPU needed:
every call here fails validation or is a pure host query)."""
import ctypes
import os
import re

import pytest

from quantized_moe_prefill_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _lib():
    if not os.path.exists(N.LIB_PATH):
        pytest.skip("library not built")
    return N.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_binding_list():
    assert _declared() == sorted(N.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 1


def _shape(**kw):
    d = dict(hidden=2048, num_experts=128, top_k=8, inter=768, group_size=128, quant=0,
             w_layout=0, shared_inter=0)
    d.update(kw)
    return N.MoeShape(**d)


def _ws(shape, T, kind=N.MOE_WS_LAYER):
    n = ctypes.c_size_t(0)
    st = _lib().moe_workspace_size(ctypes.byref(shape), T, kind, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes():
    _lib()
    st, n = _ws(_shape(), 8192)
    assert st == N.MOE_OK
    P = 8192 * 8
    # at least y_perm and h (bf16) plus the routing arrays
    assert n >= P * 2048 * 2 + P * 768 * 2 + 4 * P * 4
    st, r = _ws(_shape(), 8192, N.MOE_WS_ROUTE)
    assert st == N.MOE_OK and r >= 3 * 128 * 2048 * 2
    st, p = _ws(_shape(), 8192, N.MOE_WS_PERMUTE)
    assert st == N.MOE_OK and p >= 128 * 4
    st, f = _ws(_shape(), 8192, N.MOE_WS_EXPERT_FFN)
    assert st == N.MOE_OK and f >= P * 768 * 2
    assert n >= max(r, f, p)
    st, z = _ws(_shape(), 0)
    assert st == N.MOE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(group_size=16), N.MOE_ERR_UNSUPPORTED),
    (dict(group_size=0), N.MOE_ERR_INVALID_ARGUMENT),
    (dict(hidden=2000), N.MOE_ERR_UNSUPPORTED),
    (dict(inter=700), N.MOE_ERR_UNSUPPORTED),
    (dict(num_experts=300), N.MOE_ERR_UNSUPPORTED),
    (dict(top_k=9, num_experts=16), N.MOE_ERR_UNSUPPORTED),
    (dict(top_k=9, num_experts=8), N.MOE_ERR_INVALID_ARGUMENT),
    (dict(quant=5), N.MOE_ERR_INVALID_ARGUMENT),
    (dict(w_layout=2), N.MOE_ERR_INVALID_ARGUMENT),
    (dict(w_layout=-1), N.MOE_ERR_INVALID_ARGUMENT),
    (dict(shared_inter=100), N.MOE_ERR_UNSUPPORTED),
    (dict(shared_inter=-64), N.MOE_ERR_INVALID_ARGUMENT),
])
def test_shape_validation(kw, code):
    st, _ = _ws(_shape(**kw), 16)
    assert st == code
    assert _lib().moe_last_error()


def test_negative_T_and_null_shape():
    L = _lib()
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(_shape()), -1, 0, ctypes.byref(n)) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_workspace_size(None, 4, 0, ctypes.byref(n)) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_workspace_size(ctypes.byref(_shape()), 4, 9, ctypes.byref(n)) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_workspace_size(ctypes.byref(_shape()), (1 << 31) // 8, 0, ctypes.byref(n)) == N.MOE_ERR_UNSUPPORTED


def test_32bit_descriptor_limits():
    """Every tensor a GEMM reaches through a 32-bit buffer descriptor stays
    below 2^31 bytes: the largest T whose h (T*k*I*2 bytes) fits passes, the
    next one is refused; so are expert tensors of 2^31 bytes or more."""
    L = _lib()
    n = ctypes.c_size_t(0)
    s = _shape()  # H = 2048, E = 128, k = 8, I = 768
    t_max = ((1 << 31) - 1) // (8 * 768 * 2)  # h (T*k*I*2) is the largest descriptor-addressed activation
    assert L.moe_workspace_size(ctypes.byref(s), t_max, 0, ctypes.byref(n)) == N.MOE_OK
    assert L.moe_workspace_size(ctypes.byref(s), t_max + 1, 0, ctypes.byref(n)) == N.MOE_ERR_UNSUPPORTED
    # w13 = E * 2I * H / 2 bytes: 256 * 4096 * 2048 = 2^31
    big = _shape(num_experts=256, inter=2048, hidden=4096)
    assert L.moe_workspace_size(ctypes.byref(big), 16, 0, ctypes.byref(n)) == N.MOE_ERR_UNSUPPORTED
    ok = _shape(num_experts=128, inter=2048, hidden=4096)
    assert L.moe_workspace_size(ctypes.byref(ok), 16, 0, ctypes.byref(n)) == N.MOE_OK


FAKE = 0x10000  # an aligned non-null address that is never dereferenced


def test_route_validation_before_launch():
    L = _lib()
    s = _shape()
    # T == 0 is an OK no-op, even with NULL tensors
    assert L.moe_route(ctypes.byref(s), 0, None, None, None, None, None, None, None, None, None, 0, None) == N.MOE_OK
    # missing x
    assert L.moe_route(ctypes.byref(s), 4, None, FAKE, None, None, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT
    # misaligned x
    assert L.moe_route(ctypes.byref(s), 4, FAKE + 2, FAKE, None, None, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == N.MOE_ERR_UNSUPPORTED
    # shared_gate without shared_w
    assert L.moe_route(ctypes.byref(s), 4, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT
    # shared_gate on a shape without a shared expert (its MOE_WS_ROUTE size
    # has no room for the gate row)
    assert s.shared_inter == 0
    assert L.moe_route(ctypes.byref(s), 4, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert b"shared_inter" in L.moe_last_error()
    # workspace too small / missing
    assert L.moe_route(ctypes.byref(s), 4, FAKE, FAKE, None, None, None, FAKE, FAKE, None, FAKE, 16, None) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_route(ctypes.byref(s), 4, FAKE, FAKE, None, None, None, FAKE, FAKE, None, None, 0, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert b"workspace" in L.moe_last_error()


def _experts(**kw):
    d = dict(w13=FAKE, w13_scale=FAKE, w13_min=None, w2=FAKE, w2_scale=FAKE, w2_min=None,
             s13=None, s13_scale=None, s13_min=None, s2=None, s2_scale=None, s2_min=None)
    d.update(kw)
    return N.MoeExperts(**d)


def test_layer_forward_validation_before_launch():
    L = _lib()
    s = _shape()
    st, need = _ws(s, 4)
    args = lambda e, ws_bytes=need, sg=None, shape=s: L.moe_layer_forward(
        ctypes.byref(shape), 4, FAKE, FAKE, None, sg, ctypes.byref(e), None, FAKE, FAKE, ws_bytes, None)
    assert args(_experts(w13=None)) == N.MOE_ERR_INVALID_ARGUMENT
    assert args(_experts(w13_min=FAKE)) == N.MOE_ERR_INVALID_ARGUMENT       # min with SYM
    assert args(_experts(s13=FAKE)) == N.MOE_ERR_INVALID_ARGUMENT           # shared without shared_inter
    assert args(_experts(), ws_bytes=need - 1) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    assert args(_experts(), sg=FAKE) == N.MOE_ERR_INVALID_ARGUMENT          # gate without shared expert
    sa = _shape(quant=1)
    assert args(_experts(), shape=sa) == N.MOE_ERR_INVALID_ARGUMENT         # ASYM needs mins
    ss = _shape(shared_inter=512)
    st, need_s = _ws(ss, 4)
    ex = _experts(s13=FAKE, s13_scale=FAKE, s2=FAKE, s2_scale=FAKE)
    assert L.moe_layer_forward(ctypes.byref(ss), 4, FAKE, FAKE, None, None, ctypes.byref(ex), None,
                               FAKE, FAKE, need_s, None) == N.MOE_ERR_INVALID_ARGUMENT  # shared_gate missing
    assert L.moe_layer_forward(ctypes.byref(s), 0, None, None, None, None, None, None, None, None, 0, None) == N.MOE_OK


def test_other_entry_points_validation():
    L = _lib()
    s = _shape()
    e = _experts()
    assert L.moe_expert_ffn(ctypes.byref(s), 4, FAKE, ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, None) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_expert_ffn(ctypes.byref(s), 4, FAKE, ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_expert_ffn(ctypes.byref(s), 4, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_combine(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_combine(ctypes.byref(s), 4, None, FAKE, FAKE, None, None, None, FAKE, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_permute(ctypes.byref(s), 4, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_rmsnorm(4, 2048, FAKE, FAKE, ctypes.c_float(1e-6), FAKE, None) == N.MOE_ERR_INVALID_ARGUMENT  # aliasing
    assert L.moe_rmsnorm(4, 2047, FAKE, FAKE, ctypes.c_float(1e-6), FAKE + 64, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_rmsnorm(0, 2048, None, None, ctypes.c_float(1e-6), None, None) == N.MOE_OK
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0)
    assert L.moe_profile_read(None, ctypes.byref(n), ctypes.byref(ms)) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_profile_read(b"combine", ctypes.byref(n), ctypes.byref(ms)) == N.MOE_OK and n.value == 0


def test_integer_route_validation_before_launch():
    L = _lib()
    s = _shape()
    st, n8 = _ws(s, 8192, N.MOE_WS_LAYER_I8)
    assert st == N.MOE_OK
    P = 8192 * 8
    # int8 x, fp16 h and int8 h, fp16 y_perm and the routing arrays
    assert n8 >= 8192 * 2048 + P * 768 * 3 + P * 2048 * 2 + 4 * P * 4
    st, f8 = _ws(s, 8192, N.MOE_WS_EXPERT_FFN_I8)
    assert st == N.MOE_OK and f8 >= 8192 * 2048 + P * 768 * 3 and n8 >= f8
    # the route is defined for symmetric experts, G = 128, no shared expert
    for kw in (dict(quant=1), dict(group_size=64), dict(shared_inter=512)):
        st, _ = _ws(_shape(**kw), 16, N.MOE_WS_LAYER_I8)
        assert st == N.MOE_ERR_UNSUPPORTED, kw
        assert b"integer route" in L.moe_last_error()
    e = _experts()
    assert L.moe_layer_forward_i8(ctypes.byref(s), 4, FAKE, FAKE, None, ctypes.byref(e), None, FAKE,
                                  FAKE, 16, None) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_layer_forward_i8(ctypes.byref(s), 4, None, FAKE, None, ctypes.byref(e), None, FAKE,
                                  FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT
    sa = _shape(quant=1)
    ea = _experts(w13_min=FAKE, w2_min=FAKE)
    assert L.moe_layer_forward_i8(ctypes.byref(sa), 4, FAKE, FAKE, None, ctypes.byref(ea), None, FAKE,
                                  FAKE, 1 << 30, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_ffn_i8(ctypes.byref(s), 4, FAKE, ctypes.byref(e), FAKE, FAKE, FAKE, None, None,
                               FAKE, 1 << 30, None) == N.MOE_ERR_INVALID_ARGUMENT  # no y_perm
    assert L.moe_expert_ffn_i8(ctypes.byref(s), 4, FAKE, ctypes.byref(e), FAKE, FAKE, FAKE, FAKE,
                               FAKE + 8, FAKE, 1 << 30, None) == N.MOE_ERR_UNSUPPORTED  # misaligned h_perm
    assert L.moe_expert_ffn_i8(ctypes.byref(s), 0, None, None, None, None, None, None, None, None, 0,
                               None) == N.MOE_OK
    assert L.moe_quantize_rows_i8(4, 12, FAKE, FAKE, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_rows_i8(4, 16, FAKE, None, FAKE, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_quantize_rows_i8(0, 16, None, None, None, None) == N.MOE_OK


def test_mixed_width_validation_before_launch():
    L = _lib()
    s = _shape()
    st, need = _ws(s, 4)
    T3 = N.MoeTier * 3

    def tiers(*bits):
        return T3(*[N.MoeTier(b, 4, FAKE, FAKE, FAKE, FAKE) for b in bits] +
                  [N.MoeTier(0, 0, None, None, None, None)] * (3 - len(bits)))

    def call(tarr, n, shape=s, ws_bytes=need):
        return L.moe_layer_forward_mixed(ctypes.byref(shape), 4, FAKE, FAKE, None, tarr, n, FAKE, FAKE,
                                         None, FAKE, FAKE, ws_bytes, None)
    assert call(tiers(4, 2), 0) == N.MOE_ERR_INVALID_ARGUMENT
    assert call(tiers(4, 2), 4) == N.MOE_ERR_INVALID_ARGUMENT
    assert call(tiers(4, 4), 2) == N.MOE_ERR_INVALID_ARGUMENT        # two tiers of one width
    assert call(tiers(4, 5), 2) == N.MOE_ERR_UNSUPPORTED             # no 5-bit codes
    assert call(None, 1) == N.MOE_ERR_INVALID_ARGUMENT
    assert call(tiers(4, 3, 2), 3, shape=_shape(quant=1)) == N.MOE_ERR_UNSUPPORTED
    assert call(tiers(4, 3, 2), 3, shape=_shape(shared_inter=512)) == N.MOE_ERR_UNSUPPORTED
    assert call(tiers(4, 3, 2), 3, ws_bytes=need - 1) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    bad = T3(N.MoeTier(3, 4, None, FAKE, FAKE, FAKE), N.MoeTier(0, 0, None, None, None, None),
             N.MoeTier(0, 0, None, None, None, None))
    assert call(bad, 1) == N.MOE_ERR_INVALID_ARGUMENT                 # missing weights
    assert L.moe_expert_ffn_mixed(ctypes.byref(s), 4, FAKE, tiers(2), 1, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, 0, None) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_expert_ffn_mixed(ctypes.byref(s), 0, None, tiers(2), 1, None, None, None, None,
                                  None, None, None, 0, None) == N.MOE_OK


def test_streamed_validation_before_launch():
    L = _lib()
    s = _shape()
    n = ctypes.c_size_t(0)
    assert L.moe_stream_stage_bytes(ctypes.byref(s), 2, ctypes.byref(n)) == N.MOE_OK
    per = 2 * 768 * 2048 // 2 + 2 * 768 * 16 * 2 + 2048 * 768 // 2 + 2048 * 6 * 2
    assert n.value >= 2 * per
    E = 128
    slots = (ctypes.c_int32 * E)(*[-1] * E)
    cold = N.MoeExperts(FAKE, FAKE, None, FAKE, FAKE, None, None, None, None, None, None, None)
    st, need = _ws(s, 4)

    def call(shape=s, hot_count=0, hot_slot=slots, stage_bytes=1 << 30, ws_bytes=need + 4096):
        return L.moe_layer_forward_streamed(ctypes.byref(shape), 4, FAKE, FAKE, None, None, hot_count,
                                            ctypes.byref(cold), hot_slot, FAKE, stage_bytes, None, FAKE,
                                            FAKE, ws_bytes, None, None)
    assert call(shape=_shape(quant=1)) == N.MOE_ERR_UNSUPPORTED
    assert call(hot_slot=None) == N.MOE_ERR_INVALID_ARGUMENT
    assert call(stage_bytes=per) == N.MOE_ERR_WORKSPACE_TOO_SMALL     # not two experts
    assert call(ws_bytes=need - 1) == N.MOE_ERR_WORKSPACE_TOO_SMALL
    bad = (ctypes.c_int32 * E)(*([0] + [-1] * (E - 1)))
    assert call(hot_slot=bad, hot_count=0) == N.MOE_ERR_INVALID_ARGUMENT  # slot 0 of an empty hot set


def test_static_layer_validation_before_launch():
    """moe_layer_forward_static validates on the host like moe_layer_forward
    and refuses a call whose workspace would not fit its static array, all
    before touching a device."""
    L = _lib()
    s = _shape()  # H = 2048, E = 128, k = 8, I = 768
    n = ctypes.c_size_t(0)
    assert L.moe_layer_forward_static(ctypes.byref(s), 0, None, None, None, None, None, None, None, None) == N.MOE_OK
    # missing x
    ex = N.MoeExperts(FAKE, FAKE, None, FAKE, FAKE, None, None, None, None, None, None, None)
    assert L.moe_layer_forward_static(ctypes.byref(s), 4, None, FAKE, None, None, ctypes.byref(ex), None, FAKE, None) == N.MOE_ERR_INVALID_ARGUMENT
    # shared gate on a shape without a shared expert
    assert L.moe_layer_forward_static(ctypes.byref(s), 4, FAKE, FAKE, None, FAKE, ctypes.byref(ex), None, FAKE, None) == N.MOE_ERR_INVALID_ARGUMENT
    # the largest T whose layer workspace fits, and the next one
    assert N.MOE_STATIC_WS_BYTES == 128 << 20
    for T in (2583, 2584):
        assert L.moe_workspace_size(ctypes.byref(s), T, N.MOE_WS_LAYER, ctypes.byref(n)) == N.MOE_OK
        assert (n.value <= N.MOE_STATIC_WS_BYTES) == (T == 2583)
    assert L.moe_layer_forward_static(ctypes.byref(s), 2584, FAKE, FAKE, None, None, ctypes.byref(ex), None, FAKE, None) == N.MOE_ERR_UNSUPPORTED
    assert b"static workspace" in L.moe_last_error()


def test_tiled_layout_validation():
    """MOE_W_TILED weights: the fp16 route sizes its workspace as for row-major
    weights; the calls whose kernels read row-major weights only refuse the
    layout on the host; moe_pack_w4 checks its arguments before launching
    (include/moe.h, moe_w_layout_t and moe_pack_w4)."""
    L = _lib()
    t = _shape(w_layout=N.MOE_W_TILED)
    st, n = _ws(t, 8192)
    st0, n0 = _ws(_shape(), 8192)
    assert st == st0 == N.MOE_OK and n == n0
    st, _ = _ws(t, 16, N.MOE_WS_LAYER_I8)
    assert st == N.MOE_ERR_UNSUPPORTED and b"MOE_W_ROWS" in L.moe_last_error()
    n = ctypes.c_size_t(0)
    assert L.moe_stream_stage_bytes(ctypes.byref(t), 2, ctypes.byref(n)) == N.MOE_ERR_UNSUPPORTED
    e = _experts()
    assert L.moe_layer_forward_i8(ctypes.byref(t), 4, FAKE, FAKE, None, ctypes.byref(e), None, FAKE,
                                  FAKE, 1 << 30, None) == N.MOE_ERR_UNSUPPORTED
    # the mixed-width calls take tiled tiers (moe_pack_tier): the host checks pass
    st, n = _ws(t, 8192, N.MOE_WS_EXPERT_FFN)
    assert st == N.MOE_OK
    pk = L.moe_pack_w4
    assert pk(None, FAKE, 16, 128, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert pk(FAKE, FAKE + (1 << 24), 24, 128, None) == N.MOE_ERR_INVALID_ARGUMENT   # rows % 16
    assert pk(FAKE, FAKE + (1 << 24), 16, 192, None) == N.MOE_ERR_INVALID_ARGUMENT   # K % 128
    assert pk(FAKE, FAKE + 512, 16, 128, None) == N.MOE_ERR_INVALID_ARGUMENT         # overlap
    assert pk(FAKE + 8, FAKE + (1 << 24), 16, 128, None) == N.MOE_ERR_INVALID_ARGUMENT  # alignment
    assert pk(FAKE, FAKE + (1 << 34), 1 << 20, 1 << 12, None) == N.MOE_ERR_UNSUPPORTED  # >= 2^31 B


def test_pack_tier_validation():
    """moe_pack_tier checks its arguments before launching (include/moe.h,
    moe_pack_tier): width, row and K multiples (32 rows for a 3- or 2-bit
    gate/up matrix, whose rows interleave in 32-row groups), size, alignment
    and overlap."""
    L = _lib()
    pk = L.moe_pack_tier
    far = FAKE + (1 << 24)
    assert pk(None, FAKE, 16, 128, 4, 0, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert pk(FAKE, far, 16, 128, 5, 0, None) == N.MOE_ERR_UNSUPPORTED           # bits
    assert pk(FAKE, far, 24, 128, 3, 0, None) == N.MOE_ERR_INVALID_ARGUMENT      # rows % 16
    assert pk(FAKE, far, 16, 128, 3, 1, None) == N.MOE_ERR_INVALID_ARGUMENT      # rows % 32
    assert pk(FAKE, far, 16, 128, 2, 1, None) == N.MOE_ERR_INVALID_ARGUMENT
    assert pk(FAKE, far, 16, 192, 2, 0, None) == N.MOE_ERR_INVALID_ARGUMENT      # K % 128
    assert pk(FAKE, FAKE + 256, 32, 128, 3, 1, None) == N.MOE_ERR_INVALID_ARGUMENT  # overlap
    assert pk(FAKE + 2, far, 16, 128, 3, 0, None) == N.MOE_ERR_INVALID_ARGUMENT  # alignment
    assert pk(FAKE, FAKE + (1 << 34), 1 << 20, 1 << 13, 2, 0, None) == N.MOE_ERR_UNSUPPORTED
    assert b"moe_pack_tier" in L.moe_last_error()
