"""moe_layer_forward_static: the layer with its intermediates in the
library's static per-GPU workspace, for callers that cannot allocate. Its
output must be the bits of moe_layer_forward (the same kernels on the same
layout) on consecutive calls, the second one smaller than the first (the
array keeps the previous call's contents, which nothing may read)."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_moe_prefill_amd as qm
from quantized_moe_prefill_amd import _native as N
from synth import CONFIGS, make_layer, make_tokens

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def static_fits(shape, T):
    return qm.moe_workspace_size(shape, T) <= N.MOE_STATIC_WS_BYTES


@pytest.mark.parametrize("name,T1,T2", [
    ("a3b_pp512", 512, 77),      # the 512-row prefill chunk, then a ragged smaller batch
    ("skew_shared", 600, 16),    # shared expert, asymmetric G=32; then the small-T path
    ("tiny", 64, 5),
])
def test_static_matches_workspace_call(name, T1, T2):
    cfg = CONFIGS[name]
    shape = qm.shape_of(cfg)
    li = make_layer(cfg, device=DEV)
    ex = qm.Experts(li)
    x = make_tokens(cfg, device=DEV, rows=T1)
    assert x.shape[0] == T1 and static_fits(shape, T1)
    res = torch.randn((T1, cfg.H), device=DEV, generator=torch.Generator(device=DEV).manual_seed(3)
                      ).to(torch.bfloat16)
    for T, residual in ((T1, None), (T2, res[:T2])):
        xt = x[:T].contiguous()
        ref = qm.moe_layer_forward(shape, xt, li.w_router, li.router_bias, li.shared_gate, ex,
                                   residual=residual)
        got = qm.moe_layer_forward_static(shape, xt, li.w_router, li.router_bias,
                                          li.shared_gate, ex, residual=residual)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (name, T)
        print(f"[static] {name} T={T}: bit-equal to moe_layer_forward "
              f"(workspace {qm.moe_workspace_size(shape, T)} of {N.MOE_STATIC_WS_BYTES} bytes)")


def test_static_refuses_too_large():
    cfg = CONFIGS["a3b_pp8192"]
    shape = qm.shape_of(cfg)
    T = 4096
    assert not static_fits(shape, T)
    li = make_layer(cfg, device=DEV)
    x = make_tokens(cfg, device=DEV, rows=T)
    with pytest.raises(qm.MoeError) as e:
        qm.moe_layer_forward_static(shape, x, li.w_router, li.router_bias, None, qm.Experts(li))
    assert e.value.status == N.MOE_ERR_UNSUPPORTED
