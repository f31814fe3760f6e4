"""MoE-layer prefill benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload a3b_pp8192] [--no-cpu]

One step = one moe_layer_forward (route, permute, gate/up + SwiGLU, down,
combine) over the workload's batch, with all inputs resident in HBM. Prints
one JSON line:
  value        tokens/s of the whole layer (T / seconds per step)
  roofline     the dominant kernel (gate/up GEMM) against the bf16 MFMA peak:
               algorithmic flops per launch / its average launch time, timed
               with HIP events on the launch stream; `traffic` is the HBM
               bytes per launch from rocprofv3 counters (null until measured
               for the current kernel)
  cpu_baseline the CPU oracle (numpy float64) on the same workload on this
               host's cores
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer prefill tokens/sec at T=8192; % of bf16 MFMA peak and HBM GB/s"

# Kernel names the library reports timings under (one layer forward).
KERNELS = ("router_split", "router_gemm", "router_select", "permute_rank", "permute_scatter",
           "x_to_f16", "gateup_gemm", "down_gemm", "shared_gateup_gemm", "shared_down_gemm",
           "combine")

# HBM bytes per gate/up launch on the a3b_pp8192 workload, from rocprofv3
# FETCH_SIZE + WRITE_SIZE (scaled by the copy-kernel calibration factor);
# None until measured on the current kernel.
GATEUP_TRAFFIC_BYTES = None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="a3b_pp8192")
    ap.add_argument("--T", type=int, default=0, help="rows (default: the workload's T)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


def cpu_baseline(cfg, li, x):
    """The oracle as it stands, on the whole batch, once."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 0) for d in threadpool_info()] or [0])
    except Exception:
        blas_threads = 0
    cores = len(os.sched_getaffinity(0))
    cpu = li.to("cpu")
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    oracle.moe_layer(xb, cpu, cfg.k, cfg.G, cfg.quant)
    dt = time.perf_counter() - t0
    return {
        "value": round(x.shape[0] / dt, 2),
        "unit": "tokens/s",
        "cores": blas_threads or cores,
        "kind": "oracle",
        "sample": f"whole {x.shape[0]}-token batch, one pass of the float64 numpy oracle "
                  f"(dequantize + route + experts + combine), {dt:.1f} s; "
                  f"{cores} cores visible, BLAS threads {blas_threads}",
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the MoE layer is "
              "benchmarked on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_moe_prefill_amd as qm
    from synth import get_config, make_layer, make_tokens

    cfg = get_config(a.workload)
    T = a.T or cfg.T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    li = make_layer(cfg, device=dev)
    x = make_tokens(cfg, device=dev, rows=T)
    layer = qm.MoELayer(cfg, li, dev, T)
    out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    for _ in range(a.warmup):
        layer.forward(x, out=out)
    torch.cuda.synchronize()

    # timed region: K steps, bracketed by synchronizations
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(st)
    for _ in range(a.steps):
        layer.forward(x, out=out)
    e1.record(st)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / a.steps

    # per-kernel durations: the same K steps again with HIP events around
    # every kernel launch (recorded on the launch stream by the library)
    n_kernels = 16
    qm.profile_enable(a.steps * n_kernels)
    for _ in range(a.steps):
        layer.forward(x, out=out)
    torch.cuda.synchronize()
    kernels = {}
    for name in KERNELS:
        n, tot = qm.profile_read(name)
        if n:
            kernels[name] = round(tot / n * 1000.0, 2)  # microseconds per launch
    qm.profile_enable(0)

    P = T * cfg.k
    gu_flops = 4.0 * cfg.H * cfg.I * P
    gu_us = kernels.get("gateup_gemm")
    achieved = gu_flops / (gu_us * 1e-6) / 1e12 if gu_us else None
    layer_tflops = cfg.mfma_flops(T) / (ms * 1e-3) / 1e12
    # algorithmic HBM bytes of the layer: every active expert's packed weights
    # (all experts are active at this T) + router + x in + out
    weight_bytes = cfg.E * cfg.expert_bytes() + cfg.shared_bytes()
    io_bytes = cfg.E * cfg.H * 4 + 2 * T * cfg.H * 2
    hbm_gbs = (weight_bytes + io_bytes) / (ms * 1e-3) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one MoE FFN layer, T={T}, hidden={cfg.H}, experts={cfg.E}, "
                        f"top-{cfg.k}, inter={cfg.I}, {cfg.quant} int4 group {cfg.G}"
                        + (f", shared expert {cfg.shared_I}" if cfg.shared_I else ""),
            "T": T, "hidden": cfg.H, "experts": cfg.E, "top_k": cfg.k, "inter": cfg.I,
            "group": cfg.G, "quant": cfg.quant, "shared_inter": cfg.shared_I,
        },
        "layer_tflops": round(layer_tflops, 1),
        "layer_mfma_frac": round(layer_tflops / PEAK_BF16_TFLOPS, 4),
        "layer_hbm_gbs": round(hbm_gbs, 1),
        "layer_hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
        "kernel_us": kernels,
        "wall_s_timed": round(t_wall, 3),
        "roofline": {
            "kernel": "gateup_gemm",
            "bound": "mfma",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
            "traffic": GATEUP_TRAFFIC_BYTES if T == cfg.T else None,
            "flops_per_launch": gu_flops,
        },
        "cpu_baseline": None,
    }
    if not a.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(cfg, li, x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
