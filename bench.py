"""MoE-layer prefill benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload a3b_pp8192] [--no-cpu]
    python bench.py --route i8 ...        the integer route (moe_layer_forward_i8):
                                          8-bit activations on the int8 matrix cores,
                                          gate/up roofline against the int8 peak
    python bench.py --tiers 4:32,3:48,2:48 mixed-width experts (moe_layer_forward_mixed):
                                          the experts that receive the most rows of a
                                          calibration batch (another seed) get the
                                          first width, and so on
    python bench.py --stream-hot 32       host-resident experts streamed over PCIe
                                          (moe_layer_forward_streamed): the 32 experts
                                          that receive the most rows of the calibration
                                          batch stay on the GPU;
                                          --stage-experts sets the staging size,
                                          --copy-stream overlaps copies and kernels
    python bench.py --calib-copy ...      also run a 1 GiB device copy (counter scale)
    python bench.py --pmc-summary FETCH.csv WRITE.csv
                                          HBM bytes per launch from two rocprofv3
                                          --pmc runs (FETCH_SIZE, WRITE_SIZE)
    python bench.py --pmc-table A.csv ... per-kernel averages of every counter of
                                          rocprofv3 --pmc runs

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
               host's cores; `gemm_only` times it with the dequantized expert
               matrices prepared beforehand
  step_ms_p10_p50_p90  the spread of single steps (an event between steps)
  regimes      (default workload) the weight-streaming sweep T = 1, 4, 16 with
               the Infinity Cache evicted before each step, eager and as a
               replayed HIP graph, against 8 TB/s; and the skewed shared-expert
               layer (T = 4096) against the MFMA peak (--no-regimes skips them)
  ceilings     a bf16 8192^3 torch.matmul and a 1 GiB copy on the same box,
               as context for the fractions (--no-ceilings skips them)
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
PEAK_I8_TOPS = 5000.0       # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer prefill tokens/sec at T=8192; % of bf16 MFMA peak and HBM GB/s"

# Kernel names the library reports timings under (one layer forward).
KERNELS = ("router_split", "router_gemm", "router_select", "permute_rank", "permute_scatter",
           "x_to_f16", "gateup_gemm", "down_gemm", "shared_gateup_gemm", "shared_down_gemm",
           "combine")
KERNELS_I8 = ("router_split", "router_gemm", "router_select", "permute_rank", "permute_scatter",
              "quant_x_i8", "gateup_gemm_i8", "quant_h_i8", "down_gemm_i8", "combine")

# HBM bytes per gate/up launch on the a3b_pp8192 workload, from rocprofv3
# FETCH_SIZE + WRITE_SIZE (each scaled by the copy-kernel calibration factor),
# keyed by the hash of the expert-GEMM sources they were measured on: a
# changed kernel reports null until it is measured again.
GATEUP_TRAFFIC = {"df1d68e32e6e58bd": 660900258}   # {source sha256[:16]: bytes per launch}
GEMM_SOURCES = ("quantized_moe_prefill_amd/csrc/ffn.hip", "quantized_moe_prefill_amd/csrc/common.h",
                "quantized_moe_prefill_amd/csrc/dequant.h")
# the same for the integer route's gate/up launch
GATEUP_I8_TRAFFIC = {"3e0a6defe5a5f5a1": 525602705}
I8_SOURCES = ("quantized_moe_prefill_amd/csrc/ffn_i8.hip", "quantized_moe_prefill_amd/csrc/common.h")
CALIB_BYTES = 1 << 30
# Weight-streaming regime: with this few rows the layer reads each active
# expert's weights once, and those (tens of MB) would stay in the 256 MB
# Infinity Cache between back-to-back steps. Such runs are timed step by
# step with the cache evicted before each step by reading 1 GiB of other
# data outside the timed events, as a layer of a real model finds its
# weights in HBM after the other layers' weights went through the cache.
# (Evicting by writing instead leaves the cache full of dirty lines whose
# write-back then halves the read bandwidth of the timed step.)
STREAM_T = 16
RAMP_S = 0.2   # seconds of untimed steps before the warm-up ones (clock ramp)
FLUSH_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="a3b_pp8192")
    ap.add_argument("--T", type=int, default=0, help="rows (default: the workload's T)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--route", choices=("fp16", "i8"), default="fp16",
                    help="expert route: fp16 matrix cores (default) or the integer route")
    ap.add_argument("--stream-hot", type=int, default=-1,
                    help="stream the experts from host memory, keeping this many on the GPU")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the bf16 matmul and copy ceilings measured after the timing")
    ap.add_argument("--copy-stream", action="store_true",
                    help="with --stream-hot: copy on a second stream, overlapping the kernels")
    ap.add_argument("--stage-experts", type=int, default=32,
                    help="experts the staging buffer holds (two chunks of half of it)")
    ap.add_argument("--tiers", default="",
                    help="mixed widths, e.g. 4:32,3:48,2:48 (bits:experts, hottest first)")
    ap.add_argument("--w-layout", choices=("tiled", "rows"), default="tiled",
                    help="layout of the expert weights of the fp16 and mixed-width routes: "
                         "regrouped once by moe_pack_w4 / moe_pack_tier before the timed "
                         "steps (tiled), or row-major")
    ap.add_argument("--no-regimes", action="store_true",
                    help="skip the T=1/4/16 sweep and the skewed shared-expert layer that the "
                         "default headline run adds as extra fields")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one elementwise kernel that reads and writes 1 GiB "
                         "(counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarize two rocprofv3 counter_collection.csv files and exit")
    ap.add_argument("--pmc-table", nargs="+", metavar="CSV",
                    help="per-kernel averages of every counter in rocprofv3 "
                         "counter_collection.csv files, and exit")
    return ap.parse_args()


def gemm_source_hash(sources=GEMM_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_summary(fetch_csv: str, write_csv: str) -> None:
    """Per-kernel KiB per dispatch of FETCH_SIZE and WRITE_SIZE, and each
    scaled by the ratio of the known copy size to what the counter reads for
    the calibration copy."""
    import collections
    import csv
    import re

    def load(path, counter):
        per = collections.defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                name = re.sub(r"\(.*", "", name).replace("void ", "").strip()
                per[name].append(float(r["Counter_Value"]))
        return per

    pf = load(fetch_csv, "FETCH_SIZE")
    pw = load(write_csv, "WRITE_SIZE")
    # the calibration copy is by far the largest multiply-by-scalar dispatch
    copy_f = [max(v) for k, v in pf.items() if "MulFunctor" in k]
    copy_w = [max(v) for k, v in pw.items() if "MulFunctor" in k]
    fetch = {k: sum(v) / len(v) for k, v in pf.items() if "MulFunctor" not in k}
    write = {k: sum(v) / len(v) for k, v in pw.items() if "MulFunctor" not in k}
    nf = {k: len(v) for k, v in pf.items()}
    kib = CALIB_BYTES / 1024.0
    sf = kib / max(copy_f) if copy_f else None
    sw = kib / max(copy_w) if copy_w else None
    print(f"copy calibration ({CALIB_BYTES} B): FETCH_SIZE {max(copy_f) if copy_f else None} KiB, "
          f"WRITE_SIZE {max(copy_w) if copy_w else None} KiB -> scale fetch {sf}, write {sw}")
    print(f"{'kernel':55s} {'n':>4s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} {'scaled bytes':>14s}")
    for k in sorted(set(fetch) | set(write)):
        f, w = fetch.get(k), write.get(k)
        tot = None
        if f is not None and w is not None and sf and sw:
            tot = (f * sf + w * sw) * 1024.0
        print(f"{k[:55]:55s} {nf.get(k, 0):4d} {f if f is not None else float('nan'):12.1f} "
              f"{w if w is not None else float('nan'):12.1f} {tot if tot else float('nan'):14.4g}")
    print(f"gemm source hash {gemm_source_hash()}, integer-route gemm source hash "
          f"{gemm_source_hash(I8_SOURCES)}")


def pmc_table(csvs) -> None:
    """Per-kernel averages (over dispatches) of every counter in one or more
    rocprofv3 counter_collection.csv files, and ratios of them: non-MFMA
    VALU and LDS instructions per MFMA instruction (SQ_INSTS_VALU counts the
    MFMAs too)."""
    import collections
    import csv
    import re

    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csvs:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                name = re.sub(r"\(.*", "", name).replace("void ", "").strip()
                if "MulFunctor" in name or "at::" in name:
                    continue
                per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for k in sorted(per):
        avg = {c: sum(v) / len(v) for c, v in per[k].items()}
        n = max(len(v) for v in per[k].values())
        print(f"{k}  ({n} dispatches)")
        for c in sorted(avg):
            print(f"    {c:32s} {avg[c]:16.4g}")
        mf = avg.get("SQ_INSTS_MFMA")
        if mf:
            if "SQ_INSTS_VALU" in avg:
                print(f"    {'non-MFMA VALU per MFMA':32s} {(avg['SQ_INSTS_VALU'] - mf) / mf:16.3f}")
            if "SQ_INSTS_LDS" in avg:
                print(f"    {'LDS instructions per MFMA':32s} {avg['SQ_INSTS_LDS'] / mf:16.3f}")


def cpu_baseline(cfg, li, x, min_seconds=10.0, max_passes=8, i8=False, mixed=None):
    """The oracle as it stands, on the whole batch, repeated until about
    min_seconds of CPU work (at most max_passes passes)."""
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
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        if mixed is not None:
            oracle.moe_layer_mixed(xb, mixed, cfg.k, cfg.G)
        elif i8:
            oracle.moe_layer_i8(xb, cpu, cfg.k, cfg.G)
        else:
            oracle.moe_layer(xb, cpu, cfg.k, cfg.G, cfg.quant)
        dt += time.perf_counter() - t0
        passes += 1
    gemm_only = None
    if not i8 and mixed is None:
        # the same oracle with every expert's dequantized matrices prepared
        # before the clock starts: route, permute, the experts' products and
        # the combine (median of 3 passes)
        mo = oracle.moe_oracle
        w = mo._weights_dict(cpu)
        mats = {e: mo._expert_mats(w, e, cfg.G, cfg.quant) for e in range(cfg.E)}
        shared = (mo._expert_mats(w, None, cfg.G, cfg.quant, prefix="s")
                  if w["s13"] is not None else None)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            xf = oracle.bf16_to_f64(xb)
            L = mo.router_logits(xf, w["w_router"], w["router_bias"])
            ids, tw = oracle.select_topk(L.astype(np.float32), cfg.k)
            counts, offsets, sp, inv = oracle.permute(ids, cfg.E)
            y_perm = np.zeros((len(sp), cfg.H))
            for e in range(cfg.E):
                lo, hi = int(offsets[e]), int(offsets[e + 1])
                if lo < hi:
                    y_perm[lo:hi] = mo.swiglu_expert(xf[np.asarray(sp[lo:hi]) // cfg.k], *mats[e])[1]
            ys = sw = None
            if shared is not None:
                sw = mo.shared_gate(xf, w["shared_gate"])
                ys = mo.swiglu_expert(xf, *shared)[1]
            mo.combine(y_perm, inv, tw, ys, sw, None)
            times.append(time.perf_counter() - t0)
        t_med = sorted(times)[1]
        gemm_only = {"value": round(x.shape[0] / t_med, 2), "unit": "tokens/s",
                     "sample": "the whole batch with the experts' dequantized fp64 matrices "
                               f"prepared beforehand, median of 3 passes ({t_med:.2f} s)"}
    return {
        "value": round(passes * x.shape[0] / dt, 2),
        "unit": "tokens/s",
        "cores": blas_threads or cores,
        "kind": "oracle",
        "gemm_only": gemm_only,
        "sample": f"the whole {x.shape[0]}-token batch, {passes} passes of the float64 numpy "
                  f"oracle{' (integer route)' if i8 else (' (mixed widths)' if mixed else '')} "
                  f"(dequantize all experts + route + "
                  f"experts + combine), {dt:.1f} s in "
                  f"total; {cores} cores in the affinity mask (os.cpu_count() "
                  f"{os.cpu_count()}), BLAS threads {blas_threads}",
    }


def ceilings(dev):
    """Achievable rates on this machine, as context for the roofline fractions: a
    large bf16 matrix product (torch/hipBLASLt) and a 1 GiB device copy."""
    import torch
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    src = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_mm = rate(lambda: torch.matmul(a, b, out=c), 20)
    t_cp = rate(lambda: dst.copy_(src), 20)
    return {"bf16_matmul_8192_tflops": round(2.0 * n ** 3 / t_mm / 1e12, 1),
            "copy_1gib_gbs": round(2.0 * src.numel() * 4 / t_cp / 1e9, 1)}


def stack_cpu_baseline(cfg, layers_cpu, x, rows=32, layers=2):
    """Stacked workload: the oracle on a bounded sample (`rows` tokens through
    `layers` layers, the experts those tokens need dequantized per layer),
    scaled to tokens/s of the whole stack (tokens interact only within a
    row, so the work per token is the same for every row)."""
    import numpy as np
    import torch

    import oracle

    cores = len(os.sched_getaffinity(0))
    xb = x[:rows].view(torch.int16).cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    for li in layers_cpu[:layers]:
        w = li.norm_weight.numpy()
        xn = oracle.round_to_bf16(oracle.rmsnorm(xb, w, cfg.rms_eps))
        res = oracle.moe_layer_rows(xn, np.arange(rows), li, cfg.k, cfg.G, cfg.quant,
                                    residual_bits=xb)
        xb = oracle.round_to_bf16(res["out"])
    dt = time.perf_counter() - t0
    per_token_stack = dt / rows * (cfg.n_layers / layers)
    return {
        "value": round(1.0 / per_token_stack, 3),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{rows} tokens through {layers} of the {cfg.n_layers} layers (RMSNorm + "
                  f"routed experts + shared expert + residual, the needed experts dequantized "
                  f"per layer) in {dt:.1f} s, scaled to the whole stack",
    }


def regimes(cfg, li, x, dev, steps, tiled):
    """Driver-visible figures of the other regimes, measured after the
    headline: the weight-streaming sweep (the first T = 1, 4, 16 rows of the
    headline batch on the same weights; each step timed on its own after
    evicting the Infinity Cache, eagerly and as a replayed HIP graph) and the
    skewed shared-expert layer (T = 4096, 256 experts, asymmetric G = 32).
    Algorithmic bytes of a sweep step: the packed weights (+ scales) of the
    experts that receive rows, the router matrix, x in and out."""
    import torch

    import quantized_moe_prefill_amd as qm
    from synth import get_config, make_layer, make_tokens

    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sum = torch.empty((), dtype=torch.float32, device=dev)

    def timed(fn, evict):
        times = []
        for _ in range(steps):
            if evict:
                torch.sum(flush, dim=0, out=flush_sum)
            e0.record(st)
            fn()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2]

    res = {}
    shape = qm.shape_of(cfg)
    for T in cfg.sweep_T:
        layer = qm.MoELayer(cfg, li, dev, T, tiled=tiled)
        xt = x[:T]
        o = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)

        def step():
            layer.forward(xt, out=o)
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        ms = timed(step, True)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            step()
        st.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        gms = timed(graph.replay, True)
        _, ids, _, _ = qm.moe_route(shape, xt, li.w_router, li.router_bias, None)
        active = int(torch.unique(ids).numel())
        nbytes = active * cfg.expert_bytes() + cfg.E * cfg.H * 4 + 2 * T * cfg.H * 2
        res[f"T{T}"] = {"ms": round(ms, 4), "graph_ms": round(gms, 4),
                        "tokens_per_s": round(T / (ms * 1e-3), 1), "active_experts": active,
                        "hbm_bytes": nbytes, "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "graph_hbm_frac": round(nbytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del graph
    cfg3 = get_config("skew_shared")
    li3 = make_layer(cfg3, device=dev)
    x3 = make_tokens(cfg3, device=dev)
    layer3 = qm.MoELayer(cfg3, li3, dev, cfg3.T, tiled=tiled)
    o3 = torch.empty((cfg3.T, cfg3.H), dtype=torch.bfloat16, device=dev)
    for _ in range(20):
        layer3.forward(x3, out=o3)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(steps):
        layer3.forward(x3, out=o3)
    e1.record(st)
    torch.cuda.synchronize()
    ms3 = e0.elapsed_time(e1) / steps
    res["skew_shared"] = {"ms": round(ms3, 4), "tokens_per_s": round(cfg3.T / (ms3 * 1e-3), 1),
                          "T": cfg3.T, "mfma_frac": round(cfg3.mfma_flops() / (ms3 * 1e-3) / 1e12
                                                          / PEAK_BF16_TFLOPS, 4)}
    res["note"] = ("T1/T4/T16: the first T rows of the headline batch, median of K steps each "
                   "timed after evicting the Infinity Cache (eager, and a replayed HIP graph); "
                   "hbm_frac = algorithmic bytes (active experts + router + x + out) / time / "
                   "8 TB/s. skew_shared: T=4096, 256 experts, top-8, asym G=32, shared expert, "
                   "Zipf router bias; mfma_frac of the 2.5 PFLOP/s dense fp16/bf16 peak")
    return res


def main():
    a = parse()
    if a.pmc_summary:
        pmc_summary(*a.pmc_summary)
        return
    if a.pmc_table:
        pmc_table(a.pmc_table)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the MoE layer is "
              "benchmarked on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_moe_prefill_amd as qm
    from synth import get_config, make_layer, make_stack_layer, make_tokens

    cfg = get_config(a.workload)
    T = a.T or cfg.T
    if T > cfg.T:
        # more tokens than the workload's token tensor holds: the same layer
        # over a longer synthetic batch (drawn with the workload's seed)
        from dataclasses import replace as _replace
        cfg = _replace(cfg, T=T)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stacked = cfg.n_layers > 1
    i8 = a.route == "i8"
    tiers = [(int(b), int(n)) for b, n in (t.split(":") for t in a.tiers.split(","))] if a.tiers else []
    streamed = a.stream_hot >= 0
    # (the integer and host-streamed routes read row-major weights only)
    tiled = a.w_layout == "tiled" and not (i8 or streamed)
    if streamed and (i8 or tiers or stacked or cfg.quant != "sym" or cfg.shared_I):
        print("streamed experts need one layer of symmetric experts without a shared expert",
              file=sys.stderr)
        sys.exit(2)
    if tiers and (i8 or stacked or cfg.quant != "sym" or cfg.shared_I or
                  sum(n for _, n in tiers) != cfg.E):
        print(f"mixed widths need one layer of symmetric experts without a shared expert and "
              f"expert counts that add up to E = {cfg.E}", file=sys.stderr)
        sys.exit(2)
    if i8 and (stacked or cfg.quant != "sym" or cfg.G != 128 or cfg.shared_I):
        print(f"the integer route needs one layer of symmetric experts with group 128 and no "
              f"shared expert ({cfg.name} is not)", file=sys.stderr)
        sys.exit(2)
    x = make_tokens(cfg, device=dev, rows=T)
    if stacked:
        layers = [make_stack_layer(cfg, l, device=dev) for l in range(cfg.n_layers)]
        stack = qm.MoEStack(cfg, layers, dev, eps=cfg.rms_eps, chunk=min(cfg.chunk or T, T),
                            tiled=tiled)
        xs = torch.empty_like(x)

        def step():
            xs.copy_(x)
            stack.forward(xs)
        li = layers[0]
    else:
        li = make_layer(cfg, device=dev)
        out = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
        mixed = None
        sx = None
        # routing statistics for choosing hot (or wider) experts come from a
        # calibration batch of other tokens (another seed), routed by the
        # same router, never from the timed batch itself
        calib_seed = cfg.seed + 1

        def calib_load():
            from dataclasses import replace as _replace
            shape = qm.shape_of(cfg)
            xc = make_tokens(_replace(cfg, seed=calib_seed), device=dev, rows=T)
            _, ids0, _, _ = qm.moe_route(shape, xc, li.w_router, li.router_bias, None)
            return torch.bincount(ids0.flatten().long(), minlength=cfg.E).cpu()
        if streamed:
            shape = qm.shape_of(cfg)
            load = calib_load()
            hot = torch.argsort(-load, stable=True).tolist()[:a.stream_hot]
            sx = qm.StreamedExperts(li, hot, dev)
            stage = torch.empty(qm.moe_stream_stage_bytes(shape, a.stage_experts), dtype=torch.uint8,
                                device=dev)
            ws = torch.empty(qm.moe_workspace_size(shape, T) + 8 * cfg.E + 512, dtype=torch.uint8,
                             device=dev)

            cstream = torch.cuda.Stream(device=dev) if a.copy_stream else None

            def step():
                qm.moe_layer_forward_streamed(shape, x, li.w_router, li.router_bias, sx, stage,
                                              out=out, ws=ws, copy_stream=cstream)
        elif tiers:
            from synth.mixed import make_mixed_layer
            # widths by how many rows each expert receives in the calibration batch
            shape = qm.shape_of(cfg)
            load = calib_load()
            order = torch.argsort(-load, stable=True).tolist()
            widths = [4] * cfg.E
            pos = 0
            for b, n in tiers:
                for e in order[pos:pos + n]:
                    widths[e] = b
                pos += n
            mixed = make_mixed_layer(cfg, widths, device=dev)
            # tiled: every tier regrouped once by moe_pack_tier
            mshape = qm.shape_of(cfg, qm.MOE_W_TILED) if tiled else shape
            experts = qm.MixedExperts(qm.pack_mixed(cfg, mixed) if tiled else mixed, dev)
            ws = qm.workspace(shape, T, dev, qm.MOE_WS_LAYER)

            def step():
                qm.moe_layer_forward_mixed(mshape, x, mixed.w_router, mixed.router_bias, experts,
                                           out=out, ws=ws)
        elif i8:
            shape = qm.shape_of(cfg)
            experts = qm.Experts(li)
            ws = qm.workspace(shape, T, dev, qm.MOE_WS_LAYER_I8)

            def step():
                qm.moe_layer_forward_i8(shape, x, li.w_router, li.router_bias, experts, out=out,
                                        ws=ws)
        else:
            layer = qm.MoELayer(cfg, li, dev, T, tiled=tiled)

            def step():
                layer.forward(x, out=out)
    torch.cuda.synchronize()

    # Clock ramp: the GPU takes tens of milliseconds of sustained work to reach
    # its steady clock, longer than a few warm-up steps of a sub-millisecond
    # layer. Untimed steps for about RAMP_S seconds first (the same work as a
    # step), then the W warm-up steps, then the K timed ones.
    ramp_steps, t_ramp = 0, time.perf_counter()
    per = 1 if stacked else 10
    while time.perf_counter() - t_ramp < RAMP_S:
        for _ in range(per):
            step()
        ramp_steps += per
        torch.cuda.synchronize()
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    cold = T <= STREAM_T and not stacked
    if cold:
        flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        flush_sum = torch.empty((), dtype=torch.float32, device=dev)

        def evict():
            torch.sum(flush, dim=0, out=flush_sum)

    # timed region: K steps, bracketed by synchronizations
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(st)
    for _ in range(a.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / a.steps
    warm_ms = graph_ms = None
    if cold:
        # the same K steps one by one, each after evicting the Infinity Cache
        warm_ms = ms
        times = []
        for _ in range(a.steps):
            evict()
            e0.record(st)
            step()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        # the same step captured once as a HIP graph and replayed (launch
        # overheads of the short kernels are what the graph removes)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        times = []
        for _ in range(a.steps):
            evict()
            e0.record(st)
            graph.replay()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        graph_ms = sorted(times)[len(times) // 2]

    if stacked and T <= STREAM_T:
        # a few tokens through the whole stack (about 200 short launches per
        # step): the same step captured once as a HIP graph and replayed
        warm_ms = ms
        xs.copy_(x)
        graph = stack.capture(xs)
        times = []
        for _ in range(a.steps):
            xs.copy_(x)
            e0.record(st)
            graph.replay()
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        graph_ms = sorted(times)[len(times) // 2]
        del graph

    # the spread of single steps: K more steps, an event between consecutive
    # ones (no synchronization inside the loop)
    step_pct = None
    if not cold:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
        evs[0].record(st)
        for i in range(a.steps):
            step()
            evs[i + 1].record(st)
        torch.cuda.synchronize()
        d = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps))
        q = lambda f: d[min(len(d) - 1, int(f * len(d)))]
        step_pct = [round(q(0.1), 4), round(q(0.5), 4), round(q(0.9), 4)]

    # per-kernel durations: the same K steps again with HIP events around
    # every kernel launch (recorded on the launch stream by the library)
    launches_per_step = 16 * max(1, cfg.n_layers) * max(1, -(-T // (cfg.chunk or T)))
    qm.profile_enable(a.steps * launches_per_step)
    for _ in range(a.steps):
        if cold:
            evict()
        step()
    torch.cuda.synchronize()
    kernels = {}
    for name in (KERNELS_I8 if i8 else KERNELS) + ("rmsnorm",):
        n, tot = qm.profile_read(name)
        if n:
            # microseconds per launch (per step: a mixed-width layer launches
            # each expert GEMM once per width)
            kernels[name] = round(tot / (a.steps if (tiers or streamed) else n) * 1000.0, 2)
    qm.profile_enable(0)

    # the work of one layer application over n rows
    def layer_flops(n):
        return cfg.mfma_flops(n)

    n_apps = cfg.n_layers if stacked else 1
    P = T * cfg.k
    chunk_rows = min(cfg.chunk or T, T)
    gu_launch_rows = chunk_rows if stacked else T
    gu_flops = 4.0 * cfg.H * cfg.I * gu_launch_rows * cfg.k
    gu_name = "gateup_gemm_i8" if i8 else "gateup_gemm"
    gu_us = kernels.get(gu_name)
    achieved = gu_flops / (gu_us * 1e-6) / 1e12 if gu_us else None
    total_flops = layer_flops(T) * n_apps
    layer_tflops = total_flops / (ms * 1e-3) / 1e12
    # algorithmic HBM bytes: the packed weights of every expert that received
    # tokens (all of them at large T), router, shared expert, x in, out
    with torch.no_grad():
        logits, ids, _, _ = qm.moe_route(qm.shape_of(cfg), x, li.w_router, li.router_bias,
                                         li.shared_gate)
        active = int(torch.unique(ids).numel())
    weight_bytes = (active * cfg.expert_bytes() + cfg.shared_bytes()) * n_apps
    if tiers:
        weight_bytes = mixed.nbytes()
    io_bytes = (cfg.E * cfg.H * 4) * n_apps + 2 * T * cfg.H * 2
    hbm_gbs = (weight_bytes + io_bytes) / (ms * 1e-3) / 1e9
    # gate/up launch: the active experts' gate/up weights and scales (+ mins),
    # the token rows once, h written
    per = 2 if cfg.quant == "sym" else 4
    gu_bytes = (active * (cfg.I * cfg.H + 2 * cfg.I * (cfg.H // cfg.G) * per)
                + T * cfg.H * (1 if i8 else 2) + P * cfg.I * 2)
    if tiers:
        gu_bytes = (sum(v[0].numel() + 2 * v[1].numel() for v in mixed.tiers.values())
                    + T * cfg.H * 2 + P * cfg.I * 2)
    peak = PEAK_I8_TOPS if i8 else PEAK_BF16_TFLOPS
    if cold:
        gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9 if gu_us else None
        roofline = {"kernel": gu_name, "bound": "hbm",
                    "achieved": round(gu_gbs, 1) if gu_gbs else None, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gu_gbs / PEAK_HBM_GBS, 4) if gu_gbs else None,
                    "traffic": None, "bytes_per_launch": gu_bytes}
    else:
        roofline = {
            "kernel": gu_name,
            "bound": "mfma",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": peak,
            "unit": "TOP/s" if i8 else "TFLOP/s",
            "frac": round(achieved / peak, 4) if achieved else None,
            "traffic": ((GATEUP_I8_TRAFFIC.get(gemm_source_hash(I8_SOURCES)) if i8
                         else GATEUP_TRAFFIC.get(gemm_source_hash()))
                        if (cfg.name, T) == ("a3b_pp8192", 8192) and not (tiers or streamed)
                        else None),
            "flops_per_launch": gu_flops,
        }

    desc = (f"{cfg.name}: {'a stack of %d ' % cfg.n_layers if stacked else 'one '}MoE FFN "
            f"layer{'s with RMSNorm + residual, in %d-row chunks' % chunk_rows if stacked else ''}"
            f", T={T}, hidden={cfg.H}, experts={cfg.E}, top-{cfg.k}, inter={cfg.I}, "
            f"{cfg.quant} int4 group {cfg.G}"
            + (f", shared expert {cfg.shared_I}" if cfg.shared_I else "")
            + (", Zipf router bias" if cfg.zipf_bias else ""))
    rec = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "clock_ramp_steps": ramp_steps,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if i8 else "fp16",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "T": T, "hidden": cfg.H, "experts": cfg.E, "top_k": cfg.k, "inter": cfg.I,
            "group": cfg.G, "quant": cfg.quant, "shared_inter": cfg.shared_I,
            "layers": cfg.n_layers,
            "route": ("int8 activations" if i8 else
                      ("fp16, mixed widths " + a.tiers if tiers else
                       (f"fp16, {cfg.E - a.stream_hot} experts streamed from host memory, "
                        f"{a.stream_hot} on the GPU" if streamed else "fp16"))),
            "weights": (("every tier's matrices regrouped once into the tiled layout "
                         "(moe_pack_tier)" if tiers else
                         "4-bit matrices regrouped once into the tiled layout (moe_pack_w4)") +
                        " before the timed steps" if tiled else "row-major matrices"),
        },
        "layer_tflops": round(layer_tflops, 1),
        "layer_mfma_frac": round(layer_tflops / peak, 4),
        "active_experts": active,
        "layer_hbm_gbs": round(hbm_gbs, 1),
        "layer_hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
        "kernel_us": kernels,
        "wall_s_timed": round(t_wall, 3),
        "step_ms_p10_p50_p90": step_pct,
        "ceilings": ceilings(dev) if not a.no_ceilings else None,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if (not a.no_regimes and cfg.name == "a3b_pp8192" and T == cfg.T and not
            (i8 or tiers or streamed)):
        rec["regimes"] = regimes(cfg, li, x, dev, a.steps, tiled)
    if streamed or tiers:
        rec["calibration"] = (f"hot / wider experts chosen by their row counts in a separate "
                              f"calibration batch of {T} tokens drawn with seed {calib_seed} "
                              f"(the timed batch uses seed {cfg.seed})")
    if streamed:
        cb = sx.cold_bytes()
        rec["streamed"] = {"cold_experts": sx.n_cold, "cold_bytes": cb,
                           "pcie_gbs": round(cb / (ms * 1e-3) / 1e9, 2),
                           "note": ("host->device copies on a second stream, overlapping the "
                                    "kernels" if a.copy_stream else
                                    "host->device copies and kernels ordered on one stream")}
    if cold:
        rec["timing"] = ("median of K steps timed one by one, the Infinity Cache evicted "
                         "(1 GiB of other data read) before each; kernel_us likewise")
        rec["warm_ms_per_step"] = round(warm_ms, 4)
        rec["graph_ms_per_step"] = round(graph_ms, 4)
        rec["graph_tokens_per_s"] = round(T / (graph_ms * 1e-3), 1)
    elif graph_ms is not None:
        rec["graph_ms_per_step"] = round(graph_ms, 4)
        rec["graph_tokens_per_s"] = round(T / (graph_ms * 1e-3), 1)
        rec["graph_note"] = ("the stack step (input copy + every layer) captured as one HIP "
                             "graph, median of K replays")
    if a.calib_copy:
        # a copy kernel of known size: y = x * 1 over 1 GiB of fp32 (a memcpy
        # would go to the DMA engine, which the counters do not see)
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not a.no_cpu:
        if stacked:
            rec["cpu_baseline"] = stack_cpu_baseline(cfg, [l.to("cpu") for l in layers[:2]], x)
        else:
            rec["cpu_baseline"] = cpu_baseline(cfg, li, x, i8=i8,
                                               mixed=mixed.to("cpu") if tiers else None)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
