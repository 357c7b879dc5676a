#!/usr/bin/env python3
"""Benchmark: expanded-layout MoE layer tokens/s on one MI355X.

A step is one pass of the whole path over one batch of synthetic input
already resident in HBM: expand layout -> gate_up grouped fp8 GEMM ->
SiLU*up + fp8 quant (+ weight fold) -> down grouped fp8 GEMM -> gather.
value = valid received rows per second.

Inputs follow the seeded workload recipe (routing and top-k weights from the
numpy workload generator; activations and weights drawn from a seeded torch
generator on the GPU and quantised to fp8 with 1x128 / 128x128 scales by
plain torch ops: input preparation, not part of the timed path).

Prints one JSON line.  Extra keys: per-stage microseconds, the roofline of
the dominant kernel (gate_up GEMM) and the CPU oracle's throughput on the
host's cores.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
METRIC = "expanded MoE layer tokens/s per GPU (DSv3 shape); HBM GB/s & MFMA util vs peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dsv3")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-runs", type=int, default=3)
    return p.parse_args()


def quant_rows(x, fmt):
    """[R, H] fp32 -> fp8 codes (uint8 view) and per-1x128 scales."""
    import torch
    R, H = x.shape
    g = x.view(R, H // 128, 128)
    amax = g.abs().amax(-1, keepdim=True).clamp_min(1e-10)
    if fmt == "f32":
        q = (g * (448.0 / amax)).to(torch.float8_e4m3fn)
        s = (amax / 448.0).view(R, H // 128)
    else:
        m, e = torch.frexp(amax / 448.0)
        e = torch.where(m == 0.5, e - 1, e)                  # ceil(log2)
        q = torch.ldexp(g, (-e).float()).to(torch.float8_e4m3fn)
        s = (e + 127).to(torch.uint8).view(R, H // 128)
    return q.view(R, H).view(torch.uint8).contiguous(), s.contiguous()


def quant_blocks(w, fmt):
    """[E, N, K] fp32 -> fp8 codes and per-128x128 scales."""
    import torch
    E, N, K = w.shape
    t = w.view(E, N // 128, 128, K // 128, 128)
    amax = t.abs().amax(dim=(2, 4), keepdim=True).clamp_min(1e-10)
    if fmt == "f32":
        q = (t * (448.0 / amax)).to(torch.float8_e4m3fn)
        s = (amax / 448.0).view(E, N // 128, K // 128)
    else:
        m, e = torch.frexp(amax / 448.0)
        e = torch.where(m == 0.5, e - 1, e)
        q = torch.ldexp(t, (-e).float()).to(torch.float8_e4m3fn)
        s = (e + 127).to(torch.uint8).view(E, N // 128, K // 128)
    return q.view(E, N, K).view(torch.uint8).contiguous(), s.contiguous()


def make_inputs(wl, device):
    import numpy as np
    import torch
    import workloads as W
    d = W.generate(wl, with_weights=False, with_x=False)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    R, H, I, E = wl.rows, wl.hidden, wl.inter, wl.experts
    x = torch.randn((R, H), generator=gen, device=device, dtype=torch.float32)
    xq, xs = quant_rows(x, wl.fmt)
    del x
    nv = d["num_valid"]
    if nv < R:     # poisoned tail past the boundary (random bytes, NaN/Inf)
        xq[nv:] = torch.randint(0, 256, (R - nv, H), generator=gen, device=device,
                                dtype=torch.uint8)
        if wl.fmt == "f32":
            bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (R - nv, H // 128), generator=gen,
                                 device=device, dtype=torch.int32)
            xs[nv:] = bits.view(torch.float32)
    w13 = torch.randn((E, 2 * I, H), generator=gen, device=device) * 0.02
    w13q, w13s = quant_blocks(w13, wl.fmt)
    del w13
    w2 = torch.randn((E, H, I), generator=gen, device=device) * 0.02
    w2q, w2s = quant_blocks(w2, wl.fmt)
    del w2
    ids = torch.from_numpy(d["ids"]).to(device)
    wts = torch.from_numpy(d["w"]).to(device)
    prank = None
    if d["psum_recv_per_rank"] is not None:
        prank = torch.from_numpy(np.asarray(d["psum_recv_per_rank"])).to(device)
    torch.cuda.synchronize()
    return dict(x=xq, x_scale=xs, ids=ids, w=wts, prank=prank, w13=w13q, w13_scale=w13s,
                w2=w2q, w2_scale=w2s, num_valid=nv, data=d)


def cpu_baseline(inp, wl, runs):
    """The oracle as it stands, on this host's cores, over the same inputs."""
    import numpy as np
    from oracle import layer
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    host = {k: inp[k].cpu().numpy() for k in ("x", "x_scale", "ids", "w", "w13",
                                             "w13_scale", "w2", "w2_scale")}
    o = dict(x_q=host["x"], x_s=host["x_scale"], ids=host["ids"], w=host["w"],
             num_valid=inp["num_valid"], w13_q=host["w13"], w13_s=host["w13_scale"],
             w2_q=host["w2"], w2_s=host["w2_scale"], align=wl.align, fmt=wl.fmt)
    times = []
    for _ in range(max(1, runs)):
        t0 = time.perf_counter()
        layer.layer(o)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": inp["num_valid"] / t, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"whole {wl.name} layer ({inp['num_valid']} valid rows), "
                      f"median of {len(times)} runs, {t:.2f} s each"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path has no cross-GPU part "
              "(the dispatch/combine all-to-alls are not built); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import expanded_dispatch_layout_amd as M
    import workloads as W

    wl = W.workload(args.workload)
    dev = "cuda"
    inp = make_inputs(wl, dev)
    mod = M.ExpandedMoE(wl.rows, wl.topk, inp["w13"], inp["w13_scale"], inp["w2"],
                        inp["w2_scale"], wl.align, wl.fmt, device=dev)
    out = torch.empty((wl.rows, wl.hidden), dtype=torch.bfloat16, device=dev)
    fold = mod.row_weight if wl.fmt == "f32" else None

    def stage(i):
        if i == 0:
            mod.layout(inp["x"], inp["x_scale"], inp["ids"], inp["w"], inp["prank"])
        elif i == 1:
            M.moe_grouped_gemm_fp8(mod.ex, mod.ex_scale, wl.fmt, mod.w13, mod.w13_scale,
                                   mod.psum, mod.status, wl.align, mod.gate_up)
        elif i == 2:
            M.moe_act_quant(mod.gate_up, mod.m_indices, mod.psum, mod.status, mod.E, wl.align,
                            wl.fmt, fold, mod.dq, mod.ds)
        elif i == 3:
            M.moe_grouped_gemm_fp8(mod.dq, mod.ds, wl.fmt, mod.w2, mod.w2_scale, mod.psum,
                                   mod.status, wl.align, mod.down)
        else:
            mod.gather(inp["w"], inp["prank"], out)

    for _ in range(args.warmup):
        for i in range(5):
            stage(i)
    torch.cuda.synchronize()

    # Timed region: K whole steps; events only around the dominant kernel.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        stage(0)
        ev[s][0].record()
        stage(1)
        ev[s][1].record()
        stage(2)
        stage(3)
        stage(4)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    gemm1_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3

    # Per-stage breakdown (after the timed region; events between stages).
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(10)]
    for s in range(10):
        sev[s][0].record()
        for i in range(5):
            stage(i)
            sev[s][i + 1].record()
    torch.cuda.synchronize()
    names = ["expand_layout", "gemm_gate_up", "act_quant", "gemm_down", "gather"]
    stages_us = {n: float(np.median([sev[s][i].elapsed_time(sev[s][i + 1]) for s in range(10)]))
                 * 1e3 for i, n in enumerate(names)}

    status = mod.status.cpu().tolist()
    counts = np.bincount(inp["data"]["ids"][:inp["num_valid"]].reshape(-1)
                         .clip(-1, wl.experts - 1) + 1, minlength=wl.experts + 1)[1:]
    A = int(counts.sum())
    m_used = int(status[0])
    nonempty = int((counts > 0).sum())
    H, I = wl.hidden, wl.inter
    sb = 4 if wl.fmt == "f32" else 1
    g1_bytes = (nonempty * (2 * I * H + (2 * I // 128) * (H // 128) * sb)
                + m_used * (H + H // 128 * sb) + m_used * 2 * I * 2)
    g1_flops = 2.0 * A * 2 * I * H
    t = gemm1_us * 1e-6
    hbm_time = g1_bytes / (HBM_PEAK_GBS * 1e9)
    mfma_time = g1_flops / (FP8_PEAK_TFLOPS * 1e12)
    if hbm_time >= mfma_time:
        roof = {"bound": "hbm", "achieved": g1_bytes / t / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": g1_flops / t / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "grouped_gemm_kernel (gate_up)"
    roof["kernel_us"] = gemm1_us
    roof["algorithmic_bytes"] = int(g1_bytes)
    roof["useful_flops"] = g1_flops

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, wl, args.cpu_runs)

    res = {
        "metric": METRIC,
        "value": inp["num_valid"] / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded; routing/weights per the workload recipe)",
        "config": {"workload": wl.name, "rows": wl.rows, "valid_rows": inp["num_valid"],
                   "hidden": H, "inter": I, "experts_local": wl.experts,
                   "experts_global": wl.global_experts, "topk": wl.topk,
                   "align": wl.align, "scale_fmt": wl.fmt, "parallelism": "ep-rank share, 1 GPU",
                   "assignments": A, "expanded_rows": m_used, "capacity": mod.capacity},
        "stages_us": stages_us,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
