"""Test inputs: seeded workloads quantised by the oracle's quantiser, and
their copies on the GPU.  Every value here comes from the workload
generator and the oracle; nothing comes from the HIP path."""

import numpy as np

import workloads as W
from oracle import quant


def quantise(data, fmt=None):
    """Quantise a generated workload with the oracle (per expert / row chunk
    to bound host memory).  Returns the oracle's input dict."""
    wl = data["workload"]
    fmt = fmt or wl.fmt
    R, H = data["x"].shape
    sdt = np.float32 if fmt == "f32" else np.uint8
    g = 32 if fmt == "mxfp8" else 128
    x_q = np.empty((R, H), np.uint8)
    x_s = np.empty((R, H // g), sdt)
    for r0 in range(0, R, 2048):
        x_q[r0:r0 + 2048], x_s[r0:r0 + 2048] = quant.quantize_rows(data["x"][r0:r0 + 2048], fmt)
    W.poison_tail(data, x_q, x_s)

    def blocks(w):
        E, N, K = w.shape
        q = np.empty((E, N, K), np.uint8)
        s = np.empty((E, N, K // 32) if fmt == "mxfp8" else (E, N // 128, K // 128), sdt)
        for e in range(E):
            q[e:e + 1], s[e:e + 1] = quant.quantize_blocks(w[e:e + 1], fmt)
        return q, s
    w13_q, w13_s = blocks(data["w13"])
    w2_q, w2_s = blocks(data["w2"])
    return dict(x_q=x_q, x_s=x_s, ids=data["ids"], w=data["w"], num_valid=data["num_valid"],
                psum_recv_per_rank=data["psum_recv_per_rank"], w13_q=w13_q, w13_s=w13_s,
                w2_q=w2_q, w2_s=w2_s, align=wl.align, fmt=fmt, workload=wl)


def make(name, **over):
    wl = W.workload(name, **over)
    return quantise(W.generate(wl))


def to_gpu(inp, device="cuda"):
    import torch

    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(x=t(inp["x_q"]), x_scale=t(inp["x_s"]), ids=t(inp["ids"]), w=t(inp["w"]),
                prank=t(inp["psum_recv_per_rank"]), w13=t(inp["w13_q"]),
                w13_scale=t(inp["w13_s"]), w2=t(inp["w2_q"]), w2_scale=t(inp["w2_s"]))
