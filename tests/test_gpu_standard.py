"""GPU parity of the standard (non-EP) path through the C ABI
(moe_expand_layout_bf16 -> grouped GEMM -> act-quant without fold -> grouped
GEMM -> gather with top-k weights and the routed scaling factor) against the
oracle's standard_layer.

Bars (as for the expand path):
* layout: labels, slot map, psum, status, and the scattered rows - here the
  fp8 codes and scales the layout computes from the bf16 rows - bit-exact
  (the per-group quantisation decides every code in fp32 on both sides with
  the same operations: amax, 448 / amax, x * (448 / amax), round to nearest
  even; UE8M0: the power-of-two byte and an exact scaling);
* gather with weights and the factor, fed the oracle's down rows:
  bit-exact;
* layer output: the elementwise bar 1e-2 + 2e-2 |oracle| plus the rms
  bars of the expand-path parity tests, applied to the output divided by
  the routed scaling factor f (the path multiplies the layer output by f
  after the expert computation, so every error scales with f: the absolute
  term becomes f * 1e-2).
Full size (std_dsv3: 4096 bf16 rows, H=7168, I=2048, all 256 experts
resident, top-8, factor 2.5): the layout and the quantised rows in full,
bit-exact; the output on sampled rows against the per-token brute force,
with the weights of just those rows' experts copied to the host.
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
import workloads as W  # noqa: E402
from oracle import fp8, layer, quant  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import (SENT, _check_output, bf16_np, flipped_rows,  # noqa: E402
                                   rows_major)
from tests.test_oracle_standard import std_inputs  # noqa: E402


def to_gpu_std(inp, dev="cuda"):
    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(x=t(inp["x_bf16"].view(np.int16)).view(torch.bfloat16), ids=t(inp["ids"]),
                w=t(inp["w"]), w13=t(inp["w13_q"]), w13_scale=t(inp["w13_s"]),
                w2=t(inp["w2_q"]), w2_scale=t(inp["w2_s"]))


def run_std(inp, stop=None):
    g = to_gpu_std(inp)
    R, T = inp["ids"].shape
    mod = M.StandardMoE(R, T, g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], inp["align"],
                        inp["fmt"], inp["routed_scaling_factor"])
    for buf in (mod.ex, mod.dq):
        buf.fill_(SENT)
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device="cuda")
    mod.layout(g["x"], g["ids"], g["w"])
    if stop != "layout":
        mod.experts()
        mod.gather(g["w"], None, out)
    torch.cuda.synchronize()
    return mod, out, g


def check_layout(mod, ref):
    st = mod.status.cpu().numpy()
    assert st[0] == ref["total"] and st[1] == ref["flags"]
    assert np.array_equal(mod.psum.cpu().numpy(), ref["psum"])
    assert np.array_equal(mod.m_indices.cpu().numpy(), ref["m_indices"])
    assert np.array_equal(mod.src2dst.cpu().numpy(), ref["src2dst"])
    n = min(ref["total"], mod.capacity)
    ex = mod.ex.cpu().numpy()
    assert np.array_equal(ex[:n], ref["ex"]), np.count_nonzero(ex[:n] != ref["ex"])
    assert np.all(ex[n:] == SENT)
    assert np.array_equal(rows_major(mod.ex_scale)[:n].view(np.uint8),
                          np.ascontiguousarray(ref["ex_scale"]).view(np.uint8))


SMALL = [
    {},
    dict(fmt="ue8m0"),
    dict(rows=300, hidden=384, inter=256, experts=6, global_experts=9, topk=3, align=16,
         seed=41),
    # H = 4608: a bf16 row is two passes of 512 16-byte chunks per wave
    dict(rows=40, hidden=4608, inter=256, experts=6, global_experts=8, topk=2, align=16,
         seed=42),
    dict(rows=40, hidden=4608, inter=256, experts=6, global_experts=8, topk=2, align=16,
         fmt="ue8m0", seed=43),
    dict(rows=200, hidden=512, inter=384, experts=5, global_experts=5, topk=2, align=64,
         routed_scale=1.0, seed=44),
]
IDS = ["-".join(f"{k}{v}" for k, v in o.items()) or "std_tiny" for o in SMALL]


@pytest.mark.parametrize("over", SMALL, ids=IDS)
def test_std_layout_bit_exact(over):
    inp = std_inputs(**over)
    print(f"case {over}", flush=True)
    L = layer.standard_layer(inp)
    mod, _, _ = run_std(inp, stop="layout")
    check_layout(mod, L)


@pytest.mark.parametrize("over", SMALL, ids=IDS)
def test_std_layer_against_oracle(over):
    inp = std_inputs(**over)
    print(f"case {over}", flush=True)
    L = layer.standard_layer(inp)
    mod, out, g = run_std(inp)
    check_layout(mod, L)
    got = bf16_np(out)
    _check_output(got, L["out"], scale=inp["routed_scaling_factor"])
    # the gather alone on the oracle's down rows: bit-exact, with the factor
    n = min(L["total"], mod.capacity)
    down = torch.zeros_like(mod.down)
    down[:n] = torch.from_numpy(np.nan_to_num(L["D"], nan=0.0)).to(torch.bfloat16).cuda()
    out2 = torch.full_like(out, 3.0)
    M.moe_gather(down, mod.src2dst, g["w"], None, out2,
                 routed_scaling_factor=inp["routed_scaling_factor"])
    torch.cuda.synchronize()
    assert np.array_equal(bf16_np(out2), L["out"])


@pytest.mark.slow
def test_std_full_size():
    import bench
    wl = W.workload("std_dsv3")
    print(f"\n[std_dsv3] generating routing and bf16 rows", flush=True)
    d = W.generate(wl, with_weights=False)
    x_bf16 = fp8.bf16_bits(fp8.round_bf16(d["x"]))
    R, T = d["ids"].shape
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    print(f"[std_dsv3] drawing {wl.experts} experts' weights on the GPU", flush=True)
    w13, w13s, w2, w2s = bench.make_weights(wl, dev, gen)
    mod = M.StandardMoE(R, T, w13, w13s, w2, w2s, wl.align, wl.fmt, wl.routed_scale)
    mod.ex.fill_(SENT)
    x = torch.from_numpy(x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(d["ids"]).to(dev)
    wts = torch.from_numpy(d["w"]).to(dev)
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device=dev)
    print("[std_dsv3] running the layer on the GPU", flush=True)
    mod(x, ids, wts, out=out)
    torch.cuda.synchronize()
    # layout and quantised rows, in full
    from oracle import layout
    lay = layout.expand_layout(d["ids"], R, wl.experts, wl.align, mod.capacity)
    st = mod.status.cpu().numpy()
    assert st[0] == lay["total"] and st[1] == lay["flags"]
    assert np.array_equal(mod.psum.cpu().numpy(), lay["psum"])
    assert np.array_equal(mod.m_indices.cpu().numpy(), lay["m_indices"])
    src = mod.src2dst.cpu().numpy()
    assert np.array_equal(src, lay["src2dst"])
    x_q, x_s = layer.quantize_input(x_bf16, R, wl.fmt)
    n = lay["total"]
    ex = mod.ex[:n + 8].cpu().numpy()
    exs = mod.ex_scale.t()[:n].contiguous().cpu().numpy()
    live = src >= 0
    rr = np.nonzero(live)[0]
    dd = src[live]
    assert np.array_equal(ex[dd], x_q[rr])
    assert np.array_equal(exs[dd].view(np.uint8), np.ascontiguousarray(x_s[rr]).view(np.uint8))
    assert np.all(ex[n:] == SENT)
    print(f"[std_dsv3] layout and quantised rows bit-exact: total {n}", flush=True)
    # 256 sampled rows against the layered oracle, on host copies of the
    # experts they touch; the other rows' slots are dropped (-1) so that the
    # oracle computes only these rows (each row's result depends only on its
    # own slots)
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(R, size=256, replace=False))
    experts = np.unique(d["ids"][rows][d["ids"][rows] >= 0])
    remap = np.full(wl.experts, -1, np.int32)
    remap[experts] = np.arange(len(experts), dtype=np.int32)
    keep = np.zeros(R, bool)
    keep[rows] = True
    sub_ids = np.where((d["ids"] >= 0) & keep[:, None], remap[np.maximum(d["ids"], 0)],
                       -1).astype(np.int32)
    sel = torch.from_numpy(experts).to(dev)
    o = dict(x_bf16=x_bf16, ids=sub_ids, w=d["w"], num_valid=R,
             w13_q=w13.index_select(0, sel).cpu().numpy(),
             w13_s=w13s.index_select(0, sel).cpu().numpy(),
             w2_q=w2.index_select(0, sel).cpu().numpy(),
             w2_s=w2s.index_select(0, sel).cpu().numpy(),
             align=wl.align, fmt=wl.fmt, routed_scaling_factor=wl.routed_scale)
    print(f"[std_dsv3] oracle on {len(rows)} sampled rows ({len(experts)} experts)", flush=True)
    L = layer.standard_layer(o, workers=min(16, os.cpu_count() or 1))
    ref = L["out"][rows]
    flip = flipped_rows(src[rows], mod.dq[:n].cpu().numpy(), L["dq"], len(rows),
                        src2dst_ref=L["src2dst"][rows])
    _check_output(bf16_np(out)[rows], ref, scale=wl.routed_scale, flipped=flip,
                  label="[std_dsv3]")
