"""GPU parity of the bf16-weight standard path through the C ABI
(moe_expand_layout_bf16 with MOE_SCALE_NONE -> moe_grouped_gemm_bf16 ->
moe_silu_mul_bf16 -> moe_grouped_gemm_bf16 -> moe_gather with weights and
the routed scaling factor) against the oracle's bf16_layer.

Bars:
* layout: labels, slot map, psum, status and the scattered bf16 rows
  bit-exact (a copy);
* bf16 GEMM (fed the oracle's rows): one bf16 ulp of the oracle plus
  2^-14 * sum |a w| (the oracle rounds a float64 sum once, the matrix cores
  sum bf16 products in fp32), under 5% of the elements off at all;
* SiLU*up to bf16 (fed the oracle's G): within one bf16 ulp (the GPU's expf
  and numpy's exp may differ by an ulp, which can move a value across a bf16
  rounding boundary), under 1% of the elements off;
* layer output: the bar of the other parity tests on out / f (f the routed
  scaling factor).
Full size (std_dsv3_bf16: 4096 rows, 256 experts of bf16 weights): layout in
full, sampled rows against the per-token brute force on host copies of
their experts.
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
import workloads as W  # noqa: E402
from oracle import fp8, layer  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import _check_output, bf16_np, bf16_ulp, check_gemm  # noqa: E402
from tests.test_oracle_bf16 import bf16_inputs  # noqa: E402


def t16(bits, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def run(inp):
    R, T = inp["ids"].shape
    mod = M.StandardBf16MoE(R, T, t16(inp["w13_bf16"]), t16(inp["w2_bf16"]), inp["align"],
                            inp["routed_scaling_factor"])
    mod.ex.fill_(1.5)
    ids = torch.from_numpy(inp["ids"]).cuda()
    w = torch.from_numpy(inp["w"]).cuda()
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device="cuda")
    mod(t16(inp["x_bf16"]), ids, w, out=out)
    torch.cuda.synchronize()
    return mod, out


def abs_terms_bf16(a_bits, w_bits, m_indices, rows):
    out = np.zeros((len(rows), w_bits.shape[1]))
    for e in np.unique(m_indices[rows]):
        sel = np.nonzero(m_indices[rows] == e)[0]
        A = np.abs(fp8.bf16_from_bits(a_bits[rows[sel]]).astype(np.float64))
        Wd = np.abs(fp8.bf16_from_bits(w_bits[e]).astype(np.float64))
        out[sel] = A @ Wd.T
    return out


CASES = [{}, dict(rows=37, topk=3, align=16, seed=19),
         dict(rows=50, experts=5, global_experts=7, seed=20),
         dict(rows=120, hidden=384, inter=256, experts=6, global_experts=8, topk=3, align=16,
              seed=21)]
IDS = ["-".join(f"{k}{v}" for k, v in o.items()) or "std_bf16_tiny" for o in CASES]


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_bf16_path(over):
    inp = bf16_inputs(**over)
    print(f"case {over}", flush=True)
    L = layer.bf16_layer(inp)
    mod, out = run(inp)
    # layout: bit-exact
    st = mod.status.cpu().numpy()
    assert st[0] == L["total"] and st[1] == L["flags"]
    assert np.array_equal(mod.psum.cpu().numpy(), L["psum"])
    assert np.array_equal(mod.m_indices.cpu().numpy(), L["m_indices"])
    assert np.array_equal(mod.src2dst.cpu().numpy(), L["src2dst"])
    n = min(L["total"], mod.capacity)
    ex = mod.ex.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(ex[:n], L["ex"])
    live = L["live"]
    rows = np.nonzero(live)[0]
    # gate_up GEMM on the same (bit-identical) rows
    G = bf16_np(mod.gate_up)[:n]
    check_gemm(G[live], L["G"][live],
               abs_terms_bf16(L["ex"], inp["w13_bf16"], L["m_indices"], rows), "bf16 gate_up")
    # SiLU*up on the oracle's G
    gu = torch.zeros_like(mod.gate_up)
    gu[:n] = torch.from_numpy(np.nan_to_num(L["G"], nan=0.0)).to(torch.bfloat16).cuda()
    y = torch.zeros_like(mod.y)
    M.moe_silu_mul_bf16(gu, mod.m_indices, mod.psum, mod.status, mod.E, inp["align"], y)
    torch.cuda.synchronize()
    yg = y.view(torch.int16).cpu().numpy().view(np.uint16)[:n]
    ref_y = fp8.bf16_from_bits(L["y"][live]).astype(np.float64)
    got_y = fp8.bf16_from_bits(yg[live]).astype(np.float64)
    off = got_y != ref_y
    assert off.mean() < 0.01 and np.all(np.abs(got_y - ref_y) <= bf16_ulp(ref_y))
    # down GEMM on the oracle's y
    yy = torch.zeros_like(mod.y)
    yy[:n] = t16(L["y"])
    M.moe_grouped_gemm_bf16(yy, mod.w2, mod.psum, mod.status, inp["align"], mod.down)
    torch.cuda.synchronize()
    D = bf16_np(mod.down)[:n]
    check_gemm(D[live], L["D"][live],
               abs_terms_bf16(L["y"], inp["w2_bf16"], L["m_indices"], rows), "bf16 down")
    # layer output
    _check_output(bf16_np(out), L["out"], scale=inp["routed_scaling_factor"])


@pytest.mark.slow
def test_bf16_full_size():
    import bench
    wl = W.workload("std_dsv3_bf16")
    print("\n[std_dsv3_bf16] generating routing and bf16 rows", flush=True)
    d = W.generate(wl, with_weights=False)
    x_bf16 = fp8.bf16_bits(fp8.round_bf16(d["x"]))
    R, T = d["ids"].shape
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    print(f"[std_dsv3_bf16] drawing {wl.experts} experts' bf16 weights on the GPU", flush=True)
    w13, w2 = bench.make_weights_bf16(wl, "cuda", gen)
    mod = M.StandardBf16MoE(R, T, w13, w2, wl.align, wl.routed_scale)
    ids = torch.from_numpy(d["ids"]).cuda()
    wts = torch.from_numpy(d["w"]).cuda()
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device="cuda")
    print("[std_dsv3_bf16] running the layer on the GPU", flush=True)
    mod(t16(x_bf16), ids, wts, out=out)
    torch.cuda.synchronize()
    from oracle import layout
    lay = layout.expand_layout(d["ids"], R, wl.experts, wl.align, mod.capacity)
    src = mod.src2dst.cpu().numpy()
    assert np.array_equal(src, lay["src2dst"])
    assert np.array_equal(mod.psum.cpu().numpy(), lay["psum"])
    ex = mod.ex[:lay["total"]].view(torch.int16).cpu().numpy().view(np.uint16)
    rr = np.nonzero(src >= 0)[0]
    assert np.array_equal(ex[src[src >= 0]], x_bf16[rr])
    print(f"[std_dsv3_bf16] layout bit-exact: total {lay['total']}", flush=True)
    # 256 sampled rows against the layered oracle restricted to them (the
    # other rows' slots dropped), on host copies of the experts they touch
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(R, size=256, replace=False))
    experts = np.unique(d["ids"][rows][d["ids"][rows] >= 0])
    remap = np.full(wl.experts, -1, np.int32)
    remap[experts] = np.arange(len(experts), dtype=np.int32)
    keep = np.zeros(R, bool)
    keep[rows] = True
    sub_ids = np.where((d["ids"] >= 0) & keep[:, None], remap[np.maximum(d["ids"], 0)],
                       -1).astype(np.int32)
    sel = torch.from_numpy(experts.astype(np.int64)).cuda()
    as_bits = lambda t: t.index_select(0, sel).view(torch.int16).cpu().numpy().view(np.uint16)  # noqa
    o = dict(x_bf16=x_bf16, ids=sub_ids, w=d["w"], num_valid=R, w13_bf16=as_bits(w13),
             w2_bf16=as_bits(w2), align=wl.align, routed_scaling_factor=wl.routed_scale)
    print(f"[std_dsv3_bf16] oracle on {len(rows)} sampled rows ({len(experts)} experts)",
          flush=True)
    ref = layer.bf16_layer(o, workers=min(16, os.cpu_count() or 1))["out"][rows]
    _check_output(bf16_np(out)[rows], ref, scale=wl.routed_scale)
