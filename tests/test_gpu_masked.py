"""GPU parity of the decode path on the masked slab through the C ABI
(moe_expand_layout -> moe_expand_to_masked_slab -> moe_grouped_gemm_fp8_masked
-> moe_act_quant_masked -> moe_grouped_gemm_fp8_masked ->
moe_masked_slab_to_expand -> moe_gather) against the oracle's masked_layer.

Bars:
* the bridge into the slab: masked_m, the overflow flag, the live slab rows
  and their scales bit-exact;
* the masked GEMMs and activation against the contiguous kernels on the
  same rows: bit-identical (a row's result depends only on its own data and
  the weights, in the same accumulation order);
* the bridge back, fed the GPU's slab rows: bit-exact with the oracle's
  (fp32 product, one bf16 rounding), dropped rows zero, pads untouched;
* layer output: the bar of the other parity tests against masked_layer.
Full size (dsv3_decode: 1024 rows, 8 of 256 experts, slab height 128):
the slab in full and sampled rows against the per-token brute force.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from oracle import masked  # noqa: E402
from tests._inputs import make, to_gpu  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import SENT, _check_output, bf16_np, rows_major  # noqa: E402


def run_masked(inp, max_m):
    g = to_gpu(inp)
    R, T = inp["ids"].shape
    mod = M.MaskedMoE(R, T, g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], inp["align"],
                      max_m, inp["fmt"])
    mod.slab.fill_(SENT)
    mod.s_gate_up.fill_(1.5)
    mod.s_down.fill_(1.5)
    mod.down.fill_(1.5)
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device="cuda")
    mod(g["x"], g["x_scale"], g["ids"], g["w"], g["prank"], out=out)
    torch.cuda.synchronize()
    return mod, out, g


def oracle_of(inp, max_m):
    o = {k: v for k, v in inp.items() if k != "psum_recv_per_rank"}
    from oracle import layout
    o["num_valid"] = layout.num_valid_rows(len(inp["ids"]), inp["psum_recv_per_rank"])
    return masked.masked_layer(o, max_m)


def check_slab(mod, L, max_m):
    mm = mod.masked_m.cpu().numpy()
    assert np.array_equal(mm, L["masked_m"])
    st = mod.status.cpu().numpy()
    assert (st[1] & masked.FLAG_SLAB_OVERFLOW) == L["slab_flags"]
    slab = mod.slab.cpu().numpy()
    ss = rows_major(mod.slab_scale)
    live = L["slab_labels"] >= 0
    assert np.array_equal(slab[live], L["slab"][live])
    assert np.array_equal(ss[live].view(np.uint8), np.ascontiguousarray(L["slab_scale"][live])
                          .view(np.uint8))
    assert np.all(slab[~live] == SENT)                    # past masked_m: untouched


CASES = [
    ("tiny", {}, 0),
    ("tiny", dict(fmt="ue8m0"), 0),
    ("tiny", dict(align=16, topk=3, seed=77), 16),
    ("tiny", dict(rows=40, valid_rows=23, src_ranks=4, seed=79), 0),
    ("tiny", dict(rows=300, hidden=384, inter=256, experts=6, global_experts=9, topk=4,
                  align=16, seed=81), 32),
    # slab lower than the busiest experts: rows dropped and flagged
    ("tiny", dict(rows=300, hidden=384, inter=256, experts=6, global_experts=9, topk=4,
                  align=16, seed=81), -1),
]
IDS = [f"{n}-{'-'.join(f'{k}{v}' for k, v in o.items())}-m{m}" for n, o, m in CASES]


def _max_m(inp, extra):
    from oracle import layout
    lay = layout.expand_layout(inp["ids"], layout.num_valid_rows(len(inp["ids"]),
                               inp["psum_recv_per_rank"]), inp["w13_q"].shape[0],
                               inp["align"], 10 ** 7)
    top = int(lay["counts"].max())
    if extra < 0:            # below the busiest expert
        return max(16, (top // 2) // 16 * 16)
    return (top + extra + 15) // 16 * 16


@pytest.mark.parametrize("name,over,extra", CASES, ids=IDS)
def test_masked_layer(name, over, extra):
    inp = make(name, **over)
    max_m = _max_m(inp, extra)
    print(f"case {name} {over} max_m={max_m}", flush=True)
    L = oracle_of(inp, max_m)
    mod, out, g = run_masked(inp, max_m)
    check_slab(mod, L, max_m)
    if extra < 0:
        assert L["slab_flags"] == masked.FLAG_SLAB_OVERFLOW
    # the bridge back, on the GPU's own slab rows: bit-exact
    n = min(L["total"], mod.capacity)
    back = masked.masked_slab_to_expand(bf16_np(mod.s_down), L["psum"], L["masked_m"], max_m, n,
                                        inp["align"], row_weight=L["row_weight"])
    down = bf16_np(mod.down)[:n]
    pad = np.isnan(back[:, 0])
    assert np.array_equal(down[~pad], back[~pad])
    assert np.all(down[pad] == 1.5)                       # alignment pads: not written
    nv = L["out"].shape[0]
    got = bf16_np(out)
    _check_output(got[:nv], L["out"])
    assert np.all(got[nv:] == 7.0)


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_masked_kernels_equal_contiguous(fmt):
    """The masked GEMMs and activation give the contiguous kernels' rows bit for
    bit: run both on the same expanded rows."""
    inp = make("tiny", rows=300, hidden=384, inter=256, experts=6, global_experts=9, topk=4,
               align=16, fmt=fmt, seed=85)
    max_m = _max_m(inp, 16)
    mod, _, g = run_masked(inp, max_m)
    E, align = mod.E, inp["align"]
    # contiguous kernels on the same expanded rows (no fold: the masked path has none)
    M.moe_grouped_gemm_fp8(mod.ex, mod.ex_scale, fmt, mod.w13, mod.w13_scale, mod.psum,
                           mod.status, align, mod.gate_up)
    M.moe_act_quant(mod.gate_up, mod.m_indices, mod.psum, mod.status, E, align, fmt, None,
                    mod.dq, mod.ds)
    M.moe_grouped_gemm_fp8(mod.dq, mod.ds, fmt, mod.w2, mod.w2_scale, mod.psum, mod.status,
                           align, mod.down)
    torch.cuda.synchronize()
    psum = mod.psum.cpu().numpy()
    mm = mod.masked_m.cpu().numpy()
    st = masked.expert_starts(psum, align)
    G, Gs = mod.gate_up.view(torch.int16).cpu().numpy(), mod.s_gate_up.view(torch.int16).cpu().numpy()
    D, Ds = mod.down.view(torch.int16).cpu().numpy(), mod.s_down.view(torch.int16).cpu().numpy()
    q, qs = mod.dq.cpu().numpy(), mod.s_dq.cpu().numpy()
    sc = rows_major(mod.ds).view(np.uint8)
    scs = rows_major(mod.s_ds).view(np.uint8)
    for e in range(E):
        a, b, n = st[e], e * max_m, mm[e]
        assert np.array_equal(Gs[b:b + n], G[a:a + n])
        assert np.array_equal(qs[b:b + n], q[a:a + n])
        assert np.array_equal(scs[b:b + n], sc[a:a + n])
        assert np.array_equal(Ds[b:b + n], D[a:a + n])


@pytest.mark.slow
def test_masked_full_size():
    print("\n[dsv3_decode] quantising inputs with the oracle", flush=True)
    inp = make("dsv3_decode")
    max_m = inp["workload"].max_m
    mod, out, g = run_masked(inp, max_m)
    from oracle import layer, layout
    lay = layout.expand_layout(inp["ids"], len(inp["ids"]), mod.E, inp["align"], mod.capacity)
    mm, flags = masked.masked_counts(lay["psum"], inp["align"], max_m)
    assert flags == 0 and np.array_equal(mod.masked_m.cpu().numpy(), mm)
    st = masked.expert_starts(lay["psum"], inp["align"])
    slab = mod.slab.cpu().numpy()
    src = mod.src2dst.cpu().numpy()
    assert np.array_equal(src, lay["src2dst"])
    # every live slot's row sits in its expert's slab at its rank
    rr, kk = np.nonzero(src >= 0)
    d = src[rr, kk]
    e = inp["ids"][rr, kk]
    assert np.array_equal(slab[e * max_m + (d - st[e])], inp["x_q"][rr])
    print(f"[dsv3_decode] slab bit-exact: masked_m {mm.tolist()}", flush=True)
    print(f"[dsv3_decode] oracle on all {len(inp['ids'])} rows", flush=True)
    L = oracle_of(inp, max_m)
    got = bf16_np(out)
    _check_output(got, L["out"])
    assert not np.any(got[~(inp["ids"] >= 0).any(axis=1)])    # no local slot -> 0
