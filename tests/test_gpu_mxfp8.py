"""GPU parity of the MXFP8 format (1x32 UE8M0 groups for the activations and
every weight row) through the C ABI, against the oracle.

Bars (as for the other formats):
* layout: labels, slot map, psum, status, scattered rows and their scale
  bytes bit-exact (the expanded scales are one 4-byte word per 128-wide
  block and row: the block's four 1x32 bytes in K order);
* grouped GEMM fed the oracle's rows: one bf16 ulp + 2^-14 * sum |a w|;
* act-quant fed the oracle's G: scale bytes equal except where SiLU's exp
  moves a group's max across a power of two (then one apart, < 0.5% of the
  groups), fp8 codes equal on < 1% off, by one step or the group's scale;
* layer: the elementwise bar and the rms bars.
Full size (dsv3_mxfp8): layout bit-exact, sampled rows against the brute force.
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from oracle import fp8, layer, layout  # noqa: E402
from tests._inputs import make  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import (_check_output, _oracle_stage_inputs, abs_terms,  # noqa: E402
                                   bf16_np, check_gemm, check_layout, flipped_rows, rows_major,
                                   run_gpu)

CASES = [dict(fmt="mxfp8"), dict(fmt="mxfp8", align=16, topk=3, seed=77),
         dict(fmt="mxfp8", rows=200, hidden=512, inter=384, experts=5, global_experts=5,
              topk=2, align=64, seed=82)]
IDS = ["-".join(f"{k}{v}" for k, v in o.items()) for o in CASES]


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_mx_layout_bit_exact(over):
    inp = make("tiny", **over)
    print(f"case {over}", flush=True)
    mod, _, _ = run_gpu(inp, stop="layout")
    check_layout(mod, inp)


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_mx_stages_and_layer(over):
    inp = make("tiny", **over)
    print(f"case {over}", flush=True)
    L = _oracle_stage_inputs(inp)
    mod, out, g = run_gpu(inp)
    n = min(L["total"], mod.capacity)
    live = L["live"]
    rows = np.nonzero(live)[0]
    # each stage on the oracle's inputs, then the whole path
    M.moe_grouped_gemm_fp8(mod.ex, mod.ex_scale, "mxfp8", mod.w13, mod.w13_scale, mod.psum,
                           mod.status, inp["align"], mod.gate_up)
    torch.cuda.synchronize()
    check_gemm(bf16_np(mod.gate_up)[:n][live], L["G"][live],
               abs_terms(L["ex"], L["ex_scale"], inp["w13_q"], inp["w13_s"], L["m_indices"],
                         rows, "mxfp8"), "mx gate_up")
    gu = torch.zeros_like(mod.gate_up)
    gu[:n] = torch.from_numpy(np.nan_to_num(L["G"], nan=0.0)).to(torch.bfloat16).cuda()
    M.moe_act_quant(gu, mod.m_indices, mod.psum, mod.status, mod.E, inp["align"], "mxfp8",
                    None, mod.dq, mod.ds)
    torch.cuda.synchronize()
    dq = mod.dq.cpu().numpy()[:n]
    ds = rows_major(mod.ds)[:n].view(np.uint8)
    assert np.array_equal(dq[~live], L["dq"][~live]) and not ds[~live].any()
    sdiff = ds[live].astype(int) - L["ds"][live].astype(int)
    assert np.all(np.abs(sdiff) <= 1) and (sdiff != 0).mean() < 5e-3
    cdiff = dq[live] != L["dq"][live]
    assert cdiff.mean() < 1e-2, cdiff.mean()
    # down GEMM on the oracle's dq / ds
    mod.dq[:n] = torch.from_numpy(L["dq"]).cuda()
    mod.ds.t()[:n] = torch.from_numpy(np.ascontiguousarray(L["ds"]).view(np.int32)).cuda()
    M.moe_grouped_gemm_fp8(mod.dq, mod.ds, "mxfp8", mod.w2, mod.w2_scale, mod.psum,
                           mod.status, inp["align"], mod.down)
    torch.cuda.synchronize()
    check_gemm(bf16_np(mod.down)[:n][live], L["D"][live],
               abs_terms(L["dq"], L["ds"], inp["w2_q"], inp["w2_s"], L["m_indices"], rows,
                         "mxfp8"), "mx down")
    _check_output(bf16_np(out)[:L["out"].shape[0]], L["out"])


@pytest.mark.slow
def test_mx_full_size():
    print("\n[dsv3_mxfp8] quantising inputs with the oracle", flush=True)
    inp = make("dsv3_mxfp8")
    mod, out, _ = run_gpu(inp)
    check_layout(mod, inp)
    o = {k: v for k, v in inp.items() if k != "psum_recv_per_rank"}
    print(f"[dsv3_mxfp8] oracle on all {len(inp['ids'])} rows", flush=True)
    L = layer.layer(o, workers=min(16, os.cpu_count() or 1))
    got = bf16_np(out)
    dq = mod.dq[:min(L["total"], mod.capacity)].cpu().numpy()
    _check_output(got, L["out"], flipped=flipped_rows(L["src2dst"], dq, L["dq"], len(got)),
                  label="[dsv3_mxfp8]")
    assert not np.any(got[~(inp["ids"] >= 0).any(axis=1)])    # no local slot -> 0
