"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (ExpandedMoE, capacity from the host bound).

* The layout is compared in full, bit-exact.
* The layer output: every valid row against the layered oracle
  (``oracle.layer.layer``; per-token brute force agrees with it bit for bit
  on the CPU tests), with the bars of ``_check_output`` (the elementwise bar
  on every row whose re-quantised activations agree with the oracle's in
  every fp8 code); rows past the boundary untouched; valid rows with no local
  slot exactly zero.
* The chain: act-quant on the GPU's own G, the down GEMM on the GPU's own
  dq/ds, the gather on the GPU's own D, each against the oracle's stage on
  those inputs, element by element.
* At `large`, `dsv3_zipf_ue8m0` and `dsv3`, every stage is also fed the
  oracle's input for that stage (G, dq/ds, D and the gather, each compared
  element by element): at `large` every expert spans three 256-row GEMM
  groups, and Zipf routing overloads three experts (thousands of rows) and
  empties three.
* The padded buffers also check that a tail whose ids alias valid experts
  changes nothing.
* `prefill_h6144` is the pages' prefill trace shape (18432 expanded rows of
  H=6144).
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from oracle import layout  # noqa: E402
from tests._inputs import make, to_gpu  # noqa: E402
from tests.test_gpu_parity import (SENT, _check_output, _oracle_stage_inputs,  # noqa: E402
                                   bf16_np, check_chain, check_stages, flipped_rows,
                                   gpu_intermediates)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

WORKERS = min(16, os.cpu_count() or 1)
_outs = {}


def run_full(name):
    print(f"\n[{name}] quantising inputs with the oracle", flush=True)
    inp = make(name)
    g = to_gpu(inp)
    R, T = inp["ids"].shape
    mod = M.ExpandedMoE(R, T, g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], inp["align"],
                        inp["fmt"])
    mod.ex.fill_(SENT)
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device="cuda")
    print(f"[{name}] running the layer on the GPU", flush=True)
    mod(g["x"], g["x_scale"], g["ids"], g["w"], g["prank"], out=out)
    torch.cuda.synchronize()
    return inp, g, mod, bf16_np(out)


def check_layout(name, inp, mod):
    R, T = inp["ids"].shape
    E = inp["w13_q"].shape[0]
    nv = layout.num_valid_rows(R, inp["psum_recv_per_rank"])
    lay = layout.expand_layout(inp["ids"], nv, E, inp["align"], mod.capacity)
    st = mod.status.cpu().numpy()
    assert st[0] == lay["total"] and st[1] == lay["flags"]
    assert np.array_equal(mod.psum.cpu().numpy(), lay["psum"])
    assert np.array_equal(mod.m_indices.cpu().numpy(), lay["m_indices"])
    src = mod.src2dst.cpu().numpy()
    assert np.array_equal(src, lay["src2dst"])
    n = lay["total"]
    ex = mod.ex[:n + 8].cpu().numpy()
    exs = mod.ex_scale.t()[:n].contiguous().cpu().numpy()   # stored K-block-major
    rw = mod.row_weight[:n].cpu().numpy()
    live = src >= 0
    rr, kk = np.nonzero(live)
    d = src[live]
    assert np.array_equal(ex[d], inp["x_q"][rr])
    assert np.array_equal(exs[d], inp["x_s"][rr])
    assert np.array_equal(rw[d].view(np.uint32), inp["w"][rr, kk].view(np.uint32))
    pad = np.ones(n, bool)
    pad[d] = False
    assert not ex[:n][pad].any() and not exs[pad].any() and not rw[pad].any()
    assert np.all(ex[n:] == SENT)
    print(f"[{name}] layout bit-exact: total {n}, counts {lay['counts'].tolist()}")


def check_all_rows(name, inp, L, I, out):
    """Every valid output row against the layered oracle (I: the GPU's
    intermediates, to find the rows whose re-quantised activations differ
    from the oracle's by a rounding-boundary flip)."""
    nv = L["out"].shape[0]
    print(f"[{name}] all {nv} valid rows against the oracle", flush=True)
    flip = flipped_rows(L["src2dst"], I["dq"], L["dq"], nv)
    _check_output(out[:nv], L["out"], flipped=flip, label=f"[{name}]")
    none = ~(inp["ids"][:nv] >= 0).any(axis=1)
    assert not np.any(out[:nv][none])                 # no local slot -> 0
    if nv < out.shape[0]:
        assert np.all(out[nv:] == 7.0)                # past the boundary: untouched


FULL = ["dsv3", "dsv3_zipf_ue8m0", "large", "padded", "padded_alias", "prefill_h6144"]
STAGES = {"dsv3", "dsv3_zipf_ue8m0", "large"}


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    inp, g, mod, out = run_full(name)
    check_layout(name, inp, mod)
    print(f"[{name}] oracle layer on {WORKERS} threads", flush=True)
    L = _oracle_stage_inputs(inp, workers=WORKERS)
    I = gpu_intermediates(mod, min(L["total"], mod.capacity))
    check_all_rows(name, inp, L, I, out)
    check_chain(inp, L, I, out, workers=WORKERS, label=f"[{name}]")
    del I
    if name in STAGES:
        check_stages(inp, L, g, mod, f"[{name}]", workers=WORKERS)
    if name.startswith("padded"):
        _outs[name] = out[:inp["num_valid"]].copy()


def test_full_padded_tail_is_never_routing():
    for name in ("padded", "padded_alias"):
        if name not in _outs:
            _outs[name] = run_full(name)[3][:1536].copy()
    assert np.array_equal(_outs["padded"].view(np.uint32), _outs["padded_alias"].view(np.uint32))
