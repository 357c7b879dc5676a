"""Degenerate inputs on the GPU through the C ABI, against the oracle.

* A receive buffer with no valid rows (the per-source-rank prefix sum ends
  at 0, so R_v = 0; PaddedStandard contract of vLLM PR 54109): nothing is
  laid out (total 0) and no output row is written.
* Valid rows none of whose slots is local (every id -1): total 0, the
  GEMMs and act-quant find no rows, every valid output row is zero.
* A single received row; the standard path with a single token.
Bars as in the other parity tests: layout bit-exact, output within the
elementwise and rms bars (exactly zero where the oracle has no slot).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import layer, layout  # noqa: E402
from tests._inputs import make  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import (_check_output, _oracle_stage_inputs, bf16_np,  # noqa: E402
                                   check_layout, run_gpu)


def test_no_valid_rows():
    inp = make("tiny", rows=40, valid_rows=0, src_ranks=4, seed=95)
    assert layout.num_valid_rows(40, inp["psum_recv_per_rank"]) == 0
    print("case R_v = 0", flush=True)
    mod, out, _ = run_gpu(inp)
    ref = check_layout(mod, inp)
    assert ref["total"] == 0
    assert np.all(bf16_np(out) == 7.0)                    # nothing written


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_no_local_slots(fmt):
    inp = make("tiny", rows=32, fmt=fmt, seed=97)
    inp["ids"] = np.full_like(inp["ids"], -1)
    print(f"case no local slot, {fmt}", flush=True)
    mod, out, _ = run_gpu(inp)
    ref = check_layout(mod, inp)
    assert ref["total"] == 0
    assert np.all(mod.m_indices.cpu().numpy() == -1)
    assert np.all(bf16_np(out) == 0.0)                    # valid rows, no slot: zeros


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_single_row(fmt):
    inp = make("tiny", rows=1, topk=2, fmt=fmt, seed=96)
    print(f"case one row, {fmt}", flush=True)
    L = _oracle_stage_inputs(inp)
    mod, out, _ = run_gpu(inp)
    check_layout(mod, inp)
    _check_output(bf16_np(out), L["out"])


def test_standard_single_token():
    from tests.test_gpu_standard import check_layout as std_check_layout, run_std
    from tests.test_oracle_standard import std_inputs
    inp = std_inputs(rows=1, topk=4, seed=98)
    print("case standard path, one token", flush=True)
    L = layer.standard_layer(inp)
    mod, out, _ = run_std(inp)
    std_check_layout(mod, L)
    _check_output(bf16_np(out), L["out"], scale=inp["routed_scaling_factor"])
