"""GPU parity of the expand path on seeded random configurations, through
the C ABI, against the oracle: combinations of row count (odd ones
included), hidden and intermediate sizes (any multiple of 128), local and
global expert counts, top-k, alignment, scale format (fp32, UE8M0, MXFP8)
and a padded receive buffer that the hand-picked cases do not cover.

Each case: the layout bit-exact (labels, slot map, psum, status, scattered
rows, scales and weights, rows past the total untouched) and the layer
output within the elementwise and rms bars of the other parity tests, rows
past R_v untouched.  The configurations are drawn once from a fixed seed, so
the set is the same on every run.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests._inputs import make  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import (_check_output, _oracle_stage_inputs, bf16_np,  # noqa: E402
                                   check_layout, run_gpu)


def _cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ("f32", "ue8m0", "mxfp8")[i % 3]
        experts = int(rng.integers(1, 41))
        glob = int(experts + rng.integers(0, 2 * experts + 1))
        c = dict(rows=int(rng.integers(1, 701)), hidden=128 * int(rng.integers(1, 9)),
                 inter=128 * int(rng.integers(1, 7)), experts=experts, global_experts=glob,
                 topk=int(rng.integers(1, min(8, glob) + 1)),
                 align=int(rng.choice([16, 32, 64, 128])), fmt=fmt, seed=3000 + i)
        if rng.random() < 0.3 and c["rows"] > 4:      # padded receive buffer
            c["valid_rows"] = int(rng.integers(0, c["rows"]))
            c["src_ranks"] = int(rng.integers(1, 9))
        out.append(c)
    return out


CASES = _cases()
IDS = ["-".join(f"{k}{v}" for k, v in c.items()) for c in CASES]


@pytest.mark.parametrize("over", CASES, ids=IDS)
def test_random_config(over):
    print(f"case {over}", flush=True)
    inp = make("tiny", **over)
    L = _oracle_stage_inputs(inp)
    mod, out, _ = run_gpu(inp)
    check_layout(mod, inp)
    got = bf16_np(out)
    nv = L["out"].shape[0]
    if nv:
        _check_output(got[:nv], L["out"])
    assert np.all(got[nv:] == 7.0)                        # rows past R_v untouched


# The other paths on random configurations of their own.

def _std_cases(n=6, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        experts = int(rng.integers(1, 41))          # every expert local
        out.append(dict(rows=int(rng.integers(1, 401)), hidden=128 * int(rng.integers(1, 9)),
                        inter=128 * int(rng.integers(1, 7)), experts=experts,
                        global_experts=experts, topk=int(rng.integers(1, min(8, experts) + 1)),
                        align=int(rng.choice([16, 32, 64, 128])),
                        routed_scale=float(rng.choice([1.0, 2.5])), seed=3100 + i))
    return out


STD_CASES = _std_cases()
STD_IDS = ["-".join(f"{k}{v}" for k, v in c.items()) for c in STD_CASES]


@pytest.mark.parametrize("over", STD_CASES, ids=STD_IDS)
@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_random_standard(over, fmt):
    """The standard path (bf16 rows quantised in the layout): layout bit-exact,
    output within the bar on out / f."""
    from oracle import layer
    from tests.test_gpu_standard import check_layout as std_check_layout, run_std
    from tests.test_oracle_standard import std_inputs
    print(f"case {over} {fmt}", flush=True)
    inp = std_inputs(fmt=fmt, **over)
    L = layer.standard_layer(inp)
    mod, out, _ = run_std(inp)
    std_check_layout(mod, L)
    _check_output(bf16_np(out), L["out"], scale=inp["routed_scaling_factor"])


@pytest.mark.parametrize("over", STD_CASES, ids=STD_IDS)
def test_random_bf16_weights(over):
    """The bf16-weight path: layout (a bf16 row copy) bit-exact, output
    within the bar on out / f."""
    from oracle import layer
    from tests.test_gpu_bf16 import run as run_bf16
    from tests.test_oracle_bf16 import bf16_inputs
    print(f"case {over}", flush=True)
    inp = bf16_inputs(**over)
    L = layer.bf16_layer(inp)
    mod, out = run_bf16(inp)
    st = mod.status.cpu().numpy()
    assert st[0] == L["total"] and st[1] == L["flags"]
    assert np.array_equal(mod.src2dst.cpu().numpy(), L["src2dst"])
    n = min(L["total"], mod.capacity)
    assert np.array_equal(mod.ex.view(torch.int16).cpu().numpy().view(np.uint16)[:n], L["ex"])
    _check_output(bf16_np(out), L["out"], scale=inp["routed_scaling_factor"])


def _masked_cases(n=6, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        experts = int(rng.integers(1, 25))
        glob = int(experts + rng.integers(0, 2 * experts + 1))
        c = dict(rows=int(rng.integers(1, 401)), hidden=128 * int(rng.integers(1, 9)),
                 inter=128 * int(rng.integers(1, 7)), experts=experts, global_experts=glob,
                 topk=int(rng.integers(1, min(8, glob) + 1)),
                 align=int(rng.choice([16, 32, 64, 128])), fmt=("f32", "ue8m0")[i % 2],
                 seed=3200 + i)
        out.append((c, int(rng.choice([-1, 0, 16, 48]))))
    return out


MASKED_CASES = _masked_cases()
MASKED_IDS = ["-".join(f"{k}{v}" for k, v in c.items()) + f"-m{x}" for c, x in MASKED_CASES]


@pytest.mark.parametrize("over,extra", MASKED_CASES, ids=MASKED_IDS)
def test_random_masked(over, extra):
    """The decode path on the masked slab (slab height from the busiest
    expert: above it, or below it so rows are dropped and flagged): masked_m,
    the flag, the slab rows and scales bit-exact, output within the bar."""
    from tests.test_gpu_masked import _max_m, check_slab, oracle_of, run_masked
    inp = make("tiny", **over)
    max_m = _max_m(inp, extra)
    print(f"case {over} max_m={max_m}", flush=True)
    L = oracle_of(inp, max_m)
    mod, out, _ = run_masked(inp, max_m)
    check_slab(mod, L, max_m)
    nv = L["out"].shape[0]
    got = bf16_np(out)
    if nv:
        _check_output(got[:nv], L["out"])
    assert np.all(got[nv:] == 7.0)
