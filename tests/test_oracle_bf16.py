"""Pins for the oracle's bf16-weight path (CPU only).

The bf16-weight path (SGLang moe_runner/deep_gemm.py source,
_run_bf16_contiguous_gemm, inside the standard path) keeps the token rows and
the weights in bf16: bf16 gate_up GEMM, silu_and_mul to bf16, bf16 down GEMM,
the weighted gather with the routed scaling factor.  Pinned here by:

* the bf16 grouped GEMM on small-integer operands (exact in bf16) against an
  independent int64 matmul rounded once to bf16 (transposition, expert
  selection, skipped rows);
* the layer against a per-token brute force with no layout (bit-exact);
* one expert, top-1, weight 1: factor * dense SwiGLU MLP in float64, within
  the bf16 roundings;
A planted mistake (gate and up swapped) is caught.
"""

import numpy as np
import pytest

import workloads as W
from oracle import fp8, layer


def bf16_inputs(name="std_bf16_tiny", data=None, **over):
    wl = W.workload(name, **over)
    d = data or W.generate(wl)
    bits = lambda a: fp8.bf16_bits(fp8.round_bf16(a))  # noqa: E731
    return dict(x_bf16=bits(d["x"]), ids=d["ids"], w=d["w"], num_valid=d["num_valid"],
                w13_bf16=bits(d["w13"]), w2_bf16=bits(d["w2"]), align=wl.align,
                routed_scaling_factor=wl.routed_scale)


def test_bf16_gemm_integer_exact():
    rng = np.random.default_rng(1)
    M, N, K, E = 37, 256, 384, 3
    a = rng.integers(-4, 5, size=(M, K))
    w = rng.integers(-4, 5, size=(E, N, K))
    mi = rng.integers(-1, E, size=M).astype(np.int32)
    bits = lambda v: fp8.bf16_bits(v.astype(np.float32))  # noqa: E731  (small ints: exact)
    out = layer.bf16_grouped_gemm(bits(a), bits(w), mi, M)
    for m in range(M):
        if mi[m] < 0:
            assert np.all(np.isnan(out[m]))
        else:
            ref = fp8.round_bf16((a[m] @ w[mi[m]].T).astype(np.float64))
            assert np.array_equal(out[m], ref)


@pytest.mark.parametrize("over", [{}, dict(rows=37, topk=3, align=16, seed=19),
                                  dict(rows=50, experts=5, global_experts=7, seed=20)])
def test_bf16_layer_equals_brute_force(over):
    inp = bf16_inputs(**over)
    L = layer.bf16_layer(inp)
    assert np.array_equal(L["out"], layer.bf16_brute_force(inp))
    assert np.all(np.isfinite(L["out"])) and np.abs(L["out"]).max() > 0


def test_bf16_dense_swiglu_reduction():
    wl = W.workload("std_bf16_tiny", experts=1, global_experts=1, topk=1, seed=35)
    d = W.generate(wl)
    d["w"][:] = 1.0
    inp = bf16_inputs(data=d, experts=1, global_experts=1, topk=1, seed=35)
    out = layer.bf16_layer(inp)["out"]
    x = fp8.bf16_from_bits(inp["x_bf16"]).astype(np.float64)
    w13 = fp8.bf16_from_bits(inp["w13_bf16"][0]).astype(np.float64)
    w2 = fp8.bf16_from_bits(inp["w2_bf16"][0]).astype(np.float64)
    I = w2.shape[1]
    gate, up = x @ w13[:I].T, x @ w13[I:].T
    ref = wl.routed_scale * ((gate / (1 + np.exp(-gate)) * up) @ w2.T)
    # bf16 roundings of G, y and D (2^-9 relative each) against order-100%
    # errors for a swapped gate/up, a missing factor or a dropped term
    err = np.abs(out - ref)
    rms = np.sqrt(np.mean(ref ** 2))
    assert err.max() <= 0.05 * rms
    assert np.sqrt(np.mean(err ** 2)) <= 0.01 * rms


def test_planted_gate_up_swap_is_caught(monkeypatch):
    orig = layer.silu_mul
    monkeypatch.setattr(layer, "silu_mul", lambda g, u: orig(u, g))
    with pytest.raises(AssertionError):
        test_bf16_dense_swiglu_reduction()
