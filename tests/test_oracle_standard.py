"""Pins for the oracle's standard (non-EP) path (CPU only).

The standard path (SGLang moe_runner/deep_gemm.py source,
pre_permute_standard_to_deep_gemm / post_permute_deep_gemm_to_standard)
takes bf16 rows, quantises each per 1x128 group, runs the same layout and
expert computation, and reduces each token's rows with its top-k weights
times the routed scaling factor.  Pinned here by:

* the input quantisation's groups: within every 128-column group of a row the
  largest magnitude maps to the fp8 maximum 448, the fp32 scale is the
  group's amax / 448 (checked in float64 to within one fp32 rounding), the
  UE8M0 byte is the float64 ceil(log2(amax / 448)) + 127, and codes times
  scale reconstruct the row to half an fp8 step;
* an identity: bf16 rows that are already dequantised UE8M0 fp8 values
  requantise to the same values (the scale is a power of two and the codes
  are exact), so the standard path equals the expand path with post
  weighting on the original fp8 rows, bit for bit;
* the routed scaling factor: a power of two scales the output exactly, and
  2.5 to within the two roundings it adds;
* a per-token brute force with no layout (bit-exact);
* with one expert, top-1 and weight 1 the path is factor * dense SwiGLU MLP
  (float64 closed form, within the fp8 error).
A planted mistake (the factor ignored) is caught.
"""

import numpy as np
import pytest

import workloads as W
from oracle import fp8, layer, quant


def std_inputs(name="std_tiny", fmt=None, data=None, **over):
    wl = W.workload(name, **over)
    d = data or W.generate(wl)
    fmt = fmt or wl.fmt
    w13_q, w13_s = quant.quantize_blocks(d["w13"], fmt)
    w2_q, w2_s = quant.quantize_blocks(d["w2"], fmt)
    x_bf16 = fp8.bf16_bits(fp8.round_bf16(d["x"]))
    return dict(x_bf16=x_bf16, ids=d["ids"], w=d["w"], num_valid=d["num_valid"],
                w13_q=w13_q, w13_s=w13_s, w2_q=w2_q, w2_s=w2_s, align=wl.align, fmt=fmt,
                routed_scaling_factor=wl.routed_scale)


def _row_groups(x):
    R, H = x.shape
    return x.reshape(R, H // 128, 128)


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_input_quant_groups(fmt):
    rng = np.random.default_rng(5)
    R, H = 6, 512
    # groups of very different magnitude, so a wrong group size or axis
    # moves a scale by orders of magnitude
    mags = 2.0 ** rng.integers(-12, 10, size=(R, H // 128, 1))
    x = fp8.round_bf16((rng.standard_normal((R, H // 128, 128)) * mags).reshape(R, H))
    bits = fp8.bf16_bits(x)
    q, s = layer.quantize_input(bits, R, fmt)
    amax = np.abs(_row_groups(x.astype(np.float64))).max(axis=2)
    codes = fp8.decode_e4m3(q).reshape(R, H // 128, 128)
    if fmt == "f32":
        assert np.all(np.abs(codes).max(axis=2) == 448.0)
        ref = amax / 448.0
        assert np.all(np.abs(s.astype(np.float64) - ref) <= ref * 2.0 ** -24)
        sv = s.astype(np.float64)[:, :, None]
    else:
        m, e = np.frexp(amax / 448.0)                  # amax/448 = m * 2^e, m in [0.5, 1)
        e = np.where(m == 0.5, e - 1, e)               # exact powers of two: no round-up
        assert np.array_equal(s.astype(np.int64), e + 127)
        sv = 2.0 ** (s.astype(np.float64) - 127)[:, :, None]
        # tight: the scale is the smallest power of two with amax / s <= 448
        assert np.all(amax[:, :, None] / sv <= 448.0)
        assert np.all(amax[:, :, None] / sv > 224.0)
    rec = codes * sv
    step = np.maximum(np.abs(rec), 2.0 ** -6 * sv) * 2.0 ** -3
    assert np.all(np.abs(rec - _row_groups(x.astype(np.float64))) <= 0.5 * step + 1e-300)


def test_ue8m0_requantisation_identity():
    wl = W.workload("std_tiny", fmt="ue8m0", routed_scale=1.0)
    d = W.generate(wl)
    inp = std_inputs(data=d, fmt="ue8m0", routed_scale=1.0)
    x_q, x_s = quant.quantize_rows(d["x"], "ue8m0")
    deq = quant.dequant_rows(x_q, x_s, "ue8m0")
    assert np.array_equal(fp8.round_bf16(deq), deq)      # exact in bf16
    inp["x_bf16"] = fp8.bf16_bits(deq.astype(np.float32))
    inp["routed_scaling_factor"] = 1.0
    std = layer.standard_layer(inp)["out"]
    ex = {k: v for k, v in inp.items() if k not in ("x_bf16", "routed_scaling_factor")}
    ex.update(x_q=x_q, x_s=x_s)
    ref = layer.layer(ex, mode="post")["out"]
    assert np.array_equal(std, ref)


def test_routed_scale_power_of_two_exact():
    inp = std_inputs()
    inp["routed_scaling_factor"] = 1.0
    one = layer.standard_layer(inp)["out"]
    for f in (2.0, 0.5):
        inp["routed_scaling_factor"] = f
        assert np.array_equal(layer.standard_layer(inp)["out"], one * np.float32(f))
    assert np.abs(one).max() > 0


def test_routed_scale_general():
    inp = std_inputs()
    inp["routed_scaling_factor"] = 1.0
    one = layer.standard_layer(inp)["out"].astype(np.float64)
    inp["routed_scaling_factor"] = 2.5
    got = layer.standard_layer(inp)["out"].astype(np.float64)
    # 2.5 * bf16(acc) vs bf16(2.5 * acc): 2.5 half-ulps of acc plus half an
    # ulp of the result, at most 1.75 ulps of |2.5 * acc|
    ref = 2.5 * one
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    assert np.all(np.abs(got - ref) <= 2 * ulp)
    assert not np.array_equal(got, one)


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
@pytest.mark.parametrize("over", [{}, dict(rows=37, topk=3, align=16, seed=17)])
def test_standard_equals_brute_force(fmt, over):
    inp = std_inputs(fmt=fmt, **over)
    L = layer.standard_layer(inp)
    assert np.array_equal(L["out"], layer.brute_force(inp))
    assert np.all(np.isfinite(L["out"])) and np.abs(L["out"]).max() > 0


def test_standard_dense_swiglu_reduction():
    wl = W.workload("std_tiny", experts=1, global_experts=1, topk=1, seed=33)
    d = W.generate(wl)
    d["w"][:] = 1.0
    inp = std_inputs(data=d)
    out = layer.standard_layer(inp)["out"]
    x = fp8.bf16_from_bits(inp["x_bf16"]).astype(np.float64)
    w13 = quant.dequant_block(inp["w13_q"][0], inp["w13_s"][0], "f32")
    w2 = quant.dequant_block(inp["w2_q"][0], inp["w2_s"][0], "f32")
    I = w2.shape[1]
    gate, up = x @ w13[:I].T, x @ w13[I:].T
    ref = wl.routed_scale * ((gate / (1 + np.exp(-gate)) * up) @ w2.T)
    # Skipped by the continuous reference: the fp8 rounding of the input rows
    # and of silu(gate)*up (3 mantissa bits each, a few % rms after the
    # projections) and the bf16 roundings; a missing factor, a swapped
    # gate/up or a dropped term is off by order 100%.
    err = np.abs(out - ref)
    rms = np.sqrt(np.mean(ref ** 2))
    assert err.max() <= 0.25 * rms
    assert np.sqrt(np.mean(err ** 2)) <= 0.05 * rms


def test_planted_ignored_factor_is_caught(monkeypatch):
    orig = layer.gather
    monkeypatch.setattr(layer, "gather",
                        lambda D, s, nv, topk_weights=None, scale=1.0:
                        orig(D, s, nv, topk_weights=topk_weights))
    with pytest.raises(AssertionError):
        test_routed_scale_power_of_two_exact()
