"""Pins for the oracle's MXFP8 format (CPU only): fp8 codes with one UE8M0
scale per 1x32 group along K, for the activations and for every weight row
(SGLang moe_runner/deep_gemm.py source, DeepGemmMoeQuantInfo: MXFP8 requires
block shape [1, 32] and UE8M0 scales).

* Quantisation: every 32-wide group's largest magnitude lands in (224, 448],
  the byte is the float64 ceil(log2(amax / 448)) + 127, codes times scale
  reconstruct the values to half an fp8 step; groups differ by orders of
  magnitude, so a wrong group size or axis moves a scale by many binades.
* The grouped GEMM with small-integer codes and a random power-of-two scale
  on every 1x32 group of both operands against an independent int64 /
  float64 computation (exact: integer products times powers of two).
* The layer equals the per-token brute force (bit-exact).
A planted mistake (128-wide groups on the weights) is caught.
"""

import numpy as np
import pytest

import workloads as W
from oracle import fp8, layer, quant
from tests.test_oracle_layer import INT_CODES, _quantised_inputs


def test_mx_quant_groups():
    rng = np.random.default_rng(8)
    R, K = 5, 256
    mags = 2.0 ** rng.integers(-10, 10, size=(R, K // 32, 1))
    x = (rng.standard_normal((R, K // 32, 32)) * mags).reshape(R, K).astype(np.float32)
    q, s = quant.quantize_rows(x, "mxfp8")
    assert s.shape == (R, K // 32) and s.dtype == np.uint8
    amax = np.abs(x.astype(np.float64)).reshape(R, K // 32, 32).max(axis=2)
    m, e = np.frexp(amax / 448.0)
    e = np.where(m == 0.5, e - 1, e)
    assert np.array_equal(s.astype(np.int64), e + 127)
    sv = 2.0 ** (s.astype(np.float64) - 127)[:, :, None]
    codes = fp8.decode_e4m3(q).reshape(R, K // 32, 32)
    top = np.abs(codes).max(axis=2)
    assert np.all(top <= 448) and np.all(top >= 224)
    rec = codes * sv
    step = np.maximum(np.abs(rec), 2.0 ** -6 * sv) * 2.0 ** -3
    assert np.all(np.abs(rec - x.reshape(R, K // 32, 32)) <= 0.5 * step)
    w = rng.standard_normal((2, 128, K)).astype(np.float32)
    wq, ws = quant.quantize_blocks(w, "mxfp8")
    rq, rs = quant.quantize_rows(w.reshape(256, K), "mxfp8")     # per weight row
    assert ws.shape == (2, 128, K // 32)
    assert np.array_equal(ws.reshape(256, K // 32), rs) and np.array_equal(wq.reshape(256, K), rq)


def test_mx_gemm_integer_exact():
    rng = np.random.default_rng(9)
    M, N, K, E = 24, 256, 256, 3
    av = rng.integers(-2, 3, size=(M, K))
    wv = rng.integers(-2, 3, size=(E, N, K))
    a_q = np.vectorize(INT_CODES.get)(av).astype(np.uint8)
    w_q = np.vectorize(INT_CODES.get)(wv).astype(np.uint8)
    a_s = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    w_s = rng.integers(120, 135, size=(E, N, K // 32)).astype(np.uint8)
    mi = rng.integers(-1, E, size=M).astype(np.int32)
    out = layer.grouped_gemm(a_q, a_s, w_q, w_s, mi, M, "mxfp8")
    asc = np.repeat(2.0 ** (a_s.astype(np.float64) - 127), 32, axis=1)
    for m in range(M):
        if mi[m] < 0:
            assert np.all(np.isnan(out[m]))
            continue
        e = mi[m]
        wsc = np.repeat(2.0 ** (w_s[e].astype(np.float64) - 127), 32, axis=1)
        ref = (av[m] * asc[m])[None, :] * (wv[e] * wsc)
        assert np.array_equal(out[m], fp8.round_bf16(ref.sum(axis=1)))


@pytest.mark.parametrize("over", [{}, dict(align=16, topk=3, seed=77)])
def test_mx_layer_equals_brute_force(over):
    inp = _quantised_inputs(W.workload("tiny", **over), fmt="mxfp8")
    assert inp["x_s"].shape[1] == 256 // 32 and inp["w13_s"].shape[1:] == (256, 256 // 32)
    L = layer.layer(inp)
    assert L["mode"] == "post"
    assert L["ds"].shape[1] == 128 // 32
    assert np.array_equal(L["out"], layer.brute_force(inp))
    assert np.abs(L["out"]).max() > 0


def test_planted_weight_group_128_is_caught(monkeypatch):
    orig = quant.dequant_block

    def wrong(q, s, fmt, block=128):
        if fmt == "mxfp8":    # only every fourth 32-group's scale used, 128 wide
            s4 = np.repeat(np.asarray(s)[:, ::4], 4, axis=1)
            return quant.dequant_rows(q, s4, "mxfp8")
        return orig(q, s, fmt, block)
    monkeypatch.setattr(quant, "dequant_block", wrong)
    with pytest.raises(AssertionError):
        test_mx_gemm_integer_exact()
