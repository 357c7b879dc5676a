"""Pins for the oracle's expert computation (CPU only).

* Grouped GEMM: integer-valued fp8 operands make the product an exact
  integer matmul (numpy int64), so the transposition, the expert selection,
  the skipped rows and each 128x128 / 1x128 block scale are checked against
  an independent integer computation.
* SiLU*up against the float64 closed form; quantisation against its defining
  properties (the group's largest magnitude maps to 448, q*s reconstructs y
  to half an fp8 step, the fold multiplies the scale, UE8M0 scales are the
  tight power of two), for 1x128 rows and for 128x128 weight blocks; the
  live-row mask on a hand case and against the layout's pad rows.
* Gather against a hand-computed case.
* The whole layer equals a per-token brute force with no layout (bit-exact);
  the weight fold equals post-weighting to bf16 rounding; with one expert,
  top-1 and weight 1 the layer is a dense SwiGLU MLP (float64 closed form);
  the receive-buffer tail beyond the boundary never changes the output.
* Planted mistakes (a swapped gate/up, a transposed weight, a dropped scale)
  are caught by these pins.
"""

import numpy as np
import pytest

import workloads as W
from oracle import fp8, layer, layout, quant

INT_CODES = {-2: 0xC0, -1: 0xB8, 0: 0x00, 1: 0x38, 2: 0x40}


def int_fp8(rng, shape):
    v = rng.integers(-2, 3, size=shape)
    codes = np.vectorize(INT_CODES.get)(v).astype(np.uint8)
    return v.astype(np.int64), codes


def test_int_codes_decode():
    for v, c in INT_CODES.items():
        assert fp8.decode_e4m3(c) == v


def test_gemm_integer_exact_with_expert_selection():
    rng = np.random.default_rng(0)
    M, N, K, E = 40, 384, 256, 3
    a_int, a_q = int_fp8(rng, (M, K))
    w_int, w_q = int_fp8(rng, (E, N, K))
    a_s = np.ones((M, K // 128), np.float32)
    w_s = np.ones((E, N // 128, K // 128), np.float32)
    mi = rng.integers(-1, E, size=M).astype(np.int32)
    out = layer.grouped_gemm(a_q, a_s, w_q, w_s, mi, M, "f32")
    for m in range(M):
        if mi[m] < 0:
            assert np.all(np.isnan(out[m]))
        else:
            exact = a_int[m] @ w_int[mi[m]].T           # [N], rows x cols^T
            assert np.array_equal(out[m], fp8.round_bf16(exact.astype(np.float64)))


def test_gemm_block_scales_closed_form():
    rng = np.random.default_rng(1)
    M, N, K, E = 16, 256, 384, 2
    a_int, a_q = int_fp8(rng, (M, K))
    w_int, w_q = int_fp8(rng, (E, N, K))
    a_s = (2.0 ** rng.integers(-3, 4, size=(M, K // 128))).astype(np.float32)
    w_s = (2.0 ** rng.integers(-3, 4, size=(E, N // 128, K // 128))).astype(np.float32)
    a_s[3, 1] = 0.75
    w_s[1, 1, 2] = 1.25
    mi = (np.arange(M) % E).astype(np.int32)
    out = layer.grouped_gemm(a_q, a_s, w_q, w_s, mi, M, "f32")
    for m in range(M):
        e = mi[m]
        exact = np.zeros(N)
        for kb in range(K // 128):
            ks = slice(kb * 128, (kb + 1) * 128)
            part = a_int[m, ks] @ w_int[e, :, ks].T            # integers
            exact += part * a_s[m, kb] * np.repeat(w_s[e, :, kb], 128)
        assert np.array_equal(out[m], fp8.round_bf16(exact))


def test_gemm_ue8m0_matches_f32_of_same_values():
    rng = np.random.default_rng(2)
    M, N, K, E = 8, 128, 256, 2
    _, a_q = int_fp8(rng, (M, K))
    _, w_q = int_fp8(rng, (E, N, K))
    a_b = rng.integers(120, 134, size=(M, K // 128)).astype(np.uint8)
    w_b = rng.integers(120, 134, size=(E, N // 128, K // 128)).astype(np.uint8)
    mi = (np.arange(M) % E).astype(np.int32)
    o8 = layer.grouped_gemm(a_q, a_b, w_q, w_b, mi, M, "ue8m0")
    o32 = layer.grouped_gemm(a_q, np.ldexp(1.0, a_b.astype(int) - 127).astype(np.float32),
                             w_q, np.ldexp(1.0, w_b.astype(int) - 127).astype(np.float32),
                             mi, M, "f32")
    assert np.array_equal(o8, o32)


def test_silu_mul_closed_form():
    g = np.linspace(-20, 20, 4001).astype(np.float32)
    u = np.float32(1.5) - g * np.float32(0.1)
    ref = g.astype(np.float64) * u / (1.0 + np.exp(-g.astype(np.float64)))
    got = layer.silu_mul(g, u)
    assert np.allclose(got, ref, rtol=4e-7, atol=1e-30)
    assert layer.silu_mul(np.float32(0.0), np.float32(3.0)) == 0.0
    # each of the four float32 operations is one rounding of its exact result:
    # exp(-g) is the correctly rounded float32 of the float64 exp, then the
    # add, divide and multiply in IEEE float32 (checked here in float64 with an
    # explicit rounding after every step)
    r32 = lambda v: np.asarray(v, np.float64).astype(np.float32).astype(np.float64)  # noqa
    gg = (np.random.default_rng(4).standard_normal(200_000) * 6).astype(np.float32)
    uu = np.float32(0.75)
    e = r32(np.exp(-gg.astype(np.float64)))
    step = r32(r32(gg.astype(np.float64) / r32(1.0 + e)) * np.float64(uu))
    assert np.array_equal(layer.silu_mul(gg, uu).astype(np.float64), step)
    # silu is not symmetric in its two inputs
    assert layer.silu_mul(np.float32(-2.0), np.float32(1.0)) != \
        layer.silu_mul(np.float32(1.0), np.float32(-2.0))


def test_quant_f32_properties():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((20, 512)) * 2.0 ** rng.integers(-8, 8, (20, 1))).astype(np.float32)
    y[0, :128] = 0.0                    # an all-zero group: eps clamp
    q, s = quant.quantize_rows(y, "f32")
    deq = quant.dequant_rows(q, s, "f32")
    g = y.reshape(20, 4, 128)
    amax = np.maximum(np.abs(g).max(axis=2), np.float32(1e-10))
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    # the largest magnitude of each group lands on +-448 (code 0x7E / 0xFE)
    idx = np.abs(g).argmax(axis=2)
    qa = q.reshape(20, 4, 128)
    for r in range(1, 20):
        for j in range(4):
            assert qa[r, j, idx[r, j]] & 0x7F == 0x7E
    assert not q[0, :128].any() and s[0, 0] == np.float32(1e-10 / 448)
    # reconstruction within half an fp8 step (relative 2^-4) plus subnormal
    scaled = np.abs(y.astype(np.float64)) / np.repeat(s, 128, axis=1)
    step = np.where(scaled >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(scaled, 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - y) <= 0.5 * step * np.repeat(s, 128, axis=1) * (1 + 1e-6))


def test_quant_ue8m0_properties():
    rng = np.random.default_rng(4)
    y = (rng.standard_normal((16, 256)) * 2.0 ** rng.integers(-10, 10, (16, 1))).astype(np.float32)
    q, b = quant.quantize_rows(y, "ue8m0")
    s = fp8.e8m0_value(b)
    amax = np.abs(y.reshape(16, 2, 128)).max(axis=2).astype(np.float64)
    need = amax / 448.0
    assert np.all(s >= need * (1 - 1e-7)) and np.all(s / 2 < need)
    deq = quant.dequant_rows(q, b, "ue8m0")
    assert np.all(np.abs(deq - y) <= np.abs(y) * 2 ** -4 + np.repeat(s, 128, axis=1) * 2 ** -10)
    assert np.all(np.abs(fp8.decode_e4m3(q)) <= 448)


def test_quant_blocks_properties():
    """128x128 weight blocks: one scale per block of each expert's [N, K]
    matrix; the block's largest magnitude maps to +-448 (fp32 scales, amax /
    448 to one fp32 rounding in float64) or the UE8M0 byte is the tight power
    of two (float64 ceil(log2(amax / 448)) + 127); every code reconstructs its
    value to half an fp8 step.  Blocks are given magnitudes 2^-12 .. 2^12
    apart, so a block mixed up with its neighbour (a transposed or shifted
    block index) fails."""
    rng = np.random.default_rng(6)
    E, N, K = 2, 256, 384
    mag = 2.0 ** rng.integers(-12, 13, (E, N // 128, K // 128))
    w = (rng.standard_normal((E, N, K))
         * np.repeat(np.repeat(mag, 128, axis=1), 128, axis=2)).astype(np.float32)
    w[1, :128, 128:256] = 0.0            # an all-zero block: eps clamp
    blocks = w.astype(np.float64).reshape(E, N // 128, 128, K // 128, 128)
    amax = np.abs(blocks).max(axis=(2, 4))
    for fmt in ("f32", "ue8m0"):
        q, s = quant.quantize_blocks(w, fmt)
        assert q.shape == (E, N, K) and s.shape == (E, N // 128, K // 128)
        sv = quant.scale_values(s, fmt)
        if fmt == "f32":
            ref = np.maximum(amax, 1e-10) / 448.0
            assert np.all(np.abs(sv - ref) <= ref * 2.0 ** -23)
            qb = q.reshape(E, N // 128, 128, K // 128, 128)
            for e in range(E):
                for i in range(N // 128):
                    for j in range(K // 128):
                        if amax[e, i, j] == 0:
                            assert not qb[e, i, :, j, :].any()
                            continue
                        a = np.abs(blocks[e, i, :, j, :])
                        r, c = np.unravel_index(a.argmax(), a.shape)
                        assert qb[e, i, r, j, c] & 0x7F == 0x7E    # +-448
        else:
            live = amax > 0
            need = np.log2(amax[live] / 448.0)
            assert np.array_equal(s[live].astype(np.int64), np.ceil(need).astype(np.int64) + 127)
        deq = np.stack([quant.dequant_block(q[e], s[e], fmt) for e in range(E)])
        scale = np.repeat(np.repeat(sv, 128, axis=1), 128, axis=2)
        scaled = np.abs(w.astype(np.float64)) / scale
        step = np.where(scaled >= 2 ** -6,
                        2.0 ** (np.floor(np.log2(np.maximum(scaled, 1e-300))) - 3), 2.0 ** -9)
        assert np.all(np.abs(deq - w) <= 0.5 * step * scale * (1 + 1e-6))


def test_live_rows_hand_case():
    """Row m of expert e's block is live below psum[e]; the block's alignment
    pads and rows labelled -1 are not.  Counts 3, 0, 5 with alignment 4:
    psum = [3, 4 + 0, 4 + 5] = [3, 4, 9], blocks [0, 4), [4, 4), [4, 12)."""
    psum = np.array([3, 4, 9], np.int32)
    mi = np.array([0, 0, 0, 0, 2, 2, 2, 2, 2, 2, 2, 2, -1, -1], np.int32)
    live = layer.live_rows(mi, psum, 4, 14)
    assert live.tolist() == [1, 1, 1, 0, 1, 1, 1, 1, 1, 0, 0, 0, 0, 0]
    # a total cut short of the padded block end (capacity clamp)
    assert layer.live_rows(mi, psum, 4, 6).tolist() == [1, 1, 1, 0, 1, 1]
    # agrees with the layout's own pad rows on a random routing
    rng = np.random.default_rng(7)
    ids = rng.integers(-1, 6, (300, 3)).astype(np.int32)
    lay = layout.expand_layout(ids, 300, 6, 16, layout.capacity(300, 3, 6, 16))
    n = lay["total"]
    live = layer.live_rows(lay["m_indices"], lay["psum"], 16, n)
    src = lay["src2dst"]
    assert live.sum() == (src >= 0).sum() and np.all(live[src[src >= 0]])


def test_act_quant_fold_and_pad_rows():
    rng = np.random.default_rng(5)
    G = fp8.round_bf16(rng.standard_normal((6, 512)))
    live = np.array([1, 1, 0, 1, 0, 1], bool)
    fw = rng.random(6).astype(np.float32)
    q0, s0 = layer.act_quant(G, live, "f32")
    q1, s1 = layer.act_quant(G, live, "f32", fold_weight=fw)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1[live], (s0[live] * fw[live, None]).astype(np.float32))
    assert not q0[~live].any() and not s0[~live].any()
    y = layer.silu_mul(G[:, :256], G[:, 256:])
    qy, sy = quant.quantize_rows(y[live], "f32")
    assert np.array_equal(q0[live], qy)
    with pytest.raises(ValueError):
        layer.act_quant(G, live, "ue8m0", fold_weight=fw)


def test_gather_hand_case():
    D = fp8.round_bf16(np.array([[1.0, 2.0], [10.0, 20.0], [0.5, -0.5], [3.0, 3.0]]))
    src = np.array([[0, 1], [-1, -1], [2, -1], [3, 3]], np.int32)
    w = np.array([[0.5, 0.25], [9, 9], [2.0, 9], [1.0, 0.5]], np.float32)
    plain = layer.gather(D, src, 3)
    assert plain.tolist() == [[11.0, 22.0], [0.0, 0.0], [0.5, -0.5]]
    wtd = layer.gather(D, src, 4, topk_weights=w)
    assert wtd.tolist() == [[3.0, 6.0], [0.0, 0.0], [1.0, -1.0], [4.5, 4.5]]


def _quantised_inputs(wl, fmt=None, data=None):
    d = data or W.generate(wl)
    wl = d["workload"]
    fmt = fmt or wl.fmt
    x_q, x_s = quant.quantize_rows(d["x"], fmt)
    W.poison_tail(d, x_q, x_s)
    w13_q, w13_s = quant.quantize_blocks(d["w13"], fmt)
    w2_q, w2_s = quant.quantize_blocks(d["w2"], fmt)
    return dict(x_q=x_q, x_s=x_s, ids=d["ids"], w=d["w"],
                num_valid=d["num_valid"], w13_q=w13_q, w13_s=w13_s,
                w2_q=w2_q, w2_s=w2_s, align=wl.align, fmt=fmt)


SMALL = [
    ("tiny", {}),
    ("tiny", dict(fmt="ue8m0")),
    ("tiny", dict(align=16, topk=3, seed=77)),
    ("tiny", dict(rows=50, experts=3, global_experts=5, align=32, seed=78)),
    ("tiny", dict(rows=40, valid_rows=23, src_ranks=4, seed=79)),
    ("tiny", dict(rows=40, valid_rows=23, src_ranks=4, tail_alias=True, seed=79)),
]


@pytest.mark.parametrize("name,over", SMALL)
def test_layer_equals_brute_force(name, over):
    inp = _quantised_inputs(W.workload(name, **over))
    L = layer.layer(inp)
    assert np.array_equal(L["out"], layer.brute_force(inp))
    assert np.all(np.isfinite(L["out"]))


def test_fold_equals_post_weighting():
    inp = _quantised_inputs(W.workload("tiny", seed=123))
    fold = layer.layer(inp, mode="fold")["out"]
    Lp = layer.layer(inp, mode="post")
    post = Lp["out"]
    # Exact in real arithmetic.  In fp32/bf16 the fold adds one rounding of
    # s*w and moves the weight before the bf16 rounding of each down row, so
    # each slot's term carries a different bf16 rounding on each side (half
    # an ulp, at most 2^-8 relative, twice) and each side's output one more.
    mag = layer.gather(np.abs(Lp["D"]), Lp["src2dst"], inp["num_valid"],
                       topk_weights=np.abs(inp["w"]))
    bound = 2.0 ** -7 * (1.01 * mag + np.abs(post)) + 2.0 ** -30
    assert np.all(np.abs(fold - post) <= bound)
    rel = np.linalg.norm(fold - post) / np.linalg.norm(post)
    assert rel < 6e-3          # a few bf16 roundings (2^-9 each)


def test_dense_swiglu_reduction():
    # One expert, top-1, weight 1: the layer is silu(x W1^T) * (x W3^T) W2^T.
    wl = W.workload("tiny", experts=1, global_experts=1, topk=1, seed=31)
    d = W.generate(wl)
    d["w"][:] = 1.0
    inp = _quantised_inputs(wl, data=d)
    out = layer.layer(inp)["out"]
    x = quant.dequant_rows(inp["x_q"], inp["x_s"], "f32")
    w13 = quant.dequant_block(inp["w13_q"][0], inp["w13_s"][0], "f32")
    w2 = quant.dequant_block(inp["w2_q"][0], inp["w2_s"][0], "f32")
    I = w2.shape[1]
    gate, up = x @ w13[:I].T, x @ w13[I:].T
    ref = (gate / (1 + np.exp(-gate)) * up) @ w2.T
    # The continuous reference skips the fp8 rounding of silu(gate)*up (3
    # mantissa bits: up to 2^-4 relative per element, about 2.5% rms after
    # the down projection) and the bf16 roundings; a swapped gate/up, a
    # transposed weight or a dropped term is off by order 100%.
    err = np.abs(out - ref)
    rms = np.sqrt(np.mean(ref ** 2))
    assert err.max() <= 0.2 * rms
    assert np.sqrt(np.mean(err ** 2)) <= 0.04 * rms


def test_tail_poison_never_changes_output():
    a = _quantised_inputs(W.workload("tiny", rows=40, valid_rows=23, src_ranks=4, seed=79))
    b = _quantised_inputs(W.workload("tiny", rows=40, valid_rows=23, src_ranks=4,
                                     tail_alias=True, seed=79))
    assert not np.array_equal(a["ids"], b["ids"])
    la, lb = layer.layer(a), layer.layer(b)
    assert np.array_equal(la["out"], lb["out"])
    assert np.array_equal(la["src2dst"], lb["src2dst"])


# ---- planted mistakes: each must be caught by one of the pins above ----

def test_planted_gate_up_swap_is_caught(monkeypatch):
    orig = layer.silu_mul
    monkeypatch.setattr(layer, "silu_mul", lambda g, u: orig(u, g))
    with pytest.raises(AssertionError):
        test_dense_swiglu_reduction()


def test_planted_transposed_weight_is_caught(monkeypatch):
    orig = quant.dequant_block

    def transposed(q, s, fmt, block=128):
        w = orig(q, s, fmt, block)
        return w.T.copy() if w.shape[0] == w.shape[1] else w[::-1]
    monkeypatch.setattr(quant, "dequant_block", transposed)
    with pytest.raises(AssertionError):
        test_gemm_integer_exact_with_expert_selection()


def test_planted_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(quant, "scale_values",
                        lambda s, fmt: np.ones_like(np.asarray(s, dtype=np.float64)))
    with pytest.raises(AssertionError):
        test_gemm_block_scales_closed_form()


def test_planted_psum_without_alignment_is_caught(monkeypatch):
    monkeypatch.setattr(layout, "align_up", lambda x, a: int(x))
    with pytest.raises(AssertionError):
        from tests.test_oracle_layout import test_hand_worked_example
        test_hand_worked_example()
