"""Pins for the oracle's masked-slab decode path (CPU only).

* The bridges' index map in closed form: slab row e * max_m + i holds
  expanded row align(psum[e-1]) + i for i < masked_m[e] = min(count_e, max_m)
  (checked by carrying row numbers through the bridge), and the way back
  restores every live row, zeroes the rows the slab height dropped and
  leaves the alignment pads undefined; a hand case of masked_m and the
  overflow flag.
* The layer on the slab equals a per-token brute force with no layout or
  slab, in which each slot's down row is weighted and rounded to bf16 before
  the sum (bit-exact, fp32 and UE8M0 scales).
* Identities with the contiguous path: the slab's down rows equal the
  contiguous path's rows bit for bit (the same rows meet the same weights);
  with power-of-two top-k weights the weighted rounding is exact and the
  whole output equals the contiguous path with post-weighting.
A planted mistake (an off-by-one slab offset) is caught.
"""

import numpy as np
import pytest

import workloads as W
from oracle import fp8, layer, layout, masked, quant
from tests.test_oracle_layer import _quantised_inputs


def _psum(counts, align):
    psum, prev = [], 0
    for c in counts:
        st = layout.align_up(prev, align)
        psum.append(st + c)
        prev = st + c
    return np.array(psum, np.int32), layout.align_up(prev, align)


def test_masked_counts_hand_case():
    psum, total = _psum([3, 66, 0, 70], 64)
    assert psum.tolist() == [3, 130, 192, 262] and total == 320
    mm, flags = masked.masked_counts(psum, 64, 64)
    assert mm.tolist() == [3, 64, 0, 64] and flags == masked.FLAG_SLAB_OVERFLOW
    mm, flags = masked.masked_counts(psum, 64, 80)
    assert mm.tolist() == [3, 66, 0, 70] and flags == 0


@pytest.mark.parametrize("max_m", [16, 40, 96])
def test_bridge_index_map_and_round_trip(max_m):
    align = 16
    counts = [5, 0, 33, 17, 40, 1]
    psum, total = _psum(counts, align)
    rowid = np.arange(total, dtype=np.int64)[:, None].repeat(2, axis=1)
    slab, _, mm, flags = masked.expand_to_masked_slab(rowid, rowid[:, :1], psum, max_m, align)
    st = masked.expert_starts(psum, align)
    for e, c in enumerate(counts):
        assert mm[e] == min(c, max_m)
        for i in range(mm[e]):
            assert slab[e * max_m + i, 0] == st[e] + i          # closed form
    assert bool(flags) == (max(counts) > max_m)
    rng = np.random.default_rng(3)
    D = fp8.round_bf16(rng.standard_normal((total, 8)))
    Dslab = np.zeros((len(counts) * max_m, 8), np.float32)
    for e in range(len(counts)):
        Dslab[e * max_m: e * max_m + mm[e]] = D[st[e]: st[e] + mm[e]]
    back = masked.masked_slab_to_expand(Dslab, psum, mm, max_m, total, align)
    for e, c in enumerate(counts):
        keep = min(c, max_m)
        assert np.array_equal(back[st[e]: st[e] + keep], D[st[e]: st[e] + keep])
        assert not back[st[e] + keep: st[e] + c].any()                      # dropped
        assert np.all(np.isnan(back[st[e] + c: layout.align_up(st[e] + c, align)]))  # pads


def _masked_inputs(**over):
    return _quantised_inputs(W.workload("tiny", **over))


def _max_m(inp):
    lay = layout.expand_layout(inp["ids"], inp["num_valid"], inp["w13_q"].shape[0],
                               inp["align"], 10 ** 6)
    return int(lay["counts"].max())


@pytest.mark.parametrize("over", [{}, dict(fmt="ue8m0"), dict(align=16, topk=3, seed=77),
                                  dict(rows=40, valid_rows=23, src_ranks=4, seed=79)])
def test_masked_layer_equals_brute_force(over):
    inp = _masked_inputs(**over)
    L = masked.masked_layer(inp, max_m=_max_m(inp) + 3)
    assert L["slab_flags"] == 0
    assert np.array_equal(L["out"], layer.brute_force(inp, mode="masked"))
    assert np.abs(L["out"]).max() > 0


def test_slab_rows_equal_contiguous_rows():
    inp = _masked_inputs(seed=5)
    L = masked.masked_layer(inp, max_m=_max_m(inp))
    C = layer.layer(inp, mode="post")
    st = masked.expert_starts(L["psum"], inp["align"])
    for e, n in enumerate(L["masked_m"]):
        mx = len(L["slab_labels"]) // len(L["masked_m"])
        assert np.array_equal(L["D"][e * mx: e * mx + n], C["D"][st[e]: st[e] + n])
        assert np.array_equal(L["G"][e * mx: e * mx + n], C["G"][st[e]: st[e] + n])


def test_power_of_two_weights_equal_contiguous_post():
    inp = _masked_inputs(seed=6)
    rng = np.random.default_rng(6)
    inp["w"] = (2.0 ** rng.integers(-3, 2, size=inp["w"].shape)).astype(np.float32)
    L = masked.masked_layer(inp, max_m=_max_m(inp))
    C = layer.layer(inp, mode="post")
    assert np.array_equal(L["out"], C["out"])


def test_planted_slab_offset_is_caught(monkeypatch):
    orig = masked.expert_starts
    monkeypatch.setattr(masked, "expert_starts",
                        lambda psum, align: orig(psum, align) + 1)
    with pytest.raises(AssertionError):
        test_bridge_index_map_and_round_trip(40)
