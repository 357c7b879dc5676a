"""Pins for the oracle's expanded layout (CPU only).

* A hand-worked example (tests/golden/layout_hand.json) derived from the
  expand-mode psum definition.
* The capacity formula equals a brute-force maximum over every routing of
  tiny cases.
* Invariants on seeded random routings: every live (row, k) slot appears
  exactly once; each expert block is ceil(count/align)*align rows; the total
  is a multiple of the alignment; labels are constant on blocks with a -1
  tail; the scattered bytes equal the source rows (permute then unpermute is
  the identity); pad rows are zero; the per-row weight is the slot's weight.
* The real/padding boundary: nothing at or past it is read as routing.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "layout_hand.json")))
    ids = np.array(g["topk_ids"], dtype=np.int32)
    ex = g["expect"]
    nv = layout.num_valid_rows(len(ids), g["psum_recv_per_rank"])
    assert nv == ex["num_valid"]
    cap = layout.capacity(ids.shape[0], ids.shape[1], g["num_experts"], g["align"])
    assert cap == ex["capacity"]
    lay = layout.expand_layout(ids, nv, g["num_experts"], g["align"], cap)
    assert lay["counts"].tolist() == ex["counts"]
    assert lay["psum"].tolist() == ex["psum"]
    assert lay["total"] == ex["total"]
    assert lay["flags"] == ex["flags"]
    assert lay["src2dst"].tolist() == ex["src2dst"]
    assert lay["m_indices"].tolist() == ex["m_indices"]


def _brute_capacity(assignments, experts, align):
    best = 0
    for combo in itertools.combinations_with_replacement(range(experts), assignments):
        c = np.bincount(combo, minlength=experts)
        best = max(best, int(np.sum((c + align - 1) // align * align)))
    return best


@pytest.mark.parametrize("rows,topk,experts,align", [
    (1, 1, 1, 4), (1, 2, 3, 2), (2, 2, 3, 4), (3, 2, 4, 2), (5, 1, 3, 4),
    (4, 2, 2, 4), (3, 3, 5, 2), (2, 4, 6, 3), (7, 1, 4, 8), (6, 2, 3, 4),
])
def test_capacity_is_max_over_routings(rows, topk, experts, align):
    assert layout.capacity(rows, topk, experts, align) == \
        _brute_capacity(rows * topk, experts, align)


def _random_case(seed, rows, topk, experts, align, p_local=0.4, p_bad=0.0,
                 dup=False):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, experts, size=(rows, topk)).astype(np.int32)
    ids[rng.random((rows, topk)) > p_local] = -1
    if p_bad:
        bad = rng.random((rows, topk)) < p_bad
        ids[bad] = rng.integers(experts, experts + 5, size=int(bad.sum()))
    if not dup:
        for r in range(rows):           # make live ids distinct per row
            seen = set()
            for k in range(topk):
                if ids[r, k] >= 0 and ids[r, k] in seen:
                    ids[r, k] = -1
                seen.add(int(ids[r, k]))
    w = rng.random((rows, topk)).astype(np.float32)
    return ids, w


def _check_invariants(ids, w, x, xs, nv, E, align):
    rows, topk = ids.shape
    cap = layout.capacity(rows, topk, E, align)
    lay = layout.expand(ids, w, x, xs, nv, E, align, cap)
    live = [(r, k) for r in range(nv) for k in range(topk) if 0 <= ids[r, k] < E]
    # each live slot exactly once, nothing else
    dsts = [int(lay["src2dst"][r, k]) for r, k in live]
    assert len(set(dsts)) == len(dsts)
    assert int(np.sum(lay["src2dst"] >= 0)) == len(live)
    # block sizes and total
    counts = np.bincount([ids[r, k] for r, k in live], minlength=E)
    assert lay["counts"].tolist() == counts.tolist()
    blocks = (counts + align - 1) // align * align
    assert lay["total"] == int(blocks.sum())
    assert lay["total"] % align == 0
    starts = np.concatenate([[0], np.cumsum(blocks)[:-1]])
    assert lay["starts"].tolist() == starts.tolist()
    # labels: constant on blocks, -1 tail
    for e in range(E):
        assert np.all(lay["m_indices"][starts[e]:starts[e] + blocks[e]] == e)
    assert np.all(lay["m_indices"][lay["total"]:] == -1)
    # slots of expert e fill [start, start+count) in (row, k) order
    for e in range(E):
        mine = [int(lay["src2dst"][r, k]) for r, k in live if ids[r, k] == e]
        assert mine == list(range(starts[e], starts[e] + counts[e]))
    # data: permute then unpermute is the identity; pads are zero
    for r, k in live:
        d = lay["src2dst"][r, k]
        assert np.array_equal(lay["ex"][d], x[r])
        assert np.array_equal(lay["ex_scale"][d], xs[r])
        assert lay["row_weight"][d] == w[r, k]
    for e in range(E):
        pad = slice(starts[e] + counts[e], starts[e] + blocks[e])
        assert not lay["ex"][pad].any() and not lay["ex_scale"][pad].any()
        assert not lay["row_weight"][pad].any()
    return lay


@pytest.mark.parametrize("seed,rows,topk,E,align,nv", [
    (0, 37, 3, 5, 4, 37), (1, 64, 2, 4, 64, 64), (2, 100, 8, 8, 16, 71),
    (3, 9, 4, 3, 2, 0), (4, 50, 1, 1, 8, 50), (5, 200, 6, 16, 32, 150),
    (6, 300, 8, 1024, 16, 300),   # the most local experts, most of them empty
])
def test_layout_invariants(seed, rows, topk, E, align, nv):
    ids, w = _random_case(seed, rows, topk, E, align)
    rng = np.random.default_rng(seed + 100)
    x = rng.integers(0, 256, size=(rows, 256), dtype=np.uint8)
    xs = rng.random((rows, 2)).astype(np.float32) + 0.5
    _check_invariants(ids, w, x, xs, nv, E, align)


def test_duplicate_ids_each_get_a_row():
    ids, w = _random_case(9, 40, 4, 3, 4, p_local=0.9, dup=True)
    assert any(len(set(r[r >= 0])) < len(r[r >= 0]) for r in ids)
    rng = np.random.default_rng(1)
    x = rng.integers(0, 256, size=(40, 128), dtype=np.uint8)
    xs = np.ones((40, 1), np.float32)
    _check_invariants(ids, w, x, xs, 40, 3, 4)


def test_out_of_range_ids_are_skipped_and_flagged():
    ids, w = _random_case(12, 30, 4, 4, 8, p_bad=0.1)
    lay = layout.expand_layout(ids, 30, 4, 8, layout.capacity(30, 4, 4, 8))
    assert lay["flags"] & layout.FLAG_EXPERT_ID_RANGE
    assert np.all(lay["src2dst"][ids >= 4] == -1)
    ids2 = np.where(ids >= 4, -1, ids)
    lay2 = layout.expand_layout(ids2, 30, 4, 8, layout.capacity(30, 4, 4, 8))
    assert lay2["flags"] == 0
    assert np.array_equal(lay["src2dst"], lay2["src2dst"])


def test_boundary_tail_is_never_routing():
    # Rows at or past the boundary may hold ids that alias local experts;
    # the layout must not depend on them.
    ids, w = _random_case(21, 80, 4, 4, 16)
    nv = 50
    tail_a = ids.copy()
    tail_a[nv:] = -1
    tail_b = ids.copy()
    tail_b[nv:] = np.random.default_rng(5).integers(0, 4, size=(30, 4))
    cap = layout.capacity(80, 4, 4, 16)
    la = layout.expand_layout(tail_a, nv, 4, 16, cap)
    lb = layout.expand_layout(tail_b, nv, 4, 16, cap)
    for key in ("counts", "psum", "src2dst", "m_indices"):
        assert np.array_equal(la[key], lb[key])
    assert la["total"] == lb["total"]


def test_boundary_from_rank_prefix_sum():
    assert layout.num_valid_rows(100, None) == 100
    assert layout.num_valid_rows(100, [3, 10, 42]) == 42
    assert layout.num_valid_rows(100, [3, 10, 420]) == 100
    assert layout.num_valid_rows(100, []) == 100


def test_empty_experts_and_empty_input():
    ids = np.full((10, 2), -1, np.int32)
    ids[3, 0] = 2
    lay = layout.expand_layout(ids, 10, 4, 8, layout.capacity(10, 2, 4, 8))
    assert lay["psum"].tolist() == [0, 0, 1, 8]
    assert lay["starts"].tolist() == [0, 0, 0, 8]
    assert lay["total"] == 8
    none = layout.expand_layout(np.full((5, 3), -1, np.int32), 5, 4, 8, 40)
    assert none["total"] == 0 and np.all(none["m_indices"] == -1)


def test_capacity_overflow_drops_and_flags():
    ids = np.zeros((10, 1), np.int32)               # 10 rows to expert 0
    lay = layout.expand_layout(ids, 10, 2, 4, 8)     # capacity 8 < total 12
    assert lay["flags"] & layout.FLAG_CAPACITY_OVERFLOW
    assert lay["total"] == 12
    assert lay["src2dst"][:8, 0].tolist() == list(range(8))
    assert np.all(lay["src2dst"][8:, 0] == -1)
    assert np.all(lay["m_indices"] == 0)
