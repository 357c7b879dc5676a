"""Expanded dispatch layout (oracle; test infrastructure only).

What is computed, and where the pages define it:

* Valid slots.  Slot (r, k) of the receive buffer is live when its row lies
  below the real/padding boundary and its expert id is a local expert.
  Inactive rows carry -1 in every top-k slot, and the boundary is a device
  prefix sum over source ranks (vLLM PR 54109, Motivation: inactive rows,
  ``psum_recv_per_rank``; Design: the PaddedStandard contract obliges the
  kernel to honour -1 markers and not trust row contents).
* Expand-mode prefix sum.  ``psum[e] = align(psum[e-1]) + count[e]`` with
  ``psum[-1] = 0``: inclusive, and only the earlier experts are aligned; the
  expanded row total is ``align(psum[E-1])`` and is a multiple of the
  alignment (SGLang PR 37261, review thread: the note correcting the psum
  comment and asking for the total-rows assert).
* Row labels.  Row ``i`` of expert ``e``'s block, ``[align(psum[e-1]),
  align(psum[e]))``, is labelled ``e``; both ends round up to the alignment;
  rows past the total stay -1 so the grouped GEMM skips them (SGLang PR
  37261, Modifications/Core: labelling rows from the device psum with no
  cumsum, host copy or sentinel; SGLang moe_runner/deep_gemm.py source,
  ``pre_permute_deepep_v2_to_deep_gemm``: labels start as -1 everywhere).
* Expansion.  Each live slot becomes one row of its expert's block holding
  the token's fp8 row and its scales (SGLang PR 37261,
  SGLANG_DEEPEP_V2_PREFILL_DO_EXPAND section: per-(token, expert) rows
  grouped by expert).  Alignment gaps are zero-filled (vLLM PR 54109,
  Motivation: prefill gaps are zeroed; SGLang moe_runner/deep_gemm.py
  source, ``pre_permute_deepep_normal_to_deep_gemm``: deterministic
  zero-fill of pad slots).
* Capacity.  With the live row count known only on the device, buffers are
  sized by the largest padded total any routing of ``rows * topk``
  assignments can produce (SGLang moe_runner/deep_gemm.py source,
  ``_get_compact_all_tokens``).

Readings where the pages are silent (each listed in the design notes):
rows of one expert are in ascending (row, k) order; a pad row inside an
expert's block carries that expert's label; pad rows hold fp8 zero, scale 0
(UE8M0 byte 0) and weight 0; ids >= E are skipped and flagged; if the real
total exceeds the capacity, rows at or beyond the capacity are dropped, their
slots get -1 and the overflow flag is set.
"""

import numpy as np

FLAG_CAPACITY_OVERFLOW = 1
FLAG_EXPERT_ID_RANGE = 2


def align_up(x: int, a: int) -> int:
    return (int(x) + a - 1) // a * a


def capacity(rows: int, topk: int, num_experts: int, align: int) -> int:
    """Largest padded row total over every routing of rows*topk assignments
    onto num_experts experts, each block rounded up to `align` rows.

    With n = min(A, E) non-empty experts, each holds one assignment and one
    aligned block; the other A - n assignments add a block per `align`."""
    a = int(rows) * int(topk)
    n = min(a, int(num_experts))
    return int(align) * (n + (a - n) // int(align))


def num_valid_rows(rows: int, psum_recv_per_rank) -> int:
    """Rows below the real/padding boundary: the last entry of the per-rank
    inclusive prefix sum, clamped to [0, rows]; all rows when absent."""
    if psum_recv_per_rank is None or len(psum_recv_per_rank) == 0:
        return int(rows)
    return int(min(max(int(psum_recv_per_rank[-1]), 0), rows))


def expand_layout(topk_ids, num_valid: int, num_experts: int, align: int,
                  cap: int):
    """Integer part of the layout.  Returns a dict with
    counts [E], psum [E], starts [E], total, flags, src2dst [R, T]
    (-1 for skipped slots) and m_indices [cap]."""
    ids = np.asarray(topk_ids)
    rows, topk = ids.shape
    E = int(num_experts)
    flags = 0
    counts = [0] * E
    live = []                      # (r, k, e) in ascending (r, k) order
    for r in range(num_valid):
        for k in range(topk):
            e = int(ids[r, k])
            if e < 0:
                continue
            if e >= E:
                flags |= FLAG_EXPERT_ID_RANGE
                continue
            counts[e] += 1
            live.append((r, k, e))
    psum = [0] * E
    starts = [0] * E
    prev = 0
    for e in range(E):
        starts[e] = align_up(prev, align)
        psum[e] = starts[e] + counts[e]
        prev = psum[e]
    total = align_up(prev, align) if E else 0
    assert total % align == 0
    if total > cap:
        flags |= FLAG_CAPACITY_OVERFLOW

    src2dst = np.full((rows, topk), -1, dtype=np.int32)
    nxt = list(starts)
    for r, k, e in live:
        dst = nxt[e]
        nxt[e] += 1
        if dst < cap:
            src2dst[r, k] = dst

    m_indices = np.full(cap, -1, dtype=np.int32)
    for e in range(E):
        lo, hi = starts[e], min(align_up(psum[e], align), cap)
        if lo < hi:
            m_indices[lo:hi] = e
    return dict(counts=np.array(counts, dtype=np.int32),
                psum=np.array(psum, dtype=np.int32),
                starts=np.array(starts, dtype=np.int32),
                total=int(total), flags=int(flags),
                src2dst=src2dst, m_indices=m_indices)


def scatter_rows(lay, x, x_scale, topk_weights, align: int, cap: int):
    """Data part of the layout: copy each live slot's token row, its scales
    and its top-k weight to the slot's expanded row; zero the alignment pads.

    Only the n = min(total, cap) rows the layout defines are materialised:
    returns (ex [n, H] uint8, ex_scale [n, H/128], row_weight [n] f32,
    written [n] bool).  Every one of them is written (a slot's row or an
    alignment pad); rows from the total up to the capacity are never
    written by the library."""
    x = np.asarray(x)
    xs = np.asarray(x_scale)
    w = np.asarray(topk_weights, dtype=np.float32)
    n = min(int(lay["total"]), int(cap))
    ex = np.zeros((n, x.shape[1]), dtype=x.dtype)
    exs = np.zeros((n, xs.shape[1]), dtype=xs.dtype)
    roww = np.zeros(n, dtype=np.float32)
    written = np.zeros(n, dtype=bool)
    src = lay["src2dst"]
    rows, topk = src.shape
    for r in range(rows):
        for k in range(topk):
            d = int(src[r, k])
            if d >= 0:
                ex[d] = x[r]
                exs[d] = xs[r]
                roww[d] = w[r, k]
                written[d] = True
    for e in range(len(lay["counts"])):
        lo = int(lay["psum"][e])
        hi = min(align_up(lo, align), n)
        if lo < hi:                  # in-block alignment pad rows
            written[lo:hi] = True    # (already zero)
    return ex, exs, roww, written


def expand(topk_ids, topk_weights, x, x_scale, num_valid: int,
           num_experts: int, align: int, cap: int):
    """Whole layout step: integer layout plus the scattered data."""
    lay = expand_layout(topk_ids, num_valid, num_experts, align, cap)
    ex, exs, roww, written = scatter_rows(lay, x, x_scale, topk_weights,
                                          align, cap)
    lay.update(ex=ex, ex_scale=exs, row_weight=roww, written=written)
    return lay
