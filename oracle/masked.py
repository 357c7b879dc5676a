"""Masked-slab layout of the decode path (oracle; test infrastructure only).

Where the pages define it:

* The masked grouped GEMM takes a fixed-height slab ``[num_local_experts,
  max_m, H]`` with a per-expert row count ``masked_m``, so that the decode
  step keeps static shapes (graph capture); the expanded layout reaches it
  through two bridges, ``expand_to_masked_slab`` before the GEMMs and
  ``masked_slab_to_expand`` after (SGLang PR 37261, "Why decode stays on V1
  low_latency": the slab, the table of bridge kernels, their two extra HBM
  round trips).
* ``expand_to_masked_slab(hidden, scale, psum, E, max_m, alignment)`` returns
  the slab, its scales and ``masked_m``, which bounds each expert
  independently of the buffer capacity; ``masked_slab_to_expand(hidden,
  psum, total_expanded, alignment, topk_weights)`` brings the rows back into
  the expanded layout with the top-k weights applied, since the expanded
  combine takes none (SGLang moe_runner/deep_gemm.py source,
  ``pre_permute_deepep_v2_to_deep_gemm`` and
  ``post_permute_deep_gemm_to_deepep_v2``, masked branches).
* Between the bridges the expert computation is the contiguous one, on the
  slab's live rows (``_run_masked_gemm`` with ``masked_m``; SiLU*up and the
  per-group quantisation as in ``_run_contiguous_gemm``).

Readings (the bridge kernels' bodies are not on the pages):

* ``masked_m[e] = min(count_e, max_m)``, count_e = psum[e] - align(psum[e-1])
  (the expert's live rows); rows past ``max_m`` are dropped and flagged.
* Slab row ``e * max_m + i`` holds expanded row ``align(psum[e-1]) + i`` for
  i < masked_m[e]; the rest of the slab is never read and never written.
  Slab scales are K-block-major over all ``E * max_m`` rows, as the expanded
  ones are over the capacity.
* Back in the expanded layout, row ``align(psum[e-1]) + i`` for i <
  masked_m[e] is ``bf16(w * slab[e * max_m + i])`` with w the row's top-k
  weight (an fp32 product, one bf16 rounding), a plain copy without weights;
  rows dropped by the slab height are zero (their slots still point at
  them); alignment pad rows are not defined (no slot points at them, so the
  combine never reads them).  The combine then sums each token's rows with
  weight 1.
"""

import numpy as np

from . import fp8, layer, layout

FLAG_SLAB_OVERFLOW = 4


def expert_starts(psum, align: int):
    """First expanded row of each expert's block: align(psum[e-1])."""
    psum = np.asarray(psum, dtype=np.int64)
    return np.array([layout.align_up(psum[e - 1], align) if e else 0
                     for e in range(len(psum))], dtype=np.int64)


def masked_counts(psum, align: int, max_m: int):
    """(masked_m [E] int32, flags): live rows per expert, capped at max_m."""
    psum = np.asarray(psum, dtype=np.int64)
    counts = psum - expert_starts(psum, align)
    mm = np.minimum(counts, max_m).astype(np.int32)
    flags = FLAG_SLAB_OVERFLOW if np.any(counts > max_m) else 0
    return mm, flags


def slab_labels(masked_m, max_m: int):
    """Expert of each slab row for i < masked_m[e], -1 elsewhere."""
    E = len(masked_m)
    lab = np.full(E * max_m, -1, dtype=np.int32)
    for e in range(E):
        lab[e * max_m: e * max_m + int(masked_m[e])] = e
    return lab


def expand_to_masked_slab(ex, ex_scale, psum, max_m: int, align: int):
    """Expanded rows [n, H] and scales [n, H/128] -> slab [E*max_m, H],
    slab scales [E*max_m, H/128] (undefined rows zero), masked_m, flags."""
    ex = np.asarray(ex)
    xs = np.asarray(ex_scale)
    E = len(psum)
    mm, flags = masked_counts(psum, align, max_m)
    st = expert_starts(psum, align)
    slab = np.zeros((E * max_m, ex.shape[1]), dtype=ex.dtype)
    sscale = np.zeros((E * max_m, xs.shape[1]), dtype=xs.dtype)
    for e in range(E):
        n = int(mm[e])
        slab[e * max_m: e * max_m + n] = ex[st[e]: st[e] + n]
        sscale[e * max_m: e * max_m + n] = xs[st[e]: st[e] + n]
    return slab, sscale, mm, flags


def masked_slab_to_expand(slab_out, psum, masked_m, max_m: int, total: int, align: int,
                          row_weight=None):
    """Slab rows [E*max_m, H] (bf16 values as float32) -> expanded rows
    [total, H]: row start_e + i = bf16(row_weight[start_e + i] * slab[e*max_m
    + i]) for i < masked_m[e] (a copy without weights), zero for the rows the
    slab height dropped (masked_m[e] <= i < count_e), NaN (not defined) on
    the alignment pad rows."""
    so = np.asarray(slab_out, dtype=np.float32)
    out = np.full((int(total), so.shape[1]), np.nan, dtype=np.float32)
    st = expert_starts(psum, align)
    psum = np.asarray(psum, dtype=np.int64)
    for e in range(len(psum)):
        n = int(masked_m[e])
        out[st[e] + n: psum[e]] = 0.0
        rows = so[e * max_m: e * max_m + n]
        if row_weight is not None:
            w = np.asarray(row_weight, dtype=np.float32)[st[e]: st[e] + n]
            rows = fp8.round_bf16((rows * w[:, None]).astype(np.float32))
        out[st[e]: st[e] + n] = rows
    return out


def masked_layer(inp, max_m: int):
    """The decode path on one rank: expanded layout, bridge into the slab,
    gate_up GEMM, SiLU*up + per-group quantisation (no fold), down GEMM on
    the slab's live rows, bridge back with the top-k weights, combine with
    weight 1.  `inp` as for layer.layer.  Returns a dict of every stage."""
    fmt = inp["fmt"]
    ids = np.asarray(inp["ids"])
    R, T = ids.shape
    E = np.asarray(inp["w13_q"]).shape[0]
    align = int(inp["align"])
    cap = int(inp.get("cap") or layout.capacity(R, T, E, align))
    nv = int(inp["num_valid"])
    lay = layout.expand(ids, inp["w"], inp["x_q"], inp["x_s"], nv, E, align, cap)
    n = min(lay["total"], cap)
    slab, sscale, mm, sflags = expand_to_masked_slab(lay["ex"], lay["ex_scale"], lay["psum"],
                                                     max_m, align)
    lab = slab_labels(mm, max_m)
    live = lab >= 0
    G = layer.grouped_gemm(slab, sscale, inp["w13_q"], inp["w13_s"], lab, E * max_m, fmt,
                           live=live)
    dq, ds = layer.act_quant(G, live, fmt)
    D = layer.grouped_gemm(dq, ds, inp["w2_q"], inp["w2_s"], lab, E * max_m, fmt, live=live)
    back = masked_slab_to_expand(D, lay["psum"], mm, max_m, n, align,
                                 row_weight=lay["row_weight"])
    out = layer.gather(back, lay["src2dst"], nv)
    lay.update(slab=slab, slab_scale=sscale, masked_m=mm, slab_flags=sflags,
               slab_labels=lab, G=G, dq=dq, ds=ds, D=D, back=back, out=out, cap=cap)
    return lay
