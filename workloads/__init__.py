"""Seeded synthetic inputs for one expert-parallel rank's MoE layer.

Shared by the tests and the benchmark, imported by neither the oracle nor
the HIP library.  It holds no step of the method: it draws routing, top-k
weights and fp32 activations/weights, and the poison bytes of a padded
receive buffer.  Quantising the fp32 draws to fp8 is done by the consumer
(the oracle's quantiser in the tests, plain torch ops in the benchmark).

Workloads (names are what they are; sizes follow the pages' prefill shapes):

=================  =====================================================
tiny               64 rows, H=256, I=128, 4 local of 8 global experts,
                   top-2 uniform, alignment 64, fp32 scales
dsv3               DeepSeek-V3-shape prefill share: 4096 rows, H=7168,
                   I=2048, 8 local of 256 global experts, top-8 uniform,
                   alignment 128, fp32 scales
dsv3_zipf_ue8m0    as dsv3 with Zipf(1.2) routing that overloads three
                   local experts and empties three, UE8M0 scales
large              16384 rows, 16 local of 256 experts, rest as dsv3
padded             8192-row receive buffer, 1536 valid rows (boundary
                   from a per-source-rank prefix sum over 32 ranks),
                   random-byte tail with ids -1; rest as dsv3
padded_alias       as padded but the tail's ids alias valid local ids
dsv3_local         as dsv3 but every row has at least one local slot
std_tiny           standard (non-EP) path: bf16 input rows, 64 rows,
                   H=256, I=128, all 8 experts local, top-2, alignment
                   64, routed scaling factor 2.5
std_dsv3           standard single-GPU MoE of the DeepSeek-V3 shape: bf16
                   input, 4096 rows, H=7168, I=2048, all 256 experts on
                   the GPU (11 GB of fp8 weights), top-8 uniform,
                   alignment 128, fp32 scales, routed scaling factor 2.5
                   (the model's own)
std_bf16_tiny      standard path with bf16 weights (no quantisation
                   anywhere): std_tiny's shape
std_dsv3_bf16      standard single-GPU MoE, DeepSeek-V3 shape, bf16
                   weights (256 experts, 22.5 GB), factor 2.5
dsv3_mxfp8         as dsv3 with MXFP8 operands (1x32 UE8M0 groups for the
                   activations and every weight row)
dsv3_decode        decode share on the masked slab: 1024 received rows
                   (32 tokens from each of 32 source ranks), H=7168,
                   I=2048, 8 local of 256 experts, top-8 uniform,
                   alignment 128, fp32 scales, slab height max_m=128
                   (about four times the ~32 rows an expert expects)
prefill_h6144      the pages' prefill trace shape: 16384 received rows,
                   every one with a local slot, H=6144, I=2048, 8 local of
                   256 experts, top-8, alignment 128, fp32 scales -> 18432
                   expanded rows (their [~18432, 6144] activations and
                   [~18432, 16] down-input scales)
=================  =====================================================

Recipe (numpy PCG64, seed 1000 + index): routing by Gumbel top-T over the
global experts (sampling without replacement from the expert popularity);
the rank owns global ids [0, E), other ids become -1; top-k weights are the
softmax of T standard-normal logits, not renormalised after non-local slots
drop; x ~ N(0, 1) [R, H]; w13 ~ N(0, 0.02) [E, 2I, H]; w2 ~ N(0, 0.02)
[E, H, I], all float32.
"""

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    hidden: int
    inter: int
    experts: int            # local experts on this rank
    global_experts: int
    topk: int
    align: int
    fmt: str = "f32"        # 'f32' or 'ue8m0' scales
    routing: str = "uniform"   # 'uniform' | 'zipf' | 'local'
    valid_rows: Optional[int] = None   # None: every row is valid
    src_ranks: int = 0      # >0: boundary given as a per-rank prefix sum
    tail_alias: bool = False
    seed: int = 1000
    input: str = "fp8"      # 'fp8' (received, quantised) or 'bf16' (standard path)
    routed_scale: float = 1.0   # routed scaling factor applied in the gather
    max_m: int = 0          # >0: decode path on a masked slab of this height
    weights: str = "fp8"    # 'fp8' (block-scaled) or 'bf16' (bf16 GEMMs, no quantisation)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 128, 4, 8, 2, 64, seed=1000),
    "dsv3": Workload("dsv3", 4096, 7168, 2048, 8, 256, 8, 128, seed=1001),
    "dsv3_zipf_ue8m0": Workload("dsv3_zipf_ue8m0", 4096, 7168, 2048, 8, 256,
                                8, 128, fmt="ue8m0", routing="zipf",
                                seed=1002),
    "large": Workload("large", 16384, 7168, 2048, 16, 256, 8, 128, seed=1003),
    "padded": Workload("padded", 8192, 7168, 2048, 8, 256, 8, 128,
                       valid_rows=1536, src_ranks=32, seed=1004),
    "padded_alias": Workload("padded_alias", 8192, 7168, 2048, 8, 256, 8,
                             128, valid_rows=1536, src_ranks=32,
                             tail_alias=True, seed=1004),
    "dsv3_local": Workload("dsv3_local", 4096, 7168, 2048, 8, 256, 8, 128,
                           routing="local", seed=1005),
    "std_tiny": Workload("std_tiny", 64, 256, 128, 8, 8, 2, 64, seed=1006,
                         input="bf16", routed_scale=2.5),
    "std_dsv3": Workload("std_dsv3", 4096, 7168, 2048, 256, 256, 8, 128,
                         seed=1007, input="bf16", routed_scale=2.5),
    "std_bf16_tiny": Workload("std_bf16_tiny", 64, 256, 128, 8, 8, 2, 64, seed=1009,
                              input="bf16", routed_scale=2.5, weights="bf16"),
    "std_dsv3_bf16": Workload("std_dsv3_bf16", 4096, 7168, 2048, 256, 256, 8, 128,
                              seed=1010, input="bf16", routed_scale=2.5, weights="bf16"),
    "dsv3_mxfp8": Workload("dsv3_mxfp8", 4096, 7168, 2048, 8, 256, 8, 128, fmt="mxfp8",
                           seed=1011),
    "dsv3_decode": Workload("dsv3_decode", 1024, 7168, 2048, 8, 256, 8, 128,
                            seed=1008, max_m=128),
    "prefill_h6144": Workload("prefill_h6144", 16384, 6144, 2048, 8, 256, 8, 128,
                              routing="local", seed=1012),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _popularity(wl: Workload, rng) -> np.ndarray:
    """Selection weights over the global experts."""
    G = wl.global_experts
    if wl.routing in ("uniform", "local"):
        return np.full(G, 1.0 / G)
    if wl.routing == "zipf":
        # Zipf(1.2) over the experts that receive traffic; local experts
        # 0, 1, 2 take popularity ranks 1, 2, 3, locals 3 and 4 ranks 64 and
        # 128, the remaining locals get nothing; the other global experts
        # take the remaining ranks in a seeded random order.
        s = 1.2
        E = wl.experts
        fixed = {0: 1, 1: 2, 2: 3, 3: 64, 4: 128}
        empty = [e for e in range(E) if e not in fixed]
        n_live = G - len(empty)
        used = set(fixed.values())
        free_ranks = [r for r in range(1, n_live + 1) if r not in used]
        others = list(range(E, G))
        perm = rng.permutation(len(others))
        rank = np.zeros(G, dtype=np.int64)
        for e, r in fixed.items():
            rank[e] = r
        for i, g in enumerate(others):
            rank[g] = free_ranks[perm[i]]
        p = np.where(rank > 0, rank.astype(np.float64) ** -s, 0.0)
        return p / p.sum()
    raise ValueError(wl.routing)


def routing(wl: Workload, rng, n_rows: int):
    """Global top-T ids (Gumbel top-T, without replacement) and softmax
    weights for n_rows tokens; returns (local ids [n,T] i32, weights f32)."""
    G, T, E = wl.global_experts, wl.topk, wl.experts
    p = _popularity(wl, rng)
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    gid = np.empty((n_rows, T), dtype=np.int64)
    todo = np.arange(n_rows)
    while len(todo):
        g = rng.gumbel(size=(len(todo), G)) + logp[None, :]
        top = np.argsort(-g, axis=1, kind="stable")[:, :T]
        gid[todo] = top
        if wl.routing == "local":       # resample rows with no local slot
            todo = todo[~np.any(top < E, axis=1)]
        else:
            todo = todo[:0]
    logits = rng.standard_normal((n_rows, T))
    ez = np.exp(logits - logits.max(axis=1, keepdims=True))
    wts = (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = np.where(gid < E, gid, -1).astype(np.int32)
    return ids, wts


def generate(wl, with_weights: bool = True, with_x: bool = True):
    """Draw one workload.  Returns a dict with
    ids [R,T] i32, w [R,T] f32, num_valid, psum_recv_per_rank (or None),
    x [R,H] f32, w13 [E,2I,H] f32, w2 [E,H,I] f32 and, for padded buffers,
    the tail's poison: tail_x_bytes [R-Rv,H] u8, tail_scale_bits
    [R-Rv,H/128] u32, tail_w_bits [R-Rv,T] u32."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    R, H, I, E, T = wl.rows, wl.hidden, wl.inter, wl.experts, wl.topk
    nv = R if wl.valid_rows is None else wl.valid_rows
    ids = np.full((R, T), -1, dtype=np.int32)
    wts = np.zeros((R, T), dtype=np.float32)
    ids[:nv], wts[:nv] = routing(wl, rng, nv)
    out = dict(workload=wl, ids=ids, w=wts, num_valid=nv,
               psum_recv_per_rank=None)
    if wl.src_ranks:
        split = rng.multinomial(nv, np.full(wl.src_ranks, 1.0 / wl.src_ranks))
        out["psum_recv_per_rank"] = np.cumsum(split).astype(np.int32)
    if with_x:
        out["x"] = rng.standard_normal((R, H), dtype=np.float32)
    if with_weights:
        out["w13"] = (rng.standard_normal((E, 2 * I, H), dtype=np.float32)
                      * np.float32(0.02))
        out["w2"] = (rng.standard_normal((E, H, I), dtype=np.float32)
                     * np.float32(0.02))
    if nv < R:
        tail = R - nv
        tb = rng.integers(0, 256, size=(tail, H), dtype=np.uint8)
        sb = rng.integers(0, 2 ** 32, size=(tail, H // 128), dtype=np.uint32)
        wb = rng.integers(0, 2 ** 32, size=(tail, T), dtype=np.uint32)
        # Make sure the poison holds the nasty values: NaN and Inf scales and
        # weights, NaN fp8 codes.
        sb.flat[0:4] = [0x7FC00000, 0x7F800000, 0xFF800000, 0xFFFFFFFF]
        wb.flat[0:3] = [0x7FC00000, 0x7F800000, 0xFF800000]
        tb.flat[0:2] = [0x7F, 0xFF]
        out.update(tail_x_bytes=tb, tail_scale_bits=sb, tail_w_bits=wb)
        if wl.tail_alias:
            out["tail_ids"] = rng.integers(0, E, size=(tail, T),
                                           dtype=np.int32)
        else:
            out["tail_ids"] = np.full((tail, T), -1, dtype=np.int32)
        ids[nv:] = out["tail_ids"]
        wts[nv:] = wb.view(np.float32)
    return out


def poison_tail(data, x_q, x_s):
    """Overwrite rows past the boundary of quantised activations with the
    drawn poison bytes (in place).  x_s may hold fp32 scales, UE8M0 bytes
    (one per 1x128 group) or MXFP8 bytes (one per 1x32 group: the four bytes
    of each drawn 32-bit word)."""
    nv = data["num_valid"]
    if "tail_x_bytes" not in data:
        return
    x_q[nv:] = data["tail_x_bytes"]
    bits = data["tail_scale_bits"]
    if x_s.dtype == np.float32:
        x_s[nv:] = bits.view(np.float32)
    elif x_s.shape[1] == 4 * bits.shape[1]:
        x_s[nv:] = np.ascontiguousarray(bits).view(np.uint8).reshape(len(bits), -1)
    else:
        x_s[nv:] = (bits & 0xFF).astype(np.uint8)
