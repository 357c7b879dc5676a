"""C-ABI library checks that need no GPU.

The library loads, exports every function include/moe_expand.h declares,
its host helpers agree with the oracle's capacity bound, and every entry
point rejects bad arguments with the documented status before launching
anything (the pointers passed here are never dereferenced: each case fails
a host-side check).
"""

import ctypes

import pytest

import expanded_dispatch_layout_amd as M
from oracle import layout as olayout

FAKE = 0x100000          # 16-byte aligned, never dereferenced
MIS = FAKE + 4           # misaligned


def test_library_exports_every_header_function():
    names = M.header_functions()
    assert set(names) >= {"moe_expand_layout", "moe_expand_layout_bf16",
                          "moe_grouped_gemm_fp8", "moe_act_quant",
                          "moe_expand_to_masked_slab", "moe_grouped_gemm_fp8_masked",
                          "moe_act_quant_masked", "moe_masked_slab_to_expand",
                          "moe_grouped_gemm_bf16", "moe_silu_mul_bf16",
                          "moe_gather", "moe_expand_capacity",
                          "moe_expand_workspace_bytes", "moe_status_string"}
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in M._SIGNATURES, n


@pytest.mark.parametrize("rows,topk,E,align", [
    (64, 2, 4, 64), (4096, 8, 8, 128), (16384, 8, 16, 128), (8192, 8, 8, 128),
    (0, 8, 8, 128), (1, 1, 1, 16), (3, 2, 100, 16), (1000, 4, 7, 32)])
def test_capacity_matches_oracle(rows, topk, E, align):
    assert M.moe_expand_capacity(rows, topk, E, align) == olayout.capacity(rows, topk, E, align)


def test_capacity_bad_input():
    assert M.moe_expand_capacity(-1, 2, 4, 16) == -1
    assert M.moe_expand_capacity(4, 0, 4, 16) == -1


def test_workspace_bytes():
    assert M.moe_expand_workspace_bytes(4096, 8, 8) > 0
    assert M.moe_expand_workspace_bytes(16384, 8, 16) >= M.moe_expand_workspace_bytes(4096, 8, 8)
    assert M.moe_expand_workspace_bytes(10, 8, 0) == 0
    assert M.moe_expand_workspace_bytes(10, 99, 8) == 0


def test_status_strings():
    for c in range(8):
        assert M.status_string(c)
    assert M.status_string(99) == "unknown status"


def _layout(**kw):
    a = dict(x=FAKE, x_stride=256, x_scale=FAKE, x_scale_stride=2, fmt=0, ids=FAKE,
             w=FAKE, prank=None, nsrc=0, rows=64, hidden=256, topk=2, E=4, align=64,
             cap=320, ex=FAKE, exs=FAKE, psum=FAKE, mi=FAKE, s2d=FAKE, rw=FAKE, st=FAKE,
             ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return M.lib().moe_expand_layout(
        a["x"], a["x_stride"], a["x_scale"], a["x_scale_stride"], a["fmt"], a["ids"],
        a["w"], a["prank"], a["nsrc"], a["rows"], a["hidden"], a["topk"], a["E"],
        a["align"], a["cap"], a["ex"], a["exs"], a["psum"], a["mi"], a["s2d"], a["rw"],
        a["st"], a["ws"], a["wsb"], a["stream"])


def test_layout_rejects_bad_arguments():
    assert _layout(hidden=100) == M.MOE_ERR_SHAPE
    assert _layout(topk=0) == M.MOE_ERR_SHAPE
    assert _layout(topk=33) == M.MOE_ERR_SHAPE
    assert _layout(E=0) == M.MOE_ERR_SHAPE
    assert _layout(E=2000) == M.MOE_ERR_SHAPE
    assert _layout(align=48) == M.MOE_ERR_UNSUPPORTED
    assert _layout(align=8) == M.MOE_ERR_UNSUPPORTED
    assert _layout(cap=100) == M.MOE_ERR_SHAPE
    assert _layout(fmt=7) == M.MOE_ERR_UNSUPPORTED
    assert _layout(fmt=3, x_scale_stride=6) == M.MOE_ERR_SHAPE    # MXFP8: >= H/32 bytes
    assert _layout(fmt=3, x_scale_stride=10) == M.MOE_ERR_SHAPE   # ... and a multiple of 4
    assert _layout(x_stride=128) == M.MOE_ERR_SHAPE
    assert _layout(prank=FAKE, nsrc=0) == M.MOE_ERR_SHAPE
    assert _layout(psum=None) == M.MOE_ERR_NULL
    assert _layout(x=None) == M.MOE_ERR_NULL
    assert _layout(w=None) == M.MOE_ERR_NULL          # row_weight needs weights
    assert _layout(x=MIS) == M.MOE_ERR_ALIGNMENT
    assert _layout(x_stride=264) == M.MOE_ERR_ALIGNMENT
    assert _layout(ws=None) == M.MOE_ERR_WORKSPACE
    assert _layout(wsb=16) == M.MOE_ERR_WORKSPACE     # everything else valid


def _layout_noalloc(**kw):
    a = dict(x=FAKE, x_stride=256, x_scale=FAKE, x_scale_stride=2, fmt=0, ids=FAKE,
             w=FAKE, prank=None, nsrc=0, rows=64, hidden=256, topk=2, E=4, align=64,
             cap=320, ex=FAKE, exs=FAKE, psum=FAKE, mi=FAKE, s2d=FAKE, rw=FAKE, st=FAKE,
             stream=None)
    a.update(kw)
    return M.lib().moe_expand_layout_noalloc(
        a["x"], a["x_stride"], a["x_scale"], a["x_scale_stride"], a["fmt"], a["ids"],
        a["w"], a["prank"], a["nsrc"], a["rows"], a["hidden"], a["topk"], a["E"],
        a["align"], a["cap"], a["ex"], a["exs"], a["psum"], a["mi"], a["s2d"], a["rw"],
        a["st"], a["stream"])


def test_layout_noalloc_rejects_bad_arguments():
    """Same host checks as moe_expand_layout, all made before the scratch
    address is looked up (no GPU is touched by any of these calls)."""
    assert _layout_noalloc(hidden=100) == M.MOE_ERR_SHAPE
    assert _layout_noalloc(E=2000) == M.MOE_ERR_SHAPE
    assert _layout_noalloc(align=48) == M.MOE_ERR_UNSUPPORTED
    assert _layout_noalloc(cap=100) == M.MOE_ERR_SHAPE
    assert _layout_noalloc(psum=None) == M.MOE_ERR_NULL
    assert _layout_noalloc(x=MIS) == M.MOE_ERR_ALIGNMENT
    # valid, but the workspace would exceed the static scratch
    rows, E = 1 << 20, 256
    assert M.moe_expand_workspace_bytes(rows, 2, E) > M.MOE_NOALLOC_SCRATCH_BYTES
    cap = M.moe_expand_capacity(rows, 2, E, 64)
    assert _layout_noalloc(rows=rows, E=E, cap=cap) == M.MOE_ERR_SCRATCH
    # the largest workload sizes fit
    assert M.moe_expand_workspace_bytes(16384, 8, 16) <= M.MOE_NOALLOC_SCRATCH_BYTES
    assert M.moe_expand_workspace_bytes(8192, 8, 1024) <= M.MOE_NOALLOC_SCRATCH_BYTES


def test_gemm_rejects_bad_arguments():
    f = M.lib().moe_grouped_gemm_fp8

    def call(**kw):
        a = dict(a=FAKE, as_=FAKE, fmt=0, w=FAKE, ws=FAKE, psum=FAKE, st=FAKE,
                 cap=256, n=256, k=256, E=4, align=64, out=FAKE)
        a.update(kw)
        return f(a["a"], a["as_"], a["fmt"], a["w"], a["ws"], a["psum"], a["st"],
                 a["cap"], a["n"], a["k"], a["E"], a["align"], a["out"], None)
    assert call(n=100) == M.MOE_ERR_SHAPE
    assert call(k=192) == M.MOE_ERR_SHAPE
    assert call(cap=100) == M.MOE_ERR_SHAPE
    assert call(align=24) == M.MOE_ERR_UNSUPPORTED
    assert call(fmt=9) == M.MOE_ERR_UNSUPPORTED
    assert call(fmt=3, E=300) == M.MOE_ERR_UNSUPPORTED   # MXFP8: at most 256 experts
    assert call(psum=None) == M.MOE_ERR_NULL
    assert call(as_=FAKE + 2) == M.MOE_ERR_ALIGNMENT
    assert call(as_=FAKE + 4) == M.MOE_ERR_ALIGNMENT        # fp32 scales: 16 bytes
    assert call(as_=FAKE + 4, fmt=1, cap=0) == M.MOE_OK     # UE8M0 scales: 4 bytes
    assert call(k=512 * 128) == M.MOE_ERR_UNSUPPORTED       # item scales fit LDS
    assert call(a=MIS) == M.MOE_ERR_ALIGNMENT
    assert call(cap=0) == M.MOE_OK                  # nothing to do, nothing launched


def test_act_quant_rejects_bad_arguments():
    f = M.lib().moe_act_quant

    def call(**kw):
        a = dict(gu=FAKE, mi=FAKE, psum=FAKE, st=FAKE, cap=256, inter=128, E=4, align=64,
                 fmt=0, fw=None, out=FAKE, os=FAKE)
        a.update(kw)
        return f(a["gu"], a["mi"], a["psum"], a["st"], a["cap"], a["inter"], a["E"],
                 a["align"], a["fmt"], a["fw"], a["out"], a["os"], None)
    assert call(inter=100) == M.MOE_ERR_SHAPE
    # the weight fold needs fp32 scales (a power-of-two scale cannot absorb it)
    assert call(fmt=1, fw=FAKE) == M.MOE_ERR_UNSUPPORTED
    assert call(out=None) == M.MOE_ERR_NULL
    assert call(gu=MIS) == M.MOE_ERR_ALIGNMENT
    assert call(cap=0) == M.MOE_OK


def _layout_bf16(**kw):
    a = dict(x=FAKE, x_stride=256, fmt=0, ids=FAKE, w=FAKE, prank=None, nsrc=0, rows=64,
             hidden=256, topk=2, E=4, align=64, cap=320, ex=FAKE, exs=FAKE, psum=FAKE,
             mi=FAKE, s2d=FAKE, rw=None, st=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return M.lib().moe_expand_layout_bf16(
        a["x"], a["x_stride"], a["fmt"], a["ids"], a["w"], a["prank"], a["nsrc"], a["rows"],
        a["hidden"], a["topk"], a["E"], a["align"], a["cap"], a["ex"], a["exs"], a["psum"],
        a["mi"], a["s2d"], a["rw"], a["st"], a["ws"], a["wsb"], a["stream"])


def test_layout_bf16_rejects_bad_arguments():
    assert _layout_bf16(hidden=100) == M.MOE_ERR_SHAPE
    assert _layout_bf16(x_stride=128) == M.MOE_ERR_SHAPE      # < hidden elements
    assert _layout_bf16(x_stride=-1) == M.MOE_ERR_SHAPE
    assert _layout_bf16(x_stride=260) == M.MOE_ERR_ALIGNMENT  # 520 bytes: not 16-aligned
    assert _layout_bf16(x=MIS) == M.MOE_ERR_ALIGNMENT
    assert _layout_bf16(x=None) == M.MOE_ERR_NULL
    assert _layout_bf16(fmt=3) == M.MOE_ERR_UNSUPPORTED
    assert _layout_bf16(align=48) == M.MOE_ERR_UNSUPPORTED
    assert _layout_bf16(rw=FAKE, w=None) == M.MOE_ERR_NULL
    assert _layout_bf16(ws=None) == M.MOE_ERR_WORKSPACE
    assert _layout_bf16(wsb=16) == M.MOE_ERR_WORKSPACE       # everything else valid


def test_masked_entry_points_reject_bad_arguments():
    L = M.lib()

    def slab(**kw):
        a = dict(ex=FAKE, exs=FAKE, fmt=0, psum=FAKE, st=FAKE, cap=320, hidden=256, E=4,
                 align=64, max_m=64, slab=FAKE, ss=FAKE, mm=FAKE)
        a.update(kw)
        return L.moe_expand_to_masked_slab(a["ex"], a["exs"], a["fmt"], a["psum"], a["st"],
                                           a["cap"], a["hidden"], a["E"], a["align"],
                                           a["max_m"], a["slab"], a["ss"], a["mm"], None)
    assert slab(max_m=8) == M.MOE_ERR_SHAPE
    assert slab(max_m=40) == M.MOE_ERR_SHAPE
    assert slab(hidden=100) == M.MOE_ERR_SHAPE
    assert slab(align=48) == M.MOE_ERR_UNSUPPORTED
    assert slab(fmt=5) == M.MOE_ERR_UNSUPPORTED
    assert slab(mm=None) == M.MOE_ERR_NULL
    assert slab(slab=MIS) == M.MOE_ERR_ALIGNMENT

    def gemm(**kw):
        a = dict(a=FAKE, as_=FAKE, fmt=0, w=FAKE, ws=FAKE, mm=FAKE, max_m=64, n=256, k=256,
                 E=4, out=FAKE)
        a.update(kw)
        return L.moe_grouped_gemm_fp8_masked(a["a"], a["as_"], a["fmt"], a["w"], a["ws"],
                                             a["mm"], a["max_m"], a["n"], a["k"], a["E"],
                                             a["out"], None)
    assert gemm(max_m=40) == M.MOE_ERR_SHAPE
    assert gemm(n=100) == M.MOE_ERR_SHAPE
    assert gemm(mm=None) == M.MOE_ERR_NULL
    assert gemm(out=MIS) == M.MOE_ERR_ALIGNMENT
    assert gemm(max_m=0) == M.MOE_OK                 # nothing to do, nothing launched

    def act(**kw):
        a = dict(gu=FAKE, mm=FAKE, max_m=64, inter=128, E=4, fmt=0, out=FAKE, os=FAKE)
        a.update(kw)
        return L.moe_act_quant_masked(a["gu"], a["mm"], a["max_m"], a["inter"], a["E"],
                                      a["fmt"], a["out"], a["os"], None)
    assert act(inter=100) == M.MOE_ERR_SHAPE
    assert act(max_m=20) == M.MOE_ERR_SHAPE
    assert act(mm=None) == M.MOE_ERR_NULL
    assert act(gu=MIS) == M.MOE_ERR_ALIGNMENT
    assert act(max_m=0) == M.MOE_OK

    def back(**kw):
        a = dict(so=FAKE, mm=FAKE, max_m=64, psum=FAKE, st=FAKE, mi=FAKE, rw=None, cap=320,
                 hidden=256, E=4, align=64, out=FAKE)
        a.update(kw)
        return L.moe_masked_slab_to_expand(a["so"], a["mm"], a["max_m"], a["psum"], a["st"],
                                           a["mi"], a["rw"], a["cap"], a["hidden"], a["E"],
                                           a["align"], a["out"], None)
    assert back(max_m=0) == M.MOE_ERR_SHAPE
    assert back(mi=None) == M.MOE_ERR_NULL
    assert back(out=MIS) == M.MOE_ERR_ALIGNMENT
    assert back(cap=0) == M.MOE_OK


def test_bf16_entry_points_reject_bad_arguments():
    L = M.lib()

    def gemm(**kw):
        a = dict(a=FAKE, w=FAKE, psum=FAKE, st=FAKE, cap=320, n=256, k=256, E=4, align=64,
                 out=FAKE)
        a.update(kw)
        return L.moe_grouped_gemm_bf16(a["a"], a["w"], a["psum"], a["st"], a["cap"], a["n"],
                                       a["k"], a["E"], a["align"], a["out"], None)
    assert gemm(n=100) == M.MOE_ERR_SHAPE
    assert gemm(k=96) == M.MOE_ERR_SHAPE
    assert gemm(cap=100) == M.MOE_ERR_SHAPE
    assert gemm(align=48) == M.MOE_ERR_UNSUPPORTED
    assert gemm(psum=None) == M.MOE_ERR_NULL
    assert gemm(w=MIS) == M.MOE_ERR_ALIGNMENT
    assert gemm(cap=0) == M.MOE_OK

    def silu(**kw):
        a = dict(gu=FAKE, mi=FAKE, psum=FAKE, st=FAKE, cap=320, inter=128, E=4, align=64,
                 out=FAKE)
        a.update(kw)
        return L.moe_silu_mul_bf16(a["gu"], a["mi"], a["psum"], a["st"], a["cap"], a["inter"],
                                   a["E"], a["align"], a["out"], None)
    assert silu(inter=100) == M.MOE_ERR_SHAPE
    assert silu(st=None) == M.MOE_ERR_NULL
    assert silu(out=MIS) == M.MOE_ERR_ALIGNMENT
    assert silu(cap=0) == M.MOE_OK
    # keep-bf16 layout: ex_scale may be NULL, the plain layout refuses the format
    assert _layout_bf16(fmt=2, exs=None, wsb=16) == M.MOE_ERR_WORKSPACE
    assert _layout(fmt=2) == M.MOE_ERR_UNSUPPORTED


def test_gather_rejects_bad_arguments():
    f = M.lib().moe_gather

    def call(**kw):
        a = dict(eo=FAKE, s2d=FAKE, w=None, scale=1.0, prank=None, nsrc=0, rows=64,
                 hidden=256, topk=2, cap=320, out=FAKE)
        a.update(kw)
        return f(a["eo"], a["s2d"], a["w"], a["scale"], a["prank"], a["nsrc"], a["rows"],
                 a["hidden"], a["topk"], a["cap"], a["out"], None)
    assert call(scale=float("nan")) == M.MOE_ERR_UNSUPPORTED
    assert call(scale=float("inf")) == M.MOE_ERR_UNSUPPORTED
    assert call(hidden=100) == M.MOE_ERR_SHAPE
    assert call(topk=40) == M.MOE_ERR_SHAPE
    assert call(s2d=None) == M.MOE_ERR_NULL
    assert call(out=MIS) == M.MOE_ERR_ALIGNMENT
    assert call(rows=0) == M.MOE_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(M, "_lib", None)
    with pytest.raises(ImportError):
        M.lib()
