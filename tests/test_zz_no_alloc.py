"""moe_expand_layout_noalloc (the layout with the library's static per-GPU
scratch as its workspace) against moe_expand_layout on the same inputs,
through the C ABI: every output bit-exact, on two calls in a row, the
second with a smaller input (fewer rows and experts, a padded buffer), so
the second call runs on scratch the first one left behind.  The first call's
layout is also checked against the oracle.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from oracle import layout  # noqa: E402
from tests._inputs import make, to_gpu  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

SENT = 0x5A


def _buffers(inp, cap):
    R, T = inp["ids"].shape
    E = inp["w13_q"].shape[0]
    H = inp["x_q"].shape[1]
    sdt = torch.float32 if inp["fmt"] == "f32" else torch.uint8
    d = "cuda"
    b = dict(ex=torch.full((cap, H), SENT, dtype=torch.uint8, device=d),
             ex_scale=torch.full((H // 128, cap), 3, dtype=sdt, device=d),
             psum=torch.full((E,), -7, dtype=torch.int32, device=d),
             m_indices=torch.full((cap,), -7, dtype=torch.int32, device=d),
             src2dst=torch.full((R, T), -7, dtype=torch.int32, device=d),
             row_weight=torch.full((cap,), 5.0, dtype=torch.float32, device=d),
             status=torch.full((2,), -7, dtype=torch.int32, device=d))
    return b


def _run(inp, noalloc):
    g = to_gpu(inp)
    R, T = inp["ids"].shape
    E = inp["w13_q"].shape[0]
    cap = M.moe_expand_capacity(R, T, E, inp["align"])
    b = _buffers(inp, cap)
    args = (g["x"], g["x_scale"], inp["fmt"], g["ids"], g["w"], g["prank"], E, inp["align"],
            cap, b["ex"], b["ex_scale"], b["psum"], b["m_indices"], b["src2dst"],
            b["row_weight"], b["status"])
    if noalloc:
        M.moe_expand_layout_noalloc(*args)
    else:
        ws = torch.empty(max(M.moe_expand_workspace_bytes(R, T, E), 256), dtype=torch.uint8,
                         device="cuda")
        M.moe_expand_layout(*args, ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in b.items()}


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


CASES = [
    # a larger buffer first: 3000 rows, 16 of 48 experts, top-8
    dict(rows=3000, hidden=512, inter=128, experts=16, global_experts=48, topk=8, align=64,
         seed=201),
    # then a smaller one: a padded buffer of 700 rows (500 valid), 12 experts
    dict(rows=700, valid_rows=500, src_ranks=8, hidden=256, inter=128, experts=12,
         global_experts=30, topk=6, align=32, fmt="ue8m0", seed=202),
]


def test_noalloc_layout_matches_layout_twice():
    for i, over in enumerate(CASES):
        inp = make("tiny", **over)
        print(f"[no-alloc case {i}] rows {over['rows']} experts {over['experts']}", flush=True)
        ref = _run(inp, noalloc=False)
        got = _run(inp, noalloc=True)
        _same(got, ref)
        R, T = inp["ids"].shape
        E = inp["w13_q"].shape[0]
        nv = layout.num_valid_rows(R, inp["psum_recv_per_rank"])
        cap = M.moe_expand_capacity(R, T, E, inp["align"])
        lay = layout.expand_layout(inp["ids"], nv, E, inp["align"], cap)
        assert got["status"][0] == lay["total"] and got["status"][1] == lay["flags"]
        assert np.array_equal(got["psum"], lay["psum"])
        assert np.array_equal(got["m_indices"], lay["m_indices"])
        assert np.array_equal(got["src2dst"], lay["src2dst"])
        assert np.all(got["ex"][lay["total"]:] == SENT)   # past the total: untouched


def test_noalloc_layout_refuses_oversized_request():
    rows, T, E, align = 1 << 20, 2, 256, 64
    assert M.moe_expand_workspace_bytes(rows, T, E) > M.MOE_NOALLOC_SCRATCH_BYTES
    cap = M.moe_expand_capacity(rows, T, E, align)
    # Only host checks run: every pointer is a small valid tensor that the
    # call must not touch (it returns before any launch).
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = M._ptr(t)
    code = M.lib().moe_expand_layout_noalloc(
        p, 256, p, 2, 0, p, p, None, 0, rows, 256, T, E, align, cap,
        p, p, p, p, p, p, p, None)
    assert code == M.MOE_ERR_SCRATCH
    assert torch.count_nonzero(t).item() == 0
