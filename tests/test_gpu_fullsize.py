"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (ExpandedMoE, capacity from the host bound).

The layout is compared in full, bit-exact.  The layer output is compared on
sampled rows that the oracle evaluates one by one (per-token brute force,
bit-identical to the layered oracle on the CPU tests), with the same bars as
the small cases.  The padded buffers also check that rows past the boundary
are untouched and that a tail whose ids alias valid experts changes nothing.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from oracle import layer, layout  # noqa: E402
from tests._inputs import make, to_gpu  # noqa: E402
from tests.test_gpu_parity import SENT, _check_output, bf16_np  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

_outs = {}


def run_full(name):
    print(f"\n[{name}] quantising inputs with the oracle", flush=True)
    inp = make(name)
    g = to_gpu(inp)
    R, T = inp["ids"].shape
    mod = M.ExpandedMoE(R, T, g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], inp["align"],
                        inp["fmt"])
    mod.ex.fill_(SENT)
    out = torch.full((R, mod.H), 7.0, dtype=torch.bfloat16, device="cuda")
    print(f"[{name}] running the layer on the GPU", flush=True)
    mod(g["x"], g["x_scale"], g["ids"], g["w"], g["prank"], out=out)
    torch.cuda.synchronize()
    return inp, mod, bf16_np(out)


def check_layout(name, inp, mod):
    R, T = inp["ids"].shape
    E = inp["w13_q"].shape[0]
    nv = layout.num_valid_rows(R, inp["psum_recv_per_rank"])
    lay = layout.expand_layout(inp["ids"], nv, E, inp["align"], mod.capacity)
    st = mod.status.cpu().numpy()
    assert st[0] == lay["total"] and st[1] == lay["flags"]
    assert np.array_equal(mod.psum.cpu().numpy(), lay["psum"])
    assert np.array_equal(mod.m_indices.cpu().numpy(), lay["m_indices"])
    src = mod.src2dst.cpu().numpy()
    assert np.array_equal(src, lay["src2dst"])
    n = lay["total"]
    ex = mod.ex[:n + 8].cpu().numpy()
    exs = mod.ex_scale.t()[:n].contiguous().cpu().numpy()   # stored K-block-major
    rw = mod.row_weight[:n].cpu().numpy()
    live = src >= 0
    rr, kk = np.nonzero(live)
    d = src[live]
    assert np.array_equal(ex[d], inp["x_q"][rr])
    assert np.array_equal(exs[d], inp["x_s"][rr])
    assert np.array_equal(rw[d].view(np.uint32), inp["w"][rr, kk].view(np.uint32))
    pad = np.ones(n, bool)
    pad[d] = False
    assert not ex[:n][pad].any() and not exs[pad].any() and not rw[pad].any()
    assert np.all(ex[n:] == SENT)
    print(f"[{name}] layout bit-exact: total {n}, counts {lay['counts'].tolist()}")


def check_sampled_rows(name, inp, out):
    R, T = inp["ids"].shape
    nv = layout.num_valid_rows(R, inp["psum_recv_per_rank"])
    rng = np.random.default_rng(5)
    has = np.nonzero((inp["ids"][:nv] >= 0).any(axis=1))[0]
    none = np.nonzero(~(inp["ids"][:nv] >= 0).any(axis=1))[0]
    rows = np.concatenate([rng.choice(has, size=min(24, len(has)), replace=False),
                           rng.choice(none, size=min(4, len(none)), replace=False)])
    most = np.argsort(-(inp["ids"][:nv] >= 0).sum(axis=1), kind="stable")[:4]
    rows = np.unique(np.concatenate([rows, most]))
    o = {k: v for k, v in inp.items() if k != "psum_recv_per_rank"} | {"num_valid": nv}
    print(f"[{name}] oracle on {len(rows)} sampled rows", flush=True)
    ref = layer.brute_force(o, rows=rows)
    got = out[rows]
    _check_output(got, ref)
    assert not np.any(got[(inp["ids"][rows] < 0).all(axis=1)])   # no local slot -> 0
    if nv < R:
        assert np.all(out[nv:] == 7.0)                            # past the boundary


FULL = ["dsv3", "dsv3_zipf_ue8m0", "large", "padded", "padded_alias"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    inp, mod, out = run_full(name)
    check_layout(name, inp, mod)
    del mod
    check_sampled_rows(name, inp, out)
    if name.startswith("padded"):
        _outs[name] = out[:inp["num_valid"]].copy()


def test_full_padded_tail_is_never_routing():
    for name in ("padded", "padded_alias"):
        if name not in _outs:
            _outs[name] = run_full(name)[2][:1536].copy()
    assert np.array_equal(_outs["padded"].view(np.uint32), _outs["padded_alias"].view(np.uint32))
