"""The whole path captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: no call reads device data on the host or synchronises, so the
step records as a static graph (SGLang PR 37261, Modifications/Core: labels
from the device psum with no cumsum, host copy or sentinel; vLLM PR 54109,
Motivation: the real/padding boundary stays on the device because reading
it on the host would break graph capture).

Each path is run eagerly once, then captured, then replayed three times
with eager work of the program's own between the replays (new inputs copied
into the captured input buffers, other launches) and every replay checked
bit for bit against an eager run on the same inputs.  The library records
no memset nodes (it clears nothing with hipMemsetAsync), and the tests
capture nothing but its launches.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from tests._inputs import make, to_gpu  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _replay_check(mod, call, inputs_a, inputs_b, out):
    """Capture call() on the buffers in inputs_a; replay with a and b in turn
    (copied into those buffers) and compare each replay with an eager run."""
    bufs = inputs_a
    eager = {}
    for name, src in (("a", inputs_a), ("b", inputs_b)):
        for k in bufs:
            if bufs[k] is not None:
                bufs[k].copy_(src[k])
        call()
        torch.cuda.synchronize()
        eager[name] = out.clone()
    for k in bufs:
        if bufs[k] is not None:
            bufs[k].copy_(inputs_a[k])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()                     # warm-up on the side stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep, name in enumerate(("a", "b", "a")):
        src = inputs_a if name == "a" else inputs_b
        for k in bufs:
            if bufs[k] is not None:
                bufs[k].copy_(src[k])
        out.fill_(-3.0)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[name].view(torch.int16)), (rep, name)
    assert not torch.equal(eager["a"].view(torch.int16), eager["b"].view(torch.int16))


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_expand_path_graph_replay(fmt):
    a = make("tiny", rows=40, valid_rows=23, src_ranks=4, fmt=fmt, seed=61)
    b = make("tiny", rows=40, valid_rows=31, src_ranks=4, fmt=fmt, seed=62)
    ga, gb = to_gpu(a), to_gpu(b)
    gb["w13"], gb["w13_scale"], gb["w2"], gb["w2_scale"] = (ga["w13"], ga["w13_scale"],
                                                          ga["w2"], ga["w2_scale"])
    R, T = a["ids"].shape
    mod = M.ExpandedMoE(R, T, ga["w13"], ga["w13_scale"], ga["w2"], ga["w2_scale"],
                        a["align"], fmt)
    out = torch.zeros((R, mod.H), dtype=torch.bfloat16, device="cuda")
    ins_a = {k: ga[k].clone() for k in ("x", "x_scale", "ids", "w", "prank")}
    ins_b = {k: gb[k] for k in ins_a}

    def call():
        mod(ins_a["x"], ins_a["x_scale"], ins_a["ids"], ins_a["w"], ins_a["prank"], out=out)
    _replay_check(mod, call, ins_a, ins_b, out)


def test_masked_decode_path_graph_replay():
    a = make("tiny", rows=64, seed=63)
    b = make("tiny", rows=64, seed=64)
    ga, gb = to_gpu(a), to_gpu(b)
    R, T = a["ids"].shape
    mod = M.MaskedMoE(R, T, ga["w13"], ga["w13_scale"], ga["w2"], ga["w2_scale"], a["align"],
                      64, a["fmt"])
    out = torch.zeros((R, mod.H), dtype=torch.bfloat16, device="cuda")
    ins_a = {k: ga[k].clone() for k in ("x", "x_scale", "ids", "w")}
    ins_b = {k: gb[k] for k in ins_a}

    def call():
        mod(ins_a["x"], ins_a["x_scale"], ins_a["ids"], ins_a["w"], None, out=out)
    _replay_check(mod, call, ins_a, ins_b, out)
