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

import pytest

torch = pytest.importorskip("torch")

import expanded_dispatch_layout_amd as M  # noqa: E402
from tests._inputs import make, to_gpu  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _replay_check(mod, call, bufs, inputs_a, inputs_b, out):
    """call() reads its inputs from `bufs`.  Run it eagerly on a and on b
    (copied into bufs), capture it, then replay with a, b, a copied into the
    same buffers, each replay compared with the eager run on those inputs.
    The output is refilled with the same value before every run (rows past
    the valid boundary are never written)."""
    def load(src):
        for k in bufs:
            if bufs[k] is not None:
                bufs[k].copy_(src[k])

    eager = {}
    for name, src in (("a", inputs_a), ("b", inputs_b)):
        load(src)
        out.fill_(-3.0)
        call()
        torch.cuda.synchronize()
        eager[name] = out.clone()
    load(inputs_a)
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
        load(inputs_a if name == "a" else inputs_b)
        out.fill_(-3.0)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[name].view(torch.int16)), (rep, name)
    assert not torch.equal(eager["a"].view(torch.int16), eager["b"].view(torch.int16))


@pytest.mark.parametrize("fmt", ["f32", "ue8m0", "mxfp8"])
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
    keys = ("x", "x_scale", "ids", "w", "prank")
    bufs = {k: ga[k].clone() for k in keys}
    ins_a = {k: ga[k] for k in keys}
    ins_b = {k: gb[k] for k in keys}

    def call():
        mod(bufs["x"], bufs["x_scale"], bufs["ids"], bufs["w"], bufs["prank"], out=out)
    _replay_check(mod, call, bufs, ins_a, ins_b, out)


def test_masked_decode_path_graph_replay():
    a = make("tiny", rows=64, seed=63)
    b = make("tiny", rows=64, seed=64)
    ga, gb = to_gpu(a), to_gpu(b)
    R, T = a["ids"].shape
    mod = M.MaskedMoE(R, T, ga["w13"], ga["w13_scale"], ga["w2"], ga["w2_scale"], a["align"],
                      64, a["fmt"])
    out = torch.zeros((R, mod.H), dtype=torch.bfloat16, device="cuda")
    keys = ("x", "x_scale", "ids", "w")
    bufs = {k: ga[k].clone() for k in keys}
    ins_a = {k: ga[k] for k in keys}
    ins_b = {k: gb[k] for k in keys}

    def call():
        mod(bufs["x"], bufs["x_scale"], bufs["ids"], bufs["w"], None, out=out)
    _replay_check(mod, call, bufs, ins_a, ins_b, out)


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_standard_path_graph_replay(fmt):
    """The standard path (bf16 rows quantised in the layout, routed factor)."""
    from tests.test_gpu_standard import to_gpu_std
    from tests.test_oracle_standard import std_inputs
    a = std_inputs(fmt=fmt, rows=48, seed=65)
    b = std_inputs(fmt=fmt, rows=48, seed=66)
    ga, gb = to_gpu_std(a), to_gpu_std(b)
    R, T = a["ids"].shape
    mod = M.StandardMoE(R, T, ga["w13"], ga["w13_scale"], ga["w2"], ga["w2_scale"], a["align"],
                        fmt, a["routed_scaling_factor"])
    out = torch.zeros((R, mod.H), dtype=torch.bfloat16, device="cuda")
    keys = ("x", "ids", "w")
    bufs = {k: ga[k].clone() for k in keys}

    def call():
        mod(bufs["x"], bufs["ids"], bufs["w"], out=out)
    _replay_check(mod, call, bufs, {k: ga[k] for k in keys}, {k: gb[k] for k in keys}, out)


def test_bf16_weight_path_graph_replay():
    from tests.test_gpu_bf16 import t16
    from tests.test_oracle_bf16 import bf16_inputs
    a = bf16_inputs(rows=48, seed=67)
    b = bf16_inputs(rows=48, seed=68)
    R, T = a["ids"].shape
    mod = M.StandardBf16MoE(R, T, t16(a["w13_bf16"]), t16(a["w2_bf16"]), a["align"],
                            a["routed_scaling_factor"])
    out = torch.zeros((R, mod.H), dtype=torch.bfloat16, device="cuda")

    def dev(inp):
        return {"x": t16(inp["x_bf16"]), "ids": torch.from_numpy(inp["ids"]).cuda(),
                "w": torch.from_numpy(inp["w"]).cuda()}
    ga, gb = dev(a), dev(b)
    bufs = {k: v.clone() for k, v in ga.items()}

    def call():
        mod(bufs["x"], bufs["ids"], bufs["w"], out=out)
    _replay_check(mod, call, bufs, ga, gb, out)
