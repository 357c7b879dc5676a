"""The bench's roofline arithmetic (CPU only).

`roofline.achieved` is algorithmic bytes per launch over the measured launch
time, so the byte formula is pinned here against the per-unit figures
written out by hand for the DeepSeek-V3 share (4096 received rows, H=7168,
I=2048, 8 local experts, 1041 live rows): every non-empty expert's weights
and block scales once, each live row's operand and scales once, its bf16
output once; flops 2 * rows * N * K.  The recorded HBM traffic must be the
measured counterpart of those bytes (within a few percent), and it is only
reported while the kernel source is the one it was measured on.
"""

import bench


def test_fp32_scale_gemm_bytes_dsv3():
    b1, f1 = bench.gemm_cost(1041, 4096, 7168, 8, 4)
    assert b1 == 8 * (4096 * 7168 + 32 * 56 * 4) + 1041 * (7168 + 56 * 4) + 1041 * 4096 * 2
    assert b1 == 251_161_312                  # 251.2 MB
    assert f1 == 2.0 * 1041 * 4096 * 7168
    b2, f2 = bench.gemm_cost(1041, 7168, 2048, 8, 4)
    assert b2 == 8 * (7168 * 2048 + 56 * 16 * 4) + 1041 * (2048 + 16 * 4) + 1041 * 7168 * 2
    assert b2 == 134_591_552                  # 134.6 MB
    assert f2 == 2.0 * 1041 * 7168 * 2048


def test_other_formats():
    # UE8M0: one byte per scale
    b, _ = bench.gemm_cost(100, 256, 512, 3, 1)
    assert b == 3 * (256 * 512 + 2 * 4 * 1) + 100 * (512 + 4) + 100 * 256 * 2
    # MXFP8: one byte per 1x32 group of every weight row and activation row
    b, _ = bench.gemm_cost(100, 256, 512, 3, 4, mx=True)
    assert b == 3 * (256 * 512 + 256 * 16) + 100 * (512 + 16) + 100 * 256 * 2
    # bf16 weights: two bytes per value, no scales
    b, f = bench.gemm_cost(100, 256, 512, 3, 0, eb=2)
    assert b == 3 * 256 * 512 * 2 + 100 * 512 * 2 + 100 * 256 * 2
    assert f == 2.0 * 100 * 256 * 512


def test_recorded_traffic_matches_algorithmic_bytes():
    t = bench.measured_traffic("dsv3")
    assert t is not None, "the PMC record does not match the GEMM source"
    b1, _ = bench.gemm_cost(1041, 4096, 7168, 8, 4)
    b2, _ = bench.gemm_cost(1041, 7168, 2048, 8, 4)
    alg = (b1 + b2) / 2
    assert alg <= t <= 1.05 * alg


def test_traffic_withheld_for_another_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "grouped_gemm_dsv3_pmc.txt").write_text(
        "traffic_bytes_per_launch: 1\ngemm_source_sha256_16: 0000000000000000\n")
    csrc = tmp_path / "expanded_dispatch_layout_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "gemm.hip").write_text("// another kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("dsv3") is None
    assert bench.measured_traffic("large") is None
