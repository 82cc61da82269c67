"""Host logic of bench.py: attribution of profiled kernels to entry points,
the per-pass FLOP count, and the --gpus guard.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("name,fused,call", [
    ("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, float, false, false>(...)", True, "wtconv_fwd"),
    ("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, float, true, false>(...)", False, "wtconv_bwd_input"),
    ("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, float, false, true>(...)", False, "wtconv_fwd"),
    ("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, __half, true, true>(...)", False, "wtconv_bwd_input"),
    ("void wtc::dev::k_tile_apply<5, 3, 32, 64, 256, float, true>(...)", True, "wtconv_bwd"),
    ("void wtc::dev::k_tile_apply<5, 3, 32, 64, 256, float, true>(...)", False, "wtconv_bwd_input"),
    ("void wtc::dev::k_deep_apply<float, 5, false>(...)", True, "wtconv_fwd"),
    ("void wtc::dev::k_deep_apply<float, 5, true>(...)", False, "wtconv_bwd_input"),
    ("void wtc::dev::k_plane_bww<5, 2, 56, 56, 1, 256, float, false>(...)", False, "wtconv_bwd_weight"),
    ("void wtc::dev::k_deep_bww<5>(...)", True, "wtconv_bwd"),
    ("void wtc::dev::k_bww_final<float, 5>(...)", False, "wtconv_bwd_weight"),
    ("void wtc::dev::k_bww_final<__half, 7>(...)", True, "wtconv_bwd"),
    ("void wtc::dev::k_plane_bwd<5, 2, 56, 56, 1, 256, float, false, false>(...)", True, "wtconv_bwd"),
    ("void wtc::dev::k_plane_bwd1<5, 2, 56, 56, 1, 256, float, false, true, false>(...)", True, "wtconv_bwd"),
    ("void wtc::dev::k_plane_bwd1<5, 2, 56, 56, 1, 256, float, true, true, true>(...)", False, "wtconv_bwd"),
    ("void wtc::dev::k_plane_bwd1<5, 2, 56, 56, 1, 256, float, true, false, false>(...)", False, "wtconv_bwd_weight"),
    ("void wtc::dev::k_plane_bwd1<5, 2, 56, 56, 1, 256, float, false, false, true>(...)", False, "wtconv_bwd_weight"),
    ("void wtc::dev::k_plane_bwd1<5, 2, 56, 56, 1, 256, float, false, false, false>(...)", True, "wtconv_bwd"),
    ("void wtc::dev::k_tile_bwd1<5, 3, 32, 32, 256, float>(...)", True, "wtconv_bwd"),
    ("__amd_rocclr_copyBuffer", True, None),
    ("void at::native::roll_cuda_kernel<float>(...)", True, None),
])
def test_kernels_map_to_their_entry_point(name, fused, call):
    assert bench.call_of(name, fused) == call


def test_step_marker_is_the_forward_main_kernel():
    assert bench.is_step_marker("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, float, false, false>(x)")
    assert bench.is_step_marker("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, float, false, true>(x)")
    assert bench.is_step_marker("void wtc::dev::k_tile_apply<5, 3, 32, 64, 256, float, false>(x)")
    assert not bench.is_step_marker("void wtc::dev::k_plane_apply<5, 2, 56, 56, 1, 256, float, true, false>(x)")
    assert not bench.is_step_marker("void wtc::dev::k_tile_apply<5, 3, 32, 64, 256, float, true>(x)")
    assert not bench.is_step_marker("void wtc::dev::k_deep_apply<float, 5, false>(x)")


def test_flops_per_pixel():
    # 2 k^2 for the base conv plus 4 subbands of 2 k^2 on grids 4^l smaller:
    # 2 * 25 * (1 + 1 + 1/4) = 112.5 at k = 5, L = 2
    assert bench.conv_flops_per_pixel(2, 5) == pytest.approx(112.5)
    assert bench.conv_flops_per_pixel(1, 3) == pytest.approx(2 * 9 * 2)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a kernel\n__global__ void k(float* p) { p[0] = 1.f; }  // one\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", str(tmp_path))
    h0 = bench.source_hash()
    src.write_text("/* reworded\n   comment */\n\n__global__ void k(float* p) { p[0] = 1.f; }\n")
    assert bench.source_hash() == h0
    src.write_text("__global__ void k(float* p) { p[0] = 2.f; }\n")
    assert bench.source_hash() != h0


def test_percentiles_nearest_rank():
    v = list(range(1, 101))  # 1..100
    assert bench.percentiles(v) == {"p10": 10, "p50": 50, "p90": 90}
    assert bench.percentiles([5.0]) == {"p10": 5.0, "p50": 5.0, "p90": 5.0}
    assert bench.percentiles([3.0, 1.0, 2.0], qs=(50,)) == {"p50": 2.0}


def test_cpu_model_reads_proc_cpuinfo():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_roofline_bound_follows_arithmetic_intensity():
    # fp32 stage-1 forward: 2.17 GFLOP on 154 MB, 14 FLOP/B < 19.7: HBM-bound
    r = bench.roofline("wtconv_fwd", 2.17e9, 154e6, 50e-6, None, 1)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(154e6 / 50e-6 / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, rel=1e-3)
    # the same FLOPs on fp16 bytes (half): 28 FLOP/B > 19.7: FMA-bound
    r = bench.roofline("wtconv_fwd", 2.17e9, 77e6, 50e-6, 80e6, 10)
    assert r["bound"] == "alu" and r["unit"] == "TFLOP/s" and r["peak"] == 157.3
    assert r["traffic_bytes_per_output_element"] == pytest.approx(8e6)
    assert bench.RIDGE_FLOP_PER_BYTE == pytest.approx(157.3e12 / 8e12)
