"""bench.py's host-side logic (no GPU): the one-GPU rule, the algorithmic FLOP
and byte counts it reports, and the rule that counter-derived traffic is only
reported for the kernel sources it was taken on."""

import os
import subprocess
import sys

import bench
from wam_asp_w4a4_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "exactly one GPU" in p.stderr
    assert p.stdout == ""


def test_flop_count_of_the_layer_set():
    # 2MNK + 4MKr + 2MNr per linear, summed over the 600 linears of the set
    total = sum(bench.layer_flops(M, N, K, r) for _, M, K, N, r, *_ in synth.mot_shapes())
    assert total == 40_478_221_271_040
    # the video projection: 2*4096*3072*3072 + 4*4096*3072*32 + 2*4096*3072*32
    assert bench.layer_flops(4096, 3072, 3072, 32) == 77_309_411_328 + 1_610_612_736 + 805_306_368


def test_algorithmic_bytes_of_a_layer():
    # x bf16, y bf16, 4-bit codes and block-16 scales, bf16 W~V, float32 V, s and b
    M, N, K, r = 256, 1024, 1024, 32
    want = M * K * 2 + M * N * 2 + N * K // 2 + N * K // 16 + 2 * N * r + 4 * K * r + 4 * K + 4 * N
    assert bench.layer_bytes(M, N, K, r, 2, 2) == want == 1_843_200


def test_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    kernel, slug = "k_gemm", "probe_slug"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.kernel_source_digest(kernel)
    f = prof / f"traffic_{kernel}_{slug}.md"
    f.write_text(f"traffic_bytes_per_launch: 12345\nsource_digest: {digest}\n")
    assert bench.measured_traffic(kernel, slug) == 12345
    f.write_text("traffic_bytes_per_launch: 12345\nsource_digest: 0000000000000000\n")
    assert bench.measured_traffic(kernel, slug) is None
    f.unlink()
    assert bench.measured_traffic(kernel, slug) is None
