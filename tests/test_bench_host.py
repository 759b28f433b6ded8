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


def test_counters_only_for_matching_sources(tmp_path, monkeypatch):
    kernel, slug = "k_gemm", "probe_slug"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.kernel_source_digest(kernel)
    f = prof / f"counters_{kernel}_{slug}.md"
    f.write_text(f"mfma_busy_frac: 0.4632\nlds_bank_conflict_per_launch: 9748480\nsource_digest: {digest}\n")
    assert bench.measured_counters(kernel, slug) == {"mfma_busy_frac": 0.4632,
                                                      "lds_bank_conflict_per_launch": 9748480.0}
    f.write_text("mfma_busy_frac: 0.4632\nsource_digest: 0000000000000000\n")
    assert bench.measured_counters(kernel, slug) is None


def test_default_is_the_layer_set(monkeypatch):
    # no flags: the 600-layer set, 10 denoising steps; --workload picks a small one
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.mot and a.steps == 10 and a.warmup == 2
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "3"])
    a = bench.parse()
    assert not a.mot and a.workload == 3 and a.steps == 400


def test_every_profile_summary_names_its_command_and_kernel_sources():
    # each committed summary gives the rocprofv3 command that made it; the
    # traffic and counter summaries also carry the figure bench.py reads and
    # the digest of the kernel sources they were taken on
    prof = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(prof))
    assert names, "no profile summaries"
    for name in names:
        text = open(os.path.join(prof, name)).read()
        assert name.endswith(".md"), name
        assert "rocprofv3 " in text, name
        assert len(text) < 16_000, name
        if name.startswith("traffic_"):
            assert "traffic_bytes_per_launch:" in text and "source_digest:" in text, name
        if name.startswith("counters_"):
            assert "mfma_busy_frac:" in text and "source_digest:" in text, name


def test_calls_of_a_block_follow_its_data_flow():
    # what each projection of a transformer block reads: the block's input,
    # the conditioning context, or the output of other projections (through
    # attention, a residual add or an activation)
    needs = {
        "self_attn.q": set(), "self_attn.k": set(), "self_attn.v": set(),
        "self_attn.o": {"self_attn.q", "self_attn.k", "self_attn.v"},
        "cross_attn.q": {"self_attn.o"},
        "cross_attn.k": set(), "cross_attn.v": set(),   # the context
        "cross_attn.o": {"cross_attn.q", "cross_attn.k", "cross_attn.v"},
        "ffn.0": {"cross_attn.o"},
        "ffn.2": {"ffn.0"},
    }
    done = set()
    seen = [p for call in bench.MOT_GROUPS for p in call]
    assert sorted(seen) == sorted(needs), "every projection exactly once"
    for call in bench.MOT_GROUPS:
        for p in call:
            assert needs[p] <= done, f"{p} runs before {needs[p] - done}"
        done |= set(call)
    # one call per dependency level: nothing that could join an earlier call
    # is left for a later one
    level = {}

    def lvl(p):
        if p not in level:
            level[p] = 1 + max((lvl(q) for q in needs[p]), default=-1)
        return level[p]
    first = set(bench.MOT_GROUPS[0])
    assert first == {p for p in needs if lvl(p) == 0}
