"""bench.py's host-side logic: argument checks that end before any device is touched, the kernel
source hash that ties a counter profile to the code it was taken on, the traffic lookup, and the
thread count of the CPU baseline."""
import os

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_bad_step_counts_are_refused():
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--warmup", "-2"]) == 2


def test_kernel_sha_ignores_comments_only(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SRC, encoding="utf-8").read()
    base = bench.kernel_sha()
    commented = tmp_path / "commented.hip"
    commented.write_text("// a new comment line\n\n" + src.replace("\n", "   // trailing note\n", 1), encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(commented))
    assert bench.kernel_sha() == base
    changed = tmp_path / "changed.hip"
    changed.write_text(src + "\nstatic int extra_symbol;\n", encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(changed))
    assert bench.kernel_sha() != base


def test_counter_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    wl, kern = "bf16_b2_h16_s4096_d128", "attn_fwd_kernel"
    path = os.path.join(bench.PROFILES, f"{kern}_{wl}_pmc.txt")
    if not os.path.exists(path):
        pytest.skip("no committed HBM counter profile for the default workload")
    fields = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
    committed_sha = fields["kernel_source_sha256_16"].strip()
    got = bench.counter_traffic(kern, wl)
    if committed_sha == bench.kernel_sha():
        assert got == int(float(fields["traffic_bytes_per_launch"]))
    else:
        assert got is None
    # a profile taken on other code is not used
    src = open(bench.KERNEL_SRC, encoding="utf-8").read()
    other = tmp_path / "other.hip"
    other.write_text(src + "\nstatic int another_symbol;\n", encoding="utf-8")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(other))
    assert bench.counter_traffic(kern, wl) is None
    assert bench.counter_traffic(kern, "no_such_workload") is None


def test_cpu_share_uses_the_affinity_set(monkeypatch):
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    threads, info = bench.cpu_share()
    assert threads == len(os.sched_getaffinity(0)) and info["share"] is None
    assert info["nproc"] >= info["affinity"] >= 1
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    threads, info = bench.cpu_share()
    assert threads == 1 and info["share"] == 1
