"""Host-side logic of bench.py (no GPU): the one-GPU contract, flag validation
before any device work, the algorithmic byte and flop accounting, and the
traffic record's source digest."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=e)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = _run(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("args", [
    ["--fmt", "nvfp4"],                                   # NVFP4-style: decode only
    ["--workload", "layer", "--mode", "dense"],
    ["--workload", "moe", "--ablation", "unfused_epilogue"],
    ["--fused"],                                          # decode only
    ["--workload", "decode", "--m", "32", "--fused"],     # M <= 16
    ["--workload", "down", "--ablation", "unfused_norm"],  # down has no RMSNorm
    ["--steps", "0"],
    ["--workload", "decode", "--m", "0"],
])
def test_bad_flag_combinations_exit_before_device_work(args):
    r = _run(*args)
    assert r.returncode == 2, (r.returncode, r.stderr[-300:])


def test_algorithmic_accounting():
    b = _bench()
    # QKV: 2048 x 4096 prep with gamma; dual GEMM to 6144 with fp32 Y
    assert b.prep_bytes(2048, 4096) == 2048 * 4096 * 2 + 2048 * 4096 * 19 // 16 + 2 * 4096 == 26_746_880
    assert b.gemm_flops(2048, 6144, 4096) == 206_158_430_208
    assert b.gemm_bytes(2048, 6144, 4096) == 8_912_896 + 13_369_344 + 50_331_648
    # decode M=1, K=N=4096: the weight read once for both paths
    assert b.gemm_bytes(1, 4096, 4096) == 4352 + 8_912_896 + 16_384
    # plain FP4: 0.53125 B/elem on both sides
    assert b.gemm_bytes(2048, 6144, 4096, dense=True) == 4_456_448 + 13_369_344 + 50_331_648


def test_traffic_record_follows_the_source_digest(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    rec = tmp_path / "traffic.txt"
    monkeypatch.setattr(b, "GEMM_SRC", [str(src)])
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(rec))
    assert b.read_traffic() is None                          # no record
    rec.write_text(f"header\ntraffic: gemm_src_sha={b.source_digest([str(src)])} bytes_per_launch=12345\n")
    assert b.read_traffic() == 12345
    src.write_text("kernel v2")                              # the kernel changed since the counters
    assert b.read_traffic() is None
