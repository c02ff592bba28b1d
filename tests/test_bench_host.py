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
    """The byte and flop counts follow the method's own accounting: a
    compressed 2:4 backbone, 2.9375 B per activation element through the prep
    and 0.9375 B read by the GEMM (QKV: 24,649,728 and 71,565,312 B)."""
    b = _bench()
    # QKV: 2048 x 4096 prep with gamma; dual GEMM to 6144 with fp32 Y
    assert b.prep_bytes(2048, 4096) == 2048 * 4096 * 47 // 16 + 2 * 4096 == 24_649_728
    assert b.gemm_bytes(2048, 6144, 4096) == 7_864_320 + 13_369_344 + 50_331_648 == 71_565_312
    assert b.gemm_flops(2048, 6144, 4096) == 206_158_430_208
    assert b.gemm_useful_flops(2048, 6144, 4096) * 4 == b.gemm_flops(2048, 6144, 4096) * 3
    # the layout's own bytes: the backbone stored masked dense (0.5 B instead of 0.25)
    assert b.prep_layout_bytes(2048, 4096) == 26_746_880
    assert b.prep_layout_bytes(2048, 4096) - b.prep_bytes(2048, 4096) == 2048 * 4096 // 4
    assert b.gemm_layout_bytes(2048, 6144, 4096) == 8_912_896 + 13_369_344 + 50_331_648
    # down projection: no RMSNorm
    assert b.prep_bytes(2048, 14336, norm=False) == 86_245_376
    assert b.gemm_bytes(2048, 4096, 14336) == 92_274_688
    # gate/up and the Qwen3 MoE rows
    assert b.gemm_bytes(2048, 28672, 4096) == 305_135_616
    assert b.prep_bytes(32768, 768, norm=False) == 73_924_608
    # decode M=1, K=N=4096: the weight read once for both paths
    assert b.gemm_bytes(1, 4096, 4096) == 3840 + 8_912_896 + 16_384
    # plain FP4: 0.53125 B/elem on both sides, as stored
    assert b.gemm_bytes(2048, 6144, 4096, dense=True) == 4_456_448 + 13_369_344 + 50_331_648
    assert b.prep_bytes(2048, 4096, dense=True) == b.prep_layout_bytes(2048, 4096, dense=True)
    # NVFP4-style: 16-element scales
    assert b.prep_bytes(64, 4096, norm=False, nv=True) == 64 * 4096 * 3
    assert b.gemm_bytes(64, 4096, 4096, nv=True) == 64 * 4096 + 4096 * 4096 * 9 // 16 + 4 * 64 * 4096


def test_cpu_thread_counts():
    b = _bench()
    nproc, aff, threads = b.cpu_threads()
    assert nproc >= aff >= 1 and 1 <= threads <= min(aff, 16)


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


def test_committed_traffic_record_matches_the_sources():
    """The committed QKV counter summary carries the digest of the current GEMM
    sources, so the bench line reports its HBM traffic (after a change to those
    sources the counters are taken again, or the record re-stamped once the QKV
    kernel's instructions are shown unchanged)."""
    b = _bench()
    assert b.read_traffic() is not None, "profiles/traffic_dual_gemm_qkv.txt does not match the GEMM sources"
