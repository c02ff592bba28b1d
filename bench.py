"""Benchmark of the SharQ linear hot path on one MI355X.

One step = fused prep (RMSNorm, 2:4 mask, MXFP4 of S, residual, MXFP4 of R)
followed by the dual FP4 GEMM with its single epilogue, on one batch of the
Llama-3.1-8B fused-QKV workload (M=2048 tokens, K=4096, N=6144).  The weight
payload is packed once, outside the timed region (it is an offline step).

Inputs are seeded synthetic tensors (fp4_sparse_dense_amd.synth) and are
resident in HBM before timing starts.  Eight input/weight/output sets
(> 512 MB together) rotate from step to step so the 256 MB MALL cannot serve
a step's operands from the previous one.

Prints one JSON line.  value = layer TFLOP/s = 4*M*N*K (2*M*N*K per path) /
(wall time per step); prep GB/s and the GEMM's MFMA fraction are reported
beside it; ``roofline`` describes the dominant kernel (the dual GEMM), timed
with HIP events on the stream it is launched on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
WORKLOAD = dict(name="qkv", M=2048, K=4096, N=6144)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dual_gemm_qkv.txt")
GEMM_SRC = os.path.join(ROOT, "fp4_sparse_dense_amd", "csrc", "gemm.hip")


def prep_bytes(M, K, norm=True):
    """Algorithmic HBM bytes of one prep launch: bf16 X in, 0.9375 B/elem out, gamma once."""
    return M * K * 2 + M * K * 15 // 16 + (2 * K if norm else 0)


def gemm_flops(M, N, K):
    return 4 * M * N * K


def source_digest(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per dual-GEMM launch from the committed rocprofv3 counter
    summary, or None when the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("traffic:"):
            for kv in line.split()[1:]:
                k, _, v = kv.partition("=")
                fields[k] = v
    if fields.get("gemm_src_sha") != source_digest(GEMM_SRC):
        return None
    try:
        return int(fields["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(rows: int = 2048):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from fp4_sparse_dense_amd import synth
    from oracle import sharq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([1] + [int(p.get("num_threads", 1)) for p in threadpool_info()])
    except Exception:  # noqa: BLE001
        cores = 1
    inp = synth.layer_inputs("qkv", seed=0)
    wc, ws = O.pack_weight(inp["w"])            # offline step, not timed
    x = inp["x"][:rows]
    t0 = time.perf_counter()
    act = O.prepare(x, inp["gamma"], inp["eps"])
    O.linear(act, wc, ws)
    dt = time.perf_counter() - t0
    flops = gemm_flops(rows, inp["N"], inp["K"])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {inp['M']} token rows of the QKV workload: prep + float64 dual GEMM over all "
                      f"{inp['N']} outputs ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=8, help="rotating input/weight/output sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_sparse_dense_amd as sq
    from fp4_sparse_dense_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M, K, N = WORKLOAD["M"], WORKLOAD["K"], WORKLOAD["N"]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    sets = []
    for s in range(args.sets):
        inp = synth.layer_inputs("qkv", seed=100 + s)
        x, g = up(inp["x"]), up(inp["gamma"])
        w = sq.sharq_pack_weight(up(inp["w"]))
        act = sq.SharqAct(M, K, dev)
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        sets.append((x, g, w, act, y))
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        x, g, w, act, y = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        sq.sharq_prepare(x, g, 1e-5, out=act)
        if ev is not None:
            ev[1].record(stream)
        sq.sharq_linear(act, w, out=y)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: wall clock over exactly `steps` steps
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-kernel durations: HIP events on the launch stream, same steps again
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    ms_per_step = wall * 1e3 / args.steps
    flops = gemm_flops(M, N, K)
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    pbytes = prep_bytes(M, K)
    prep_gbs = pbytes / (prep_ms * 1e-3) / 1e9

    cpu = None if args.no_cpu_baseline else cpu_baseline()

    rec = {
        "metric": "SharQ linear TFLOPS + prep GB/s (fraction of peak), Llama-8B shapes M=2048",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B fused QKV projection: M=2048 tokens, K=4096, N=6144; RMSNorm; "
                               "2:4 mask; MXFP4 activations and weight; fp32 output",
                   "M": M, "K": K, "N": N, "pattern": "2:4", "format": "MXFP4", "rotating_sets": args.sets},
        "prep": {"us": round(prep_ms * 1e3, 3), "GB/s": round(prep_gbs, 1),
                 "frac_hbm": round(prep_gbs / PEAK_HBM_GBS, 4), "bytes": pbytes},
        "gemm": {"us": round(gemm_ms * 1e3, 3), "TFLOP/s": round(gemm_tflops, 1),
                 "frac_mfma": round(gemm_tflops / PEAK_FP4_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": read_traffic()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
