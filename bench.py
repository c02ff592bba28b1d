"""Benchmark of the SharQ linear hot path on one MI355X.

One step = fused prep (RMSNorm, 2:4 mask, MXFP4 of S, residual, MXFP4 of R)
followed by the dual FP4 GEMM with its single epilogue, on one batch of a
workload.  The default workload -- the headline line -- is the Llama-3.1-8B
fused QKV projection (M=2048 tokens, K=4096, N=6144, RMSNorm).  Other
workloads (``--workload``): gateup (N=28672, RMSNorm), down (K=14336, N=4096,
SiLU-product inputs, no norm), decode (``--m`` in 1, 8, 32, 64; K=N=4096, no
norm; ``--fmt nvfp4`` runs it in the NVFP4-style format: E4M3 scale per 16,
binary32 tensor scales, fp16 MFMA on exactly expanded codes) and moe (Qwen3-30B-A3B-shaped expert layer: 4096 tokens routed top-8 of
128 experts with Zipf(1.1) loads; step = prep of the tokens + grouped gate/up
(K=2048, N_e=1536) + prep of the 32768 expert-sorted down rows + grouped down
(K=768, N_e=2048)) and moe_mlp (the same experts as one MLP: prep of the tokens
+ grouped gate/up whose SwiGLU epilogue prepares the down rows, h =
SiLU(gate) * up never stored + grouped down on them).  ``--mode dense`` times the plain MXFP4 linear instead
(pattern 0:4: no backbone, MXFP4 of the normalised row, one GEMM) -- the dense
FP4 baseline SharQ is compared against; its flops are 2*M*N*K.  Weight payloads
are packed once, outside the timed region (an offline step).

Inputs are seeded synthetic tensors (fp4_sparse_dense_amd.synth for
activations and the router; weights N(0, 0.02) drawn on the device from a
seeded generator and rounded to bf16) and are resident in HBM before timing
starts.  Input/weight/output sets rotate from step to step, enough of them
(> 512 MB together) that the 256 MB MALL cannot serve a step's operands from
an earlier one.

Prints one JSON line.  value = layer TFLOP/s = 4*M*N*K (2*M*N*K per path) /
(wall time per step); prep GB/s and the GEMM's fractions are reported beside
it; ``roofline`` describes the dominant kernel (the dual GEMM), timed with HIP
events on the stream it is launched on.  Bytes are the method's algorithmic
bytes (a compressed 2:4 backbone: 2.9375 B per activation element through the
prep, 0.9375 B read by the GEMM); the layout's own bytes (the backbone stored
masked dense) are reported beside them.  The GEMM's fraction is given on the
metric's 4*M*N*K and on the method's useful 3*M*N*K, against the published
peaks and against the peaks measured on the same device in the same run
(``measured_peaks``; ``--no-peaks`` skips that).
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
PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 MFMA (the NVFP4-style GEMM runs the fp16 one)
WORKLOADS = {
    "qkv": dict(M=2048, K=4096, N=6144, norm=True, law="outlier",
                desc="Llama-3.1-8B fused QKV projection: M=2048 tokens, K=4096, N=6144; RMSNorm"),
    "gateup": dict(M=2048, K=4096, N=28672, norm=True, law="outlier",
                   desc="Llama-3.1-8B MLP gate/up: M=2048, K=4096, N=28672; RMSNorm"),
    "down": dict(M=2048, K=14336, N=4096, norm=False, law="silu",
                 desc="Llama-3.1-8B MLP down: M=2048, K=14336, N=4096; SiLU(g)*u inputs, no norm"),
    "decode": dict(M=None, K=4096, N=4096, norm=False, law="outlier",
                   desc="decode: M rows, K=N=4096, no norm"),
}
MOE = dict(tokens=4096, experts=128, top_k=8, d_model=2048, d_ff=768)
ROTATE_BYTES = 600 << 20       # rotating sets exceed the 256 MB MALL
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dual_gemm_qkv.txt")
# the dual GEMM's source: its kernel file and the headers it compiles with
GEMM_SRC = [os.path.join(ROOT, "fp4_sparse_dense_amd", "csrc", f)
            for f in ("gemm.hip", "gemm_common.h", "device_common.h", "launch.h")]


def prep_bytes(M, K, norm=True, nv=False, dense=False):
    """Algorithmic HBM bytes of one prep, as the method counts them: bf16 X in
    once, gamma once, and out per activation element the compressed 2:4
    backbone (K/2 kept codes: 0.25 B), its metadata (0.125 B), the residual's
    codes (0.5 B) and both block-scale arrays (1/32 B each for MXFP4, 1/16 B
    each for the NVFP4-style format): 2.9375 B per element in all for MXFP4
    (3.0 for NVFP4-style).  Plain FP4 (no backbone): 2 + 0.53125 B."""
    if dense:
        out = M * K * 17 // 32
    else:
        out = M * K * 15 // 16 if not nv else M * K
    return M * K * 2 + out + (2 * K if norm else 0)


def prep_layout_bytes(M, K, norm=True, nv=False, dense=False):
    """Bytes the preparation actually moves in this library's layout: the
    backbone is stored masked dense (0.5 B per element instead of 0.25, gfx950
    has no sparse FP4 MFMA to consume a compressed one), so MXFP4 writes
    1.1875 B per element (NVFP4-style 1.25; plain FP4 0.53125)."""
    out = M * K * 5 // 4 if nv else (M * K * 17 // 32 if dense else M * K * 19 // 16)
    return M * K * 2 + out + (2 * K if norm else 0)


def gemm_flops(M, N, K):
    """The metric's count: 2*M*N*K per path, 4*M*N*K for the dual GEMM."""
    return 4 * M * N * K


def gemm_useful_flops(M, N, K):
    """The method's own work: the backbone keeps K/2 of every row, so the sparse
    path is M*N*K and the dense path 2*M*N*K.  gfx950 has no sparse FP4 MFMA,
    so 4*M*N*K execute and 0.75 of the MFMA peak is this count's ceiling."""
    return 3 * M * N * K


def gemm_bytes(M, N, K, out_bytes=4, nv=False, dense=False):
    """Algorithmic HBM bytes of one dual GEMM: the prepared A with a compressed
    backbone (0.9375 B per element: backbone codes 0.25, metadata 0.125, residual
    codes 0.5, scales 1/32 each; NVFP4-style 1.0), the packed weight read once
    for both paths (MXFP4 0.53125 B/elem; NVFP4-style 0.5625), Y.  Plain FP4:
    0.53125 B/elem on both sides."""
    if dense:
        return M * K * 17 // 32 + N * K * 17 // 32 + out_bytes * M * N
    if nv:
        return M * K + N * K * 9 // 16 + out_bytes * M * N
    return M * K * 15 // 16 + N * K * 17 // 32 + out_bytes * M * N


def gemm_layout_bytes(M, N, K, out_bytes=4, nv=False, dense=False):
    """Bytes the GEMM actually reads in this library's layout: the masked dense
    backbone (0.5 B per element) and no metadata, so 1.0625 B per activation
    element for MXFP4 (NVFP4-style 1.125)."""
    if dense:
        return gemm_bytes(M, N, K, out_bytes, dense=True)
    if nv:
        return M * K * 9 // 8 + N * K * 9 // 16 + out_bytes * M * N
    return M * K * 17 // 16 + N * K * 17 // 32 + out_bytes * M * N


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


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


def cpu_threads():
    """(nproc, affinity count, threads used by the all-core legs)."""
    nproc = os.cpu_count() or 1
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        aff = nproc
    return nproc, aff, max(1, min(aff, 16))


def cpu_baseline(prep_rows: int = 128, gemm_rows: int = 512, min_s: float = 3.0):
    """The oracle as it stands, on bounded samples of the QKV workload, in
    three legs: the preparation single-threaded, the preparation on all
    allowed cores (row blocks on a thread pool: numpy releases the GIL inside
    its array operations, and the preparation is row-local), and the float64
    dual GEMM with the BLAS library's threads.  Each leg repeats whole passes
    until min_s of wall time."""
    import concurrent.futures as cf

    import numpy as np
    from fp4_sparse_dense_amd import synth
    from oracle import sharq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([1] + [int(p.get("num_threads", 1)) for p in threadpool_info()])
    except Exception:  # noqa: BLE001
        blas = 1
    nproc, aff, threads = cpu_threads()
    inp = synth.layer_inputs("qkv", seed=0)
    M, K, N = inp["M"], inp["K"], inp["N"]
    wc, ws = O.pack_weight(inp["w"])            # offline step, not timed

    def loop(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return n, dt

    x1 = inp["x"][:prep_rows]
    n1, t1 = loop(lambda: O.prepare(x1, inp["gamma"], inp["eps"]))
    prep1 = prep_bytes(prep_rows, K) * n1 / t1 / 1e9
    xa = inp["x"][:prep_rows * threads]
    chunks = np.array_split(xa, threads)
    with cf.ThreadPoolExecutor(threads) as ex:
        na, ta = loop(lambda: list(ex.map(lambda c: O.prepare(c, inp["gamma"], inp["eps"]), chunks)))
    prep_all = prep_bytes(xa.shape[0], K) * na / ta / 1e9
    act = O.prepare(inp["x"][:gemm_rows], inp["gamma"], inp["eps"])
    ng, tg = loop(lambda: O.linear(act, wc, ws))
    gemm_tf = gemm_flops(gemm_rows, N, K) * ng / tg / 1e12
    # the whole layer on all cores, per token row: prep (all cores) + GEMM
    s_row = prep_bytes(1, K, norm=False) / (prep_all * 1e9) + gemm_flops(1, N, K) / (gemm_tf * 1e12)
    return {"value": gemm_flops(1, N, K) / s_row / 1e12, "unit": "TFLOP/s", "cores": max(threads, blas),
            "kind": "oracle",
            "sample": f"QKV workload (K={K}, N={N}): prep of {prep_rows} rows single-threaded ({n1} passes, "
                      f"{t1:.1f} s), prep of {xa.shape[0]} rows on {threads} threads ({na} passes, {ta:.1f} s), "
                      f"float64 dual GEMM of {gemm_rows} rows x all {N} outputs with {blas} BLAS threads "
                      f"({ng} passes, {tg:.1f} s); value = 4*N*K flops per row over the all-core prep time "
                      f"plus the GEMM time per row",
            "prep_1thread_GB/s": round(prep1, 4), "prep_allcores_GB/s": round(prep_all, 4),
            "gemm_fp64_TFLOP/s": round(gemm_tf, 5), "nproc": nproc, "affinity": aff,
            "prep_threads": threads, "blas_threads": blas}


def measure_peaks(reps: int = 5):
    """FP4 MFMA rate on random operand bytes and streaming read bandwidth over
    1 GiB (past the 256 MB last-level cache), measured on this device with the
    library's measurement kernels; HIP events on the stream they run on."""
    import torch

    import fp4_sparse_dense_amd as sq
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    ops = torch.randint(0, 256, (6144,), dtype=torch.uint8, device="cuda", generator=gen)
    # the same bytes with the first operands in the backbone's pattern: in every
    # group of four codes (16 bits) two are zero, the kept pair drawn at random
    keep = torch.tensor([0x00FF, 0x0F0F, 0xF00F, 0x0FF0, 0xF0F0, 0xFF00], dtype=torch.int32, device="cuda")
    pick = keep[torch.randint(0, 6, (2048,), device="cuda", generator=gen)]
    half = ops[:4096].view(2048, 2).to(torch.int32)
    masked_a = torch.stack([half[:, 0] & (pick & 0xFF), half[:, 1] & (pick >> 8)], 1).reshape(-1).to(torch.uint8)
    ops_masked = torch.cat([masked_a, ops[4096:]])
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    buf = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device="cuda", generator=gen)
    stream = torch.cuda.current_stream()

    def rate(launch):
        launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        work = sum(launch() for _ in range(reps))
        e1.record(stream)
        torch.cuda.synchronize()
        return work / (e0.elapsed_time(e1) * 1e-3)

    fp4 = rate(lambda: sq.peak_fp4_mfma(ops, 4096, sink)) / 1e12
    fp4_masked = rate(lambda: sq.peak_fp4_mfma(ops_masked, 4096, sink)) / 1e12
    rd = rate(lambda: sq.peak_read(buf, sink)) / 1e9
    del buf
    torch.cuda.empty_cache()
    # the dual GEMM runs half its MFMAs on the backbone, half on the residual
    mix = 2.0 / (1.0 / fp4 + 1.0 / fp4_masked)
    return {"fp4_mfma_TFLOP/s": round(fp4, 1), "fp4_mfma_backbone_TFLOP/s": round(fp4_masked, 1),
            "fp4_mfma_dual_mix_TFLOP/s": round(mix, 1), "hbm_read_GB/s": round(rd, 1),
            "how": "back-to-back v_mfma_scale_f32_16x16x128_f8f6f4, 16 waves per CU, on random E2M1 bytes, and "
                   "with two of every four first-operand codes zero (the backbone); the dual mix is their "
                   "harmonic mean (one MFMA of each kind per output block and K tile); "
                   "16-byte loads streaming 1 GiB"}


def device_weight(gen, N, K):
    """W ~ N(0, 0.02) rounded to bf16, drawn on the device from a seeded generator."""
    import torch
    return (torch.randn(N, K, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)


def timed(step, steps, warmup, graph=False):
    """Wall time per step over `steps` steps after `warmup`, bracketed by
    synchronisations, then per-kernel HIP-event times over the same steps: for
    each part of the step, that part's launches of all the steps run back to
    back between two events (an event between every kernel would add its own
    dispatch gap to each), giving the average duration of one launch.

    graph=True (workloads whose kernels are shorter than a host launch): the
    steps are captured once in a HIP graph and replayed, so the timed region
    holds device work only; per-kernel times then come from graphs holding only
    that kernel's launches, timed with events around the replay."""
    import numpy as np
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if not graph:
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        parts = []
        for j in range(step.parts):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                step(i, part=j)
            e1.record(stream)
            torch.cuda.synchronize()
            parts.append([e0.elapsed_time(e1) / steps])
        return wall * 1e3 / steps, parts

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        return g

    def replay_ms(g, reps=5):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / steps

    g_all = capture(lambda i: step(i))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_all.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    parts = []
    for j in range(step.parts):
        gj = capture(lambda i, j=j: step(i, part=j))
        parts.append([replay_ms(gj)])
    return wall * 1e3 / steps, parts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qkv", choices=sorted(list(WORKLOADS) + ["moe", "moe_mlp", "layer"]))
    ap.add_argument("--m", type=int, default=1, help="rows of the decode workload")
    ap.add_argument("--fmt", default="mxfp4", choices=["mxfp4", "nvfp4"],
                    help="FP4 format (nvfp4: the decode workload only)")
    ap.add_argument("--mode", default="sharq", choices=["sharq", "dense"],
                    help="dense: the plain MXFP4 linear (no backbone), the baseline SharQ is compared against")
    ap.add_argument("--fused", action="store_true",
                    help="decode with M <= 16: the whole layer in one launch (sharq_linear_fused; MXFP4 or --fmt nvfp4)")
    ap.add_argument("--ablation", default="none", choices=["none", "unfused_norm", "unfused_epilogue"],
                    help="fusion ablations: a standalone RMSNorm writing bf16 before the preparation, or "
                         "the two GEMM paths as separate launches and an add")
    ap.add_argument("--sets", type=int, default=0, help="rotating input/weight/output sets (0: enough for > 512 MB)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the timed steps in a HIP graph and replay it (always on for decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the FP4 MFMA rate and read bandwidth on this device")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.fmt == "nvfp4" and args.workload != "decode":
        print("the NVFP4-style path is built for the decode workload (--workload decode)", file=sys.stderr)
        sys.exit(2)
    special = args.workload in ("moe", "moe_mlp", "layer")
    if special and (args.fmt != "mxfp4" or args.mode != "sharq" or args.fused or args.ablation != "none"):
        print("the moe, moe_mlp and layer workloads run the default MXFP4 SharQ layers", file=sys.stderr)
        sys.exit(2)
    if args.mode == "dense" and (args.fmt != "mxfp4" or args.workload in ("moe", "moe_mlp")):
        print("the plain FP4 linear is built for MXFP4 dense layers", file=sys.stderr)
        sys.exit(2)
    if args.fused and (args.workload != "decode" or args.m > 16 or args.mode != "sharq" or args.ablation != "none"):
        print("--fused is the one-launch layer (MXFP4 or NVFP4-style) for the decode workload with --m <= 16",
              file=sys.stderr)
        sys.exit(2)
    if args.ablation != "none" and (args.fmt != "mxfp4" or args.mode != "sharq" or args.workload in ("moe", "moe_mlp") or
                                    (args.ablation == "unfused_norm" and not WORKLOADS[args.workload]["norm"])):
        print("the fusion ablations run the MXFP4 SharQ layer (unfused_norm needs a workload with RMSNorm)",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.m < 1 or args.sets < 0:
        print("--steps and --m must be >= 1, --warmup and --sets >= 0", file=sys.stderr)
        sys.exit(2)

    import torch

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    args.measured_peaks = None if args.no_peaks else measure_peaks()
    if args.workload in ("moe", "moe_mlp"):
        rec = run_moe(args)
    elif args.workload == "layer":
        rec = run_layer(args)
    else:
        rec = run_dense(args)
    print(json.dumps(rec), flush=True)


def run_dense(args):
    import numpy as np
    import torch

    import fp4_sparse_dense_amd as sq
    from fp4_sparse_dense_amd import synth

    wl = dict(WORKLOADS[args.workload])
    M = args.m if args.workload == "decode" else wl["M"]
    K, N, norm = wl["K"], wl["N"], wl["norm"]
    nv = args.fmt == "nvfp4"
    fmt = sq.FMT_NVFP4 if nv else sq.FMT_MXFP4
    dense = args.mode == "dense"
    pat_n = 0 if dense else 2

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    per_set = M * K * 2 + gemm_bytes(M, N, K, nv=nv, dense=dense)
    nsets = args.sets or max(2, min(64, -(-ROTATE_BYTES // per_set)))
    nx = min(nsets, 4)                       # distinct activation draws (CPU-generated)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    xs, gammas = [], []
    for s in range(nx):
        if args.workload == "qkv":
            inp = synth.layer_inputs("qkv", seed=100 + s, with_weight=False)
        else:
            rng = np.random.default_rng(200 + s)
            x = synth.outlier_activations(rng, M, K) if wl["law"] == "outlier" else synth.silu_product_activations(rng, M, K)
            inp = dict(x=x, gamma=synth.norm_weight(rng, K) if norm else None)
        xs.append(up(inp["x"]))
        gammas.append(up(inp["gamma"]) if norm else None)
    ablation = args.ablation
    sets = []
    for s in range(nsets):
        w = sq.sharq_pack_weight(device_weight(gen, N, K), fmt=fmt)
        act = sq.SharqAct(M, K, torch.device("cuda"), n=pat_n, fmt=fmt)
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        extra = {}
        if ablation == "unfused_norm":
            extra["xb"] = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        if ablation == "unfused_epilogue":
            extra["ys"] = torch.empty(M, N, dtype=torch.float32, device="cuda")
            extra["yr"] = torch.empty(M, N, dtype=torch.float32, device="cuda")
            extra["pb"], extra["pr"] = sq.path_act(act, "backbone"), sq.path_act(act, "residual")
        sets.append((w, act, y, extra))
    torch.cuda.synchronize()

    # the step as a list of launches; the first n_prep are the preparation side
    def launches(i):
        w, act, y, ex = sets[i % nsets]
        x, g = xs[i % nx], gammas[i % nx]
        if ablation == "unfused_norm":
            return [lambda: sq.sharq_rmsnorm(x, g, 1e-5, out=ex["xb"]),
                    lambda: sq.sharq_prepare(ex["xb"], None, 1e-5, out=act),
                    lambda: sq.sharq_linear(act, w, out=y)]
        if ablation == "unfused_epilogue":
            return [lambda: sq.sharq_prepare(x, g, 1e-5, out=act),
                    lambda: sq.sharq_linear(ex["pb"], w, out=ex["ys"]),
                    lambda: sq.sharq_linear(ex["pr"], w, out=ex["yr"]),
                    lambda: sq.sharq_add_f32(ex["ys"], ex["yr"], out=y)]
        if args.fused:
            return [lambda: sq.sharq_linear_fused(x, w, g, 1e-5, out=y)]
        return [lambda: sq.sharq_prepare(x, g, 1e-5, n=pat_n, fmt=fmt, out=act),
                lambda: sq.sharq_linear(act, w, out=y)]
    part_names = ["layer"] if args.fused else {"unfused_norm": ["rmsnorm", "prep", "gemm"],
                  "unfused_epilogue": ["prep", "gemm_backbone", "gemm_residual", "add"]}.get(ablation, ["prep", "gemm"])
    n_prep = 0 if args.fused else (2 if ablation == "unfused_norm" else 1)

    def step(i, part=None):
        for j, fn in enumerate(launches(i)):
            if part in (None, j):
                fn()
    step.parts = len(part_names)

    graph = args.workload == "decode" or args.graph
    ms, parts = timed(step, args.steps, args.warmup, graph=graph)
    part_ms = [float(np.mean(p)) for p in parts]
    prep_ms, gemm_ms = sum(part_ms[:n_prep]), sum(part_ms[n_prep:])
    flops = gemm_flops(M, N, K) // (2 if dense else 1)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    # the one-launch layer reads X (bf16) instead of the prepared activation
    # (NVFP4-style weight: 0.5625 B/elem, MXFP4: 0.53125)
    wbytes = N * K * 9 // 16 if nv else N * K * 17 // 32
    gbytes = (M * K * 2 + wbytes + 4 * M * N) if args.fused else gemm_bytes(M, N, K, nv=nv, dense=dense)
    glayout = (M * K * 2 + wbytes + 4 * M * N) if args.fused else gemm_layout_bytes(M, N, K, nv=nv, dense=dense)
    gemm_gbs = gbytes / (gemm_ms * 1e-3) / 1e9
    pbytes = prep_bytes(M, K, norm, nv=nv, dense=dense)
    playout = prep_layout_bytes(M, K, norm, nv=nv, dense=dense)
    prep_gbs = pbytes / (prep_ms * 1e-3) / 1e9 if prep_ms > 0 else 0.0
    peak_mfma = PEAK_F16_TFLOPS if nv else PEAK_FP4_TFLOPS
    useful = flops if dense else gemm_useful_flops(M, N, K)
    useful_frac = useful / (gemm_ms * 1e-3) / 1e12 / peak_mfma
    # fractions of the peaks measured on this device in the same run (the FP4
    # MFMA rate of the GEMM's own operand mix: half backbone, half residual for
    # the SharQ layer, dense operands for the plain FP4 layer; streaming read
    # bandwidth for the HBM-bound kernels)
    mp = getattr(args, "measured_peaks", None)
    m_fp4 = (mp["fp4_mfma_TFLOP/s"] if dense else mp["fp4_mfma_dual_mix_TFLOP/s"]) if mp and not nv else None
    m_hbm = mp["hbm_read_GB/s"] if mp else None

    def frac(a, peak):
        return round(a / peak, 4) if peak else None
    hbm_bound = gbytes / (PEAK_HBM_GBS * 1e9) > flops / (peak_mfma * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gemm_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                "peak_measured": m_hbm, "frac_measured": frac(gemm_gbs, m_hbm)}
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": round(gemm_tflops / peak_mfma, 4),
                "traffic": read_traffic() if (args.workload == "qkv" and not dense and ablation == "none") else None,
                "frac_useful": round(useful_frac, 4), "peak_measured": m_fp4,
                "frac_measured": frac(gemm_tflops, m_fp4)}
    cpu = None if (args.no_cpu_baseline or args.workload != "qkv" or dense or ablation != "none") else cpu_baseline()
    wname = args.workload if args.workload != "decode" else f"decode{M}"
    if dense:
        wname += "-plainfp4"
    if args.fused:
        wname += "-fused"
    if ablation != "none":
        wname += "-" + ablation.replace("_", "-")
    return {
        "metric": ("plain MXFP4 linear TFLOPS (dense FP4 baseline, 2*M*N*K), Llama-8B shapes" if dense else
                   "SharQ linear TFLOPS + prep GB/s (fraction of peak), Llama-8B shapes M=2048"),
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4" if nv else "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"{wname}{'-nvfp4' if nv else ''}: " +
                               wl["desc"].split(": ", 1)[1].replace("M rows", f"M={M}") +
                               ("; 2:4 mask; NVFP4-style activations and weight (E4M3 scale per 16, binary32 tensor "
                                "scales, fp16 MFMA on exactly expanded codes); fp32 output" if nv else
                                "; no backbone (plain MXFP4 of the row), MXFP4 weight; fp32 output" if dense else
                                "; 2:4 mask; MXFP4 activations and weight; fp32 output"),
                   "M": M, "K": K, "N": N, "pattern": "0:4" if dense else "2:4",
                   "format": "NVFP4-style" if nv else "MXFP4",
                   "rotating_sets": nsets},
        "prep": None if args.fused else {"us": round(prep_ms * 1e3, 3), "GB/s": round(prep_gbs, 1),
                                         "frac_hbm": round(prep_gbs / PEAK_HBM_GBS, 4),
                                         "frac_hbm_measured": frac(prep_gbs, m_hbm), "bytes": pbytes,
                                         "layout_bytes": playout, "layout_overhead_bytes": playout - pbytes},
        "gemm": {"us": round(gemm_ms * 1e3, 3), "TFLOP/s": round(gemm_tflops, 1),
                 "frac_mfma": round(gemm_tflops / peak_mfma, 4), "frac_useful": round(useful_frac, 4),
                 "frac_mfma_measured": frac(gemm_tflops, m_fp4), "GB/s": round(gemm_gbs, 1),
                 "frac_hbm": round(gemm_gbs / PEAK_HBM_GBS, 4), "bytes": gbytes, "layout_bytes": glayout},
        "roofline": roof,
        "measured_peaks": mp,
        "cpu_baseline": cpu,
        "parts_us": {k: round(v * 1e3, 3) for k, v in zip(part_names, part_ms)},
    }


LAYER = dict(M=2048, d=4096, qkv=6144, ff=14336)


def run_layer(args):
    """A synthetic Llama-3.1-8B decoder layer of SharQ linears, batch 1 x 2048
    tokens, random weights: prep(x, g1) -> QKV -> [attention stand-in: the Q
    columns of the bf16 QKV output, a strided view] -> prep -> O with the
    residual add in its epilogue -> prep(h, g2) -> gate/up whose SwiGLU
    epilogue prepares the down projection's activation (the MLP's hidden
    activation is never stored) -> down with the residual add.  Attention
    itself is not part of the SharQ hot path."""
    import numpy as np
    import torch

    import fp4_sparse_dense_amd as sq
    from fp4_sparse_dense_amd import synth

    M, d, nq, ff = LAYER["M"], LAYER["d"], LAYER["qkv"], LAYER["ff"]
    dev = torch.device("cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    inp = synth.layer_inputs("qkv", seed=300, with_weight=False)
    x = up(inp["x"])
    g1 = up(inp["gamma"])
    g2 = up(synth.norm_weight(np.random.default_rng(301), d))
    w_bytes = (nq * d + d * d + 2 * ff * d + d * ff) * 17 // 32
    nsets = args.sets or max(2, -(-ROTATE_BYTES // w_bytes))
    sets = []
    for s_ in range(nsets):
        wgu = sq.interleave_gate_up(device_weight(gen, ff, d), device_weight(gen, ff, d))
        sets.append(dict(qkv=sq.sharq_pack_weight(device_weight(gen, nq, d)),
                         o=sq.sharq_pack_weight(device_weight(gen, d, d)),
                         gu=sq.sharq_pack_weight(wgu),
                         down=sq.sharq_pack_weight(device_weight(gen, d, ff))))
        del wgu
    b = dict(a1=sq.SharqAct(M, d, dev), a2=sq.SharqAct(M, d, dev), a3=sq.SharqAct(M, d, dev),
             a4=sq.SharqAct(M, ff, dev),
             qkv=torch.empty(M, nq, dtype=torch.bfloat16, device=dev),
             h=torch.empty(M, d, dtype=torch.bfloat16, device=dev),
             out=torch.empty(M, d, dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    names = ["prep_qkv", "gemm_qkv", "prep_o", "gemm_o_residual", "prep_gateup", "gemm_gateup_swiglu_prep",
             "gemm_down_residual"]

    def launches(i):
        w = sets[i % nsets]
        return [lambda: sq.sharq_prepare(x, g1, 1e-5, out=b["a1"]),
                lambda: sq.sharq_linear(b["a1"], w["qkv"], out=b["qkv"], out_dtype=sq.OUT_BF16),
                lambda: sq.sharq_prepare(b["qkv"][:, :d], None, 1e-5, out=b["a2"]),
                lambda: sq.sharq_linear_residual(b["a2"], w["o"], x, out=b["h"]),
                lambda: sq.sharq_prepare(b["h"], g2, 1e-5, out=b["a3"]),
                lambda: sq.sharq_linear_swiglu_prep(b["a3"], w["gu"], out=b["a4"]),
                lambda: sq.sharq_linear_residual(b["a4"], w["down"], b["h"], out=b["out"])]

    def step(i, part=None):
        for j, fn in enumerate(launches(i)):
            if part in (None, j):
                fn()
    step.parts = len(names)

    ms, parts = timed(step, args.steps, args.warmup)
    part_ms = [float(np.mean(p)) for p in parts]
    shapes = {"gemm_qkv": nq * d, "gemm_o": d * d, "gemm_gateup": 2 * ff * d, "gemm_down": d * ff}
    flops = sum(4 * M * nk for nk in shapes.values())
    j = names.index("gemm_gateup_swiglu_prep")
    gu_tflops = 4 * M * 2 * ff * d / (part_ms[j] * 1e-3) / 1e12
    return {
        "metric": "SharQ decoder layer TFLOPS (4*M*N*K summed over the layer's four SharQ linears)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"layer: synthetic Llama-3.1-8B decoder layer of SharQ linears, batch 1 x {M} tokens "
                               "(QKV 6144, O 4096 and down 4096 with the residual adds in their epilogues, gate/up 2x14336 "
                               "whose SwiGLU epilogue prepares the down projection's activation); attention "
                               "replaced by the Q columns of the QKV output; random weights; 2:4 mask; MXFP4",
                   "M": M, "rotating_sets": nsets},
        "roofline": {"bound": "mfma", "achieved": round(gu_tflops, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tflops / PEAK_FP4_TFLOPS, 4), "traffic": None,
                     "kernel": "gate/up GEMM with the SwiGLU epilogue preparing the down activation"},
        "cpu_baseline": None,
        "parts_us": {k: round(v * 1e3, 3) for k, v in zip(names, part_ms)},
    }


def run_moe(args):
    import numpy as np
    import torch

    import fp4_sparse_dense_amd as sq
    from fp4_sparse_dense_amd import synth

    T, E, k, dm, dff = MOE["tokens"], MOE["experts"], MOE["top_k"], MOE["d_model"], MOE["d_ff"]
    rows = T * k
    mlp = args.workload == "moe_mlp"
    rng = np.random.default_rng(300)
    expert, token, seg = synth.zipf_router(rng, T, E, k)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    x_tok = up(synth.outlier_activations(rng, T, dm))
    x_down = up(synth.outlier_activations(rng, rows, dff))
    seg_d = torch.from_numpy(seg).cuda()
    ri = torch.from_numpy(token.astype(np.int32)).cuda()
    n_gu, n_d = 2 * dff, dm
    # moe_mlp: each expert's 2*dff gate/up rows are taken as gate and up rows
    # interleaved in 16-row blocks (random weights either way)
    per_set = (E * n_gu * dm + E * n_d * dff) * 17 // 32 + 4 * rows * n_d + (rows * dff * 19 // 16 if mlp else 4 * rows * n_gu)
    nsets = args.sets or max(2, -(-ROTATE_BYTES // per_set))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    sets = []
    for s in range(nsets):
        wgu = sq.sharq_pack_weight(device_weight(gen, E * n_gu, dm))
        wd = sq.sharq_pack_weight(device_weight(gen, E * n_d, dff))
        mid = sq.SharqAct(rows, dff, torch.device("cuda")) if mlp else torch.empty(rows, n_gu, device="cuda")
        sets.append((wgu, wd, mid, torch.empty(rows, n_d, device="cuda")))
    a_tok = sq.SharqAct(T, dm, torch.device("cuda"))
    a_down = sq.SharqAct(rows, dff, torch.device("cuda"))
    ws = torch.empty(max(sq.grouped_workspace_bytes(rows, E, dm), sq.grouped_workspace_bytes(rows, E, dff)),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step(i, part=None):
        wgu, wd, mid, yd = sets[i % nsets]
        if mlp:
            fns = [lambda: sq.sharq_prepare(x_tok, None, out=a_tok),
                   lambda: sq.sharq_linear_grouped_swiglu_prep(a_tok, wgu, seg_d, E, row_index=ri, rows=rows, out=mid,
                                                               workspace=ws),
                   lambda: sq.sharq_linear_grouped(mid, wd, seg_d, E, rows=rows, out=yd, workspace=ws)]
        else:
            fns = [lambda: sq.sharq_prepare(x_tok, None, out=a_tok),
                   lambda: sq.sharq_linear_grouped(a_tok, wgu, seg_d, E, row_index=ri, rows=rows, out=mid,
                                                   workspace=ws),
                   lambda: sq.sharq_prepare(x_down, None, out=a_down),
                   lambda: sq.sharq_linear_grouped(a_down, wd, seg_d, E, rows=rows, out=yd, workspace=ws)]
        for j, fn in enumerate(fns):
            if part in (None, j):
                fn()
    step.parts = 3 if mlp else 4

    ms, parts = timed(step, args.steps, args.warmup)
    t = [float(np.mean(p)) for p in parts]
    # moe_mlp parts: token prep, gate/up (+ SwiGLU + down prep), down
    t_gu, t_d = t[1], (t[2] if mlp else t[3])
    f_gu, f_d = gemm_flops(rows, n_gu, dm), gemm_flops(rows, n_d, dff)
    # algorithmic bytes (the method's count, a compressed backbone: 0.9375 B per
    # activation element): prepared rows read once (distinct tokens for
    # gate/up), all experts' weights once, Y (or, for moe_mlp, the prepared
    # down rows) written once
    b_gu = T * dm * 15 // 16 + E * n_gu * dm * 17 // 32 + (rows * dff * 15 // 16 if mlp else 4 * rows * n_gu)
    b_d = rows * dff * 15 // 16 + E * n_d * dff * 17 // 32 + 4 * rows * n_d
    gbs_gu = b_gu / (t_gu * 1e-3) / 1e9
    tf_gu = f_gu / (t_gu * 1e-3) / 1e12
    hbm_bound = b_gu / (PEAK_HBM_GBS * 1e9) > f_gu / (PEAK_FP4_TFLOPS * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs_gu, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs_gu / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(tf_gu, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf_gu / PEAK_FP4_TFLOPS, 4), "traffic": None,
                "frac_useful": round(f_gu * 3 // 4 / (t_gu * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, 4)}
    loads = np.diff(seg)
    if mlp:
        desc = (f"moe_mlp: Qwen3-30B-A3B-shaped expert MLP, {T} tokens top-{k} of {E} experts "
                f"(Zipf(1.1) loads, max {int(loads.max())} min {int(loads.min())} rows), gate/up K={dm} "
                f"N_e={n_gu} with the SwiGLU epilogue preparing the down rows, down K={dff} N_e={n_d}; "
                f"no norm; 2:4 mask; MXFP4; fp32 output")
        prep = {"tokens_us": round(t[0] * 1e3, 3),
                "GB/s": round(prep_bytes(T, dm, False) / (t[0] * 1e-3) / 1e9, 1)}
        gemm = {"gate_up_swiglu_prep_us": round(t_gu * 1e3, 3), "down_us": round(t_d * 1e3, 3)}
    else:
        desc = (f"moe: Qwen3-30B-A3B-shaped expert layer, {T} tokens top-{k} of {E} experts "
                f"(Zipf(1.1) loads, max {int(loads.max())} min {int(loads.min())} rows), "
                f"gate/up K={dm} N_e={n_gu}, down K={dff} N_e={n_d}; no norm; 2:4 mask; MXFP4; fp32 output")
        prep = {"tokens_us": round(t[0] * 1e3, 3), "down_rows_us": round(t[2] * 1e3, 3),
                "GB/s": round((prep_bytes(T, dm, False) + prep_bytes(rows, dff, False)) / ((t[0] + t[2]) * 1e-3) / 1e9, 1)}
        gemm = {"gate_up_us": round(t_gu * 1e3, 3), "down_us": round(t_d * 1e3, 3)}
    gemm.update({"gate_up_TFLOP/s": round(tf_gu, 1), "down_TFLOP/s": round(f_d / (t_d * 1e-3) / 1e12, 1),
                 "gate_up_GB/s": round(gbs_gu, 1), "down_GB/s": round(b_d / (t_d * 1e-3) / 1e9, 1)})
    return {
        "metric": "SharQ linear TFLOPS + prep GB/s (fraction of peak), Llama-8B shapes M=2048",
        "value": round((f_gu + f_d) / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": desc, "rows": rows, "experts": E, "rotating_sets": nsets},
        "prep": prep,
        "gemm": gemm,
        "roofline": roof,
        "cpu_baseline": None,
        "parts_us": {n: round(v * 1e3, 3) for n, v in zip(
            ["prep_tokens", "gate_up_swiglu_prep", "down"] if mlp else ["prep_tokens", "gate_up", "prep_down", "down"],
            t)},
    }


if __name__ == "__main__":
    main()
