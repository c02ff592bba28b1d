"""The library on the caller's stream and under HIP graph capture: results on a
side stream (passed explicitly or current through torch.cuda.stream) equal the
default stream's; independent layers on two streams at once equal the same
calls run alone; a captured graph of the preparation, the layer, the grouped
layer, the grouped SwiGLU-prep layer and the one-launch decode layer, replayed several times with new inputs
copied in and eager work in between, equals the eager result every time."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(seed, M=256, K=1024, N=512):
    rng = np.random.default_rng(seed)
    return synth.outlier_activations(rng, M, K), synth.norm_weight(rng, K), synth.linear_weight(rng, N, K)


def test_side_stream_equals_default():
    import torch
    print("side stream", flush=True)
    x, g, w = _inputs(1, M=300, K=512, N=384)
    xd, gd, wt = dev_bf16(x), dev_bf16(g), sq.sharq_pack_weight(dev_bf16(w))
    y0 = sq.sharq_linear(sq.sharq_prepare(xd, gd, 1e-5), wt)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    y1 = sq.sharq_linear(sq.sharq_prepare(xd, gd, 1e-5, stream=s), wt, stream=s)
    with torch.cuda.stream(s):
        y2 = sq.sharq_linear(sq.sharq_prepare(xd, gd, 1e-5), wt)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)


def test_two_streams_concurrently():
    """Independent layers on two streams at once (default priority), nothing
    ordering one stream's kernels against the other's: the 2:4 MXFP4 layer, the
    NVFP4-style layer and the grouped layer on each, with different inputs,
    four rounds; every output equals the same call run alone on the default
    stream (the library keeps no state that calls share)."""
    import torch
    print("two streams", flush=True)
    work = []
    for seed in (11, 12):
        x, g, w = _inputs(seed, M=384, K=768, N=640)
        rng = np.random.default_rng(seed + 100)
        expert, token, seg = synth.zipf_router(rng, 96, 5, 2)
        we = np.concatenate([synth.linear_weight(rng, 64, 768) for _ in range(5)])
        work.append(dict(x=dev_bf16(x), g=dev_bf16(g), wt=sq.sharq_pack_weight(dev_bf16(w)),
                         wtn=sq.sharq_pack_weight(dev_bf16(w), fmt=sq.FMT_NVFP4),
                         xe=dev_bf16(x[:96]), we=sq.sharq_pack_weight(dev_bf16(we)),
                         seg=torch.from_numpy(seg).cuda(), ri=torch.from_numpy(token.astype(np.int32)).cuda()))

    def run(d, stream=None):
        y = sq.sharq_linear(sq.sharq_prepare(d["x"], d["g"], 1e-5, stream=stream), d["wt"], stream=stream)
        yn = sq.sharq_linear(sq.sharq_prepare(d["x"], d["g"], 1e-5, fmt=sq.FMT_NVFP4, stream=stream), d["wtn"],
                             stream=stream)
        ye = sq.sharq_linear_grouped(sq.sharq_prepare(d["xe"], None, stream=stream), d["we"], d["seg"], 5,
                                     row_index=d["ri"], rows=int(d["seg"][-1]), stream=stream)
        return y, yn, ye

    refs = [run(d) for d in work]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for rnd in range(4):
        outs = [run(d, stream=st) for d, st in zip(work, streams)]
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            for a, b in zip(o, r):
                assert torch.equal(a, b), f"round {rnd}, stream {i}"


def test_graph_replay_matches_eager():
    import torch
    print("graph replay", flush=True)
    xs = [_inputs(s)[0] for s in (2, 3)]
    _, g, w = _inputs(2)
    gd, wt = dev_bf16(g), sq.sharq_pack_weight(dev_bf16(w))
    wt_nv = sq.sharq_pack_weight(dev_bf16(w), fmt=sq.FMT_NVFP4)
    # grouped: 4 experts of 128 weight rows over the 256 rows, sorted
    rng = np.random.default_rng(9)
    we = np.concatenate([synth.linear_weight(rng, 128, 1024) for _ in range(4)])
    wg = sq.sharq_pack_weight(dev_bf16(we))
    seg = torch.tensor([0, 40, 40, 201, 256], dtype=torch.int64, device="cuda")
    # grouped gate/up with the SwiGLU-prep epilogue: 2 experts (F = 128) over 250
    # routed rows (a ragged last block: the padding-row fill runs too)
    wga = np.concatenate([synth.linear_weight(rng, 128, 1024) for _ in range(2)])
    wua = np.concatenate([synth.linear_weight(rng, 128, 1024) for _ in range(2)])
    wgu = sq.sharq_pack_weight(sq.interleave_gate_up(dev_bf16(wga), dev_bf16(wua), experts=2))
    seg2 = torch.tensor([0, 90, 250], dtype=torch.int64, device="cuda")
    ri = torch.arange(255, 5, -1, dtype=torch.int32, device="cuda")
    x_dec = dev_bf16(xs[0][:1])

    xd = dev_bf16(xs[0])                                   # static input of the graph

    def work(x, xdec):
        act = sq.sharq_prepare(x, gd, 1e-5)
        h = sq.sharq_linear_grouped_swiglu_prep(act, wgu, seg2, 2, row_index=ri, rows=250)
        return (sq.sharq_linear(act, wt),
                sq.sharq_linear_grouped(act, wg, seg, 4),
                sq.sharq_linear_fused(xdec, wt, gd, 1e-5),
                sq.sharq_linear_fused(xdec, wt_nv, gd, 1e-5),
                h.s_codes, h.s_meta, h.s_scales, h.r_codes, h.r_scales)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            work(xd, x_dec)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = work(xd, x_dec)
    for it, i in enumerate([0, 1, 0, 1]):
        xd.copy_(dev_bf16(xs[i]))
        x_dec.copy_(dev_bf16(xs[i][:1]))
        graph.replay()
        ref = work(dev_bf16(xs[i]), dev_bf16(xs[i][:1]))   # eager work between replays
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (it, k)


def _segment_stream(t):
    """The stream torch's caching allocator attached to the block holding t."""
    import torch
    p = t.data_ptr()
    for seg in torch.cuda.memory_snapshot():
        if seg["address"] <= p < seg["address"] + seg["total_size"]:
            return seg["stream"]
    raise AssertionError("block not found in the allocator snapshot")


def test_binding_allocates_on_the_callers_stream():
    """Buffers the binding allocates for a call on an explicit stream belong to
    that stream, so a block freed when the call returns (the grouped layer's
    workspace) is handed only to later work ordered on that stream."""
    import torch
    print("binding allocation stream", flush=True)
    x, g, w = _inputs(4, M=64, K=512, N=256)
    xd, gd, wt = dev_bf16(x), dev_bf16(g), sq.sharq_pack_weight(dev_bf16(w))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    act = sq.sharq_prepare(xd, gd, 1e-5, stream=s)
    y = sq.sharq_linear(act, wt, stream=s)
    seg = torch.tensor([0, 20, 64], dtype=torch.int64, device="cuda")
    s.wait_stream(torch.cuda.current_stream())
    yg = sq.sharq_linear_grouped(act, sq.sharq_pack_weight(dev_bf16(np.concatenate([w[:128], w[128:]]))), seg, 2,
                                 stream=s)
    assert torch.cuda.current_stream() == torch.cuda.default_stream()
    for t in (act.r_codes, act.s_codes, y, yg):
        assert _segment_stream(t) == s.cuda_stream
    torch.cuda.synchronize()
    y0 = sq.sharq_linear(sq.sharq_prepare(xd, gd, 1e-5), wt)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
