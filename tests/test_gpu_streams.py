"""The library on the caller's stream and under HIP graph capture: results on a
side stream (passed explicitly or current through torch.cuda.stream) equal the
default stream's; a captured graph of the preparation, the layer, the grouped
layer and the one-launch decode layer, replayed several times with new inputs
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
    x_dec = dev_bf16(xs[0][:1])

    xd = dev_bf16(xs[0])                                   # static input of the graph

    def work(x, xdec):
        act = sq.sharq_prepare(x, gd, 1e-5)
        return (sq.sharq_linear(act, wt),
                sq.sharq_linear_grouped(act, wg, seg, 4),
                sq.sharq_linear_fused(xdec, wt, gd, 1e-5),
                sq.sharq_linear_fused(xdec, wt_nv, gd, 1e-5))

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
