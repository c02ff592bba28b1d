"""GPU parity of the grouped expert layer: every routed row of every expert
against the oracle's SharQ linear layer of that row with that expert's weight
(|y_gpu - y_ref| <= 1e-5 * sum|terms| + 1e-6), for gathered token rows
(gate/up) and expert-sorted rows (down), with empty experts, experts spanning
several M tiles, ragged N tiles, bf16 and strided outputs, and out-of-range
row indices."""
import numpy as np
import pytest

import fp4_sparse_dense_amd as sq
from fp4_sparse_dense_amd import synth
from oracle import sharq_oracle as O
from tests.gpu_helpers import assert_linear_close, dev_bf16

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def _reference(ref_act, src_rows, seg, w_stack, experts):
    """Per expert: oracle linear of its routed source rows with its weight slice."""
    ne = w_stack.shape[0] // experts
    rows = seg[-1]
    y = np.zeros((rows, ne))
    b = np.zeros((rows, ne))
    for e in range(experts):
        lo, hi = seg[e], seg[e + 1]
        if hi == lo:
            continue
        wc, ws = O.pack_weight(w_stack[e * ne:(e + 1) * ne])
        idx = src_rows[lo:hi]
        ok = (idx >= 0) & (idx < ref_act["s_codes"].shape[0])
        if ok.any():
            ye, be = O.linear(ref_act, wc, ws, rows=idx[ok])
            y[lo:hi][ok] = ye
            b[lo:hi][ok] = be
    return y, b


def _run(x, w_stack, experts, seg, row_index, rows=None):
    import torch
    act = sq.sharq_prepare(dev_bf16(x), None)
    wt = sq.sharq_pack_weight(dev_bf16(w_stack))
    seg_d = _dev(seg, torch.int64)
    ri = None if row_index is None else _dev(row_index.astype(np.int32), torch.int32)
    y = sq.sharq_linear_grouped(act, wt, seg_d, experts, row_index=ri, rows=int(seg[-1]) if rows is None else rows)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_gate_up_gathered(seed):
    print(f"grouped gate/up seed {seed}", flush=True)
    rng = np.random.default_rng(100 + seed)
    tokens, experts, top_k, d_model, d_ff = 512, 12, 4, 256, 64
    expert, token, seg = synth.zipf_router(rng, tokens, experts, top_k)
    x = synth.outlier_activations(rng, tokens, d_model)
    w = np.concatenate([synth.linear_weight(rng, 2 * d_ff, d_model) for _ in range(experts)])
    assert int(np.diff(seg).max()) > 256            # some expert spans several M tiles
    yg = _run(x, w, experts, seg, token)
    ref = O.prepare(x, None)
    yr, b = _reference(ref, token.astype(np.int64), seg, w, experts)
    assert_linear_close(yg, yr, b, f"gate/up seed {seed}")


def test_grouped_down_sorted_rows_with_empty_experts():
    print("grouped down", flush=True)
    rng = np.random.default_rng(7)
    experts, d_model, d_ff = 10, 256, 96
    counts = np.array([0, 37, 300, 0, 1, 16, 15, 513, 0, 40])      # empty, tiny, multi-tile
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = synth.outlier_activations(rng, int(seg[-1]), d_ff)
    w = np.concatenate([synth.linear_weight(rng, d_model, d_ff) for _ in range(experts)])
    yg = _run(x, w, experts, seg, None)
    ref = O.prepare(x, None)
    yr, b = _reference(ref, np.arange(seg[-1]), seg, w, experts)
    assert_linear_close(yg, yr, b, "down")


def test_grouped_partial_k_tile():
    """K = 160: the last 128-wide K tile holds 32 real columns and zero padding,
    through the gather (token rows) and the in-place read (sorted rows)."""
    print("grouped partial K tile", flush=True)
    rng = np.random.default_rng(51)
    tokens, experts, top_k, d_model, n_e = 140, 7, 3, 160, 48
    expert, token, seg = synth.zipf_router(rng, tokens, experts, top_k)
    x = synth.outlier_activations(rng, tokens, d_model)
    w = np.concatenate([synth.linear_weight(rng, n_e, d_model) for _ in range(experts)])
    ref = O.prepare(x, None)
    yg = _run(x, w, experts, seg, token)
    yr, b = _reference(ref, token.astype(np.int64), seg, w, experts)
    assert_linear_close(yg, yr, b, "partial K tile, gathered")
    xs = x[token]                                         # the same rows, already in expert order
    ys = _run(xs, w, experts, seg, None)
    yr2, b2 = _reference(O.prepare(xs, None), np.arange(len(xs)), seg, w, experts)
    assert_linear_close(ys, yr2, b2, "partial K tile, in order")


def test_grouped_out_of_range_rows_read_zero():
    print("grouped out-of-range rows", flush=True)
    rng = np.random.default_rng(11)
    experts, d_model, n_e, tokens = 3, 128, 32, 40
    x = synth.outlier_activations(rng, tokens, d_model)
    w = np.concatenate([synth.linear_weight(rng, n_e, d_model) for _ in range(experts)])
    row_index = np.array([0, 5, 39, 40, -1, 7, 1000, 3, 2], dtype=np.int64)
    seg = np.array([0, 3, 3, 9], dtype=np.int64)
    yg = _run(x, w, experts, seg, row_index)
    ref = O.prepare(x, None)
    yr, b = _reference(ref, row_index, seg, w, experts)
    bad = (row_index < 0) | (row_index >= tokens)
    assert np.all(yg[bad] == 0.0)
    assert_linear_close(yg, yr, b, "out-of-range rows")


def test_grouped_ragged_tiles_bf16_and_strided_outputs():
    """N_e = 80 (a last N tile past N_e) and experts ending inside a 16-row block:
    fp32 output against the oracle; the bf16 output is the fp32 one rounded to
    nearest even; outputs with a padded row stride (16-byte rows: the LDS-staged
    epilogue; odd stride: the element-wise one) equal the dense ones and leave
    the padding untouched."""
    import torch
    print("grouped ragged tiles / bf16 / strided", flush=True)
    rng = np.random.default_rng(21)
    tokens, experts, top_k, d_model, n_e = 300, 6, 3, 384, 80
    expert, token, seg = synth.zipf_router(rng, tokens, experts, top_k)
    x = synth.outlier_activations(rng, tokens, d_model)
    w = np.concatenate([synth.linear_weight(rng, n_e, d_model) for _ in range(experts)])
    act = sq.sharq_prepare(dev_bf16(x), None)
    wt = sq.sharq_pack_weight(dev_bf16(w))
    seg_d = _dev(seg, torch.int64)
    ri = _dev(token.astype(np.int32), torch.int32)
    rows = int(seg[-1])
    y32 = sq.sharq_linear_grouped(act, wt, seg_d, experts, row_index=ri, rows=rows)
    y16 = sq.sharq_linear_grouped(act, wt, seg_d, experts, row_index=ri, rows=rows, out_dtype=sq.OUT_BF16)
    outs = {}
    for pad in (8, 1):
        for dt, code in ((torch.float32, sq.OUT_F32), (torch.bfloat16, sq.OUT_BF16)):
            big = torch.full((rows, n_e + pad), 3.0, dtype=dt, device="cuda")
            sq.sharq_linear_grouped(act, wt, seg_d, experts, row_index=ri, rows=rows, out=big[:, :n_e], out_dtype=code)
            outs[(pad, code)] = big
    torch.cuda.synchronize()
    ref = O.prepare(x, None)
    yr, b = _reference(ref, token.astype(np.int64), seg, w, experts)
    assert_linear_close(y32.cpu().numpy(), yr, b, "ragged grouped fp32")
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    for (pad, code), big in outs.items():
        want = y32 if code == sq.OUT_F32 else y16
        assert torch.equal(big[:, :n_e].contiguous(), want), (pad, code)
        assert torch.all(big[:, n_e:] == 3.0), (pad, code)


def test_grouped_malformed_offsets_are_clamped():
    """Segment offsets outside the contract (seg[0] != 0, decreasing, negative,
    past rows, seg[E] != rows, more experts than a wave has lanes) act as their
    sanitised form: clamped into [0, rows], seg[0] = 0, seg[E] = rows, then the
    running maximum.  The output equals the oracle's over those segments."""
    print("grouped malformed offsets", flush=True)
    rng = np.random.default_rng(31)
    experts, d_model, n_e = 70, 128, 16
    rows = 300
    seg = np.sort(rng.integers(0, rows, experts + 1)).astype(np.int64)
    seg[5] = seg[4] - 30          # decreasing
    seg[9] = -7                   # negative
    seg[40] = rows + 25           # past rows (clamps to rows: the experts after it are empty ...)
    seg[41:60] = seg[41:60] - rows  # ... whatever follows it below
    seg[0], seg[-1] = 17, rows - 40
    clean = np.clip(seg, 0, rows)
    clean[0], clean[-1] = 0, rows
    clean = np.maximum.accumulate(clean)
    x = synth.outlier_activations(rng, rows, d_model)
    w = np.concatenate([synth.linear_weight(rng, n_e, d_model) for _ in range(experts)])
    yg = _run(x, w, experts, seg, None, rows=rows)
    yc = _run(x, w, experts, clean, None, rows=rows)
    assert np.array_equal(yg, yc)
    ref = O.prepare(x, None)
    yr, b = _reference(ref, np.arange(rows), clean, w, experts)
    assert_linear_close(yg, yr, b, "malformed offsets")


def test_grouped_most_experts():
    """The largest expert count the layer takes (1024): the setup's scans then
    hold 17 offsets per lane.  Zipf-routed token rows (most experts empty, a few
    spanning several M tiles); every routed row against the oracle."""
    print("grouped 1024 experts", flush=True)
    rng = np.random.default_rng(41)
    tokens, experts, top_k, d_model, n_e = 600, 1024, 4, 128, 16
    expert, token, seg = synth.zipf_router(rng, tokens, experts, top_k)
    assert (np.diff(seg) == 0).sum() > 100 and np.diff(seg).max() > 128
    x = synth.outlier_activations(rng, tokens, d_model)
    w = np.concatenate([synth.linear_weight(rng, n_e, d_model) for _ in range(experts)])
    yg = _run(x, w, experts, seg, token)
    ref = O.prepare(x, None)
    yr, b = _reference(ref, token.astype(np.int64), seg, w, experts)
    assert_linear_close(yg, yr, b, "1024 experts")


def test_grouped_full_size_sampled():
    """The Qwen3-30B-A3B-shaped expert layer at full size (4096 tokens, top-8 of
    128 experts with Zipf(1.1) loads; gate/up K = 2048, N_e = 1536 over routed
    token rows, down K = 768, N_e = 2048 over expert-sorted rows), the launch
    configuration the benchmark times; the oracle recomputes sampled routed
    rows (the largest and smallest experts, segment edges, random ones) at
    sampled columns from each row's expert weight."""
    import torch
    print("grouped full size sampled", flush=True)
    inp = synth.moe_inputs(seed=4)
    E, seg, token = 128, inp["seg"], inp["token"]
    rows = int(seg[-1])
    sizes = np.diff(seg)
    rng = np.random.default_rng(5)
    big, small = int(np.argmax(sizes)), int(np.argmin(np.where(sizes > 0, sizes, 1 << 30)))
    pick = [seg[big], seg[big + 1] - 1, seg[small], seg[small + 1] - 1, 0, rows - 1]
    pick += list(rng.choice(rows, 18, replace=False))
    pick = np.unique(np.array(pick, dtype=np.int64))
    expert_of = np.searchsorted(seg, pick, side="right") - 1
    seg_d = _dev(seg, torch.int64)
    for name, x, w, src in (("gate/up", inp["x_tok"], inp["w_gu"], token.astype(np.int64)),
                            ("down", inp["x_down"], inp["w_d"], np.arange(rows))):
        ne = w.shape[1]
        act = sq.sharq_prepare(dev_bf16(x), None)
        wt = sq.sharq_pack_weight(dev_bf16(w.reshape(E * ne, -1)))
        ri = _dev(token.astype(np.int32), torch.int32) if name == "gate/up" else None
        y = sq.sharq_linear_grouped(act, wt, seg_d, E, row_index=ri, rows=rows)
        torch.cuda.synchronize()
        cols = np.unique(np.concatenate([np.arange(16), np.arange(ne - 16, ne), rng.choice(ne, 96, replace=False)]))
        got = y.cpu().numpy()[np.ix_(pick, cols)]
        ref = O.prepare(x[src[pick]], None)
        yr = np.zeros_like(got, dtype=np.float64)
        b = np.zeros_like(yr)
        for j, e in enumerate(expert_of):
            wc, ws = O.pack_weight(w[e][cols])
            yj, bj = O.linear(ref, wc, ws, rows=np.array([j]))
            yr[j], b[j] = yj[0], bj[0]
        assert_linear_close(got, yr, b, f"full-size {name}")
        del act, wt, y
