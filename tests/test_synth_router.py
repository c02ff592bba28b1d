"""The seeded expert router used for the grouped workload: its invariants
(every token routed to top_k distinct experts, rows sorted by expert then
token, segment offsets consistent with the rows, Zipf popularity ordering)."""
import numpy as np

from fp4_sparse_dense_amd import synth


def test_router_invariants():
    rng = np.random.default_rng(0)
    tokens, experts, top_k = 1024, 64, 8
    expert, token, seg = synth.zipf_router(rng, tokens, experts, top_k)
    assert expert.shape == token.shape == (tokens * top_k,)
    assert seg.shape == (experts + 1,) and seg[0] == 0 and seg[-1] == tokens * top_k
    assert np.all(np.diff(seg) >= 0)
    # rows sorted by (expert, token), each expert's rows inside its segment
    assert np.all(np.lexsort((token, expert)) == np.arange(tokens * top_k))
    for e in range(experts):
        assert np.all(expert[seg[e]:seg[e + 1]] == e)
    # each token: top_k distinct experts
    per_token = {}
    for e, t in zip(expert, token):
        per_token.setdefault(int(t), set()).add(int(e))
    assert len(per_token) == tokens and all(len(v) == top_k for v in per_token.values())


def test_router_is_seeded_and_skewed():
    a = synth.zipf_router(np.random.default_rng(5), 2048, 128, 8)
    b = synth.zipf_router(np.random.default_rng(5), 2048, 128, 8)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    loads = np.diff(a[2])
    # Zipf(1.1) popularity over 128 experts: the busiest expert carries several
    # times the mean load, the quietest far less than it
    assert loads.max() > 4 * loads.mean() and loads.min() < loads.mean() / 2
