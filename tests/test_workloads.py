"""The seeded input generators have the structure their workloads claim (no GPU)."""
import numpy as np

import workloads as W


def test_hot_4gram_workload_is_hot():
    """Every request of the boilerplate workload ends in the fixed 4-gram, which the 1M-token
    corpus holds followed by a real token more than 10^5 times."""
    w = W.WORKLOADS[6]
    c = W.join_docs(W.corpus_docs(6))
    H = W.hot_gram(w.V)
    at = (c[:-4] == H[0]) & (c[1:-3] == H[1]) & (c[2:-2] == H[2]) & (c[3:-1] == H[3]) & \
        (c[4:] >= 0)
    assert 0.9e6 < len(c) < 1.2e6
    assert int(at.sum()) > 100_000
    n, tok, samp = W.make_batch(6, B=16)
    for b in range(16):
        ctx = np.concatenate([tok[b, : n[b]], samp[b][samp[b] >= 0]])
        assert np.array_equal(ctx[-4:], H)
        assert (ctx >= 0).all() and w.n_lo <= n[b] <= w.n_hi


def test_inputs_are_seeded():
    a = W.make_batch(6, set_index=1, B=4)
    b = W.make_batch(6, set_index=1, B=4)
    c = W.make_batch(6, set_index=2, B=4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[1], c[1])
