"""HIP-graph capture of the drafter step (RFC page, Design: the proposer runs inside captured
decode graphs; suffix-gpu page, Highlights: static shapes, no host synchronisation, index swapped
without moving buffers).

sfx_propose is captured once and replayed while the program's own eager work runs between the
replays: new documents are harvested (so the next replay must find them in the delta), rebuilds
are swapped in, and the input rows are rewritten in place.  Every replay must equal an eager call
and the oracle on the live corpus.  A step captured while an ingest is pending records the passes
that index the delta by tail pair, and its replays run them; one captured with nothing pending
records none, and its replays scan the delta instead."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pending", [False, True])
def test_captured_propose_follows_corpus_and_inputs(pending):
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import suffix_match_drafter_amd as sfx

    knobs = dict(k=16, max_tree_depth=24, num_backoff=4, max_occurrences=128, mode=1,
                 spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
    B, S, cap = 32, 4096, 1 << 17
    d = sfx.Drafter(sfx.Config(max_batch=B, max_seq=S, max_sampled=1, corpus_capacity=cap,
                               **knobs))
    docs = W.corpus_docs(3)
    lc = O.LiveCorpus(cap)
    d.ingest_docs(docs[:100])
    lc.ingest(docs[:100])
    d.rebuild()
    if pending:  # documents past the live index at capture time
        d.ingest_docs(docs[400:420])
        lc.ingest(docs[400:420])
    p = O.params_from(knobs)

    n0, tok0, samp0 = W.make_batch(2, set_index=0, B=B)
    dn = torch.from_numpy(n0).cuda()
    dt = torch.from_numpy(tok0).cuda()
    ds = torch.from_numpy(samp0).cuda()
    draft = torch.empty((B, 16), dtype=torch.int32, device="cuda")
    nv = torch.empty((B,), dtype=torch.int32, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.propose(dn, dt, ds, draft, nv)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.propose(dn, dt, ds, draft, nv)
    torch.cuda.synchronize()

    inputs = [(n0, tok0, samp0)] + [W.make_batch(2, set_index=i, B=B) for i in (1, 2)]
    for step in range(6):
        # eager work between replays: new documents, sometimes a rebuild, new rows in place
        new = docs[100 + 40 * step: 140 + 40 * step]
        d.ingest_docs(new)
        lc.ingest(new)
        if step % 2 == 1:
            d.rebuild()
        n, tok, samp = inputs[step % len(inputs)]
        dn.copy_(torch.from_numpy(n))
        dt.copy_(torch.from_numpy(tok))
        ds.copy_(torch.from_numpy(samp))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_d, got_n = draft.cpu().numpy().copy(), nv.cpu().numpy().copy()
        eager_d, eager_n = d.propose(dn, dt, ds)
        torch.cuda.synchronize()
        exp_d, exp_n = O.propose(p, n, tok, samp, corpus=lc.text(), num_threads=8)
        assert np.array_equal(got_d, eager_d.cpu().numpy()), f"replay {step} vs eager"
        assert np.array_equal(got_n, eager_n.cpu().numpy()), f"replay {step} vs eager counts"
        assert np.array_equal(got_d, exp_d) and np.array_equal(got_n, exp_n), \
            f"replay {step} vs oracle"
    d.close()


def test_captured_call_forms_and_acceptance():
    """The counted and masked call forms and the acceptance calls captured together in one graph
    (each uses context-owned scratch, so none synchronises or allocates) and replayed between
    eager ingests, rebuilds and rewritten inputs.  Every replay equals the same calls made
    eagerly on a second context that follows the same corpus, and the oracle."""
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import suffix_match_drafter_amd as sfx

    knobs = dict(k=12, max_tree_depth=16, num_backoff=3, max_occurrences=64, mode=1,
                 spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
    B, S, T, k2, cap = 24, 512, 2, 7, 1 << 16
    cfg = sfx.Config(max_batch=B, max_seq=S, max_sampled=T, corpus_capacity=cap, **knobs)
    d, e = sfx.Drafter(cfg), sfx.Drafter(cfg)  # captured, and its eager mirror
    rng = np.random.default_rng(77)
    V = 6
    docs = [rng.integers(0, V, size=int(rng.integers(5, 200))).astype(np.int32)
            for _ in range(210)]
    lc = O.LiveCorpus(cap)
    for x in (d, e):
        x.ingest_docs(docs[:60])
        x.rebuild()
    lc.ingest(docs[:60])
    p = O.params_from(knobs)

    def draw():
        tok = rng.integers(0, V, size=(B, S)).astype(np.int32)
        n = rng.integers(0, S + 1, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, T)).astype(np.int32)
        samp[rng.random(B) < 0.3, 1] = -1
        counts = rng.integers(0, T + 1, size=B).astype(np.int32)
        mask = (rng.random(B) < 0.8).astype(np.int32)
        acc = rng.integers(-1, k2 + 2, size=B).astype(np.int32)
        return n, tok, samp, counts, mask, acc

    host = draw()
    dev_in = [torch.from_numpy(a).cuda() for a in host]
    dn, dt, ds, dc, dm, da = dev_in
    d1 = torch.empty((B, k2), dtype=torch.int32, device="cuda")
    v1 = torch.empty((B,), dtype=torch.int32, device="cuda")
    est = torch.empty((B, knobs["k"]), dtype=torch.int32, device="cuda")
    d2 = torch.empty((B, knobs["k"]), dtype=torch.int32, device="cuda")
    v2 = torch.empty((B,), dtype=torch.int32, device="cuda")

    def calls(x, o1, w1, oe, o2, w2):
        x.propose_counts(k2, dn, dt, ds, dc, o1, w1)
        x.accept_estimate(B, oe)
        x.accept_feedback(da)
        x.propose_masked(dn, dt, dm, o2, w2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(d, d1, v1, est, d2, v2)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    d.accept_reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(d, d1, v1, est, d2, v2)
    torch.cuda.synchronize()

    for step in range(5):
        new = docs[60 + 30 * step: 90 + 30 * step]
        for x in (d, e):
            x.ingest_docs(new)
            if step % 2 == 1:
                x.rebuild()
        lc.ingest(new)
        host = draw()
        for t_dev, a in zip(dev_in, host):
            t_dev.copy_(torch.from_numpy(a))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy().copy() for t in (d1, v1, est, d2, v2)]
        m1 = torch.empty_like(d1), torch.empty_like(v1)
        me = torch.empty_like(est)
        m2 = torch.empty_like(d2), torch.empty_like(v2)
        calls(e, m1[0], m1[1], me, m2[0], m2[1])
        torch.cuda.synchronize()
        mirror = [t.cpu().numpy() for t in (m1[0], m1[1], me, m2[0], m2[1])]
        for name, a, b in zip(("counted draft", "counted valid", "estimate", "masked draft",
                               "masked valid"), got, mirror):
            assert np.array_equal(a, b), f"replay {step}: {name} differs from the eager calls"
        assert np.array_equal(d.accept_counts().cpu().numpy(), e.accept_counts().cpu().numpy()), \
            f"replay {step}: acceptance counts"
        n, tok, samp, counts, mask, _ = host
        ed, en = O.propose_counts(p, k2, n, tok, samp, counts, corpus=lc.text())
        assert np.array_equal(got[0], ed) and np.array_equal(got[1], en), f"replay {step} counted"
        ed, en = O.propose_masked(p, n, tok, mask, corpus=lc.text())
        assert np.array_equal(got[3], ed) and np.array_equal(got[4], en), f"replay {step} masked"
    d.close()
    e.close()
