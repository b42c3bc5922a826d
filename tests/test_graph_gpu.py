"""HIP-graph capture of the drafter step (RFC page, Design: the proposer runs inside captured
decode graphs; suffix-gpu page, Highlights: static shapes, no host synchronisation, index swapped
without moving buffers).

sfx_propose is captured once and replayed while the program's own eager work runs between the
replays: new documents are harvested (so the next replay must see them through the delta scan),
rebuilds are swapped in, and the input rows are rewritten in place.  Every replay must equal an
eager call and the oracle on the live corpus."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def test_captured_propose_follows_corpus_and_inputs():
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
