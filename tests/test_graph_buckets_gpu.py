"""Batch-bucketed graphs of the drafter step (RFC page "[RFC]: Suffix decoding on GPU
(suffix_gpu)", Design, Proposer bullet: the draft chain is captured per batch-size bucket at
warm-up and runs eagerly where capture fails or graphs are off).

A graph set is created over persistent buffers whose rows past the live batch hold junk.  Each
call runs the smallest bucket >= B with rows B.. emptied, and must equal an eager call on the
first B rows and the oracle on the live corpus; the emptied rows must read as empty (length 0,
no sampled id, draft -1, count 0) and rows past the bucket must be left alone.  Between calls
the corpus grows (a pending delta) and rebuilds are swapped in.  The fallback is exercised by
the disabled mode and by captures that are broken on purpose from the host."""
import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

KNOBS = dict(k=16, max_tree_depth=24, num_backoff=4, max_occurrences=128, mode=1,
             spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
MAXB, S, T, CAP = 64, 4096, 1, 1 << 17
BUCKETS = [8, 16, 32]
SENTINEL = 7


def _drafter():
    import suffix_match_drafter_amd as sfx

    d = sfx.Drafter(sfx.Config(max_batch=MAXB, max_seq=S, max_sampled=T, corpus_capacity=CAP,
                               **KNOBS))
    docs = W.corpus_docs(3)
    lc = O.LiveCorpus(CAP)
    d.ingest_docs(docs[:150])
    lc.ingest(docs[:150])
    d.rebuild()
    return d, lc, docs


def _buffers():
    import torch

    nt = torch.zeros((MAXB,), dtype=torch.int32, device="cuda")
    tok = torch.zeros((MAXB, S), dtype=torch.int32, device="cuda")
    smp = torch.full((MAXB, T), -1, dtype=torch.int32, device="cuda")
    draft = torch.full((MAXB, KNOBS["k"]), SENTINEL, dtype=torch.int32, device="cuda")
    nv = torch.full((MAXB,), SENTINEL, dtype=torch.int32, device="cuda")
    return nt, tok, smp, draft, nv


def _fill(bufs, B, step, rng):
    """Rows 0..B-1 from a fresh input set; every other row junk; outputs set to a sentinel."""
    import torch

    nt, tok, smp, draft, nv = bufs
    n, t, s = W.make_batch(3, set_index=step, B=B)
    junk_n = rng.integers(1, S + 1, size=MAXB).astype(np.int32)
    junk_s = rng.integers(0, 32000, size=(MAXB, T)).astype(np.int32)
    junk_n[:B], junk_s[:B] = n, s
    nt.copy_(torch.from_numpy(junk_n))
    smp.copy_(torch.from_numpy(junk_s))
    tok[:B].copy_(torch.from_numpy(t))
    tok[B:].copy_(torch.from_numpy(rng.integers(0, 32000, size=(MAXB - B, S)).astype(np.int32)))
    draft.fill_(SENTINEL)
    nv.fill_(SENTINEL)
    return n, t, s, junk_n, junk_s


def _bucket(B):
    return next((b for b in BUCKETS if b >= B), None)


def _check_call(d, lc, bufs, B, inputs, replayed=True):
    import torch

    nt, tok, smp, draft, nv = bufs
    n, t, s, junk_n, junk_s = inputs
    torch.cuda.synchronize()
    got_d, got_n = draft.cpu().numpy(), nv.cpu().numpy()
    eager_d, eager_n = d.propose(torch.from_numpy(n).cuda(), torch.from_numpy(t).cuda(),
                                 torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got_d[:B], eager_d.cpu().numpy()), f"B={B}: draft vs eager"
    assert np.array_equal(got_n[:B], eager_n.cpu().numpy()), f"B={B}: num_valid vs eager"
    exp_d, exp_n = O.propose(O.params_from(KNOBS), n, t, s, corpus=lc.text(), num_threads=8)
    assert np.array_equal(got_d[:B], exp_d) and np.array_equal(got_n[:B], exp_n), \
        f"B={B}: drafts vs oracle"
    # a replay runs the bucket with its rows past B emptied; an eager call runs B rows
    bp = (_bucket(B) or B) if replayed else B
    # emptied rows of the bucket: no prefix, no sampled id, nothing proposed
    assert (nt.cpu().numpy()[B:bp] == 0).all() and (smp.cpu().numpy()[B:bp] == -1).all()
    assert (got_d[B:bp] == -1).all() and (got_n[B:bp] == 0).all()
    # rows past the bucket untouched
    assert (nt.cpu().numpy()[bp:] == junk_n[bp:]).all()
    assert (smp.cpu().numpy()[bp:] == junk_s[bp:]).all()
    assert (got_d[bp:] == SENTINEL).all() and (got_n[bp:] == SENTINEL).all()


@pytest.mark.parametrize("delta_index", [False, True])
def test_bucketed_graphs_follow_batch_and_corpus(delta_index):
    import suffix_match_drafter_amd as sfx

    d, lc, docs = _drafter()
    bufs = _buffers()
    flags = sfx.GRAPHS_DELTA_INDEX if delta_index else 0
    gs = d.graphs(BUCKETS, *bufs, flags=flags)
    st = gs.stats()
    assert st["buckets"] == 3 and st["exact_mask"] == 0b111 and st["padded_mask"] == 0b111
    rng = np.random.default_rng(11)
    seq = [8, 5, 16, 13, 1, 32, 20, 50, 3, 32, 64, 9]
    for step, B in enumerate(seq):
        if step % 3 == 1:  # documents past the live index: the next calls find them in the delta
            new = docs[150 + 20 * step: 170 + 20 * step]
            d.ingest_docs(new)
            lc.ingest(new)
        if step % 4 == 3:
            d.rebuild()
        inputs = _fill(bufs, B, step, rng)
        gs.propose(B)
        _check_call(d, lc, bufs, B, inputs)
    st = gs.stats()
    big = sum(1 for B in seq if B > BUCKETS[-1])
    assert st["replays"] == len(seq) - big and st["eager_calls"] == big
    gs.close()
    d.close()


@pytest.mark.parametrize("mode", ["eager", "break_odd"])
def test_bucketed_graphs_fallback(mode):
    import suffix_match_drafter_amd as sfx

    d, lc, _ = _drafter()
    bufs = _buffers()
    flags = sfx.GRAPHS_EAGER if mode == "eager" else sfx.GRAPHS_DEBUG_BREAK_ODD
    gs = d.graphs(BUCKETS, *bufs, flags=flags)
    st = gs.stats()
    want = 0 if mode == "eager" else 0b101
    assert st["exact_mask"] == want and st["padded_mask"] == want
    rng = np.random.default_rng(5)
    seq = [8, 12, 16, 30, 2]
    for step, B in enumerate(seq):
        inputs = _fill(bufs, B, 20 + step, rng)
        gs.propose(B)
        _check_call(d, lc, bufs, B, inputs, replayed=mode != "eager" and not 8 < B <= 16)
    st = gs.stats()
    eager = len(seq) if mode == "eager" else sum(1 for B in seq if 8 < B <= 16)
    assert st["eager_calls"] == eager and st["replays"] == len(seq) - eager
    gs.close()
    d.close()


def test_bucketed_graphs_with_state_update():
    import torch

    import suffix_match_drafter_amd as sfx

    d, lc, _ = _drafter()
    bufs = _buffers()
    nt, tok, smp, draft, nv = bufs
    nout = torch.full((MAXB,), SENTINEL, dtype=torch.int32, device="cuda")
    gs = d.graphs(BUCKETS, *bufs, num_tokens_out=nout, flags=sfx.GRAPHS_UPDATE_STATE)
    rng = np.random.default_rng(3)
    for step, B in enumerate([16, 11, 40]):
        inputs = _fill(bufs, B, 40 + step, rng)
        n, t, s, junk_n, junk_s = inputs
        tok_before = tok.clone()
        nout.fill_(SENTINEL)
        gs.propose(B)
        torch.cuda.synchronize()
        # the step itself as an eager call on copies of the first B rows
        tcopy = torch.from_numpy(t).cuda()
        exp_n = sfx.update_state(tcopy, torch.from_numpy(n).cuda(), torch.from_numpy(s).cuda())
        torch.cuda.synchronize()
        bp = next((b for b in BUCKETS if b >= B), B)
        assert torch.equal(tok[:B], tcopy), f"B={B}: written-back rows"
        assert torch.equal(nout[:B], exp_n), f"B={B}: new lengths"
        assert torch.equal(tok[B:], tok_before[B:]), f"B={B}: rows past B changed"
        assert (nout[B:bp].cpu().numpy() == 0).all()
        assert (nout[bp:].cpu().numpy() == SENTINEL).all()
        # drafts are those of the step before the write-back
        got_d = draft.cpu().numpy()[:B]
        exp_d, _ = O.propose(O.params_from(KNOBS), n, t, s, corpus=lc.text(), num_threads=8)
        assert np.array_equal(got_d, exp_d), f"B={B}: drafts vs oracle"
    gs.close()
    d.close()
