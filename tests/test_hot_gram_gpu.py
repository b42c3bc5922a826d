"""GPU parity on corpora whose request tails end in a hot 4-gram (suffix-gpu page, How it works
step 2: the tail is searched in the shared corpus's suffix array, every pattern length at once).

Above 1024 live occurrences of the tail's 4-gram, the library takes the supports of lengths
>= 5 from bound searches of the suffix array and the earliest sites from the smallest
positions of a range (or, for a range above 2048 entries, from the position-ordered scan).
These tests put tails on both sides of both thresholds: the boilerplate workload (a 4-gram
over 10^5 times in a 1M-token corpus), and a small corpus where the token before the 4-gram
makes supports of about 3000, 500 and 1100; with and without a delta (the general path), in
both modes, on both context paths.  Drafts must equal the oracle's bit for bit."""
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

NTHREADS = min(16, len(os.sched_getaffinity(0)))
FLAGS = [0, 1]  # staged context, streamed context


def _run(knobs, n, tok, samp, docs, delta_docs=(), flags=0, cap=1 << 21):
    import torch

    import suffix_match_drafter_amd as sfx

    B, S = tok.shape
    d = sfx.Drafter(sfx.Config(max_batch=B, max_seq=S, max_sampled=samp.shape[1],
                               corpus_capacity=cap, flags=flags, **knobs))
    d.ingest_docs(docs)
    d.rebuild()
    if delta_docs:
        d.ingest_docs(list(delta_docs))
    draft, nv = d.propose(*(torch.from_numpy(np.ascontiguousarray(x)).cuda()
                            for x in (n, tok, samp)))
    torch.cuda.synchronize()
    out = draft.cpu().numpy(), nv.cpu().numpy()
    d.close()
    return out


def _check(knobs, n, tok, samp, docs, delta_docs=(), flags=0):
    got = _run(knobs, n, tok, samp, docs, delta_docs, flags)
    corpus = W.join_docs(list(docs) + list(delta_docs))
    exp = O.propose(O.params_from(knobs), n, tok, samp, corpus=corpus, num_threads=NTHREADS)
    bad = np.nonzero((got[0] != exp[0]).any(axis=1) | (got[1] != exp[1]))[0]
    assert bad.size == 0, (f"{bad.size} rows differ; row {bad[0]}: gpu {got[0][bad[0]].tolist()}"
                           f"/{got[1][bad[0]]} oracle {exp[0][bad[0]].tolist()}/{exp[1][bad[0]]}")
    return exp


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("delta", [False, True])
def test_boilerplate_workload(flags, delta):
    w = W.WORKLOADS[6]
    docs = W.corpus_docs(6)
    n, tok, samp = W.make_batch(6, set_index=2, B=32)
    base, extra = (docs[:1600], docs[1600:]) if delta else (docs, [])
    exp = _check(w.knobs(), n, tok, samp, base, extra, flags)
    assert (exp[1] > 0).all()


def _small_corpus(rng, H, segs, weights):
    """Documents of segments: 0..2 noise tokens, a token drawn by `weights`, then H."""
    toks = np.array(list(weights.keys()), np.int32)
    p = np.array(list(weights.values()), np.float64)
    p /= p.sum()
    docs, cur = [], []
    for _ in range(segs):
        cur += list(rng.integers(100, 400, size=int(rng.integers(0, 3))))
        cur.append(int(rng.choice(toks, p=p)))
        cur += H
        if len(cur) > 200:
            docs.append(np.array(cur, np.int32))
            cur = []
    if cur:
        docs.append(np.array(cur, np.int32))
    return docs


def _rows(rng, B, S, H, before):
    """Rows of noise ending in `before[b]` tokens then H; some rows repeat a corpus stretch."""
    n = np.full(B, S - 1, np.int32)
    tok = rng.integers(100, 400, size=(B, S)).astype(np.int32)
    samp = np.zeros((B, 1), np.int32)
    for b in range(B):
        ctx = list(tok[b, : S - len(before[b]) - len(H)]) + list(before[b]) + H
        tok[b, : S - 1] = ctx[: S - 1]
        samp[b, 0] = ctx[S - 1]
    return n, tok, samp


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("delta", [False, True])
def test_supports_around_thresholds(flags, mode, delta):
    rng = np.random.default_rng(41)
    H = [11, 12, 13, 14]
    # support of "7 H" about 3000 (scan), of "9 H" about 500 (selection); H over 1024 in all
    docs = _small_corpus(rng, H, 5000, {7: 0.6, 9: 0.1, 20: 0.1, 21: 0.1, 22: 0.1})
    B, S = 24, 256
    before = []
    for b in range(B):
        x = [7, 9, 20][b % 3]
        before.append([int(rng.integers(100, 400)), x] if b % 2 else [x])
    n, tok, samp = _rows(rng, B, S, H, before)
    # a few rows end in a long stretch of a document, so long matches exist too
    for b in range(0, B, 5):
        d = docs[b % len(docs)]
        tail = list(d[-60:]) if len(d) >= 60 else list(d)
        ctx = list(tok[b, : S - 1]) + [int(samp[b, 0])]
        ctx = (ctx + tail)[-S:]
        tok[b, : S - 1] = ctx[: S - 1]
        samp[b, 0] = ctx[-1]
    if mode == 0:
        knobs = dict(k=8, max_tree_depth=24, num_backoff=1, max_occurrences=128, mode=0)
    else:
        knobs = dict(k=16, max_tree_depth=24, num_backoff=4, max_occurrences=128, mode=1,
                     spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
    base, extra = (docs[:-20], docs[-20:]) if delta else (docs, [])
    _check(knobs, n, tok, samp, base, extra, flags)


@pytest.mark.parametrize("segs", [1000, 1100, 1200])
def test_group_size_near_switch(segs):
    """The tail's 4-gram just below and just above 1024 live occurrences."""
    rng = np.random.default_rng(segs)
    H = [31, 32, 33, 34]
    docs = _small_corpus(rng, H, segs, {5: 0.5, 6: 0.3, 7: 0.2})
    B, S = 12, 128
    before = [[int(rng.integers(100, 400)), [5, 6, 7][b % 3]] for b in range(B)]
    n, tok, samp = _rows(rng, B, S, H, before)
    knobs = dict(k=16, max_tree_depth=24, num_backoff=4, max_occurrences=128, mode=1,
                 spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
    _check(knobs, n, tok, samp, docs)
