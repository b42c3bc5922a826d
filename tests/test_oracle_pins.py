"""Pins of the CPU oracle against facts fixed outside it (CPU only).

* hand-worked examples in tests/golden/worked_examples.json;
* brute force on tiny inputs (tests/bruteforce.py: substring enumeration, continuation trie,
  Python-ordered suffixes);
* closed forms (periodic rows, all-distinct rows, a corpus holding the tail once);
* a cross-path invariant: corpus matching against the one-document corpus [ctx, -1] equals
  self matching for lengths >= 2, computed by two independent oracle routines.
"""
import json
import os

import numpy as np
import pytest

from tests import bruteforce as bf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def knobs(k, D=24, nb=1, M=128, mode=0, factor=1_000_000, prob=100_000, offset=0, tree=0):
    return dict(k=k, max_tree_depth=D, num_backoff=nb, max_occurrences=M, mode=mode,
                spec_factor_ppm=factor, spec_offset_ppm=offset, min_token_prob_ppm=prob,
                min_self_match=1, min_corpus_match=2, tree_depth_cap=tree)


# ------------------------------------------------------------------ hand-worked golden cases
@pytest.mark.parametrize("case", GOLD["local"], ids=lambda c: c["name"])
def test_golden_local(orc, case):
    ctx, t = orc.context(case["row"], case["n"], case["sampled"])
    assert t == len(case["sampled"])
    mb = orc.match_back(ctx, case["D"])
    assert mb.tolist() == case["mb"]
    for i, (l, sup, sites) in enumerate(zip(case["ladder"], case["support"], case["sites"])):
        assert orc.kth_largest(mb, i + 1) == l
        assert orc.count_at_least(mb, l) == sup
        assert orc.first_sites(mb, l, 128).tolist() == sites
    row = np.array(case["row"], np.int32)[None]
    samp = np.array(case["sampled"], np.int32)[None]
    n = np.array([case["n"]], np.int32)
    for key, exp in case.items():
        if key.startswith("expand_l"):
            l = int(key.split("_")[1][1:])
            k = int(key.split("_k")[1])
            sites = case["sites"][case["ladder"].index(l)]
            toks, counts, snum = orc.expand(ctx, sites, k)
            assert toks.tolist() == exp["tokens"] and counts.tolist() == exp["counts"]
            assert snum == exp["snum"]
        if key.startswith("longest_fill_k"):
            p = orc.make_params(int(key.split("_k")[1]), max_tree_depth=case["D"])
            d, nv = orc.propose(p, n, row, samp)
            assert d[0].tolist() == exp["draft"] and nv[0] == exp["num_valid"]
        if key.startswith("scored_"):
            parts = key.split("_")
            nb = int(parts[1][2:]) if parts[1].startswith("nb") else 1
            kk = int([x for x in parts if x.startswith("k")][0][1:])
            factor = int([x for x in parts if x.startswith("factor")][0][6:]) * 1_000_000
            prob = int([x for x in parts if x.startswith("prob")][0][4:])
            p = orc.make_params(kk, max_tree_depth=case["D"], num_backoff=nb, mode=1,
                                spec_factor_ppm=factor, min_token_prob_ppm=prob)
            d, nv, info = orc.propose(p, n, row, samp, with_info=True)
            assert d[0].tolist() == exp["draft"] and nv[0] == exp["num_valid"]
            if "snum" in exp:
                assert info[0].snum == exp["snum"] and info[0].c0 == exp["c0"]


@pytest.mark.parametrize("case", GOLD["global"], ids=lambda c: c["name"])
def test_golden_global(orc, case):
    C = np.array(case["text"], np.int32)
    lc = orc.LiveCorpus(10**6)
    lc.ingest(case["docs"])
    assert lc.text().tolist() == case["text"]
    ctx, _ = orc.context(case["row"], case["n"], case["sampled"])
    m = orc.corpus_match(C, ctx, case["D"])
    assert m.tolist() == case["corpus_m"]
    for i, (l, sup, sites) in enumerate(zip(case["ladder"], case["support"], case["sites"])):
        assert orc.kth_largest(m, i + 1) == l
        assert orc.count_at_least(m, l) == sup
        assert orc.first_sites(m, l, 128).tolist() == sites
    toks, counts, snum = orc.expand(C, case["sites"][0], 8)
    assert toks.tolist() == case["expand"]["tokens"]
    assert counts.tolist() == case["expand"]["counts"] and snum == case["expand"]["snum"]
    p = orc.make_params(4, max_tree_depth=case["D"])
    d, nv = orc.propose(p, np.array([case["n"]]), np.array([case["row"]]),
                        np.array([case["sampled"]]), corpus=C)
    assert d[0].tolist() == case["longest_fill_k4"]["draft"]
    assert nv[0] == case["longest_fill_k4"]["num_valid"]


@pytest.mark.parametrize("case", GOLD["selection"], ids=lambda c: c["name"])
def test_golden_selection(orc, case):
    lc = orc.LiveCorpus(10**6)
    lc.ingest([np.array(x, np.int32) for x in case["docs"]])
    C = lc.text()
    p = orc.make_params(**case["knobs"])
    d, nv = orc.propose(p, np.array([case["n"]]), np.array([case["row"]], np.int32),
                        np.array([case["sampled"]], np.int32), corpus=C if len(C) else None)
    assert d[0].tolist() == case["expect"]["draft"]
    assert nv[0] == case["expect"]["num_valid"]


@pytest.mark.parametrize("case", GOLD["suffix_array"], ids=lambda c: str(c["text"]))
def test_golden_suffix_array(orc, case):
    assert orc.suffix_array(case["text"]).tolist() == case["sa"]


# ------------------------------------------------------------------ brute force, tiny inputs
def _rand_ctx(rng, V, L):
    return rng.integers(0, V, size=L).astype(np.int32)


def test_match_back_and_ladder_bruteforce(orc):
    rng = np.random.default_rng(11)
    for it in range(400):
        V = int(rng.choice([2, 3, 4, 16]))
        L = int(rng.integers(1, 48))
        D = int(rng.choice([1, 2, 3, 5, 8, 24]))
        ctx = _rand_ctx(rng, V, L)
        mb = orc.match_back(ctx, D)
        assert mb.tolist() == bf.local_mb(ctx.tolist(), D), (it, ctx, D)
        for t in range(1, 6):
            l = bf.ladder(lambda x: len(bf.local_occ_ends(ctx.tolist(), x)), min(D, L - 1), t)
            assert orc.kth_largest(mb, t) == l, (it, t)
            if l >= 1:
                ends = bf.local_occ_ends(ctx.tolist(), l)
                assert orc.count_at_least(mb, l) == len(ends)
                M = int(rng.integers(1, 6))
                assert orc.first_sites(mb, l, M).tolist() == [j + 1 for j in ends][:M]


def _rand_corpus(rng, V, ndocs, lo, hi):
    docs = [rng.integers(0, V, size=int(rng.integers(lo, hi + 1))).astype(np.int32)
            for _ in range(ndocs)]
    lc = __import__("oracle").LiveCorpus(10**9)
    lc.ingest(docs)
    return lc.text()


def test_corpus_match_bruteforce(orc):
    rng = np.random.default_rng(12)
    for it in range(300):
        V = int(rng.choice([2, 3, 5]))
        C = _rand_corpus(rng, V, int(rng.integers(0, 6)), 0, 12)
        L = int(rng.integers(1, 10))
        D = int(rng.choice([2, 3, 4, 6, 24]))
        ctx = _rand_ctx(rng, V, L)
        if it % 3 == 0:  # a -1 inside the context never matches a document separator
            ctx = rng.integers(-1, V, size=L).astype(np.int32)
        m = orc.corpus_match(C, ctx, D)
        for t in range(1, 5):
            l = bf.ladder(lambda x: len(bf.corpus_occ_starts(C.tolist(), ctx.tolist(), x)),
                          min(D, L), t)
            assert orc.kth_largest(m, t) == l, (it, C, ctx, D, t)
            if l >= 1:
                starts = bf.corpus_occ_starts(C.tolist(), ctx.tolist(), l)
                assert orc.count_at_least(m, l) == len(starts)
                assert orc.first_sites(m, l, 3).tolist() == sorted(i + l for i in starts)[:3]


def test_expand_matches_trie(orc):
    rng = np.random.default_rng(13)
    for it in range(400):
        V = int(rng.choice([2, 3, 4]))
        X = rng.integers(-1, V, size=int(rng.integers(1, 40))).astype(np.int32)
        nsites = int(rng.integers(1, 8))
        sites = np.sort(rng.choice(len(X), size=min(nsites, len(X)), replace=False))
        cap = int(rng.integers(0, 10))
        scored = bool(rng.integers(0, 2))
        prob = int(rng.choice([0, 100_000, 300_000, 500_000, 1_000_000]))
        toks, counts, snum = orc.expand(X, sites, cap, scored, prob)
        bt, bc, bs = bf.trie_expand(X.tolist(), sites.tolist(), cap, scored, prob)
        assert toks.tolist() == bt and counts.tolist() == bc and snum == bs, (it, X, sites)


def test_cross_path_one_document_corpus(orc):
    """Corpus matching against [ctx, -1] and self matching share no code in the oracle but
    must find the same occurrences for every length >= 2."""
    rng = np.random.default_rng(14)
    for it in range(300):
        V = int(rng.choice([2, 3, 4]))
        L = int(rng.integers(2, 40))
        D = int(rng.choice([2, 3, 6, 24]))
        ctx = _rand_ctx(rng, V, L)
        C = np.concatenate([ctx, [-1]]).astype(np.int32)
        mb = orc.match_back(ctx, D)
        m = orc.corpus_match(C, ctx, D)
        # corpus end e = local end j; the local cap is min(D, j+1), the corpus one min(D, L)
        # and e+1, which agree on every end j <= L-2.
        assert np.array_equal(np.minimum(m[: L - 1], D), mb), (it, ctx)
        for t in range(1, 4):
            lt, gt = orc.kth_largest(mb, t), orc.kth_largest(m, t)
            if lt >= 2 or gt >= 2:
                assert lt == gt
                assert (orc.first_sites(mb, lt, 5).tolist()
                        == orc.first_sites(m, gt, 5).tolist())


@pytest.mark.parametrize("mode", [0, 1])
def test_propose_bruteforce(orc, mode):
    rng = np.random.default_rng(15 + mode)
    for it in range(150):
        V = int(rng.choice([2, 3, 4, 6]))
        B = 3
        S = int(rng.integers(1, 30))
        T = int(rng.integers(0, 3))
        k = int(rng.integers(1, 7))
        nb = 1 if mode == 0 else int(rng.integers(1, 5))
        M = int(rng.choice([1, 2, 3, 128]))
        D = int(rng.choice([2, 3, 5, 24]))
        kn = knobs(k, D=D, nb=nb, M=M, mode=mode,
                   factor=int(rng.choice([500_000, 1_000_000, 2_000_000])),
                   prob=int(rng.choice([0, 100_000, 400_000])),
                   offset=int(rng.choice([0, 1_000_000])), tree=int(rng.integers(0, 2)))
        tok = rng.integers(0, V, size=(B, S)).astype(np.int32)
        n = rng.integers(-2, S + 3, size=B).astype(np.int32)
        samp = rng.integers(-1, V, size=(B, T)).astype(np.int32)
        C = _rand_corpus(rng, V, int(rng.integers(0, 5)), 0, 10) if rng.integers(0, 2) else None
        d, nv = orc.propose(orc.params_from(kn), n, tok, samp, corpus=C)
        for b in range(B):
            ed, en = bf.propose_row(kn, tok[b].tolist(), n[b], samp[b].tolist(),
                                    None if C is None else C.tolist())
            assert d[b].tolist() == ed and nv[b] == en, (it, b, kn, tok[b], n[b], samp[b], C)


def test_suffix_array_bruteforce(orc):
    rng = np.random.default_rng(16)
    for it in range(200):
        V = int(rng.choice([1, 2, 3, 5]))
        n = int(rng.integers(0, 200))
        text = rng.integers(-1, V, size=n).astype(np.int32)
        assert orc.suffix_array(text).tolist() == bf.suffix_array(text.tolist())


# ------------------------------------------------------------------ closed forms
@pytest.mark.parametrize("p,r,D", [(3, 5, 24), (4, 6, 5), (5, 3, 24), (2, 20, 7), (7, 4, 3)])
def test_periodic_row_closed_form(orc, p, r, D):
    """Row (0..p-1)^r: an earlier copy of the tail ends every p tokens.  l1 = min(D, L-p); the
    sites with that length are ends j = L-1-m*p (m >= 1, j >= l1-1); from site L-m*p the
    continuation is 0,1,2,... for m*p tokens, so c_d = c0 - floor(d/p) and token d = d mod p."""
    ctx = np.tile(np.arange(p, dtype=np.int32), r)
    L = len(ctx)
    l1 = min(D, L - p)
    mb = orc.match_back(ctx, D)
    assert orc.kth_largest(mb, 1) == l1
    ms = [m for m in range(1, r) if L - 1 - m * p >= l1 - 1]
    assert orc.count_at_least(mb, l1) == len(ms)
    sites = orc.first_sites(mb, l1, 128)
    assert sites.tolist() == sorted(L - m * p for m in ms)
    k = 3 * p + 2
    toks, counts, snum = orc.expand(ctx, sites, k)
    c0 = len(ms)
    nexp = min(k, c0 * p)
    assert toks.tolist() == [d % p for d in range(nexp)]
    assert counts.tolist() == [c0 - d // p for d in range(nexp)]
    assert snum == sum(c0 - d // p for d in range(nexp))
    # whole call, longest-match mode: the draft continues the period, the rest is the fill
    row = ctx[:-1][None]
    d, nv = orc.propose(orc.make_params(k, max_tree_depth=D), np.array([L - 1]), row,
                        ctx[-1:][None])
    assert nv[0] == nexp and d[0, :nexp].tolist() == [x % p for x in range(nexp)]
    assert (d[0, nexp:] == ctx[-1]).all()
    # scored mode: cap = floor(factor * l1); stop when c_d / c0 < 0.5
    pr = orc.make_params(k, max_tree_depth=D, mode=1, spec_factor_ppm=1_000_000,
                         min_token_prob_ppm=500_000)
    d, nv, info = orc.propose(pr, np.array([L - 1]), row, ctx[-1:][None], with_info=True)
    n2 = 0
    while n2 < min(k, l1, c0 * p) and (c0 - n2 // p) * 2 >= c0:
        n2 += 1
    assert nv[0] == n2 and info[0].snum == sum(c0 - x // p for x in range(n2))
    assert (d[0, n2:] == -1).all()


def test_all_distinct_row(orc):
    for L in (1, 2, 17, 300):
        ctx = np.arange(L, dtype=np.int32) + 5
        for mode in (0, 1):
            d, nv = orc.propose(orc.make_params(6, mode=mode, num_backoff=1 + 2 * mode),
                                np.array([L - 1]), ctx[:-1][None] if L > 1 else
                                np.zeros((1, 1), np.int32), ctx[-1:][None])
            assert nv[0] == 0
            assert (d[0] == (ctx[-1] if mode == 0 else -1)).all()


def test_unique_corpus_occurrence(orc):
    """A corpus that holds the tail exactly once: the draft is that document's continuation,
    every chain probability is 1 (c_d = 1) and the draft stops at the document's end."""
    rng = np.random.default_rng(17)
    for it in range(50):
        tail = rng.choice(np.arange(100, 200), size=int(rng.integers(2, 8)),
                          replace=False).astype(np.int32)
        cont = rng.integers(300, 400, size=int(rng.integers(1, 12))).astype(np.int32)
        docs = [rng.integers(500, 600, size=10).astype(np.int32),
                np.concatenate([rng.integers(700, 800, size=3), tail, cont]).astype(np.int32)]
        lc = orc.LiveCorpus(10**6)
        lc.ingest(docs)
        C = lc.text()
        row = np.concatenate([rng.integers(900, 1000, size=5), tail[:-1]]).astype(np.int32)
        k = 8
        for mode in (0, 1):
            p = orc.make_params(k, mode=mode, num_backoff=1 + mode, spec_factor_ppm=10**8,
                                min_token_prob_ppm=10**6)
            d, nv, info = orc.propose(p, np.array([len(row)]), row[None], tail[-1:][None],
                                      corpus=C, with_info=True)
            n = min(k, len(cont))
            assert nv[0] == n and d[0, :n].tolist() == cont[:n].tolist()
            assert info[0].snum == n and info[0].c0 == 1
            assert info[0].chosen_len == len(tail)


# ------------------------------------------------------------------ state update, corpus model
def test_update_state(orc):
    rng = np.random.default_rng(18)
    for it in range(100):
        B, S, T = 4, int(rng.integers(1, 12)), int(rng.integers(0, 4))
        tok = rng.integers(0, 9, size=(B, S)).astype(np.int32)
        n = rng.integers(-2, S + 2, size=B).astype(np.int32)
        samp = rng.integers(-1, 9, size=(B, T)).astype(np.int32)
        new, nn = orc.update_state(tok, n, samp)
        for b in range(B):
            nb_ = max(0, min(int(n[b]), S))
            t = 0
            while t < T and samp[b, t] >= 0:
                t += 1
            w = min(t, S - nb_)
            assert nn[b] == nb_ + w
            assert new[b, nb_:nb_ + w].tolist() == samp[b, :w].tolist()
            assert new[b, :nb_].tolist() == tok[b, :nb_].tolist()
            assert new[b, nb_ + w:].tolist() == tok[b, nb_ + w:].tolist()


def test_live_corpus_eviction(orc):
    rng = np.random.default_rng(19)
    for it in range(100):
        cap = int(rng.integers(0, 60))
        lc = orc.LiveCorpus(cap)
        hist = []
        for step in range(int(rng.integers(1, 6))):
            docs = [rng.integers(0, 9, size=int(rng.integers(0, 15))).astype(np.int32)
                    for _ in range(int(rng.integers(0, 4)))]
            lc.ingest(docs)
            hist += [d.tolist() for d in docs]
            # the live set is the longest run of most recent documents that fits
            tot, live = 0, []
            for d in reversed(hist):
                if tot + len(d) + 1 > cap:
                    break
                tot += len(d) + 1
                live.insert(0, d)
            exp = [x for d in live for x in d + [-1]]
            assert lc.text().tolist() == exp
            assert len(exp) <= cap


def test_inflight_ingest_hand_example(orc):
    """In-flight ingest (RFC page, Design: in-flight responses ingested, finished ones
    final-flushed), worked by hand from the rule: chunks past the cursor of at least min_chunk
    tokens, a final flush takes any remainder and resets the cursor, a shorter length restarts
    the row, a repeated row counts at its first entry, unknown rows are ignored."""
    tok = np.array([[10, 11, 12, 13, 14, 15], [20, 21, 22, 23, 24, 25],
                    [30, 31, 32, 33, 34, 35]], np.int32)
    m = orc.InflightIngest(max_rows=3)
    calls = [  # (rows, lengths, final, min_chunk) -> documents
        (([0], [1], None, 2), []),
        (([0], [3], None, 2), [[10, 11, 12]]),
        (([0], [4], None, 2), []),
        (([0], [5], [1], 2), [[13, 14]]),
        (([0], [2], None, 2), [[10, 11]]),
        (([0], [1], None, 2), []),             # shorter than the cursor: restart, 1 < 2
        (([1, 1, 2], [3, 5, 2], None, 1), [[20, 21, 22], [30, 31]]),
        (([1], [6], None, 4), []),             # 3 tokens past the cursor, below min_chunk
        (([1, 4, -1, 2], [6, 6, 6, 2], [1, 1, 1, 1], 4), [[23, 24, 25]]),  # row 2: nothing left
        (([2], [3], [1], 9), [[30, 31, 32]]),  # row 2's cursor was reset by the empty flush
        (([0, 1], [6, 2], None, 2), [[10, 11, 12, 13, 14, 15], [20, 21]]),
    ]
    for i, ((rows, lens, fin, mc), exp) in enumerate(calls):
        got = m.docs(tok, rows, lens, final=fin, min_chunk=mc)
        assert [d.tolist() for d in got] == exp, f"call {i}"
    assert m.cursor == [6, 2, 0]


def test_inflight_ingest_invariants(orc):
    """Random decode traces: with min_chunk 1 and a flush at every request's end, each request's
    chunks concatenate to its whole response; with any min_chunk only a final flush may append
    fewer than min_chunk tokens."""
    rng = np.random.default_rng(23)
    for it in range(60):
        B, S = int(rng.integers(1, 6)), 64
        mc = int(rng.integers(0, 6))
        m = orc.InflightIngest(max_rows=B)
        tok = np.zeros((B, S), np.int32)
        n = np.zeros(B, np.int64)
        got = {b: [] for b in range(B)}   # chunks of the current request of each row
        done = []                         # (response, chunks) of finished requests
        for step in range(30):
            fin = np.zeros(B, np.int32)
            for b in range(B):
                grow = int(rng.integers(0, 5))
                tok[b, n[b]:n[b] + grow] = rng.integers(0, 1000, size=min(grow, S - n[b]))
                n[b] = min(S, n[b] + grow)
                fin[b] = int(rng.random() < 0.15 or n[b] == S)
            order = rng.permutation(B)
            docs = m.docs(tok, order, n[order], final=fin[order], min_chunk=mc)
            k = 0
            for b in order:  # attribute the documents back to rows (entry order)
                before = sum(len(c) for c in got[b])
                if k < len(docs) and before < n[b] and \
                        docs[k].tolist() == tok[b, before:before + len(docs[k])].tolist() and \
                        (len(docs[k]) >= max(mc, 1) or fin[b]):
                    got[b].append(docs[k])
                    k += 1
                if fin[b]:
                    done.append((tok[b, :n[b]].copy(), got[b]))
                    got[b], n[b] = [], 0
            assert k == len(docs)
        for resp, chunks in done:
            cat = np.concatenate(chunks) if chunks else np.zeros(0, np.int32)
            assert cat.tolist() == resp.tolist()
            assert all(len(c) >= max(mc, 1) for c in chunks[:-1])


def test_accept_model_hand_values(orc):
    """Acceptance estimate (vLLM docs, adaptive verification): values worked by hand from
    Laplace's rule, (accepted + 1) / (proposed + 2) in ppm, with prefix acceptance."""
    m = orc.AcceptModel()
    m.record([(1, 5, 3), None, (0, 5, 2)])
    assert m.estimate(3, 4).tolist() == [[500000, 500000, 500000, 0], [0] * 4,
                                         [500000, 500000, 0, 0]]
    m.feedback([2, 7, 0])   # row 0 accepts slots 0 and 1 of 3; row 1 has no draft; row 2 none
    assert m.counts[1, 5, :3].tolist() == [[1, 1], [1, 1], [1, 0]]
    assert m.counts[0, 5, :2].tolist() == [[1, 0], [1, 0]]
    m.feedback([3, 3, 3])   # consumed: nothing more is counted
    assert int(m.counts.sum()) == 3 + 2 + 2
    m.record([(1, 5, 3)])
    # slot 0: 2/3 -> 666666; slot 2: 1/3 -> 333333
    assert m.estimate(1, 3).tolist() == [[666666, 666666, 333333]]
    for _ in range(8):      # eight more fully accepted drafts: (9 + 1) / (9 + 2)
        m.record([(1, 5, 1)])
        m.feedback([1])
    m.record([(1, 5, 1)])
    assert m.estimate(1, 2).tolist() == [[10 * 1000000 // 11, 0]]


def test_masked_form_matches_updated_state(orc):
    """The masked form (PyPI page, Quickstart: propose(num_tokens_no_spec, token_ids,
    combined_mask)) after the state update equals the ordinary step on the state before it: the
    update writes the sampled id at n, and the masked call reads it back as the context's last
    token.  Rows with mask 0, and empty rows, get no draft."""
    rng = np.random.default_rng(29)
    for mode, nb in ((0, 1), (1, 3)):
        kn = dict(k=6, max_tree_depth=8, num_backoff=nb, max_occurrences=16, mode=mode,
                  spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
        p = orc.params_from(kn)
        B, S, V = 12, 80, 4
        tok = rng.integers(0, V, size=(B, S)).astype(np.int32)
        n = rng.integers(0, S, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, 1)).astype(np.int32)
        corpus = orc.LiveCorpus(1000)
        corpus.ingest([rng.integers(0, V, size=30).astype(np.int32) for _ in range(5)])
        exp_d, exp_n = orc.propose(p, n, tok, samp, corpus=corpus.text())
        tok2, n2 = orc.update_state(tok, n, samp)
        mask = np.ones(B, np.int32)
        got_d, got_n = orc.propose_masked(p, n2, tok2, mask, corpus=corpus.text())
        assert np.array_equal(got_d, exp_d) and np.array_equal(got_n, exp_n)
        mask[::3] = 0
        got_d, got_n = orc.propose_masked(p, n2, tok2, mask, corpus=corpus.text())
        assert (got_d[::3] == -1).all() and (got_n[::3] == 0).all()
        keep = mask != 0
        assert np.array_equal(got_d[keep], exp_d[keep]) and np.array_equal(got_n[keep], exp_n[keep])
        empty = orc.propose_masked(p, np.zeros(B, np.int32), tok2, np.ones(B, np.int32))
        assert (empty[0] == -1).all() and (empty[1] == 0).all()


def test_counted_form(orc):
    """The counted form (RFC page, Design: propose(k, num_tokens_no_spec, token_ids, sampled,
    counts)): counts equal to the padding's own count reproduce the ordinary step; entries past
    counts are ignored; in LONGEST_FILL mode (no score, no cap but k) a narrower k gives the
    first k tokens of the wider draft."""
    rng = np.random.default_rng(31)
    B, S, T, V = 10, 60, 3, 4
    tok = rng.integers(0, V, size=(B, S)).astype(np.int32)
    n = rng.integers(0, S + 1, size=B).astype(np.int32)
    samp = rng.integers(0, V, size=(B, T)).astype(np.int32)
    lead = rng.integers(0, T + 1, size=B)
    for b in range(B):
        samp[b, lead[b]:] = -1
    for mode, nb in ((0, 1), (1, 3)):
        kn = dict(k=8, max_tree_depth=8, num_backoff=nb, max_occurrences=16, mode=mode,
                  spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
        p = orc.params_from(kn)
        exp = orc.propose(p, n, tok, samp)
        got = orc.propose_counts(p, 8, n, tok, samp, lead)
        assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1])
        junk = samp.copy()
        junk[junk < 0] = 3  # entries past counts are never read
        got = orc.propose_counts(p, 8, n, tok, junk, lead)
        assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1])
        if mode == 0:
            for k in (1, 3, 5):
                d, nv = orc.propose_counts(p, k, n, tok, samp, lead)
                assert np.array_equal(d, exp[0][:, :k])
                assert np.array_equal(nv, np.minimum(exp[1], k))


def test_tree_depth_cap(orc):
    """Tree-depth cap (gitcode blog, section 4, parameter table: max_tree_depth bounds the match
    length plus the draft length).  Hand case: the tail "1 2 3" matches at the row start (length
    3, D = 6), whose continuation 4 5 6 7 8 1 2 3 would fill k = 8 slots; with the cap only
    D - 3 = 3 tokens remain.  On random rows in LONGEST_FILL mode the winner does not depend on
    the cap (it is chosen by length), so the capped draft is the uncapped one cut to D - l tokens
    and filled; in both modes no draft exceeds D - l for its winner's length l."""
    row = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 1, 2]], np.int32)
    samp = np.array([[3]], np.int32)
    n = np.array([10], np.int32)
    base = knobs(8, D=6)
    d, nv = orc.propose(orc.params_from(base), n, row, samp)
    assert d[0].tolist() == [4, 5, 6, 7, 8, 1, 2, 3] and nv[0] == 8
    d, nv = orc.propose(orc.params_from(dict(base, tree_depth_cap=1)), n, row, samp)
    assert d[0].tolist() == [4, 5, 6, 3, 3, 3, 3, 3] and nv[0] == 3
    # the flag bit of a config reaches the same parameter
    assert orc.params_from(dict(base, flags=orc.TREE_DEPTH_CAP_FLAG)).tree_depth_cap == 1

    rng = np.random.default_rng(33)
    B, S, V = 16, 80, 3
    for mode, nb in ((0, 1), (1, 3)):
        for D in (2, 5, 9, 24):
            kn = knobs(10, D=D, nb=nb, M=16, mode=mode, factor=4_000_000)
            tok = rng.integers(0, V, size=(B, S)).astype(np.int32)
            n = rng.integers(0, S + 1, size=B).astype(np.int32)
            samp = rng.integers(0, V, size=(B, 1)).astype(np.int32)
            C = _rand_corpus(rng, V, 6, 0, 30)
            free = orc.propose(orc.params_from(kn), n, tok, samp, corpus=C, with_info=True)
            capd = orc.propose(orc.params_from(dict(kn, tree_depth_cap=1)), n, tok, samp,
                               corpus=C, with_info=True)
            for b in range(B):
                r = capd[2][b]
                if r.chosen >= 0:
                    assert capd[1][b] <= max(0, D - r.chosen_len)
                if mode == 0:
                    l = free[2][b].chosen_len
                    keep = min(int(free[1][b]), max(0, D - l)) if free[2][b].chosen >= 0 else 0
                    assert capd[1][b] == keep
                    fill = capd[0][b][-1] if keep < 10 else None
                    assert capd[0][b][:keep].tolist() == free[0][b][:keep].tolist()
                    if fill is not None:
                        assert (capd[0][b][keep:] == samp[b, 0]).all()


# ------------------------------------------------------------------ algorithmic-byte counter
def test_alg_words_context_and_io(orc):
    # categories 0 and 1 in closed form; no corpus: no probe or interval words
    rng = np.random.default_rng(41)
    B, S, T, k = 5, 60, 2, 6
    tok = rng.integers(0, 4, size=(B, S)).astype(np.int32)
    n = np.array([0, 7, 60, 33, 12], np.int32)
    samp = np.array([[1, 2], [3, -1], [-1, 5], [0, 0], [2, -1]], np.int32)
    w = orc.alg_words(orc.make_params(k), n, tok, samp)
    t = np.array([2, 1, 0, 2, 1])
    assert w["context"] == int((n + t)[t > 0].sum())
    assert w["io"] == B * (2 + T + k + 1)
    assert w["sa_probes"] == 0 and w["interval_scans"] == 0


def test_alg_words_single_site_votes(orc):
    # the worked example "single earlier occurrence of the tail": one site, the continuation
    # 1 2 4 1 2 3 has no negative id, so a k=4 longest-match vote reads one word per depth
    case = GOLD["local"][0]
    w = orc.alg_words(orc.make_params(4, max_tree_depth=case["D"]), np.array([case["n"]]),
                      np.array([case["row"]], np.int32), np.array([case["sampled"]], np.int32))
    assert w["voted_tokens"] == 4


def test_alg_words_probe_closed_form(orc):
    # every corpus token is smaller than the tail's tokens, and the corpus holds 2^5 - 1 tokens:
    # each lower-bound search halves [0, N) five times, always to the right, reading one
    # suffix-array word and one token per step; the upper bound then starts at N (no step)
    N = 31
    C = np.array([i % 3 for i in range(N - 1)] + [-1], np.int32)
    row = np.array([[7, 8, 9, 7, 8, 9]], np.int32)
    for D, L_tail in ((24, 7), (4, 4), (2, 2)):
        w = orc.alg_words(orc.make_params(3, max_tree_depth=D), np.array([6]), row,
                          np.array([[9]], np.int32), corpus=C)
        lengths = len(range(2, min(D, 7) + 1))
        assert w["sa_probes"] == lengths * 5 * 2, (D, w)
        assert w["interval_scans"] == 0


def test_alg_words_interval_is_occurrence_count(orc):
    # the interval scanned for the corpus candidate holds every occurrence of its g-gram (the
    # suffixes starting with it), counted here by direct substring comparison
    rng = np.random.default_rng(43)
    for it in range(60):
        V = int(rng.choice([2, 3]))
        C = _rand_corpus(rng, V, int(rng.integers(1, 8)), 0, 25)
        if len(C) == 0:
            continue
        row = rng.integers(0, V, size=(1, 20)).astype(np.int32)
        samp = rng.integers(0, V, size=(1, 1)).astype(np.int32)
        p = orc.make_params(4, max_tree_depth=6)
        w = orc.alg_words(p, np.array([20]), row, samp, corpus=C)
        ctx, _ = orc.context(row[0], 20, samp[0])
        m = orc.corpus_match(C, ctx, 6)
        g = orc.kth_largest(m, 1)
        if g < 2:
            assert w["interval_scans"] == 0
            continue
        pat = ctx[len(ctx) - g:].tolist()
        occ = sum(1 for i in range(len(C)) if C[i:i + g].tolist() == pat)
        assert w["interval_scans"] == occ, (it, g)


def test_alg_bytes_file_is_current(orc):
    # the stored algorithmic bytes the benchmark reads were written by oracle/alg_bytes.py from
    # the current oracle and generators: recompute two of its workloads' sets
    import workloads as W

    stored = json.load(open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle",
                                         "alg_bytes.json")))["workloads"]
    for cid, set_index in ((1, 0), (1, 3), (3, 0)):
        w = W.WORKLOADS[cid]
        C = W.join_docs(W.corpus_docs(cid)) if w.corpus else None
        n, tok, samp = W.make_batch(cid, set_index=set_index)
        words = orc.alg_words(orc.params_from(w.knobs()), n, tok, samp, corpus=C, num_threads=8)
        exp = [s for s in stored[w.name]["sets"] if s["set_index"] == set_index][0]["bytes"]
        assert {k: 4 * v for k, v in words.items()} == {k: v for k, v in exp.items()
                                                         if k != "total"}
