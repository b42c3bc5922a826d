"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle, bit-exact.

Drafts, valid counts, suffix arrays, updated rows and live corpora must be identical element by
element on the same seeded inputs.  Sizes span several tiles with ragged tails; the workload
configurations run at full size."""
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

NTHREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def S():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import suffix_match_drafter_amd as sfx

    sfx.load()
    return sfx


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(S, knobs, n, tok, samp, corpus_docs=None, capacity=0, drafter=None, flags=0):
    import torch

    B, Sq = tok.shape
    T = samp.shape[1]
    d = drafter
    if d is None:
        cfg = S.Config(max_batch=max(B, 1), max_seq=max(Sq, 1), max_sampled=max(T, 1),
                       corpus_capacity=capacity, flags=flags, **knobs)
        d = S.Drafter(cfg)
        if corpus_docs is not None:
            d.ingest_docs(corpus_docs)
            d.rebuild()
    draft, nv = d.propose(dev(n), dev(tok), dev(samp))
    torch.cuda.synchronize()
    return draft.cpu().numpy(), nv.cpu().numpy(), d


def assert_same(got, exp, what=""):
    gd, gn = got
    ed, en = exp
    bad = np.nonzero((gd != ed).any(axis=1) | (gn != en))[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows differ, first {bad[:5].tolist()}; "
                           f"row {bad[0]}: gpu {gd[bad[0]].tolist()}/{gn[bad[0]]} "
                           f"oracle {ed[bad[0]].tolist()}/{en[bad[0]]}")


def knobs_of(w):
    return w.knobs()


# Both context paths: staged in LDS (flags 0, rows up to about 19K tokens) and read from device
# memory (flags 1, FLAG_STREAM_CONTEXT, the path of longer rows).
FLAGS = [0, 1]


# ------------------------------------------------------------------ hand-worked selection cases
GOLD = __import__("json").load(open(os.path.join(os.path.dirname(__file__), "golden",
                                                 "worked_examples.json")))


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("case", GOLD["selection"], ids=lambda c: c["name"])
def test_golden_selection_gpu(S, case, flags):
    n = np.array([case["n"]], np.int32)
    tok = np.array([case["row"]], np.int32)
    samp = np.array([case["sampled"]], np.int32)
    docs = [np.array(x, np.int32) for x in case["docs"]]
    got = run_gpu(S, case["knobs"], n, tok, samp, corpus_docs=docs if docs else None,
                  capacity=1024 if docs else 0, flags=flags)
    assert got[0][0].tolist() == case["expect"]["draft"], case["name"]
    assert got[1][0] == case["expect"]["num_valid"], case["name"]


# ------------------------------------------------------------------ fuzz and edge cases
@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("mode", [0, 1])
def test_fuzz_small(S, mode, flags):
    rng = np.random.default_rng(100 + mode)
    for it in range(40):
        V = int(rng.choice([2, 3, 5, 50]))
        B = int(rng.integers(1, 9))
        Sq = int(rng.integers(1, 300))
        T = int(rng.integers(0, 4))
        nb = 1 if mode == 0 else int(rng.integers(1, 9))
        kn = dict(k=int(rng.integers(1, 33)), max_tree_depth=int(rng.choice([1, 2, 3, 7, 24, 64])),
                  num_backoff=nb, max_occurrences=int(rng.choice([1, 2, 5, 64, 128])), mode=mode,
                  spec_factor_ppm=int(rng.choice([0, 500_000, 2_000_000])),
                  spec_offset_ppm=int(rng.choice([0, 1_000_000])),
                  min_token_prob_ppm=int(rng.choice([0, 100_000, 500_000, 1_000_000])),
                  min_self_match=int(rng.choice([1, 1, 2])))
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(-3, Sq + 4, size=B).astype(np.int32)
        samp = rng.integers(-1, V, size=(B, T)).astype(np.int32)
        exp = O.propose(O.params_from(kn), n, tok, samp)
        got = run_gpu(S, kn, n, tok, samp, flags=flags)[:2]
        assert_same(got, exp, f"fuzz it={it} kn={kn} B={B} S={Sq} T={T} flags={flags}")


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("mode", [0, 1])
def test_fuzz_with_corpus(S, mode, flags):
    rng = np.random.default_rng(200 + mode)
    for it in range(25):
        V = int(rng.choice([2, 3, 6, 40]))
        B = int(rng.integers(1, 7))
        Sq = int(rng.integers(2, 200))
        nb = 1 if mode == 0 else int(rng.integers(1, 9))
        D = int(rng.choice([2, 3, 4, 5, 6, 9, 24]))
        kn = dict(k=int(rng.integers(1, 17)), max_tree_depth=D, num_backoff=nb,
                  max_occurrences=int(rng.choice([1, 3, 128])), mode=mode,
                  spec_factor_ppm=int(rng.choice([1_000_000, 2_000_000])),
                  min_token_prob_ppm=int(rng.choice([0, 100_000, 400_000])),
                  min_corpus_match=int(rng.integers(2, D + 1)))
        docs = [rng.integers(0, V, size=int(rng.integers(0, 60))).astype(np.int32)
                for _ in range(int(rng.integers(1, 40)))]
        lc = O.LiveCorpus(10**7)
        lc.ingest(docs)
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(0, Sq + 1, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, 1)).astype(np.int32)
        exp = O.propose(O.params_from(kn), n, tok, samp, corpus=lc.text())
        got = run_gpu(S, kn, n, tok, samp, corpus_docs=docs, capacity=1 << 14, flags=flags)[:2]
        assert_same(got, exp, f"corpus fuzz it={it} kn={kn} flags={flags}")


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("mode", [0, 1])
def test_tree_depth_cap(S, mode, flags):
    """SFX_FLAG_TREE_DEPTH_CAP (gitcode blog, section 4: match length plus draft length at most
    max_tree_depth) on random rows with a corpus, and in the counted form with a narrower k:
    drafts equal the oracle's with the same cap."""
    import torch

    rng = np.random.default_rng(400 + mode)
    for it in range(12):
        V = int(rng.choice([2, 3, 6]))
        B, Sq = int(rng.integers(1, 9)), int(rng.integers(2, 160))
        nb = 1 if mode == 0 else int(rng.integers(1, 6))
        D = int(rng.choice([2, 4, 7, 12, 24]))
        kn = dict(k=int(rng.integers(1, 33)), max_tree_depth=D, num_backoff=nb,
                  max_occurrences=int(rng.choice([2, 16, 128])), mode=mode,
                  spec_factor_ppm=int(rng.choice([1_000_000, 4_000_000])),
                  min_token_prob_ppm=int(rng.choice([0, 100_000])))
        f = flags | S.FLAG_TREE_DEPTH_CAP
        docs = [rng.integers(0, V, size=int(rng.integers(0, 50))).astype(np.int32)
                for _ in range(int(rng.integers(1, 30)))]
        lc = O.LiveCorpus(10**7)
        lc.ingest(docs)
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(0, Sq + 1, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, 1)).astype(np.int32)
        p = O.params_from(dict(kn, flags=f))
        assert p.tree_depth_cap == 1
        exp = O.propose(p, n, tok, samp, corpus=lc.text())
        got = run_gpu(S, kn, n, tok, samp, corpus_docs=docs, capacity=1 << 14, flags=f)
        assert_same(got[:2], exp, f"tree cap it={it} kn={kn} flags={f}")
        k2 = int(rng.integers(1, kn["k"] + 1))
        cnt = np.ones(B, np.int32)
        dd, dn = got[2].propose_counts(k2, dev(n), dev(tok), dev(samp), dev(cnt))
        torch.cuda.synchronize()
        exp2 = O.propose_counts(p, k2, n, tok, samp, cnt, corpus=lc.text())
        assert_same((dd.cpu().numpy(), dn.cpu().numpy()), exp2, f"tree cap counts it={it} k={k2}")
        got[2].close()


@pytest.mark.parametrize("flags", FLAGS)
def test_max_sampled_width(S, flags):
    """T = 16, the largest sampled width: contexts extend the row prefix by up to 16 sampled ids
    (n up to S, so a context can be 16 tokens longer than the row), with padding at random
    points, k = 32 and D = 64, with a corpus."""
    rng = np.random.default_rng(404)
    B, Sq, T, V = 16, 300, 16, 3
    tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
    n = np.concatenate([np.full(4, Sq), rng.integers(0, Sq + 1, size=B - 4)]).astype(np.int32)
    samp = rng.integers(0, V, size=(B, T)).astype(np.int32)
    lead = rng.integers(0, T + 1, size=B)
    lead[:3] = T
    for b in range(B):
        samp[b, lead[b]:] = -1
    docs = [rng.integers(0, V, size=int(rng.integers(0, 80))).astype(np.int32) for _ in range(50)]
    lc = O.LiveCorpus(10**7)
    lc.ingest(docs)
    for mode, nb in ((0, 1), (1, 8)):
        kn = dict(k=32, max_tree_depth=64, num_backoff=nb, max_occurrences=128, mode=mode,
                  spec_factor_ppm=4_000_000, min_token_prob_ppm=50_000)
        exp = O.propose(O.params_from(kn), n, tok, samp, corpus=lc.text())
        got = run_gpu(S, kn, n, tok, samp, corpus_docs=docs, capacity=1 << 14, flags=flags)
        assert_same(got[:2], exp, f"T=16 mode={mode} flags={flags}")
        got[2].close()


@pytest.mark.parametrize("flags", FLAGS)
def test_degenerate_rows(S, flags):
    """Empty rows, rows with no sampled token, a single repeated token (every position
    matches), n above S, S not a multiple of 4, T=0."""
    B, Sq = 6, 301
    tok = np.full((B, Sq), 7, np.int32)
    n = np.array([0, 1, 301, 400, -5, 150], np.int32)
    samp = np.array([[7, -1], [-1, 3], [7, 7], [2, -1], [7, -1], [7, 7]], np.int32)
    for mode in (0, 1):
        kn = dict(k=32, max_tree_depth=64, num_backoff=1 + 7 * mode, max_occurrences=128,
                  mode=mode, spec_factor_ppm=10**7, min_token_prob_ppm=0)
        exp = O.propose(O.params_from(kn), n, tok, samp)
        assert_same(run_gpu(S, kn, n, tok, samp, flags=flags)[:2], exp, f"degenerate mode {mode}")
    kn = dict(k=4, max_tree_depth=24, num_backoff=1, max_occurrences=128, mode=0)
    e0 = O.propose(O.params_from(kn), n, tok, samp[:, :0])
    assert_same(run_gpu(S, kn, n, tok, samp[:, :0], flags=flags)[:2], e0, "T=0")


@pytest.mark.parametrize("flags", FLAGS)
def test_full_depth_match(S, flags):
    """max_tree_depth at its limit (64): an early copy of the last 63 context tokens (preceded by
    another token) continues with Y, a later copy of all 64 continues with X.  The longest match
    is the 64-token one, so the draft starts with X; a ladder that stops at 63 would take the
    earlier site and draft Y.  Locally, in the corpus snapshot, split between snapshot and delta,
    and in the delta alone."""
    import torch

    rng = np.random.default_rng(64)
    V, n = 5000, 400
    row = rng.integers(0, V, size=n).astype(np.int32)
    samp = np.array([[int(rng.integers(0, V))]], np.int32)
    tail = np.concatenate([row, samp[0]])[-64:]
    X, Y = 4242, 4243
    other = (int(tail[0]) + 1) % V
    loc = row.copy()
    loc[19] = other
    loc[20:83] = tail[1:]
    loc[83] = Y
    loc[150:214] = tail
    loc[214] = X
    doc_a = np.concatenate([rng.integers(0, V, 30), [other], tail[1:], [Y],
                            rng.integers(0, V, 20)]).astype(np.int32)
    doc_b = np.concatenate([rng.integers(0, V, 30), tail, [X],
                            rng.integers(0, V, 20)]).astype(np.int32)
    text = W.join_docs([doc_a, doc_b])
    nn = np.array([n], np.int32)
    for mode, nb in ((0, 1), (1, 4)):
        kn = dict(k=8, max_tree_depth=64, num_backoff=nb, max_occurrences=128, mode=mode,
                  spec_factor_ppm=10**7, min_token_prob_ppm=0)
        p = O.params_from(kn)
        exp = O.propose(p, nn, loc[None], samp)
        assert exp[0][0, 0] == X
        assert_same(run_gpu(S, kn, nn, loc[None], samp, flags=flags)[:2], exp,
                    f"local mode {mode}")
        exp = O.propose(p, nn, row[None], samp, corpus=text)
        assert exp[0][0, 0] == X
        got = run_gpu(S, kn, nn, row[None], samp, corpus_docs=[doc_a, doc_b],
                      capacity=1 << 12, flags=flags)
        assert_same(got[:2], exp, f"corpus snapshot mode {mode}")
        got[2].close()
        cfg = S.Config(max_batch=1, max_seq=n, max_sampled=1, corpus_capacity=1 << 12,
                       flags=flags, **kn)
        for split in (True, False):
            d = S.Drafter(cfg)
            if split:
                d.ingest_docs([doc_a])
                d.rebuild()
                d.ingest_docs([doc_b])
            else:
                d.ingest_docs([doc_a, doc_b])
            dd, dn = d.propose(dev(nn), dev(row[None]), dev(samp))
            torch.cuda.synchronize()
            assert_same((dd.cpu().numpy(), dn.cpu().numpy()), exp,
                        f"corpus delta split={split} mode {mode}")
            d.close()


# Above this many rows a context keeps no pair index of the delta, and every request scans the
# delta itself: the tests below run both ways.
NO_INDEX_BATCH = 1100


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("index", [True, False])
@pytest.mark.parametrize("mode", [0, 1])
def test_fuzz_with_delta(S, mode, index, flags):
    """Documents ingested after the last rebuild (the delta) from small vocabularies, so that
    many requests share a tail pair, many pairs collide, and a pair occurs thousands of times;
    rows without sampled tokens, with a negative token before the sampled one, shorter than two
    tokens; rings that wrap and evict, down to a ring shorter than two 64-position runs.  Drafts
    equal the oracle's on the live corpus, with the
    per-call pair index and with the scan of the whole delta."""
    import torch

    rng = np.random.default_rng(500 + 2 * mode + index)
    for it in range(12):
        V = int(rng.choice([2, 3, 5, 12, 40]))
        B = int(rng.integers(1, 160))
        Sq = int(rng.integers(2, 300))
        T = int(rng.integers(1, 4))
        nb = 1 if mode == 0 else int(rng.integers(1, 9))
        D = int(rng.choice([2, 3, 5, 9, 24]))
        kn = dict(k=int(rng.integers(1, 17)), max_tree_depth=D, num_backoff=nb,
                  max_occurrences=int(rng.choice([1, 5, 128])), mode=mode,
                  spec_factor_ppm=int(rng.choice([1_000_000, 2_000_000])),
                  min_token_prob_ppm=int(rng.choice([0, 100_000, 400_000])),
                  min_corpus_match=int(rng.integers(2, D + 1)))
        cap = int(rng.choice([70, 3000, 1 << 14]))  # 70: ring slots wrap inside one 64-run
        seed = [rng.integers(0, V, size=int(rng.integers(0, 80))).astype(np.int32)
                for _ in range(int(rng.integers(0, 30)))]
        delta = [rng.integers(0, V, size=int(rng.integers(0, 400))).astype(np.int32)
                 for _ in range(int(rng.integers(1, 40)))]
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(0, Sq + 1, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, T)).astype(np.int32)
        samp[rng.random((B, T)) < 0.15] = -1           # some rows stop early or draft nothing
        neg = rng.random(B) < 0.05                     # a negative token before the sampled one
        for b in np.nonzero(neg)[0]:
            if n[b] > 0:
                tok[b, n[b] - 1] = -3
        cfg = S.Config(max_batch=NO_INDEX_BATCH if not index else max(B, 1), max_seq=Sq,
                       max_sampled=T, corpus_capacity=cap, **kn)
        d = S.Drafter(cfg)
        lc = O.LiveCorpus(cap)
        if seed:
            d.ingest_docs(seed)
            lc.ingest(seed)
        d.rebuild()
        d.ingest_docs(delta)
        lc.ingest(delta)
        exp = O.propose(O.params_from(kn), n, tok, samp, corpus=lc.text())
        dd, dn = d.propose(dev(n), dev(tok), dev(samp))
        torch.cuda.synchronize()
        assert_same((dd.cpu().numpy(), dn.cpu().numpy()), exp,
                    f"delta fuzz it={it} V={V} B={B} cap={cap} kn={kn}")
        d.close()


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("index", [True, False])
@pytest.mark.parametrize("wrap", [False, True])
def test_delta_many_short_matches(S, flags, wrap, index):
    """A delta with 20000 occurrences of exactly the last two context tokens, then three of the
    last 24: far more short occurrences than any wavefront keeps, so the long candidate's sites
    lie past every kept record and must be found again.  With wrap the delta runs across the end
    of the ring and the oldest documents are evicted.  Run with the per-call pair index and with
    the scan of the whole delta."""
    import torch

    rng = np.random.default_rng(77)
    V, n = 1000, 200
    row = rng.integers(0, V, size=(2, n)).astype(np.int32)
    samp = rng.integers(0, V, size=(2, 1)).astype(np.int32)
    ctx = np.concatenate([row[0], samp[0]])
    tail = ctx[::-1][:24]
    z = next(v for v in range(V) if v not in (tail[0], tail[1], tail[2]))
    short = np.tile(np.array([tail[1], tail[0], z], np.int32), 20000)
    longs = [np.concatenate([rng.integers(0, V, 50), ctx[-24:], [1000 + i],
                             rng.integers(0, V, 50)]).astype(np.int32) for i in range(3)]
    seed = [rng.integers(0, V, 3000).astype(np.int32) for _ in range(10)]
    cap = 1 << 16 if wrap else 1 << 18
    nn = np.full(2, n, np.int32)
    for mode, nb in ((0, 1), (1, 4)):
        kn = dict(k=8, max_tree_depth=24, num_backoff=nb, max_occurrences=128, mode=mode,
                  spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
        cfg = S.Config(max_batch=2 if index else NO_INDEX_BATCH, max_seq=n, max_sampled=1,
                       corpus_capacity=cap, flags=flags, **kn)
        d = S.Drafter(cfg)
        lc = O.LiveCorpus(cap)
        d.ingest_docs(seed)
        lc.ingest(seed)
        d.rebuild()
        d.ingest_docs([short] + longs)
        lc.ingest([short] + longs)
        assert (lc.evicted() > 0) == wrap
        exp = O.propose(O.params_from(kn), nn, row, samp, corpus=lc.text())
        if mode == 0:  # the longest match wins; SCORED prefers the unanimous short one
            assert exp[0][0, 0] in (1000, 1001, 1002)
        dd, dn = d.propose(dev(nn), dev(row), dev(samp))
        torch.cuda.synchronize()
        assert_same((dd.cpu().numpy(), dn.cpu().numpy()), exp, f"mode {mode}")
        d.close()


def test_long_repeated_rows(S):
    """Rows of one repeated token at full length (every end position is a hit), a long row that
    starts with a repeated run, and rows of period 2, in both context paths and at the largest
    row capacity."""
    B, Sq = 4, 32768
    tok = np.full((B, Sq), 5, np.int32)
    tok[1, 20000:] = np.arange(Sq - 20000) % 97 + 10
    tok[2, :] = np.arange(Sq) % 2
    tok[3, :] = np.arange(Sq) % 3
    n = np.array([Sq, Sq, Sq - 1, 20001], np.int32)
    samp = np.array([[5], [5], [1], [2]], np.int32)
    for mode in (0, 1):
        kn = dict(k=32, max_tree_depth=64, num_backoff=1 + 7 * mode, max_occurrences=128,
                  mode=mode, spec_factor_ppm=10**7, min_token_prob_ppm=0)
        exp = O.propose(O.params_from(kn), n, tok, samp, num_threads=NTHREADS)
        # a 32768-token row only runs on the streaming path; 16384 fits either
        assert_same(run_gpu(S, kn, n, tok, samp)[:2], exp, f"long rows mode {mode}")
        h = Sq // 2
        n2 = np.minimum(n, h)
        exp2 = O.propose(O.params_from(kn), n2, tok[:, :h], samp, num_threads=NTHREADS)
        for flags in FLAGS:
            assert_same(run_gpu(S, kn, n2, np.ascontiguousarray(tok[:, :h]), samp,
                                flags=flags)[:2], exp2, f"half rows mode {mode} flags {flags}")


# ------------------------------------------------------------------ workload configurations
@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("cid", [1, 2])
def test_config_self_match(S, cid, flags):
    w = W.WORKLOADS[cid]
    n, tok, samp = W.make_batch(cid)
    exp = O.propose(O.params_from(w.knobs()), n, tok, samp, num_threads=NTHREADS)
    got = run_gpu(S, w.knobs(), n, tok, samp, flags=flags)[:2]
    assert_same(got, exp, f"config {cid} flags {flags}")
    assert (got[1] <= w.k).all()
    assert (got[0] != W.POISON).all()


@pytest.mark.parametrize("cid,flags", [(3, 0), (4, 0), (4, 1)])
def test_config_corpus(S, cid, flags):
    import torch

    w = W.WORKLOADS[cid]
    docs = W.corpus_docs(cid)
    text = W.join_docs(docs)
    n, tok, samp = W.make_batch(cid)
    cap = 1 << 20
    got_d, got_n, d = run_gpu(S, w.knobs(), n, tok, samp, corpus_docs=docs, capacity=cap,
                              flags=flags)
    snap = d.corpus_snapshot().cpu().numpy()
    assert np.array_equal(snap, text)
    # the live index: its snapshot text and suffix array, and its doubling rounds: the first
    # sort by one token plus one round per h = 1, 2, 4, ... up to the longest common prefix of
    # two suffixes (lam), i.e. floor(log2(lam)) + 2
    itext, isa = (x.cpu().numpy() for x in d.debug_index())
    assert np.array_equal(itext, text)
    osa = O.suffix_array(itext)
    assert np.array_equal(isa, osa)
    lam = _max_adjacent_lcp(itext, osa)
    rounds, ntok = d.rebuild_stats()
    assert ntok == len(itext)
    assert rounds == (int(np.floor(np.log2(lam))) + 2 if lam >= 1 else 1), (rounds, lam)
    exp = O.propose(O.params_from(w.knobs()), n, tok, samp, corpus=text, num_threads=NTHREADS)
    assert_same((got_d, got_n), exp, f"config {cid}")
    assert (got_d != W.POISON).all()
    # a second call on the same context is identical (no state leaks between calls)
    d2, n2 = d.propose(dev(n), dev(tok), dev(samp))
    torch.cuda.synchronize()
    assert np.array_equal(d2.cpu().numpy(), got_d) and np.array_equal(n2.cpu().numpy(), got_n)
    d.close()


def _max_adjacent_lcp(text, sa):
    # longest common prefix of suffixes adjacent in suffix-array order (the longest of any two)
    best = 0
    t = text.astype(np.int64)
    n = len(t)
    a, b = sa[:-1].astype(np.int64), sa[1:].astype(np.int64)
    lcp = np.zeros(len(a), np.int64)
    alive = np.ones(len(a), bool)
    k = 0
    while alive.any():
        ia, ib = a + k, b + k
        ok = alive & (ia < n) & (ib < n)
        eq = np.zeros(len(a), bool)
        eq[ok] = t[ia[ok]] == t[ib[ok]]
        lcp += eq
        alive = eq
        k += 1
    best = int(lcp.max()) if len(lcp) else 0
    return best


def test_config_ingest_under_load(S):
    """Workload 5: a 2^22-token ring seeded with the template corpus; every step harvests 256
    finished rows and starts an asynchronous rebuild while B=512 requests of up to 32768 tokens
    propose.  At several steps (with a rebuild in flight, so part of the corpus is only in the
    delta, and after the ring has started to evict) every row must equal the oracle on the live
    corpus, whatever rebuild is live at that moment."""
    import torch

    w = W.WORKLOADS[5]
    cfg = S.Config(max_batch=w.B, max_seq=w.S, max_sampled=w.T,
                   corpus_capacity=w.ring_capacity, **w.knobs())
    d = S.Drafter(cfg)
    seed = W.corpus_docs(5)
    d.ingest_docs(seed)
    d.rebuild()
    lc = O.LiveCorpus(w.ring_capacity)
    lc.ingest(seed)
    n, tok, samp = W.make_batch(5)
    dn, dt, ds = dev(n), dev(tok), dev(samp)
    p = O.params_from(w.knobs())
    checks = 0
    for step in range(12):
        itok, rows, lens = W.ingest_batch(5, step)
        d.harvest_finished(dev(rows), dev(lens), dev(itok))
        lc.ingest([itok[r, :lens[r]] for r in rows])
        if step % 2 == 0:
            d.wait_rebuild()
            d.rebuild_async()
        if step in (0, 5, 11):
            got_d, got_n = d.propose(dn, dt, ds)
            torch.cuda.synchronize()
            exp = O.propose(p, n, tok, samp, corpus=lc.text(), num_threads=NTHREADS)
            assert_same((got_d.cpu().numpy(), got_n.cpu().numpy()), exp, f"step {step}")
            assert (got_n.cpu().numpy() <= w.k).all()
            checks += 1
    d.wait_rebuild()
    snap = d.corpus_snapshot().cpu().numpy()
    assert np.array_equal(snap, lc.text())
    assert lc.evicted() > 0, "the ring should have started evicting"
    # after the wrap and the eviction: a rebuild of the live corpus, and its suffix array at the
    # ring's size against the oracle's
    d.rebuild()
    itext, isa = (x.cpu().numpy() for x in d.debug_index())
    assert np.array_equal(itext, lc.text())
    assert itext.shape[0] > (3 * w.ring_capacity) // 4
    assert np.array_equal(isa, O.suffix_array(itext))
    d.close()
    assert checks == 3


# ------------------------------------------------------------------ large token ids
# Ids at and above 2^24 and next to INT32_MAX: the vote's hash path then takes the count and the
# token from two reductions (they no longer pack into one word), the first suffix-array sort
# uses all 32 key bits, and the n-gram hash sees full-width keys.  A few frequent symbols give
# candidates with many more than 24 alive sites and split votes.
BIG_IDS = np.array([(1 << 24) + 7919 * i for i in range(24)] +
                   [(1 << 30) + 104729 * i for i in range(8)] +
                   [2**31 - 1 - i for i in range(8)], np.int64).astype(np.int32)


def _big_rows(rng, B, Sq, nsym):
    p = 1.0 / np.arange(1, nsym + 1) ** 0.8
    p /= p.sum()
    sym = rng.choice(nsym, size=(B, Sq), p=p)
    return BIG_IDS[sym]


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("mode", [0, 1])
def test_large_token_ids(S, mode, flags):
    rng = np.random.default_rng(900 + mode)
    B, Sq = 8, 3000
    tok = _big_rows(rng, B, Sq, 40)
    n = rng.integers(Sq // 2, Sq, size=B).astype(np.int32)
    samp = BIG_IDS[rng.integers(0, 40, size=(B, 1))]
    docs = [_big_rows(rng, 1, int(rng.integers(50, 200)), 40)[0] for _ in range(300)]
    kn = dict(k=16, max_tree_depth=24, num_backoff=1 if mode == 0 else 4, max_occurrences=128,
              mode=mode, spec_factor_ppm=2_000_000, min_token_prob_ppm=0)
    lc = O.LiveCorpus(10**7)
    lc.ingest(docs)
    exp = O.propose(O.params_from(kn), n, tok, samp, corpus=lc.text(), num_threads=NTHREADS)
    got = run_gpu(S, kn, n, tok, samp, corpus_docs=docs, capacity=1 << 17, flags=flags)[:2]
    assert_same(got, exp, f"large ids mode={mode} flags={flags}")
    # without the corpus as well (local candidates only)
    exp = O.propose(O.params_from(kn), n, tok, samp, num_threads=NTHREADS)
    got = run_gpu(S, kn, n, tok, samp, flags=flags)[:2]
    assert_same(got, exp, f"large ids, no corpus, mode={mode} flags={flags}")


def test_large_token_ids_suffix_array(S):
    rng = np.random.default_rng(77)
    docs = [_big_rows(rng, 1, int(rng.integers(20, 400)), 40)[0] for _ in range(400)]
    text = W.join_docs(docs)
    sa = S.build_suffix_array(dev(text)).cpu().numpy()
    assert np.array_equal(sa, O.suffix_array(text))
    # the full signed range: INT32_MIN .. INT32_MAX in one text
    wide = np.concatenate([BIG_IDS, -BIG_IDS, [np.iinfo(np.int32).min, -1, 0]]).astype(np.int32)
    wide = rng.choice(wide, size=50000)
    sa = S.build_suffix_array(dev(wide)).cpu().numpy()
    assert np.array_equal(sa, O.suffix_array(wide))


# ------------------------------------------------------------------ suffix arrays
@pytest.mark.parametrize("n,V", [(1, 5), (2, 1), (17, 2), (1000, 3), (4097, 2), (70001, 50),
                                 (250000, 7)])
def test_suffix_array_random(S, n, V):
    rng = np.random.default_rng(n)
    text = rng.integers(-1, V, size=n).astype(np.int32)
    sa = S.build_suffix_array(dev(text)).cpu().numpy()
    assert np.array_equal(sa, O.suffix_array(text))


def test_suffix_array_repetitive(S):
    # long repeats force many doubling rounds
    base = np.arange(37, dtype=np.int32)
    text = np.concatenate([np.tile(base, 60), [-1], np.tile(base[:5], 300), [-1]]).astype(np.int32)
    sa = S.build_suffix_array(dev(text)).cpu().numpy()
    assert np.array_equal(sa, O.suffix_array(text))


def test_suffix_array_template_corpus(S):
    text = W.join_docs(W.corpus_docs(4))
    sa = S.build_suffix_array(dev(text)).cpu().numpy()
    assert np.array_equal(sa, O.suffix_array(text))


# ------------------------------------------------------------------ state update
def test_update_state(S):
    import torch

    rng = np.random.default_rng(5)
    B, Sq, T = 37, 129, 3
    tok = rng.integers(0, 100, size=(B, Sq)).astype(np.int32)
    n = rng.integers(-2, Sq + 3, size=B).astype(np.int32)
    samp = rng.integers(-1, 100, size=(B, T)).astype(np.int32)
    exp_tok, exp_n = O.update_state(tok, n, samp)
    t = dev(tok)
    got_n = S.update_state(t, dev(n), dev(samp))
    torch.cuda.synchronize()
    assert np.array_equal(t.cpu().numpy(), exp_tok)
    assert np.array_equal(got_n.cpu().numpy(), exp_n)


# ------------------------------------------------------------------ ingest, eviction, rebuild
def test_ring_eviction_and_delta(S):
    """Documents appended past the capacity evict the oldest; drafts are defined on the live
    corpus whether a document is indexed (rebuilt) or still in the delta."""
    import torch

    rng = np.random.default_rng(9)
    V = 6
    kn = dict(k=6, max_tree_depth=8, num_backoff=3, max_occurrences=7, mode=1,
              spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
    cap = 3000
    cfg = S.Config(max_batch=16, max_seq=256, max_sampled=1, corpus_capacity=cap, **kn)
    d = S.Drafter(cfg)
    live = O.LiveCorpus(cap)
    B, Sq = 16, 256
    for step in range(12):
        R = int(rng.integers(1, 9))
        rows = rng.integers(0, V, size=(R, 200)).astype(np.int32)
        lens = rng.integers(-5, 230, size=R).astype(np.int32)
        idx = rng.permutation(R).astype(np.int32)
        d.harvest_finished(dev(idx), dev(lens), dev(rows))
        live.ingest(O.harvest_docs(rows, idx, lens))
        if step % 3 == 1:
            d.wait_rebuild()
            d.rebuild()
        if step % 4 == 2:
            d.rebuild_async()
            if step % 8 == 2:
                d.wait_rebuild()
        assert np.array_equal(d.corpus_snapshot().cpu().numpy(), live.text()), step
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(0, Sq + 1, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, 1)).astype(np.int32)
        exp = O.propose(O.params_from(kn), n, tok, samp, corpus=live.text())
        got = run_gpu(S, kn, n, tok, samp, drafter=d)[:2]
        assert_same(got, exp, f"ring step {step}")
        d.poll()
    d.wait_rebuild()
    torch.cuda.synchronize()
    d.close()


@pytest.mark.parametrize("flags", FLAGS)
def test_masked_form(S, flags):
    """sfx_propose_masked (PyPI page, Quickstart: propose(num_tokens_no_spec, token_ids,
    combined_mask)) against the oracle's masked form, with a corpus, random masks and empty
    rows; and, on the GPU alone, the masked call after update_state equals the ordinary call
    on the state before it."""
    import torch

    rng = np.random.default_rng(57)
    V, B, Sq = 6, 40, 300
    docs = [rng.integers(0, V, size=int(rng.integers(1, 90))).astype(np.int32)
            for _ in range(30)]
    text = W.join_docs(docs)
    for mode, nb in ((0, 1), (1, 4)):
        kn = dict(k=10, max_tree_depth=12, num_backoff=nb, max_occurrences=64, mode=mode,
                  spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
        p = O.params_from(kn)
        cfg = S.Config(max_batch=B, max_seq=Sq, max_sampled=1, corpus_capacity=1 << 14,
                       flags=flags, **kn)
        d = S.Drafter(cfg)
        d.ingest_docs(docs)
        d.rebuild()
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(-2, Sq + 3, size=B).astype(np.int32)
        n[:3] = 0
        mask = (rng.random(B) < 0.7).astype(np.int32)
        gd, gn = d.propose_masked(dev(n), dev(tok), dev(mask))
        torch.cuda.synchronize()
        exp = O.propose_masked(p, n, tok, mask, corpus=text)
        assert_same((gd.cpu().numpy(), gn.cpu().numpy()), exp, f"masked mode {mode}")
        # after the state update, the masked call equals the ordinary one before it
        n0 = rng.integers(0, Sq, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, 1)).astype(np.int32)
        td = dev(tok)
        od, on = d.propose(dev(n0), td, dev(samp))
        n1 = S.update_state(td, dev(n0), dev(samp))
        md, mn = d.propose_masked(n1, td, dev(np.ones(B, np.int32)))
        torch.cuda.synchronize()
        assert np.array_equal(od.cpu().numpy(), md.cpu().numpy())
        assert np.array_equal(on.cpu().numpy(), mn.cpu().numpy())
        d.close()


@pytest.mark.parametrize("flags", FLAGS)
def test_counted_form(S, flags):
    """sfx_propose_counts (RFC page, Design: propose(k, num_tokens_no_spec, token_ids, sampled,
    counts)) against the oracle's counted form: counts below, at and above the valid entries,
    negative counts, non-negative junk past the count, and every call width k up to the
    configured one, in both modes, with a corpus."""
    import torch

    rng = np.random.default_rng(61)
    V, B, Sq, T = 6, 36, 200, 3
    docs = [rng.integers(0, V, size=int(rng.integers(1, 70))).astype(np.int32)
            for _ in range(25)]
    text = W.join_docs(docs)
    for mode, nb in ((0, 1), (1, 4)):
        kn = dict(k=12, max_tree_depth=10, num_backoff=nb, max_occurrences=64, mode=mode,
                  spec_factor_ppm=1_500_000, min_token_prob_ppm=100_000)
        p = O.params_from(kn)
        cfg = S.Config(max_batch=B, max_seq=Sq, max_sampled=T, corpus_capacity=1 << 14,
                       flags=flags, **kn)
        d = S.Drafter(cfg)
        d.ingest_docs(docs)
        d.rebuild()
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(0, Sq + 1, size=B).astype(np.int32)
        samp = rng.integers(0, V, size=(B, T)).astype(np.int32)
        samp[rng.random((B, T)) < 0.15] = -1
        counts = rng.integers(-1, T + 2, size=B).astype(np.int32)
        for k in (1, 5, 12):
            gd, gn = d.propose_counts(k, dev(n), dev(tok), dev(samp), dev(counts))
            torch.cuda.synchronize()
            exp = O.propose_counts(p, k, n, tok, samp, counts, corpus=text)
            assert_same((gd.cpu().numpy(), gn.cpu().numpy()), exp, f"counted k={k} mode {mode}")
        with pytest.raises(S.SfxError) as ei:
            d.propose_counts(13, dev(n), dev(tok), dev(samp), dev(counts))
        assert ei.value.code == S.ECAPACITY
        d.close()


@pytest.mark.parametrize("flags", FLAGS)
def test_delta_walk_with_and_without_early_region(S, flags):
    """Long staged rows leave no LDS for the early delta walk's own region (the delta is walked
    after the local sites, in the hit lists' space); streamed rows leave room (the wavefronts
    that vote no local candidate walk it beside them).  Both against the oracle, with the pair
    index, on a corpus with a delta of template documents."""
    import torch

    knobs = dict(k=16, max_tree_depth=24, num_backoff=4, max_occurrences=128, mode=1,
                 spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
    B, Sq, cap = 16, 16384, 1 << 18
    n, tok, samp = W.make_batch(4, set_index=3, B=B)
    docs = W.corpus_docs(4)
    d = S.Drafter(S.Config(max_batch=B, max_seq=Sq, max_sampled=1, corpus_capacity=cap,
                           flags=flags, **knobs))
    lc = O.LiveCorpus(cap)
    d.ingest_docs(docs[:300])
    lc.ingest(docs[:300])
    d.rebuild()
    d.ingest_docs(docs[300:420])
    lc.ingest(docs[300:420])
    dd, dn = d.propose(dev(n), dev(tok), dev(samp))
    torch.cuda.synchronize()
    exp = O.propose(O.params_from(knobs), n, tok, samp, corpus=lc.text(), num_threads=NTHREADS)
    assert_same((dd.cpu().numpy(), dn.cpu().numpy()), exp, f"flags={flags}")
