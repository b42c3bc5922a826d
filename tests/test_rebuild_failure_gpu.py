"""Failure of an index rebuild (suffix-gpu page, How it works step 4: the index is rebuilt on a
side stream and double-buffered; the one in use stays in place until the new one is swapped
in).  With the test hook set, a rebuild fails after building into the inactive buffer: the
synchronous call returns EHIP; the asynchronous one reports EHIP from poll (nothing swapped in)
or from wait.  Throughout, drafts equal the oracle's on the live corpus (the old index plus the
delta), and the next rebuild works."""
import ctypes

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

KN = dict(k=6, max_tree_depth=8, num_backoff=3, max_occurrences=16, mode=1,
          spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
V = 5


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


def docs(rng, count):
    return [rng.integers(0, V, size=int(rng.integers(1, 60))).astype(np.int32)
            for _ in range(count)]


def check(d, lc, inputs, what):
    import torch

    n, tok, samp = inputs
    dd, dn = d.propose(dev(n), dev(tok), dev(samp))
    torch.cuda.synchronize()
    ed, en = O.propose(O.params_from(KN), n, tok, samp, corpus=lc.text())
    assert np.array_equal(dd.cpu().numpy(), ed) and np.array_equal(dn.cpu().numpy(), en), what


def test_injected_rebuild_failures(S):
    import torch

    rng = np.random.default_rng(61)
    B, Sq = 12, 96
    inputs = (rng.integers(1, Sq + 1, size=B).astype(np.int32),
              rng.integers(0, V, size=(B, Sq)).astype(np.int32),
              rng.integers(0, V, size=(B, 1)).astype(np.int32))
    d = S.Drafter(S.Config(max_batch=B, max_seq=Sq, max_sampled=1, corpus_capacity=4000, **KN))
    lc = O.LiveCorpus(4000)
    first = docs(rng, 30)
    d.ingest_docs(first)
    lc.ingest(first)
    d.rebuild()
    check(d, lc, inputs, "after the first rebuild")

    # synchronous rebuild: fails, the new documents stay reachable through the delta
    more = docs(rng, 20)
    d.ingest_docs(more)
    lc.ingest(more)
    d.debug_fail_next_rebuild()
    with pytest.raises(S.SfxError) as ei:
        d.rebuild()
    assert ei.value.code == S.EHIP and "injected" in str(ei.value)
    check(d, lc, inputs, "after a failed synchronous rebuild")
    d.rebuild()
    check(d, lc, inputs, "after the next synchronous rebuild")

    # asynchronous rebuild, seen by poll: error, nothing swapped in; proposes meanwhile and after
    more = docs(rng, 20)
    d.ingest_docs(more)
    lc.ingest(more)
    d.debug_fail_next_rebuild()
    d.rebuild_async()
    check(d, lc, inputs, "while the failing rebuild runs")
    L = S.load()
    sw = ctypes.c_int32(7)
    rc = 0
    for _ in range(2000):
        rc = L.sfx_poll(d._h, ctypes.byref(sw), S._stream(None))
        if rc != 0 or sw.value:
            break
        torch.cuda.synchronize()
    assert rc == S.EHIP and sw.value == 0, (rc, sw.value)
    check(d, lc, inputs, "after poll reported the failure")
    # the state is idle again: a new rebuild starts, and wait swaps it in
    d.rebuild_async()
    d.wait_rebuild()
    check(d, lc, inputs, "after the next asynchronous rebuild")

    # asynchronous rebuild, seen by wait
    more = docs(rng, 20)
    d.ingest_docs(more)
    lc.ingest(more)
    d.debug_fail_next_rebuild()
    d.rebuild_async()
    with pytest.raises(S.SfxError) as ei:
        d.wait_rebuild()
    assert ei.value.code == S.EHIP
    check(d, lc, inputs, "after wait reported the failure")
    d.rebuild()
    check(d, lc, inputs, "after the rebuild that follows")
    d.close()


def test_hook_needs_a_corpus(S):
    bare = S.Drafter(S.Config(max_batch=1, max_seq=8, max_sampled=1, corpus_capacity=0, **KN))
    with pytest.raises(S.SfxError) as ei:
        bare.debug_fail_next_rebuild()
    assert ei.value.code == S.ESTATE
    bare.close()
