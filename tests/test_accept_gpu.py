"""Per-slot acceptance estimate (vLLM docs "Suffix Decoding", Use adaptive verification at
higher concurrency: a running estimate per draft position, keyed by the draft's source, its match
length and the position).

Each step proposes on the GPU and in the oracle (whose row information names the winning
candidate), then compares the estimates with the oracle's acceptance model, feeds the same
synthetic verifier results to both, and compares the whole counts table.  This also checks the
source and length the propose kernel records for every row."""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("mode,nb", [(0, 1), (1, 4)])
def test_estimates_follow_feedback(S, mode, nb):
    import torch

    rng = np.random.default_rng(41 + mode)
    V, Sq, MB = 8, 128, 32
    kn = dict(k=8, max_tree_depth=16, num_backoff=nb, max_occurrences=32, mode=mode,
              spec_factor_ppm=2_000_000, min_token_prob_ppm=100_000)
    k = kn["k"]
    docs = [rng.integers(0, V, size=int(rng.integers(5, 80))).astype(np.int32)
            for _ in range(60)]
    lc = O.LiveCorpus(1 << 14)
    lc.ingest(docs)
    d = S.Drafter(S.Config(max_batch=MB, max_seq=Sq, max_sampled=1, corpus_capacity=1 << 14,
                           **kn))
    d.ingest_docs(docs)
    d.rebuild()
    model = O.AcceptModel()
    p = O.params_from(kn)
    for step in range(8):
        B = [24, 16, 32, 5][step % 4]
        tok = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
        n = rng.integers(0, Sq + 1, size=B).astype(np.int32)
        samp = rng.integers(-1, V, size=(B, 1)).astype(np.int32)
        dd, dn = d.propose(dev(n), dev(tok), dev(samp))
        ed, en, info = O.propose(p, n, tok, samp, corpus=lc.text(), with_info=True)
        torch.cuda.synchronize()
        assert np.array_equal(dd.cpu().numpy(), ed) and np.array_equal(dn.cpu().numpy(), en)
        model.record(O.picks_from_info(info, nb))
        est = d.accept_estimate(B)
        torch.cuda.synchronize()
        assert np.array_equal(est.cpu().numpy(), model.estimate(B, k)), f"step {step} estimates"
        na = rng.integers(-1, k + 2, size=B).astype(np.int32)
        d.accept_feedback(dev(na))
        model.feedback(na)
        d.accept_feedback(dev(na))  # the records are consumed: counted once
        counts = d.accept_counts().cpu().numpy()
        assert np.array_equal(counts, model.counts), f"step {step} counts"
    counts = d.accept_counts().cpu().numpy()
    assert counts[..., 0].sum() > 0 and (counts[..., 1] <= counts[..., 0]).all()
    if mode == 1:
        assert counts[0, ..., 0].sum() > 0 and counts[1, ..., 0].sum() > 0, "both sources"
    d.accept_reset()
    assert int(d.accept_counts().sum()) == 0
    assert int(d.accept_estimate(MB).abs().sum()) == 0
    d.close()


def test_accept_argument_checks(S):
    kn = dict(k=4, max_tree_depth=8, num_backoff=1, max_occurrences=8, mode=0)
    d = S.Drafter(S.Config(max_batch=4, max_seq=8, max_sampled=1, corpus_capacity=0, **kn))
    with pytest.raises(S.SfxError) as ei:
        d.accept_estimate(5)
    assert ei.value.code == S.ECAPACITY
    with pytest.raises(S.SfxError) as ei:
        d.accept_feedback(dev(np.zeros(5, np.int32)))
    assert ei.value.code == S.ECAPACITY
    # without a corpus every draft is local; before any propose there is nothing to estimate
    assert int(d.accept_estimate(4).abs().sum()) == 0
    d.close()
