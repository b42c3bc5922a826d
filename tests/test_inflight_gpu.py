"""In-flight ingest (RFC page "[RFC]: Suffix decoding on GPU (suffix_gpu)", Design: in-flight
responses are ingested off the critical path, finished requests are final-flushed before their
batch rows are reused).

Random decode traces drive sfx_ingest_inflight and the oracle's cursor model side by side: rows
grow by a few tokens per step, some finish (final flush) and are reused, some calls list a row
twice or name rows outside the batch, min_chunk varies, finished rows are also harvested, and
rebuilds come and go while the small ring evicts.  After every call the device's live corpus
must equal the oracle's, and drafts must equal the oracle's on that corpus."""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

KN = dict(k=6, max_tree_depth=8, num_backoff=3, max_occurrences=16, mode=1,
          spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)


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


@pytest.mark.parametrize("cap", [1 << 14, 1500])
def test_inflight_trace(S, cap):
    import torch

    rng = np.random.default_rng(31 + cap)
    B, Sq, V = 12, 96, 5
    d = S.Drafter(S.Config(max_batch=B, max_seq=Sq, max_sampled=1, corpus_capacity=cap, **KN))
    lc, model = O.LiveCorpus(cap), O.InflightIngest(max_rows=B)
    tok = np.zeros((B, Sq), np.int32)
    n = np.zeros(B, np.int32)
    checks = 0
    for step in range(40):
        for b in range(B):
            g = int(rng.integers(0, 7))
            g = min(g, Sq - int(n[b]))
            tok[b, n[b]:n[b] + g] = rng.integers(0, V, size=g)
            n[b] += g
        fin = ((rng.random(B) < 0.1) | (n == Sq)).astype(np.int32)
        # entries: a random subset of rows in random order, sometimes a repeat or a stranger
        rows = rng.permutation(B)[: int(rng.integers(1, B + 1))].astype(np.int32)
        if rng.random() < 0.3:
            rows = np.concatenate([rows, rows[:1], [B + 3, -2]]).astype(np.int32)
        lens = np.where((rows >= 0) & (rows < B), n[np.clip(rows, 0, B - 1)], 7).astype(np.int32)
        fl = np.where((rows >= 0) & (rows < B), fin[np.clip(rows, 0, B - 1)], 1).astype(np.int32)
        mc = int(rng.choice([0, 1, 3, 8]))
        d.ingest_inflight(dev(rows), dev(lens), dev(tok), final=dev(fl), min_chunk=mc)
        lc.ingest(model.docs(tok, rows, lens, final=fl, min_chunk=mc))
        # rows whose final entry was taken this call start a new request (the first listing
        # of a row is the one that counts)
        seen = set()
        for r, row in enumerate(rows.tolist()):
            if 0 <= row < B and row not in seen:
                seen.add(row)
                if fl[r]:
                    if rng.random() < 0.5:  # also harvest the whole finished response
                        d.harvest_finished(dev(np.array([row], np.int32)),
                                           dev(np.array([n[row]], np.int32)), dev(tok))
                        lc.ingest([tok[row, :n[row]].copy()])
                    n[row] = 0
        if step % 7 == 3:
            d.rebuild()
        snap = d.corpus_snapshot().cpu().numpy()
        assert np.array_equal(snap, lc.text()), f"step {step}: live corpus differs"
        if step % 5 == 4:
            q = rng.integers(0, V, size=(B, Sq)).astype(np.int32)
            qn = rng.integers(1, Sq + 1, size=B).astype(np.int32)
            qs = rng.integers(0, V, size=(B, 1)).astype(np.int32)
            dd, dn = d.propose(dev(qn), dev(q), dev(qs))
            torch.cuda.synchronize()
            ed, en = O.propose(O.params_from(KN), qn, q, qs, corpus=lc.text())
            assert np.array_equal(dd.cpu().numpy(), ed) and np.array_equal(dn.cpu().numpy(), en), \
                f"step {step}: drafts differ"
            checks += 1
    assert checks == 8
    if cap == 1500:
        assert lc.evicted() > 0
    d.close()


def test_inflight_argument_checks(S):
    d = S.Drafter(S.Config(max_batch=4, max_seq=8, max_sampled=1, corpus_capacity=100, **KN))
    rows = dev(np.zeros(1, np.int32))
    tok = dev(np.zeros((4, 8), np.int32))
    with pytest.raises(S.SfxError) as ei:
        d.ingest_inflight(rows, rows, tok, min_chunk=-1)
    assert ei.value.code == S.EINVAL
    big = dev(np.zeros(65537, np.int32))
    with pytest.raises(S.SfxError) as ei:
        d.ingest_inflight(big, big, tok)
    assert ei.value.code == S.ECAPACITY
    bare = S.Drafter(S.Config(max_batch=4, max_seq=8, max_sampled=1, corpus_capacity=0, **KN))
    with pytest.raises(S.SfxError) as ei:
        bare.ingest_inflight(rows, rows, tok)
    assert ei.value.code == S.ESTATE
    d.close()
    bare.close()
