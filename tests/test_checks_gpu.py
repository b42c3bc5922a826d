"""Optional input checks and the sticky device error word (RFC page "[RFC]: Suffix decoding on
GPU (suffix_gpu)", Design: the drafter runs on device tensors without host synchronisation, so
lengths the host cannot see are clamped on the device; the checks report such inputs).

With SFX_FLAG_CHECK_INPUTS each call sets the documented bit for every clamped or ignored
input, the bits accumulate until sfx_debug_errors reads and clears them, and results equal
those of a context without the flag (and the oracle's on the clamped inputs).  Without the flag
the word stays 0."""
import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

KN = dict(k=6, max_tree_depth=8, num_backoff=3, max_occurrences=16, mode=1,
          spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
B, SQ, T, V = 8, 64, 2, 5


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


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def make(S, flags, cap=4096):
    return S.Drafter(S.Config(max_batch=B, max_seq=SQ, max_sampled=T, corpus_capacity=cap,
                              flags=flags, **KN))


def clean_inputs(seed):
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, V, size=(B, SQ)).astype(np.int32)
    n = rng.integers(0, SQ + 1, size=B).astype(np.int32)
    samp = rng.integers(0, V, size=(B, T)).astype(np.int32)
    samp[1, 1] = -1  # trailing padding is not an error
    return n, tok, samp


def docs(seed):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, V, size=int(rng.integers(1, 50))).astype(np.int32) for _ in range(20)]


def test_clean_inputs_raise_nothing(S):
    d = make(S, S.FLAG_CHECK_INPUTS)
    d.ingest_docs(docs(1))
    d.rebuild()
    n, tok, samp = clean_inputs(2)
    d.propose(dev(n), dev(tok), dev(samp))
    d.propose_masked(dev(n), dev(tok), dev(np.ones(B, np.int32)))
    d.propose_counts(4, dev(n), dev(tok), dev(samp), dev(np.full(B, T, np.int32)))
    d.harvest_finished(dev(np.arange(3, dtype=np.int32)), dev(n[:3]), dev(tok))
    d.ingest_inflight(dev(np.arange(B, dtype=np.int32)), dev(n), dev(tok))
    assert d.debug_errors() == 0
    d.close()


def test_propose_bits_and_unchanged_results(S):
    n, tok, samp = clean_inputs(3)
    n[2], n[5] = SQ + 7, -4
    samp[3] = [-1, 2]  # a valid id after the padding: ignored
    checked, plain = make(S, S.FLAG_CHECK_INPUTS), make(S, 0)
    lc = O.LiveCorpus(4096)
    for x in (checked, plain):
        x.ingest_docs(docs(4))
        x.rebuild()
    lc.ingest(docs(4))
    outs = []
    for x in (checked, plain):
        dd, dn = x.propose(dev(n), dev(tok), dev(samp))
        outs.append((host(dd), host(dn)))
    ed, en = O.propose(O.params_from(KN), n, tok, samp, corpus=lc.text())
    for dd, dn in outs:
        assert np.array_equal(dd, ed) and np.array_equal(dn, en)
    assert checked.debug_errors() == S.ERR_LENGTH | S.ERR_SAMPLED_AFTER_PAD
    assert checked.debug_errors() == 0, "the read clears the word"
    assert plain.debug_errors() == 0, "no checks without the flag"
    # sticky: bits of several calls accumulate until read
    n2 = np.clip(n, 0, SQ)
    checked.propose(dev(n2), dev(tok), dev(samp))
    tok2 = tok.copy()
    tok2[0, max(int(n2[0]) - 1, 0)] = -3
    n3 = n2.copy()
    n3[0] = max(int(n2[0]), 1)
    checked.propose(dev(n3), dev(tok2), dev(np.clip(samp, 0, None)))
    assert checked.debug_errors() == S.ERR_SAMPLED_AFTER_PAD | S.ERR_NEGATIVE_TOKEN
    # a negative id past the row prefix is not read, so it is no error
    tok3 = np.clip(tok, 0, None)
    n4 = np.full(B, SQ // 2, np.int32)
    tok3[:, SQ // 2:] = -9
    checked.propose(dev(n4), dev(tok3), dev(np.clip(samp, 0, None)))
    assert checked.debug_errors() == 0
    checked.close()
    plain.close()


def test_other_call_forms(S):
    d = make(S, S.FLAG_CHECK_INPUTS)
    n, tok, samp = clean_inputs(5)
    d.propose_masked(dev(np.where(np.arange(B) == 1, SQ + 1, n).astype(np.int32)), dev(tok),
                     dev(np.ones(B, np.int32)))
    assert d.debug_errors() == S.ERR_LENGTH
    s2 = samp.copy()
    s2[4] = [-1, 3]
    cnt = np.full(B, T, np.int32)
    cnt[4] = 1  # the id after the padding does not count: no error
    d.propose_counts(4, dev(n), dev(tok), dev(s2), dev(cnt))
    assert d.debug_errors() == 0
    cnt[4] = 2
    d.propose_counts(4, dev(n), dev(tok), dev(s2), dev(cnt))
    assert d.debug_errors() == S.ERR_SAMPLED_AFTER_PAD
    cnt[4], cnt[6] = 1, T + 1
    d.propose_counts(4, dev(n), dev(tok), dev(s2), dev(cnt))
    assert d.debug_errors() == S.ERR_LENGTH
    d.close()


def test_ingest_bits(S):
    d = make(S, S.FLAG_CHECK_INPUTS)
    _, tok, _ = clean_inputs(6)
    rows = np.array([0, B + 2, 3], np.int32)
    d.harvest_finished(dev(rows), dev(np.array([5, 5, 5], np.int32)), dev(tok))
    assert d.debug_errors() == S.ERR_ROW_INDEX
    d.harvest_finished(dev(rows[:1]), dev(np.array([SQ + 1], np.int32)), dev(tok))
    assert d.debug_errors() == S.ERR_LENGTH
    d.ingest_inflight(dev(np.array([1, -1], np.int32)), dev(np.array([4, 4], np.int32)),
                      dev(tok))
    assert d.debug_errors() == S.ERR_ROW_INDEX
    d.ingest_inflight(dev(np.array([2], np.int32)), dev(np.array([-2], np.int32)), dev(tok))
    assert d.debug_errors() == S.ERR_LENGTH
    # the corpus got exactly the documented (clamped) documents
    lc = O.LiveCorpus(4096)
    lc.ingest([tok[0, :5], np.zeros(0, np.int32), tok[3, :5], tok[0, :SQ], tok[1, :4]])
    assert np.array_equal(host(d.corpus_snapshot()), lc.text())
    d.close()


def test_negative_ids_in_documents(S):
    """Documents with negative ids are reported (the context is closed without proposing)."""
    d = make(S, S.FLAG_CHECK_INPUTS)
    _, tok, _ = clean_inputs(7)
    tok[2, 3] = -6
    d.harvest_finished(dev(np.array([2], np.int32)), dev(np.array([10], np.int32)), dev(tok))
    assert d.debug_errors() == S.ERR_NEGATIVE_TOKEN
    d.harvest_finished(dev(np.array([2], np.int32)), dev(np.array([3], np.int32)), dev(tok))
    assert d.debug_errors() == 0, "the negative id is past the document"
    import torch

    toks = torch.tensor([1, 2, -4, 3, 0, 1], dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, 2, 4, 3, 6], dtype=torch.int64, device="cuda")  # 4 -> 3 decreases
    assert S.load().sfx_ingest(d._h, 4, S._ptr(offs), S._ptr(toks), S._stream(None)) == S.OK
    assert d.debug_errors() == S.ERR_NEGATIVE_TOKEN | S.ERR_LENGTH
    d.close()


def test_debug_errors_without_flag(S):
    d = make(S, 0, cap=0)
    n, tok, samp = clean_inputs(8)
    n[0] = -1
    d.propose(dev(n), dev(tok), dev(samp))
    assert d.debug_errors() == 0
    d.close()
