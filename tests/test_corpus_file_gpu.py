"""Save and load of the corpus (suffix-gpu page, TODO: the cross-request global memory --
corpus ring, suffix array and delta -- persisted and restored across sessions).

A restored context must equal the saved one and the oracle on the live corpus, at once and after
further ingest and rebuilds.  The file is read here with numpy from the layout sfx.h documents,
independently of the library: its live tokens must be the oracle's live corpus, its suffix array
the oracle's suffix array of the saved index text, and its checksum the documented FNV-1a.
Corrupt, truncated or mismatched files are refused and leave the target context unchanged."""
import struct

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

KN = dict(k=6, max_tree_depth=8, num_backoff=3, max_occurrences=7, mode=1,
          spec_factor_ppm=3_000_000, min_token_prob_ppm=100_000)
CAP = 3000
V = 6


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


def make(S, cap=CAP):
    return S.Drafter(S.Config(max_batch=16, max_seq=256, max_sampled=1, corpus_capacity=cap,
                              **KN))


def batch(seed):
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, V, size=(16, 256)).astype(np.int32)
    n = rng.integers(0, 257, size=16).astype(np.int32)
    samp = rng.integers(0, V, size=(16, 1)).astype(np.int32)
    return n, tok, samp


def propose(d, inputs):
    import torch

    n, tok, samp = inputs
    dd, dn = d.propose(dev(n), dev(tok), dev(samp))
    torch.cuda.synchronize()
    return dd.cpu().numpy(), dn.cpu().numpy()


def expect(lc, inputs):
    n, tok, samp = inputs
    return O.propose(O.params_from(KN), n, tok, samp, corpus=lc.text())


def same(got, exp, what):
    assert np.array_equal(got[0], exp[0]) and np.array_equal(got[1], exp[1]), what


def docs_for(rng, count):
    return [rng.integers(0, V, size=int(rng.integers(0, 120))).astype(np.int32)
            for _ in range(count)]


def fill(d, lc, rng, steps):
    """Ingest in steps, rebuilding every third one; ends with documents in the delta."""
    for s in range(steps):
        docs = docs_for(rng, int(rng.integers(1, 12)))
        d.ingest_docs(docs)
        lc.ingest(docs)
        if s % 3 == 1:
            d.rebuild()


def fnv32(payload: bytes) -> int:
    h = 14695981039346656037
    for w in np.frombuffer(payload, "<u4"):
        h = ((h ^ int(w)) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def read_file(path):
    raw = open(path, "rb").read()
    cap, head, tail, dh, dt, s0, s1, checksum = struct.unpack("<7qQ", raw[8:72])
    nl, nd, ni = head - tail, dh - dt, s1 - s0
    off = 72
    live = np.frombuffer(raw, "<i4", nl, off)
    off += 4 * nl
    starts = np.frombuffer(raw, "<i8", nd, off)
    off += 8 * nd
    text = np.frombuffer(raw, "<i4", ni, off)
    off += 4 * ni
    sa = np.frombuffer(raw, "<i4", ni, off)
    off += 4 * ni
    return dict(raw=raw, magic=raw[:8], cap=cap, head=head, tail=tail, doc_head=dh, doc_tail=dt,
                snap=(s0, s1), checksum=checksum, live=live, starts=starts, text=text, sa=sa,
                size=off)


def write_file(path, f, live=None, starts=None, text=None, sa=None):
    """Re-encode a parsed file with some sections replaced and a correct checksum."""
    live = f["live"] if live is None else live
    starts = f["starts"] if starts is None else starts
    text = f["text"] if text is None else text
    sa = f["sa"] if sa is None else sa
    payload = (np.asarray(live, "<i4").tobytes() + np.asarray(starts, "<i8").tobytes()
               + np.asarray(text, "<i4").tobytes() + np.asarray(sa, "<i4").tobytes())
    head = struct.pack("<7qQ", f["cap"], f["head"], f["tail"], f["doc_head"], f["doc_tail"],
                       f["snap"][0], f["snap"][1], fnv32(payload))
    open(path, "wb").write(f["magic"] + head + payload)


def test_save_load_roundtrip(S, tmp_path):
    rng = np.random.default_rng(11)
    d, lc = make(S), O.LiveCorpus(CAP)
    fill(d, lc, rng, 14)
    extra = docs_for(rng, 4)  # documents in the delta, past the live index
    d.ingest_docs(extra)
    lc.ingest(extra)
    assert lc.evicted() > 0
    inputs = [batch(s) for s in (1, 2)]
    before = [propose(d, x) for x in inputs]
    for x, got in zip(inputs, before):
        same(got, expect(lc, x), "saved context vs oracle")
    path = str(tmp_path / "corpus.sfx")
    d.save(path)

    # the file, read independently: layout, live corpus, suffix array, checksum
    f = read_file(path)
    assert f["magic"] == b"SFXCORP1" and f["cap"] == CAP and f["size"] == len(f["raw"])
    assert np.array_equal(f["live"], lc.text())
    assert f["doc_head"] - f["doc_tail"] == int((lc.text() == -1).sum())
    assert f["starts"][0] == f["tail"]
    ends = np.nonzero(f["live"] == -1)[0] + f["tail"] + 1  # position after each separator
    assert np.array_equal(f["starts"][1:], ends[:-1])
    s0, s1 = f["snap"]
    assert 0 < s1 - s0 and s1 < f["head"], "the index should lag the delta"
    assert np.array_equal(f["sa"], O.suffix_array(f["text"].copy()))
    lo = max(s0, f["tail"])
    assert np.array_equal(f["text"][lo - s0:], f["live"][lo - f["tail"]:s1 - f["tail"]])
    assert f["checksum"] == fnv32(f["raw"][72:])

    # restored: same corpus, same drafts, now and after more ingest and rebuilds
    d2 = make(S)
    d2.load(path)
    assert np.array_equal(d2.corpus_snapshot().cpu().numpy(), lc.text())
    for x, got in zip(inputs, before):
        same(propose(d2, x), got, "restored context vs saved")
    for step in range(4):
        docs = docs_for(rng, 5)
        for dd in (d, d2):
            dd.ingest_docs(docs)
        lc.ingest(docs)
        if step % 2 == 0:
            d.rebuild()
            d2.rebuild()
        for x in inputs:
            exp = expect(lc, x)
            same(propose(d, x), exp, f"saved context, step {step}")
            same(propose(d2, x), exp, f"restored context, step {step}")
    # both rebuilt at the same point: their files are byte-identical
    d.rebuild()
    d2.rebuild()
    p1, p2 = str(tmp_path / "a.sfx"), str(tmp_path / "b.sfx")
    d.save(p1)
    d2.save(p2)
    assert open(p1, "rb").read() == open(p2, "rb").read()
    d.close()
    d2.close()


def test_save_during_async_rebuild_and_empty(S, tmp_path):
    rng = np.random.default_rng(12)
    d, lc = make(S), O.LiveCorpus(CAP)
    fill(d, lc, rng, 6)
    extra = docs_for(rng, 6)
    d.ingest_docs(extra)
    lc.ingest(extra)
    d.rebuild_async()
    path = str(tmp_path / "c.sfx")
    d.save(path)  # the rebuild in flight is not saved; its documents are in the saved delta
    d.wait_rebuild()
    d2 = make(S)
    d2.load(path)
    x = batch(3)
    exp = expect(lc, x)
    same(propose(d, x), exp, "source after its rebuild")
    same(propose(d2, x), exp, "restored from a save taken mid-rebuild")
    # an empty corpus round-trips too
    e, e2 = make(S), make(S)
    pe = str(tmp_path / "empty.sfx")
    e.save(pe)
    f = read_file(pe)
    assert f["head"] == f["tail"] == 0 and f["size"] == 72 == len(f["raw"])
    e2.ingest_docs(docs_for(rng, 3))
    e2.rebuild()
    e2.load(pe)
    assert e2.corpus_snapshot().numel() == 0
    same(propose(e2, x), expect(O.LiveCorpus(CAP), x), "restored empty corpus")
    for c in (d, d2, e, e2):
        c.close()


def test_load_refuses_bad_files(S, tmp_path):
    rng = np.random.default_rng(13)
    src, lc = make(S), O.LiveCorpus(CAP)
    fill(src, lc, rng, 8)
    path = str(tmp_path / "good.sfx")
    src.save(path)
    f = read_file(path)

    # the target keeps its own corpus through every refused load
    tgt, tlc = make(S), O.LiveCorpus(CAP)
    fill(tgt, tlc, np.random.default_rng(14), 5)
    x = batch(4)
    ref = propose(tgt, x)
    same(ref, expect(tlc, x), "target before")

    def refused(raw_or_writer, code, what):
        p = str(tmp_path / "bad.sfx")
        if callable(raw_or_writer):
            raw_or_writer(p)
        else:
            open(p, "wb").write(raw_or_writer)
        with pytest.raises(S.SfxError) as ei:
            tgt.load(p)
        assert ei.value.code == code, (what, str(ei.value))
        same(propose(tgt, x), ref, f"target unchanged after {what}")

    raw = f["raw"]
    refused(raw[:-4], S.EIO, "truncated")
    refused(raw[:40], S.EIO, "truncated header")
    refused(raw + b"\0\0\0\0", S.EIO, "trailing bytes")
    refused(b"XFXCORP1" + raw[8:], S.EIO, "bad magic")
    flipped = bytearray(raw)
    flipped[72] ^= 1
    refused(bytes(flipped), S.EIO, "checksum")
    hdr = bytearray(raw)
    hdr[16:24] = struct.pack("<q", f["tail"] - 1)  # head below tail
    refused(bytes(hdr), S.EIO, "inconsistent counters")
    # contents that pass the checksum but are not a valid corpus
    sa = f["sa"].copy()
    sa[0] = sa[1]
    refused(lambda p: write_file(p, f, sa=sa), S.EIO, "suffix array not a permutation")
    starts = f["starts"].copy()
    starts[1] += 1
    refused(lambda p: write_file(p, f, starts=starts), S.EIO, "document start off a separator")
    text = f["text"].copy()
    text[-2] = (text[-2] + 1) % V if text[-2] >= 0 else 0
    refused(lambda p: write_file(p, f, text=text), S.EIO, "index text differs from corpus")
    live = f["live"].copy()
    live[-1] = 0
    refused(lambda p: write_file(p, f, live=live), S.EIO, "unterminated last document")
    with pytest.raises(S.SfxError) as ei:
        make(S, cap=CAP + 1).load(path)
    assert ei.value.code == S.EINVAL
    with pytest.raises(S.SfxError) as ei:
        tgt.load(str(tmp_path / "missing.sfx"))
    assert ei.value.code == S.EIO
    # a rebuild in flight, and a context without a corpus
    tgt.rebuild_async()
    with pytest.raises(S.SfxError) as ei:
        tgt.load(path)
    assert ei.value.code == S.ESTATE
    tgt.wait_rebuild()
    bare = S.Drafter(S.Config(max_batch=1, max_seq=8, max_sampled=1, corpus_capacity=0, **KN))
    for call in (bare.save, bare.load):
        with pytest.raises(S.SfxError) as ei:
            call(path)
        assert ei.value.code == S.ESTATE
    # the good file still loads
    tgt.load(path)
    same(propose(tgt, x), expect(lc, x), "target after loading the good file")
    for c in (src, tgt, bare):
        c.close()
