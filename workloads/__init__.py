"""Seeded synthetic workloads for the suffix-match drafter.

This module only draws random inputs; it holds none of the drafter's arithmetic and is shared
by the tests, the benchmark and the smoke check.  The pages measure on Spec-Bench, GSM8K and
agentic traces, which are not available here; these generators stand in for them:

* rows imitate within-request repetition: a row is built segment by segment; with probability
  p_copy a span of U[8,64] tokens is copied from earlier in the same row, otherwise U[4,32]
  fresh tokens are drawn Zipf(s=1.1) over the vocabulary;
* the corpus imitates cross-request reuse: 2000 documents of U[200,800] tokens stitched from a
  pool of 500 shared template spans of U[16,128] tokens, with 20% of tokens replaced by fresh
  Zipf noise;
* the hot-4-gram variant imitates boilerplate-heavy traces (tool calls, agentic loops): rows and
  documents are made of short segments, each U[0,2] Zipf noise tokens, then one of 400 shared
  prefixes of U[2,8] tokens (drawn Zipf(s=1.1) over the pool), then one fixed 4-gram H; every
  request's context ends with a prefix and H.  The 1M-token corpus then holds H over 10^5
  times.

All ranges are inclusive.  Randomness is numpy PCG64 seeded by SeedSequence(1000 + config id),
spawned into independent streams (lengths, rows, templates, documents, ingest).
"""
from __future__ import annotations

import dataclasses
from functools import lru_cache

import numpy as np

POISON = -7  # fills the unused tail of every row; never part of any context


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    B: int
    S: int
    T: int
    n_lo: int
    n_hi: int
    V: int
    p_copy: float
    corpus: bool
    # drafter knobs
    k: int
    max_tree_depth: int
    num_backoff: int
    max_occurrences: int
    mode: int  # 0 longest-match + fill, 1 scored
    spec_factor_ppm: int = 1_000_000
    spec_offset_ppm: int = 0
    min_token_prob_ppm: int = 100_000
    min_self_match: int = 1
    min_corpus_match: int = 2
    # ingest under load
    ring_capacity: int = 0
    ingest_rows: int = 0
    ingest_len_lo: int = 0
    ingest_len_hi: int = 0
    ingest_S: int = 0

    def knobs(self) -> dict:
        return dict(k=self.k, max_tree_depth=self.max_tree_depth, num_backoff=self.num_backoff,
                    max_occurrences=self.max_occurrences, mode=self.mode,
                    spec_factor_ppm=self.spec_factor_ppm, spec_offset_ppm=self.spec_offset_ppm,
                    min_token_prob_ppm=self.min_token_prob_ppm,
                    min_self_match=self.min_self_match, min_corpus_match=self.min_corpus_match)


WORKLOADS = {
    1: Workload(1, "self-B4-S512-V1024", B=4, S=512, T=1, n_lo=128, n_hi=512, V=1024, p_copy=0.5,
                corpus=False, k=8, max_tree_depth=24, num_backoff=1, max_occurrences=128, mode=0),
    2: Workload(2, "self-B64-S4096-V32000", B=64, S=4096, T=1, n_lo=1024, n_hi=4096, V=32000,
                p_copy=0.5, corpus=False, k=8, max_tree_depth=24, num_backoff=1,
                max_occurrences=128, mode=0),
    3: Workload(3, "self+corpus-B64-S4096-V32000", B=64, S=4096, T=1, n_lo=1024, n_hi=4096,
                V=32000, p_copy=0.5, corpus=True, k=8, max_tree_depth=24, num_backoff=1,
                max_occurrences=128, mode=0),
    4: Workload(4, "scored-B256-S16384-V151936-corpus1M", B=256, S=16384, T=1, n_lo=4096,
                n_hi=16384, V=151936, p_copy=0.6, corpus=True, k=16, max_tree_depth=24,
                num_backoff=4, max_occurrences=128, mode=1, spec_factor_ppm=2_000_000,
                spec_offset_ppm=0, min_token_prob_ppm=100_000),
    5: Workload(5, "ingest-ring4M-B512-S32768-V151936", B=512, S=32768, T=1, n_lo=8192,
                n_hi=32768, V=151936, p_copy=0.6, corpus=True, k=32, max_tree_depth=24,
                num_backoff=4, max_occurrences=128, mode=1, spec_factor_ppm=2_000_000,
                spec_offset_ppm=0, min_token_prob_ppm=100_000, ring_capacity=1 << 22,
                ingest_rows=256, ingest_len_lo=512, ingest_len_hi=2048, ingest_S=2048),
    6: Workload(6, "hot4gram-B256-S16384-V151936-corpus1M", B=256, S=16384, T=1, n_lo=4096,
                n_hi=16384, V=151936, p_copy=0.6, corpus=True, k=16, max_tree_depth=24,
                num_backoff=4, max_occurrences=128, mode=1, spec_factor_ppm=2_000_000,
                spec_offset_ppm=0, min_token_prob_ppm=100_000),
}

N_TEMPLATES = 500
TEMPLATE_LO, TEMPLATE_HI = 16, 128
N_DOCS = 2000
DOC_LO, DOC_HI = 200, 800
NOISE = 0.2


@lru_cache(maxsize=8)
def zipf_cdf(V: int, s: float = 1.1) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def zipf(rng: np.random.Generator, V: int, size: int) -> np.ndarray:
    """Token ids with P(id = r-1) proportional to r^-1.1, r = 1..V (inverse CDF)."""
    u = rng.random(size)
    t = np.searchsorted(zipf_cdf(V), u, side="right")
    return np.minimum(t, V - 1).astype(np.int32)


def gen_row(rng: np.random.Generator, length: int, V: int, p_copy: float) -> np.ndarray:
    out = np.empty(length + 64, np.int32)
    m0 = int(rng.integers(4, 33))
    out[:m0] = zipf(rng, V, m0)
    n = m0
    while n < length:
        if rng.random() < p_copy:
            m = int(rng.integers(8, 65))
            if n >= m:
                s = int(rng.integers(0, n - m + 1))
                if n + m > len(out):
                    out = np.concatenate([out, np.empty(len(out), np.int32)])
                out[n:n + m] = out[s:s + m]
                n += m
                continue
        m = int(rng.integers(4, 33))
        if n + m > len(out):
            out = np.concatenate([out, np.empty(len(out), np.int32)])
        out[n:n + m] = zipf(rng, V, m)
        n += m
    return out[:length].copy()


def _streams(cid: int, n: int = 5):
    ss = np.random.SeedSequence(1000 + cid)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


HOT_PREFIXES = 400
HOT_PREFIX_LO, HOT_PREFIX_HI = 2, 8
HOT_NOISE_HI = 2
HOT_DOCS = 2000


def hot_gram(V: int) -> np.ndarray:
    """The fixed boilerplate 4-gram of the hot-4-gram workload (four distinct mid-range ids)."""
    return np.array([V // 7 + 11, V // 5 + 13, V // 3 + 17, V // 2 + 19], np.int32)


@lru_cache(maxsize=2)
def hot_prefixes(V: int):
    r = _streams(6)[2]
    return [zipf(r, V, int(r.integers(HOT_PREFIX_LO, HOT_PREFIX_HI + 1)))
            for _ in range(HOT_PREFIXES)]


def hot_row(rng: np.random.Generator, length: int, V: int, p_copy: float) -> np.ndarray:
    """A row of boilerplate segments (noise, a shared prefix, the hot 4-gram), with spans copied
    from earlier in the row as gen_row does, ending with a prefix and the 4-gram."""
    H, pre = hot_gram(V), hot_prefixes(V)
    parts, n = [], 0
    while n < length:
        if n >= 8 and rng.random() < p_copy:
            m = int(rng.integers(8, 65))
            if n >= m:
                row = np.concatenate(parts)
                s = int(rng.integers(0, n - m + 1))
                parts = [row, row[s:s + m].copy()]
                n += m
                continue
        seg = [zipf(rng, V, int(rng.integers(0, HOT_NOISE_HI + 1))),
               pre[int(zipf(rng, HOT_PREFIXES, 1)[0])], H]
        parts.extend(seg)
        n += sum(len(x) for x in seg)
    row = np.concatenate(parts)[:length].copy()
    tail = np.concatenate([pre[int(zipf(rng, HOT_PREFIXES, 1)[0])], H])
    m = min(len(tail), length)
    row[length - m:] = tail[len(tail) - m:]
    return row


def make_batch(cid: int, set_index: int = 0, B: int | None = None):
    """Propose inputs for workload cid: (num_tokens [B], token_ids [B,S], sampled [B,T]).

    set_index selects an independent input set (used to rotate buffers in the benchmark)."""
    w = WORKLOADS[cid]
    B = w.B if B is None else B
    ss = np.random.SeedSequence([1000 + cid, 17, set_index])
    r_len, r_row = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(2)]
    n = r_len.integers(w.n_lo, w.n_hi + 1, size=B).astype(np.int32)
    tok = np.full((B, w.S), POISON, np.int32)
    samp = np.full((B, w.T), -1, np.int32)
    gen = hot_row if cid == 6 else gen_row
    for b in range(B):
        row = gen(r_row, int(n[b]) + w.T, w.V, w.p_copy)
        tok[b, : n[b]] = row[: n[b]]
        samp[b, :] = row[n[b]: n[b] + w.T]
    return n, tok, samp


def template_docs(V: int, cid: int = 4):
    """The 2000 template-stitched documents (without separators)."""
    _, _, r_tpl, r_doc, _ = _streams(cid)
    tpls = [zipf(r_tpl, V, int(r_tpl.integers(TEMPLATE_LO, TEMPLATE_HI + 1)))
            for _ in range(N_TEMPLATES)]
    docs = []
    for _ in range(N_DOCS):
        target = int(r_doc.integers(DOC_LO, DOC_HI + 1))
        parts, got = [], 0
        while got < target:
            t = tpls[int(r_doc.integers(0, N_TEMPLATES))]
            parts.append(t)
            got += len(t)
        d = np.concatenate(parts)[:target].copy()
        mask = r_doc.random(target) < NOISE
        d[mask] = zipf(r_doc, V, int(mask.sum()))
        docs.append(d.astype(np.int32))
    return docs


def hot_docs(V: int):
    """The hot-4-gram corpus: HOT_DOCS documents of U[200,800] tokens made of boilerplate
    segments (without separators)."""
    r = _streams(6)[3]
    H, pre = hot_gram(V), hot_prefixes(V)
    docs = []
    for _ in range(HOT_DOCS):
        target = int(r.integers(DOC_LO, DOC_HI + 1))
        parts, got = [], 0
        while got < target:
            seg = [zipf(r, V, int(r.integers(0, HOT_NOISE_HI + 1))),
                   pre[int(zipf(r, HOT_PREFIXES, 1)[0])], H]
            parts.extend(seg)
            got += sum(len(x) for x in seg)
        docs.append(np.concatenate(parts)[:target].astype(np.int32))
    return docs


def join_docs(docs) -> np.ndarray:
    parts = []
    for d in docs:
        parts.append(np.asarray(d, np.int32))
        parts.append(np.array([-1], np.int32))
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


def corpus_docs(cid: int):
    """Corpus documents of a workload (configs 3/4/5), or [] when it has no corpus."""
    w = WORKLOADS[cid]
    if not w.corpus:
        return []
    if cid == 6:
        return hot_docs(w.V)
    return template_docs(w.V, cid=3 if cid == 3 else 4)


def ingest_batch(cid: int, step: int):
    """Finished rows harvested at one step of the ingest workload:
    (token_ids [R, ingest_S], row_indices [R], lengths [R])."""
    w = WORKLOADS[cid]
    ss = np.random.SeedSequence([1000 + cid, 29, step])
    r = np.random.Generator(np.random.PCG64(ss))
    R = w.ingest_rows
    lengths = r.integers(w.ingest_len_lo, w.ingest_len_hi + 1, size=R).astype(np.int32)
    tok = np.full((R, w.ingest_S), POISON, np.int32)
    for i in range(R):
        tok[i, : lengths[i]] = gen_row(r, int(lengths[i]), w.V, w.p_copy)
    rows = np.arange(R, dtype=np.int32)
    return tok, rows, lengths
