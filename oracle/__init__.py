"""Plain CPU oracle of the suffix-match drafter (ctypes wrapper over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY.  The tests, the package smoke check, the benchmark's CPU-baseline
leg and ``alg_bytes.py`` (which writes the stored algorithmic bytes the benchmark reads) are its
only users; the GPU product path never imports it.  The arithmetic lives in ``oracle.c`` (plain
C loops written from the pages' definitions), ``alg_bytes.c`` (the instrumented word count of a
call) and ``corpus.py`` (the live-document bookkeeping of the shared corpus).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .accept import AcceptModel, picks_from_info  # noqa: F401
from .corpus import InflightIngest, LiveCorpus, harvest_docs  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

MODE_LONGEST_FILL = 0
MODE_SCORED = 1
MAX_NB = 8
# bit of a drafter config's `flags` that asks for the tree-depth cap (read by params_from)
TREE_DEPTH_CAP_FLAG = 4


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, OpenMP only to spread rows over threads)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-shared", "-fPIC",
               "-o", _SO + ".tmp", os.path.join(_HERE, "oracle.c"),
               os.path.join(_HERE, "alg_bytes.c")]
        subprocess.check_call(cmd)
        os.replace(_SO + ".tmp", _SO)
    return _SO


BUILD_FLAGS = "gcc -O2 -std=c11 -fopenmp"


class Params(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_int32),
        ("max_tree_depth", ctypes.c_int32),
        ("num_backoff", ctypes.c_int32),
        ("max_occurrences", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("min_self_match", ctypes.c_int32),
        ("min_corpus_match", ctypes.c_int32),
        ("tree_depth_cap", ctypes.c_int32),
        ("spec_factor_ppm", ctypes.c_int64),
        ("spec_offset_ppm", ctypes.c_int64),
        ("min_token_prob_ppm", ctypes.c_int64),
    ]


class RowInfo(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32),
        ("t", ctypes.c_int32),
        ("local_len", ctypes.c_int32 * MAX_NB),
        ("local_support", ctypes.c_int32 * MAX_NB),
        ("global_len", ctypes.c_int32 * MAX_NB),
        ("global_support", ctypes.c_int32 * MAX_NB),
        ("chosen", ctypes.c_int32),
        ("chosen_len", ctypes.c_int32),
        ("c0", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("snum", ctypes.c_int64),
    ]


_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        L.orc_context.restype = ctypes.c_int32
        L.orc_context.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P, _I32P,
                                  _I32P, _I32P]
        L.orc_match_back.restype = None
        L.orc_match_back.argtypes = [_I32P, ctypes.c_int32, ctypes.c_int32, _I32P]
        L.orc_corpus_match.restype = None
        L.orc_corpus_match.argtypes = [_I32P, ctypes.c_int64, _I32P, ctypes.c_int32,
                                       ctypes.c_int32, _I32P]
        L.orc_kth_largest.restype = ctypes.c_int32
        L.orc_kth_largest.argtypes = [_I32P, ctypes.c_int64, ctypes.c_int32]
        L.orc_count_at_least.restype = ctypes.c_int64
        L.orc_count_at_least.argtypes = [_I32P, ctypes.c_int64, ctypes.c_int32]
        L.orc_first_sites.restype = ctypes.c_int32
        L.orc_first_sites.argtypes = [_I32P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      _I32P]
        L.orc_spec_cap.restype = ctypes.c_int32
        L.orc_spec_cap.argtypes = [ctypes.POINTER(Params), ctypes.c_int32]
        L.orc_expand.restype = ctypes.c_int32
        L.orc_expand.argtypes = [_I32P, ctypes.c_int64, _I32P, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int64, _I32P, _I32P, _I64P]
        L.orc_propose.restype = ctypes.c_int
        L.orc_propose.argtypes = [ctypes.POINTER(Params), ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, _I32P, _I32P, _I32P, _I32P, ctypes.c_int64,
                                  _I32P, _I32P, ctypes.POINTER(RowInfo), ctypes.c_int32]
        L.orc_update_state.restype = None
        L.orc_update_state.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P,
                                       _I32P, _I32P, _I32P]
        L.orc_suffix_array.restype = ctypes.c_int
        L.orc_suffix_array.argtypes = [_I32P, ctypes.c_int64, _I32P]
        L.orc_alg_words.restype = ctypes.c_int
        L.orc_alg_words.argtypes = [ctypes.POINTER(Params), ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _I32P, _I32P, _I32P, _I32P, ctypes.c_int64,
                                    _I32P, _I64P, ctypes.c_int32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_I32P)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def make_params(k, max_tree_depth=24, num_backoff=1, max_occurrences=128, mode=MODE_LONGEST_FILL,
                min_self_match=1, min_corpus_match=2, spec_factor_ppm=1_000_000,
                spec_offset_ppm=0, min_token_prob_ppm=100_000, tree_depth_cap=0) -> Params:
    return Params(k, max_tree_depth, num_backoff, max_occurrences, mode, min_self_match,
                  min_corpus_match, int(bool(tree_depth_cap)), spec_factor_ppm, spec_offset_ppm,
                  min_token_prob_ppm)


def params_from(cfg) -> Params:
    """Build oracle parameters from any object/dict with the drafter knob names."""
    g = (lambda n, d=None: cfg.get(n, d)) if isinstance(cfg, dict) else \
        (lambda n, d=None: getattr(cfg, n, d))
    return make_params(g("k"), g("max_tree_depth", 24), g("num_backoff", 1),
                       g("max_occurrences", 128), g("mode", MODE_LONGEST_FILL),
                       g("min_self_match", 1), g("min_corpus_match", 2),
                       g("spec_factor_ppm", 1_000_000), g("spec_offset_ppm", 0),
                       g("min_token_prob_ppm", 100_000),
                       g("tree_depth_cap", 0) or (int(g("flags", 0) or 0) & TREE_DEPTH_CAP_FLAG))


# --------------------------------------------------------------------------- building blocks
def context(row, n, sampled, S=None):
    row = _i32(row)
    samp = _i32(sampled)
    S = len(row) if S is None else S
    ctx = np.zeros(S + len(samp) + 1, np.int32)
    t = ctypes.c_int32(0)
    L = lib().orc_context(S, len(samp), int(n), _p(row), _p(samp), _p(ctx), ctypes.byref(t))
    return ctx[:L].copy(), t.value


def match_back(ctx, D):
    ctx = _i32(ctx)
    L = len(ctx)
    mb = np.zeros(max(L - 1, 1), np.int32)
    lib().orc_match_back(_p(ctx), L, D, _p(mb))
    return mb[: max(L - 1, 0)]


def corpus_match(C, ctx, D):
    C = _i32(C)
    ctx = _i32(ctx)
    m = np.zeros(max(len(C), 1), np.int32)
    lib().orc_corpus_match(_p(C), len(C), _p(ctx), len(ctx), D, _p(m))
    return m[: len(C)]


def kth_largest(vals, t):
    v = _i32(vals)
    return lib().orc_kth_largest(_p(v) if len(v) else None, len(v), t)


def count_at_least(vals, l):
    v = _i32(vals)
    return lib().orc_count_at_least(_p(v) if len(v) else None, len(v), l)


def first_sites(vals, l, M):
    v = _i32(vals)
    out = np.zeros(max(M, 1), np.int32)
    c = lib().orc_first_sites(_p(v) if len(v) else None, len(v), l, M, _p(out))
    return out[:c].copy()


def spec_cap(params: Params, l):
    return lib().orc_spec_cap(ctypes.byref(params), l)


def expand(X, sites, cap, scored=False, min_prob_ppm=0):
    X = _i32(X)
    sites = _i32(sites)
    out = np.zeros(max(cap, 1), np.int32)
    counts = np.zeros(max(cap, 1), np.int32)
    snum = ctypes.c_int64(0)
    n = lib().orc_expand(_p(X), len(X), _p(sites) if len(sites) else None, len(sites), cap,
                         int(scored), int(min_prob_ppm), _p(out), _p(counts), ctypes.byref(snum))
    return out[:n].copy(), counts[:n].copy(), snum.value


# --------------------------------------------------------------------------- whole calls
def propose(params: Params, num_tokens, token_ids, sampled, corpus=None, num_threads=1,
            with_info=False):
    """Run the drafter on host arrays. token_ids [B,S], sampled [B,T], corpus 1-D or None."""
    tok = _i32(token_ids)
    samp = _i32(sampled)
    nt = _i32(num_tokens)
    B, S = tok.shape
    T = samp.shape[1] if samp.ndim == 2 else 0
    if samp.size == 0:
        samp = np.zeros((B, max(T, 1)), np.int32)
    draft = np.empty((B, params.k), np.int32)
    nv = np.empty(B, np.int32)
    info = (RowInfo * max(B, 1))() if with_info else None
    if corpus is not None and len(corpus):
        C = _i32(corpus)
        cp, N = _p(C), len(C)
    else:
        C, cp, N = None, None, 0
    rc = lib().orc_propose(ctypes.byref(params), B, S, T, _p(nt), _p(tok), _p(samp), cp, N,
                           _p(draft), _p(nv), info, num_threads)
    if rc != 0:
        raise ValueError("oracle rejected the parameters")
    if with_info:
        return draft, nv, [info[b] for b in range(B)]
    return draft, nv


def propose_masked(params: Params, num_tokens, token_ids, mask, corpus=None, num_threads=1):
    """The masked form (PyPI page "suffix-gpu 0.1.1", Quickstart: propose(num_tokens_no_spec,
    token_ids, combined_mask)): row b's context is token_ids[b, 0:clamp(n_b, 0, S)] alone, and
    rows with mask 0 get no draft.  Reading taken: otherwise the drafter step as usual, the
    context's last token taking the role of the last sampled id (fill, C-14)."""
    tok = _i32(token_ids)
    B, S = tok.shape
    n = np.clip(np.asarray(num_tokens, np.int64), 0, S)
    m = np.asarray(mask)
    prefix = np.zeros(B, np.int32)
    last = np.full((B, 1), -1, np.int32)
    for b in range(B):
        if m[b] != 0 and n[b] > 0:
            prefix[b] = n[b] - 1
            last[b, 0] = tok[b, n[b] - 1]
        else:
            prefix[b] = n[b]
    return propose(params, prefix, tok, last, corpus=corpus, num_threads=num_threads)


def propose_counts(params: Params, k, num_tokens, token_ids, sampled, counts, corpus=None,
                   num_threads=1):
    """The counted form (RFC page "[RFC]: Suffix decoding on GPU (suffix_gpu)", Design: the
    ngram_gpu contract propose(k, num_tokens_no_spec, token_ids, sampled, counts)).  Reading
    taken: counts[b], clamped to [0, T], is the number of valid entries of sampled[b] in place of
    the -1 padding, and k is the call's draft width (the spec cap of SCORED mode is taken
    against it)."""
    samp = _i32(sampled)
    B, T = samp.shape
    c = np.clip(np.asarray(counts, np.int64), 0, T)
    cut = np.where(np.arange(T)[None, :] < c[:, None], samp, -1).astype(np.int32)
    pk = Params()
    ctypes.memmove(ctypes.byref(pk), ctypes.byref(params), ctypes.sizeof(Params))
    pk.k = int(k)
    return propose(pk, num_tokens, token_ids, cut, corpus=corpus, num_threads=num_threads)


def update_state(token_ids, num_tokens, sampled):
    tok = _i32(token_ids).copy()
    samp = _i32(sampled)
    nt = _i32(num_tokens)
    B, S = tok.shape
    T = samp.shape[1]
    out = np.empty(B, np.int32)
    lib().orc_update_state(B, S, T, _p(tok), _p(nt), _p(samp), _p(out))
    return tok, out


ALG_CATEGORIES = ("context", "io", "sa_probes", "interval_scans", "voted_tokens")


def alg_words(params: Params, num_tokens, token_ids, sampled, corpus=None, sa=None,
              num_threads=1):
    """Words one call must touch, by category (alg_bytes.c); sa: the corpus's suffix array
    (computed here when not given)."""
    tok = _i32(token_ids)
    samp = _i32(sampled)
    nt = _i32(num_tokens)
    B, S = tok.shape
    T = samp.shape[1]
    out = np.zeros(5, np.int64)
    if corpus is not None and len(corpus):
        C = _i32(corpus)
        SA = _i32(sa) if sa is not None else suffix_array(C)
        cp, N, sp = _p(C), len(C), _p(SA)
    else:
        cp, N, sp = None, 0, None
    rc = lib().orc_alg_words(ctypes.byref(params), B, S, T, _p(nt), _p(tok), _p(samp), cp, N, sp,
                             out.ctypes.data_as(_I64P), num_threads)
    if rc != 0:
        raise ValueError("bad arguments")
    return dict(zip(ALG_CATEGORIES, (int(x) for x in out)))


def suffix_array(text):
    t = _i32(text)
    sa = np.empty(max(len(t), 1), np.int32)
    rc = lib().orc_suffix_array(_p(t) if len(t) else None, len(t), _p(sa))
    if rc != 0:
        raise ValueError("text too long")
    return sa[: len(t)].copy()
