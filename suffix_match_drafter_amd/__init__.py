"""suffix_match_drafter_amd -- MI355X (gfx950) suffix-match drafter.

Thin ctypes binding over ``libsfx.so`` (C-ABI in ``include/sfx.h``).  This module only
marshals arguments: every step of the drafter runs in the library's HIP kernels.  PyTorch is
used for device memory and streams.  There is no CPU fallback: if the library is missing the
calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsfx.so")

MODE_LONGEST_FILL = 0
MODE_SCORED = 1

OK, EINVAL, ENOMEM, ECAPACITY, EHIP, ESTATE, EIO = 0, -1, -2, -3, -4, -5, -6
_NAMES = {EINVAL: "EINVAL", ENOMEM: "ENOMEM", ECAPACITY: "ECAPACITY", EHIP: "EHIP",
          ESTATE: "ESTATE", EIO: "EIO"}

# every entry point declared in include/sfx.h
EXPORTS = ("sfx_create", "sfx_destroy", "sfx_last_error", "sfx_propose", "sfx_propose_masked",
           "sfx_propose_counts",
           "sfx_update_state", "sfx_harvest_finished", "sfx_ingest_inflight", "sfx_ingest",
           "sfx_rebuild", "sfx_rebuild_async", "sfx_poll", "sfx_wait_rebuild",
           "sfx_accept_estimate", "sfx_accept_feedback", "sfx_accept_reset", "sfx_accept_counts",
           "sfx_corpus_snapshot", "sfx_save", "sfx_load", "sfx_debug_errors",
           "sfx_debug_fail_next_rebuild", "sfx_debug_index", "sfx_rebuild_stats",
           "sfx_suffix_array_workspace_bytes", "sfx_build_suffix_array",
           "sfx_build_suffix_array_noalloc", "sfx_graphs_create", "sfx_graphs_propose",
           "sfx_graphs_stats", "sfx_graphs_destroy")


FLAG_STREAM_CONTEXT = 1  # read contexts from device memory instead of staging them in LDS
FLAG_CHECK_INPUTS = 2    # check device-resident inputs into the sticky error word
FLAG_TREE_DEPTH_CAP = 4  # match length plus draft length at most max_tree_depth

# flags of a batch-bucketed graph set (include/sfx.h)
GRAPHS_EAGER = 1             # capture nothing: every call runs eagerly
GRAPHS_UPDATE_STATE = 2      # the chain ends with the state update
GRAPHS_DELTA_INDEX = 4       # every chain groups the delta by tail pair first
GRAPHS_DEBUG_BREAK_ODD = 8   # test hook: captures of odd-indexed buckets fail

# bits of the sticky error word (include/sfx.h)
ERR_LENGTH, ERR_NEGATIVE_TOKEN, ERR_SAMPLED_AFTER_PAD, ERR_ROW_INDEX = 1, 2, 4, 8
ERR_SYNC_TIMEOUT = 16    # a propose workgroup's bounded internal wait ran out


class SfxError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_int32),
        ("max_tree_depth", ctypes.c_int32),
        ("num_backoff", ctypes.c_int32),
        ("max_occurrences", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("min_self_match", ctypes.c_int32),
        ("min_corpus_match", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_seq", ctypes.c_int32),
        ("max_sampled", ctypes.c_int32),
        ("spec_factor_ppm", ctypes.c_int64),
        ("spec_offset_ppm", ctypes.c_int64),
        ("min_token_prob_ppm", ctypes.c_int64),
        ("corpus_capacity", ctypes.c_int64),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


@dataclasses.dataclass
class Config:
    k: int
    max_tree_depth: int = 24
    num_backoff: int = 1
    max_occurrences: int = 128
    mode: int = MODE_LONGEST_FILL
    min_self_match: int = 1
    min_corpus_match: int = 2
    max_batch: int = 256
    max_seq: int = 16384
    max_sampled: int = 1
    spec_factor_ppm: int = 1_000_000
    spec_offset_ppm: int = 0
    min_token_prob_ppm: int = 100_000
    corpus_capacity: int = 0
    flags: int = 0
    reserved: int = 0

    def _c(self) -> _Config:
        return _Config(*[getattr(self, f[0]) for f in _Config._fields_])


_V = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_lib = None


def load(path: str = LIB_PATH):
    """Load libsfx.so (torch is imported first so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m suffix_match_drafter_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    sig = {
        "sfx_create": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_V)]),
        "sfx_destroy": (None, [_V]),
        "sfx_last_error": (ctypes.c_char_p, []),
        "sfx_propose": (ctypes.c_int, [_V, _I32, _I32, _I32, _V, _V, _V, _V, _V, _V]),
        "sfx_propose_masked": (ctypes.c_int, [_V, _I32, _I32, _V, _V, _V, _V, _V, _V]),
        "sfx_propose_counts": (ctypes.c_int, [_V, _I32, _I32, _I32, _I32, _V, _V, _V, _V, _V,
                                              _V, _V]),
        "sfx_update_state": (ctypes.c_int, [_I32, _I32, _I32, _V, _V, _V, _V, _V]),
        "sfx_harvest_finished": (ctypes.c_int, [_V, _I32, _V, _V, _V, _I32, _I32, _V]),
        "sfx_ingest": (ctypes.c_int, [_V, _I32, _V, _V, _V]),
        "sfx_ingest_inflight": (ctypes.c_int, [_V, _I32, _V, _V, _V, _V, _I32, _I32, _I32, _V]),
        "sfx_rebuild": (ctypes.c_int, [_V, _V]),
        "sfx_rebuild_async": (ctypes.c_int, [_V, _V]),
        "sfx_poll": (ctypes.c_int, [_V, ctypes.POINTER(_I32), _V]),
        "sfx_wait_rebuild": (ctypes.c_int, [_V, _V]),
        "sfx_corpus_snapshot": (ctypes.c_int, [_V, _V, _I64, ctypes.POINTER(_I64), _V]),
        "sfx_accept_estimate": (ctypes.c_int, [_V, _I32, _V, _V]),
        "sfx_accept_feedback": (ctypes.c_int, [_V, _I32, _V, _V]),
        "sfx_accept_reset": (ctypes.c_int, [_V, _V]),
        "sfx_accept_counts": (ctypes.c_int, [_V, _V, _V]),
        "sfx_save": (ctypes.c_int, [_V, ctypes.c_char_p, _V]),
        "sfx_load": (ctypes.c_int, [_V, ctypes.c_char_p, _V]),
        "sfx_debug_errors": (ctypes.c_int, [_V, ctypes.POINTER(ctypes.c_uint32), _V]),
        "sfx_debug_fail_next_rebuild": (ctypes.c_int, [_V]),
        "sfx_debug_index": (ctypes.c_int, [_V, _V, _V, _I64, ctypes.POINTER(_I64), _V]),
        "sfx_rebuild_stats": (ctypes.c_int, [_V, ctypes.POINTER(_I32), ctypes.POINTER(_I64)]),
        "sfx_suffix_array_workspace_bytes": (ctypes.c_size_t, [_I64]),
        "sfx_build_suffix_array": (ctypes.c_int, [_V, _I64, _V, _V, ctypes.c_size_t, _V]),
        "sfx_build_suffix_array_noalloc": (ctypes.c_int, [_V, _I64, _V, _V]),
        "sfx_graphs_create": (ctypes.c_int, [_V, _I32, ctypes.POINTER(_I32), _I32, _I32, _V, _V,
                                             _V, _V, _V, _V, _I32, _V, ctypes.POINTER(_V)]),
        "sfx_graphs_propose": (ctypes.c_int, [_V, _I32, _V]),
        "sfx_graphs_stats": (ctypes.c_int, [_V, ctypes.POINTER(_I32),
                                            ctypes.POINTER(ctypes.c_uint64),
                                            ctypes.POINTER(ctypes.c_uint64),
                                            ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
        "sfx_graphs_destroy": (None, [_V]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc):
    if rc != OK:
        raise SfxError(rc, load().sfx_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _V(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _i32(t: torch.Tensor, name: str, ndim: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda:
        raise TypeError(f"{name} must be an int32 CUDA/HIP tensor")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D tensor")
    return t


def _ptr(t):
    return _V(t.data_ptr()) if t is not None and t.numel() else _V(0)


class Drafter:
    """One drafter context: configuration, corpus ring and double-buffered corpus index."""

    def __init__(self, cfg: Config):
        L = load()
        self.cfg = cfg
        h = _V()
        _check(L.sfx_create(ctypes.byref(cfg._c()), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            load().sfx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def propose(self, num_tokens, token_ids, sampled, draft=None, num_valid=None, stream=None):
        tok = _i32(token_ids, "token_ids", 2)
        B, S = tok.shape
        samp = _i32(sampled, "sampled", 2)
        nt = _i32(num_tokens, "num_tokens_no_spec", 1)
        if samp.shape[0] != B or nt.shape[0] != B:
            raise ValueError("batch sizes differ")
        if draft is None:
            draft = torch.empty((B, self.cfg.k), dtype=torch.int32, device=tok.device)
        if num_valid is None:
            num_valid = torch.empty((B,), dtype=torch.int32, device=tok.device)
        _i32(draft, "draft", 2)
        _i32(num_valid, "num_valid", 1)
        if draft.shape != (B, self.cfg.k) or num_valid.shape != (B,):
            raise ValueError("draft must be [B,k] and num_valid [B]")
        _check(load().sfx_propose(self._h, B, S, samp.shape[1], _ptr(nt), _ptr(tok), _ptr(samp),
                                  _ptr(draft), _ptr(num_valid), _stream(stream)))
        return draft, num_valid

    def propose_masked(self, num_tokens, token_ids, mask, draft=None, num_valid=None,
                       stream=None):
        """The masked form: contexts are the rows themselves; rows with mask 0 get no draft."""
        tok = _i32(token_ids, "token_ids", 2)
        B, S = tok.shape
        nt = _i32(num_tokens, "num_tokens_no_spec", 1)
        m = _i32(mask, "mask", 1)
        if nt.shape[0] != B or m.shape[0] != B:
            raise ValueError("num_tokens_no_spec, mask and token_ids disagree on B")
        if draft is None:
            draft = torch.empty((B, self.cfg.k), dtype=torch.int32, device=tok.device)
        if num_valid is None:
            num_valid = torch.empty((B,), dtype=torch.int32, device=tok.device)
        _check(load().sfx_propose_masked(self._h, B, S, _ptr(nt), _ptr(tok), _ptr(m),
                                         _ptr(draft), _ptr(num_valid), _stream(stream)))
        return draft, num_valid

    def propose_counts(self, k, num_tokens, token_ids, sampled, counts, draft=None,
                       num_valid=None, stream=None):
        """The counted form: counts[b] valid entries of sampled[b]; drafts of width k."""
        tok = _i32(token_ids, "token_ids", 2)
        B, S = tok.shape
        samp = _i32(sampled, "sampled", 2)
        nt = _i32(num_tokens, "num_tokens_no_spec", 1)
        cnt = _i32(counts, "counts", 1)
        if samp.shape[0] != B or nt.shape[0] != B or cnt.shape[0] != B:
            raise ValueError("num_tokens_no_spec, token_ids, sampled and counts disagree on B")
        if draft is None:
            draft = torch.empty((B, k), dtype=torch.int32, device=tok.device)
        if num_valid is None:
            num_valid = torch.empty((B,), dtype=torch.int32, device=tok.device)
        _check(load().sfx_propose_counts(self._h, int(k), B, S, samp.shape[1], _ptr(nt),
                                         _ptr(tok), _ptr(samp), _ptr(cnt), _ptr(draft),
                                         _ptr(num_valid), _stream(stream)))
        return draft, num_valid

    def graphs(self, buckets, num_tokens, token_ids, sampled, draft, num_valid,
               num_tokens_out=None, flags=0, stream=None) -> "GraphSet":
        """Pre-capture the step for each batch bucket over these persistent buffers."""
        return GraphSet(self, buckets, num_tokens, token_ids, sampled, draft, num_valid,
                        num_tokens_out, flags, stream)

    def propose_with_update(self, num_tokens, token_ids, sampled, stream=None):
        draft, nv = self.propose(num_tokens, token_ids, sampled, stream=stream)
        new_n = update_state(token_ids, num_tokens, sampled, stream=stream)
        return draft, nv, new_n

    def harvest_finished(self, row_indices, lengths, token_ids, stream=None):
        rows = _i32(row_indices, "row_indices", 1)
        lens = _i32(lengths, "lengths", 1)
        tok = _i32(token_ids, "token_ids", 2)
        if rows.shape != lens.shape:
            raise ValueError("row_indices and lengths differ in size")
        _check(load().sfx_harvest_finished(self._h, rows.shape[0], _ptr(rows), _ptr(lens),
                                           _ptr(tok), tok.shape[0], tok.shape[1],
                                           _stream(stream)))

    def ingest_inflight(self, row_indices, lengths, token_ids, final=None, min_chunk=1,
                        stream=None):
        """Append each listed row's tokens past its ingest cursor as one document once at least
        min_chunk have accumulated; rows with final != 0 flush what is left and restart."""
        rows = _i32(row_indices, "row_indices", 1)
        lens = _i32(lengths, "lengths", 1)
        tok = _i32(token_ids, "token_ids", 2)
        if rows.shape != lens.shape:
            raise ValueError("row_indices and lengths differ in size")
        fin = None
        if final is not None:
            fin = _i32(final, "final", 1)
            if fin.shape != rows.shape:
                raise ValueError("final and row_indices differ in size")
        _check(load().sfx_ingest_inflight(self._h, rows.shape[0], _ptr(rows), _ptr(lens),
                                          _ptr(fin), _ptr(tok), tok.shape[0], tok.shape[1],
                                          int(min_chunk), _stream(stream)))

    def ingest(self, doc_offsets, tokens, stream=None):
        offs = doc_offsets
        if offs.dtype != torch.int64 or not offs.is_cuda or offs.dim() != 1:
            raise TypeError("doc_offsets must be a 1-D int64 CUDA/HIP tensor")
        tok = _i32(tokens, "tokens", 1)
        _check(load().sfx_ingest(self._h, offs.shape[0] - 1, _ptr(offs), _ptr(tok),
                                 _stream(stream)))

    def ingest_docs(self, docs, stream=None):
        """Convenience: ingest a list of 1-D int sequences (host) as packed documents."""
        import numpy as np

        lens = [len(d) for d in docs]
        offs = np.zeros(len(docs) + 1, np.int64)
        offs[1:] = np.cumsum(lens)
        flat = np.concatenate([np.asarray(d, np.int32) for d in docs]) if docs else \
            np.zeros(0, np.int32)
        dev = torch.device("cuda")
        self.ingest(torch.from_numpy(offs).to(dev), torch.from_numpy(flat).to(dev), stream)

    def rebuild(self, stream=None):
        _check(load().sfx_rebuild(self._h, _stream(stream)))

    def rebuild_async(self, stream=None):
        _check(load().sfx_rebuild_async(self._h, _stream(stream)))

    def poll(self, stream=None) -> bool:
        sw = _I32(0)
        _check(load().sfx_poll(self._h, ctypes.byref(sw), _stream(stream)))
        return bool(sw.value)

    def wait_rebuild(self, stream=None):
        _check(load().sfx_wait_rebuild(self._h, _stream(stream)))

    def accept_estimate(self, B, est_ppm=None, stream=None):
        """[B, k] int32 per-slot acceptance estimates (ppm) of the last propose's drafts."""
        if est_ppm is None:
            est_ppm = torch.empty((B, self.cfg.k), dtype=torch.int32, device="cuda")
        _check(load().sfx_accept_estimate(self._h, B, _ptr(est_ppm), _stream(stream)))
        return est_ppm

    def accept_feedback(self, num_accepted, stream=None):
        """Count the verifier's accepted tokens [B] against the last propose's drafts."""
        na = _i32(num_accepted, "num_accepted", 1)
        _check(load().sfx_accept_feedback(self._h, na.shape[0], _ptr(na), _stream(stream)))

    def accept_reset(self, stream=None):
        _check(load().sfx_accept_reset(self._h, _stream(stream)))

    def accept_counts(self, stream=None) -> torch.Tensor:
        """The counts table as int64 [2, 65, 32, 2] (proposed, accepted)."""
        out = torch.empty((2, 65, 32, 2), dtype=torch.int64, device="cuda")
        _check(load().sfx_accept_counts(self._h, _ptr(out), _stream(stream)))
        return out

    def save(self, path, stream=None):
        """Write the corpus (live documents, counters, live index) to the host file `path`."""
        _check(load().sfx_save(self._h, os.fsencode(path), _stream(stream)))

    def load(self, path, stream=None):
        """Replace the corpus with the one saved in `path` (same corpus_capacity)."""
        _check(load().sfx_load(self._h, os.fsencode(path), _stream(stream)))

    def debug_fail_next_rebuild(self):
        """Test hook: the next rebuild fails with EHIP before its swap (the live index stays)."""
        _check(load().sfx_debug_fail_next_rebuild(self._h))

    def debug_errors(self, stream=None) -> int:
        """Read and clear the sticky ERR_* bits raised since the last read (synchronises)."""
        v = ctypes.c_uint32(0)
        _check(load().sfx_debug_errors(self._h, ctypes.byref(v), _stream(stream)))
        return v.value

    def corpus_snapshot(self, stream=None) -> torch.Tensor:
        cap = max(int(self.cfg.corpus_capacity), 1)
        out = torch.empty(cap, dtype=torch.int32, device="cuda")
        n = _I64(0)
        _check(load().sfx_corpus_snapshot(self._h, _ptr(out), cap, ctypes.byref(n),
                                          _stream(stream)))
        return out[: n.value]

    def rebuild_stats(self):
        """sfx_rebuild_stats: (doubling rounds, snapshot tokens) of the last index build."""
        r, n = _I32(0), _I64(0)
        _check(load().sfx_rebuild_stats(self._h, ctypes.byref(r), ctypes.byref(n)))
        return r.value, n.value

    def debug_index(self, stream=None):
        """sfx_debug_index: (snapshot text, suffix array) of the live corpus index."""
        cap = max(int(self.cfg.corpus_capacity), 1)
        text = torch.empty(cap, dtype=torch.int32, device="cuda")
        sa = torch.empty(cap, dtype=torch.int32, device="cuda")
        n = _I64(0)
        _check(load().sfx_debug_index(self._h, _ptr(text), _ptr(sa), cap, ctypes.byref(n),
                                      _stream(stream)))
        return text[: n.value], sa[: n.value]


class GraphSet:
    """Graphs of the drafter step captured per batch-size bucket over persistent buffers
    (sfx_graphs_create); propose(B) replays the smallest bucket >= B with rows B.. emptied, or
    runs eagerly where no graph was captured."""

    def __init__(self, drafter, buckets, num_tokens, token_ids, sampled, draft, num_valid,
                 num_tokens_out=None, flags=0, stream=None):
        buckets = [int(x) for x in buckets]
        nt = _i32(num_tokens, "num_tokens", 1)
        tok = _i32(token_ids, "token_ids", 2)
        smp = _i32(sampled, "sampled", 2)
        dr = _i32(draft, "draft", 2)
        nv = _i32(num_valid, "num_valid", 1)
        nout = None if num_tokens_out is None else _i32(num_tokens_out, "num_tokens_out", 1)
        rows = max(buckets) if buckets else 0
        for name, t in (("num_tokens", nt), ("token_ids", tok), ("sampled", smp),
                        ("draft", dr), ("num_valid", nv), ("num_tokens_out", nout)):
            if t is not None and t.shape[0] < rows:
                raise ValueError(f"{name} has {t.shape[0]} rows, the largest bucket {rows}")
        if dr.shape[1] != drafter.cfg.k:
            raise ValueError(f"draft must have k={drafter.cfg.k} columns")
        # the buffers stay referenced while the graphs exist
        self._keep = (drafter, nt, tok, smp, dr, nv, nout)
        arr = (_I32 * max(len(buckets), 1))(*buckets)
        h = _V()
        _check(load().sfx_graphs_create(drafter._h, len(buckets), arr, tok.shape[1],
                                        smp.shape[1], _ptr(nt), _ptr(tok), _ptr(smp), _ptr(dr),
                                        _ptr(nv), _ptr(nout), int(flags), _stream(stream),
                                        ctypes.byref(h)))
        self._h = h

    def propose(self, B, stream=None):
        _check(load().sfx_graphs_propose(self._h, int(B), _stream(stream)))

    def stats(self):
        nb, em, pm = _I32(), ctypes.c_uint64(), ctypes.c_uint64()
        rep, eag = _I64(), _I64()
        _check(load().sfx_graphs_stats(self._h, ctypes.byref(nb), ctypes.byref(em),
                                       ctypes.byref(pm), ctypes.byref(rep), ctypes.byref(eag)))
        return {"buckets": nb.value, "exact_mask": em.value, "padded_mask": pm.value,
                "replays": rep.value, "eager_calls": eag.value}

    def close(self):
        if getattr(self, "_h", None):
            load().sfx_graphs_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def update_state(token_ids, num_tokens, sampled, num_tokens_out=None, stream=None):
    tok = _i32(token_ids, "token_ids", 2)
    samp = _i32(sampled, "sampled", 2)
    nt = _i32(num_tokens, "num_tokens_no_spec", 1)
    B, S = tok.shape
    if num_tokens_out is None:
        num_tokens_out = torch.empty((B,), dtype=torch.int32, device=tok.device)
    _check(load().sfx_update_state(B, S, samp.shape[1], _ptr(tok), _ptr(nt), _ptr(samp),
                                   _ptr(num_tokens_out), _stream(stream)))
    return num_tokens_out


NOALLOC_MAX_TOKENS = 1 << 20  # largest text of build_suffix_array_noalloc


def build_suffix_array_noalloc(text: torch.Tensor, sa: torch.Tensor, stream=None) -> None:
    """sfx_build_suffix_array_noalloc: the suffix array of text into the caller's sa (same
    length), with no allocation; sa is ready once `stream` reaches the call."""
    t = _i32(text, "text", 1)
    out = _i32(sa, "sa", 1)
    if out.shape[0] != t.shape[0]:
        raise ValueError("sa must have text's length")
    _check(load().sfx_build_suffix_array_noalloc(_ptr(t), t.shape[0], _ptr(out), _stream(stream)))


def build_suffix_array(text: torch.Tensor, stream=None) -> torch.Tensor:
    t = _i32(text, "text", 1)
    n = t.shape[0]
    sa = torch.empty(n, dtype=torch.int32, device=t.device)
    L = load()
    wsb = L.sfx_suffix_array_workspace_bytes(n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=t.device)
    _check(L.sfx_build_suffix_array(_ptr(t), n, _ptr(sa), _ptr(ws), wsb, _stream(stream)))
    return sa
