"""Live-document bookkeeping of the shared corpus (oracle side; test infrastructure only).

SuffixGPU page, How it works step 4: finished sequences are appended as new documents and the
oldest documents are evicted when the ring is full; vLLM docs "Suffix Decoding", Model Runner
V2: the corpus keeps finished responses up to a token budget, oldest first out.

Readings taken:
  * each document occupies len + 1 tokens: its tokens and one -1 separator after it;
  * after documents are appended, the oldest are dropped while the total exceeds the capacity,
    so the live set is always the longest run of most recent documents that fits (a document
    larger than the capacity therefore never stays live);
  * the live corpus text is the live documents in ingest order, each followed by -1.
"""
from __future__ import annotations

from collections import deque

import numpy as np


def harvest_docs(token_ids, row_indices, lengths):
    """Documents of harvest_finished: row r's first clamp(len, 0, S) tokens, in the given order.

    SuffixGPU page, Quickstart: harvest_finished(row_indices, lengths, token_ids)."""
    tok = np.asarray(token_ids, dtype=np.int32)
    S = tok.shape[1]
    docs = []
    for r, ln in zip(np.asarray(row_indices).tolist(), np.asarray(lengths).tolist()):
        ln = max(0, min(int(ln), S))
        docs.append(tok[int(r), :ln].copy())
    return docs


class LiveCorpus:
    def __init__(self, capacity: int):
        if capacity < 0:
            raise ValueError("capacity must be >= 0")
        self.capacity = int(capacity)
        self.docs: deque[np.ndarray] = deque()
        self.total = 0
        self.dropped = 0

    def ingest(self, docs) -> None:
        for d in docs:
            d = np.asarray(d, dtype=np.int32)
            self.docs.append(d)
            self.total += len(d) + 1
        while self.docs and self.total > self.capacity:
            old = self.docs.popleft()
            self.total -= len(old) + 1
            self.dropped += 1

    def evicted(self) -> int:
        """Number of documents dropped so far."""
        return self.dropped

    def text(self) -> np.ndarray:
        if not self.docs:
            return np.zeros(0, np.int32)
        parts = []
        for d in self.docs:
            parts.append(d)
            parts.append(np.array([-1], np.int32))
        return np.concatenate(parts).astype(np.int32)


class InflightIngest:
    """Per-row ingest cursors of in-flight responses (RFC page "[RFC]: Suffix decoding on GPU
    (suffix_gpu)", Design: in-flight responses are ingested off the critical path and finished
    requests are final-flushed before their batch rows are reused; the ingest-chunk knob).

    Reading taken (the page gives no document semantics for partial responses): an ingest call
    appends, for every listed row, the tokens past the row's cursor as one separate document once
    at least max(min_chunk, 1) of them have accumulated, or on a final flush whenever any are
    left.  The cursor then moves to the row's length, or back to 0 after a final flush.  A length
    below the cursor means the row was reused without a flush, and the row restarts at 0.  A row
    listed twice in one call counts once, at its first entry; rows outside
    [0, min(num_rows, max_rows)) are ignored.  docs() returns the call's documents in entry order,
    to be given to LiveCorpus.ingest."""

    def __init__(self, max_rows: int):
        self.max_rows = int(max_rows)
        self.cursor = [0] * self.max_rows

    def docs(self, token_ids, row_indices, lengths, final=None, min_chunk=1):
        tok = np.asarray(token_ids, dtype=np.int32)
        num_rows, S = tok.shape
        limit = min(num_rows, self.max_rows)
        need = max(int(min_chunk), 1)
        seen = set()
        out = []
        for r, (row, ln) in enumerate(zip(np.asarray(row_indices).tolist(),
                                          np.asarray(lengths).tolist())):
            row = int(row)
            if row < 0 or row >= limit or row in seen:
                continue
            seen.add(row)
            n = max(0, min(int(ln), S))
            c = self.cursor[row]
            if n < c:
                c = 0
            fin = final is not None and int(final[r]) != 0
            chunk = n - c
            take = chunk >= need or (fin and chunk > 0)
            if take:
                out.append(tok[row, c:n].copy())
            self.cursor[row] = 0 if fin else (n if take else c)
        return out
