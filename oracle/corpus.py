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
