"""Per-slot acceptance estimate, learned online (oracle side; test infrastructure only).

vLLM docs "Suffix Decoding", Use adaptive verification at higher concurrency: a running
estimate of each draft position's chance of acceptance, keyed by the draft's source, its match
length and the position.

Readings taken:
  * a draft's source is its winning candidate's: 0 for the request's own context, 1 for the
    corpus; its length is that candidate's match length; its slots are 0 .. num_valid - 1;
  * the verifier accepts a prefix of the draft, so slot d counts as accepted when the number of
    accepted tokens exceeds d;
  * the estimate of a (source, length, slot) cell is Laplace's rule of succession,
    (accepted + 1) / (proposed + 2), floored to parts per million (an unseen cell is one half);
  * feedback refers to the last propose of each row and is counted once.
"""
from __future__ import annotations

import numpy as np

LENS, SLOTS = 65, 32


def picks_from_info(info, nb):
    """(source, length, num_valid) of each row's winner, None where no candidate won; `info` as
    returned by propose(..., with_info=True)."""
    out = []
    for r in info:
        out.append(None if r.chosen < 0 else (int(r.chosen >= nb), int(r.chosen_len), int(r.n)))
    return out


class AcceptModel:
    def __init__(self):
        self.counts = np.zeros((2, LENS, SLOTS, 2), np.int64)  # [..., 0] proposed, [..., 1] accepted
        self.picks = {}

    def record(self, picks):
        """The rows' winners of a propose call (rows beyond the call keep theirs)."""
        for b, p in enumerate(picks):
            self.picks[b] = p

    def feedback(self, num_accepted):
        for b, na in enumerate(np.asarray(num_accepted).tolist()):
            p = self.picks.get(b)
            if p is None:
                continue
            self.picks[b] = None
            src, ln, nv = p
            na = max(0, min(int(na), nv))
            for d in range(nv):
                self.counts[src, ln, d, 0] += 1
                if d < na:
                    self.counts[src, ln, d, 1] += 1

    def estimate(self, B, k):
        est = np.zeros((B, k), np.int64)
        for b in range(B):
            p = self.picks.get(b)
            if p is None:
                continue
            src, ln, nv = p
            for d in range(min(nv, k)):
                prop, acc = self.counts[src, ln, d]
                est[b, d] = (1_000_000 * (int(acc) + 1)) // (int(prop) + 2)
        return est.astype(np.int32)
