"""Independent brute-force formulations used to pin the oracle (tests only).

These restate the drafter's definitions in a different form from oracle.c -- substring
enumeration instead of incremental backward scans, an explicit continuation trie instead of an
alive set, Python list ordering for suffixes -- so that a dropped term, a wrong index or a
swapped tie rule in the oracle shows up as a disagreement.  Only for tiny inputs.
"""
from __future__ import annotations

from collections import Counter


def local_occ_ends(ctx, l):
    """Ends j <= L-2 of earlier occurrences of the last l tokens (SuffixGPU page, How it works
    step 1; vLLM docs Suffix Decoding, Model Runner V2)."""
    L = len(ctx)
    if l < 1 or l > L:
        return []
    tail = list(ctx[L - l:])
    return [j for j in range(l - 1, L - 1) if list(ctx[j - l + 1:j + 1]) == tail]


def local_mb(ctx, D):
    L = len(ctx)
    out = []
    for j in range(L - 1):
        best = 0
        for m in range(1, min(D, j + 1) + 1):
            if list(ctx[j - m + 1:j + 1]) == list(ctx[L - m:]):
                best = m
        out.append(best)
    return out


def corpus_occ_starts(C, ctx, l):
    """Starts i of corpus occurrences of the last l tokens that are followed by a real token."""
    N, L = len(C), len(ctx)
    if l < 1 or l > L:
        return []
    tail = list(ctx[L - l:])
    return [i for i in range(0, N - l) if list(C[i:i + l]) == tail and C[i + l] != -1
            and -1 not in C[i:i + l]]


def ladder(count_of_len, max_len, t):
    """Largest length with at least t occurrences (0 if none)."""
    best = 0
    for l in range(1, max_len + 1):
        if count_of_len(l) >= t:
            best = l
    return best


def trie_expand(X, sites, cap, scored=False, prob_ppm=0):
    """Greedy descent of the continuation trie of the sites (SuffixGPU page, How it works
    step 3): each trie node counts the sites whose continuation passes through it; the child
    with the largest count (then the smallest token id) is taken while the count-based
    probability count/c0 stays >= min_token_prob."""
    c0 = len(sites)
    strs = []
    for p in sites:
        s, q = [], p
        while q < len(X) and X[q] != -1 and len(s) < cap:
            s.append(int(X[q]))
            q += 1
        strs.append(tuple(s))
    cnt = Counter()
    for s in strs:
        for d in range(1, len(s) + 1):
            cnt[s[:d]] += 1
    out, counts, prefix = [], [], ()
    while len(prefix) < cap:
        kids = [(c, key[-1]) for key, c in cnt.items()
                if len(key) == len(prefix) + 1 and key[:-1] == prefix]
        if not kids:
            break
        c, tok = max(kids, key=lambda x: (x[0], -x[1]))
        if scored and c * 10**6 < prob_ppm * c0:
            break
        out.append(tok)
        counts.append(c)
        prefix = prefix + (tok,)
    return out, counts, sum(counts)


def propose_row(knobs, row, n, sampled, C=None):
    """Whole drafter call for one row, from the brute-force pieces above."""
    k, D, nb, M, mode = (knobs["k"], knobs["max_tree_depth"], knobs["num_backoff"],
                         knobs["max_occurrences"], knobs["mode"])
    S = len(row)
    n = max(0, min(int(n), S))
    t = 0
    while t < len(sampled) and sampled[t] >= 0:
        t += 1
    ctx = [int(x) for x in row[:n]] + [int(x) for x in sampled[:t]]
    L = len(ctx)
    if t == 0:
        return [-1] * k, 0
    fill = ctx[-1] if mode == 0 else -1

    def cap_of(l):
        cap = k
        if mode == 1:
            cap = max(0, min(k, (knobs["spec_factor_ppm"] * l + knobs.get("spec_offset_ppm", 0))
                             // 10**6))
        if knobs.get("tree_depth_cap"):
            # the tree's depth (match length plus drafted tokens) stays within max_tree_depth
            cap = min(cap, max(0, D - l))
        return cap

    cands = []
    for ti in range(1, nb + 1):
        l = ladder(lambda x: len(local_occ_ends(ctx, x)), min(D, L - 1), ti)
        if l >= knobs.get("min_self_match", 1) and l >= 1:
            sites = sorted(j + 1 for j in local_occ_ends(ctx, l))[:M]
            toks, _, snum = trie_expand(ctx, sites, cap_of(l), mode == 1,
                                        knobs.get("min_token_prob_ppm", 0))
            cands.append((l, len(sites), snum, toks))
        else:
            cands.append(None)
    for ti in range(1, nb + 1):
        if C is None or len(C) == 0:
            cands.append(None)
            continue
        l = ladder(lambda x: len(corpus_occ_starts(C, ctx, x)), min(D, L), ti)
        if l >= knobs.get("min_corpus_match", 2):
            sites = sorted(i + l for i in corpus_occ_starts(C, ctx, l))[:M]
            toks, _, snum = trie_expand(C, sites, cap_of(l), mode == 1,
                                        knobs.get("min_token_prob_ppm", 0))
            cands.append((l, len(sites), snum, toks))
        else:
            cands.append(None)
    win = None
    if mode == 0:
        lc, gc = cands[0], cands[nb]
        if lc is not None and (gc is None or lc[0] >= gc[0]):
            win = lc
        elif gc is not None:
            win = gc
    else:
        for c in cands:
            if c is None:
                continue
            # score = snum / c0, compared as fractions
            if win is None or c[2] * win[1] > win[2] * c[1]:
                win = c
    toks = win[3] if win is not None else []
    return toks + [fill] * (k - len(toks)), len(toks)


def suffix_array(text):
    t = [int(x) for x in text]
    return sorted(range(len(t)), key=lambda i: t[i:])
