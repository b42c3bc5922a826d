"""Benchmark of the drafter step on one MI355X.

A step is one sfx_propose over one batch: every request's self match, corpus probes, vote and
selection.  Default workload: B=256 requests, S=16384 resident tokens (valid lengths
U[4096,16384]), V=151936, k=16, scored mode, and a 1M-token template corpus indexed on the
device.  Inputs are synthetic (seeded generators in workloads/) and already resident in HBM when
the timed region starts; the token buffers rotate over enough copies to exceed the 256 MB
Infinity Cache, so each step streams its rows from HBM.

Prints one JSON line (metric, value, roofline, cpu_baseline, ...).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_SOURCES = ("suffix_match_drafter_amd/csrc/propose.hip",
                  "suffix_match_drafter_amd/csrc/propose.h",
                  "suffix_match_drafter_amd/csrc/delta_index.h",
                  "suffix_match_drafter_amd/csrc/sfx_internal.h")


REBUILD_BYTES_PER_TOKEN_ROUND = 8 + 4 * 32 + 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n, samp, B, T, k):
    """Words the method must touch per call: each request's context (its row prefix and the
    sampled ids appended to it), its length, and the [k] draft plus valid count written back.
    Corpus words are not counted (a conservative floor)."""
    t = (samp >= 0).cumprod(axis=1).sum(axis=1)
    L = np.minimum(np.maximum(n, 0), 1 << 30) + t
    return int(4 * L.sum() + 4 * B * (1 + T) + 4 * B * (k + 1)), int(L.sum())


def exact_alg_bytes(workload, nsets):
    """The exact algorithmic bytes per call of the first `nsets` input sets of a workload, by
    category, as the oracle's instrumented counter wrote them to oracle/alg_bytes.json (the
    benchmark only reads that file); None when the file does not cover these sets."""
    path = os.path.join(ROOT, "oracle", "alg_bytes.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        entry = json.load(fh)["workloads"].get(workload)
    if entry is None:
        return None
    sets = [s for s in entry["sets"] if s["set_index"] < nsets]
    if len(sets) != nsets:
        return None
    return {k: float(np.mean([s["bytes"][k] for s in sets])) for k in sets[0]["bytes"]}


def kernel_source_hash():
    """sha256 over the propose kernel's sources: a traffic figure taken from hardware counters
    holds only for the kernel it was taken on."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per propose launch from the committed counter summary for this workload
    (FETCH_SIZE + WRITE_SIZE per dispatch, scaled by a plain copy of known size), or None when
    there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"propose_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def copy_calibration(torch, dev, mib, reps):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE and WRITE_SIZE
    counters (run outside the timed region, only when asked for)."""
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {mib} MiB")
    del src, dst


def copy_bandwidth_gbs(torch, dev, stream, mib=512, reps=10):
    """Achievable HBM bandwidth on this machine: a plain device-to-device copy of `mib` MiB (read
    plus write counted), HIP events on `stream`, outside the timed region."""
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = event_ms(torch, stream, lambda: dst.copy_(src), reps)
    del src, dst
    return 2 * mib * (1 << 20) / (ms * 1e-3) / 1e9


def event_ms(torch, stream, fn, reps):
    """Mean milliseconds of fn() over reps back-to-back calls, HIP events on `stream`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_calls_per_s(torch, d, bufs, draft, nv, per_graph=32, replays=60):
    """The same rotating calls captured once in a HIP graph (per_graph propose launches over
    successive buffers) and replayed: per-call launch overhead removed."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(per_graph):
            b = bufs[i % len(bufs)]
            d.propose(b[0], b[1], b[2], draft, nv, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cur = torch.cuda.current_stream()
        for i in range(per_graph):
            b = bufs[i % len(bufs)]
            d.propose(b[0], b[1], b[2], draft, nv, cur)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    g.replay()
    torch.cuda.synchronize()
    ms = event_ms(torch, stream, g.replay, replays)
    return per_graph / (ms * 1e-3)


def bucketed_graph_calls_per_s(torch, d, bufs, draft, nv, B, buckets, calls=600):
    """The library's batch-bucketed graphs (sfx_graphs_create at warm-up, sfx_graphs_propose
    per call), one graph set per rotating buffer, over copies of the lengths and sampled ids
    (a padded bucket empties its rows past B): calls/s at batch B, with how many calls replayed
    a graph."""
    stream = torch.cuda.current_stream()
    sets = []
    for b in bufs:
        nt, sm = b[0].clone(), b[2].clone()
        sets.append((d.graphs(buckets, nt, b[1], sm, draft, nv, stream=stream), nt, sm))
    torch.cuda.synchronize()
    k = [0]

    def one():
        sets[k[0] % len(sets)][0].propose(B, stream)
        k[0] += 1

    event_ms(torch, stream, one, 2 * len(sets))
    ms = event_ms(torch, stream, one, calls)
    replayed = sum(s[0].stats()["replays"] for s in sets)
    for s in sets:
        s[0].close()
    return 1e3 / ms, replayed / k[0]


def other_workloads(torch, sfx, W, dev, calls=200):
    """Workloads 1-3 (self match, self match + template corpus) in calls/s, one resident input
    set each."""
    out = {}
    stream = torch.cuda.current_stream()
    for cid in (1, 2, 3):
        w = W.WORKLOADS[cid]
        n, tok, samp = W.make_batch(cid)
        dn, dt, ds = (torch.from_numpy(x).to(dev) for x in (n, tok, samp))
        d = sfx.Drafter(sfx.Config(max_batch=w.B, max_seq=w.S, max_sampled=w.T,
                                   corpus_capacity=(1 << 20) if w.corpus else 0, **w.knobs()))
        if w.corpus:
            d.ingest_docs(W.corpus_docs(cid))
            d.rebuild()
        draft = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
        nv = torch.empty((w.B,), dtype=torch.int32, device=dev)
        fn = lambda: d.propose(dn, dt, ds, draft, nv, stream)  # noqa: E731
        event_ms(torch, stream, fn, 20)
        out[w.name] = round(1e3 / event_ms(torch, stream, fn, calls), 1)
        d.close()
    return out


def hot_gram_workload(torch, sfx, W, dev, sets=4, copies=2, calls=100):
    """The boilerplate workload: the workload-4 shape over a 1M-token corpus in which every
    request's last 4-gram occurs over 10^5 times; calls/s over rotating input buffers."""
    w = W.WORKLOADS[6]
    docs = W.corpus_docs(6)
    d = sfx.Drafter(sfx.Config(max_batch=w.B, max_seq=w.S, max_sampled=w.T,
                               corpus_capacity=1 << 21, **w.knobs()))
    d.ingest_docs(docs)
    d.rebuild()
    bufs = []
    for s in range(sets):
        arrs = W.make_batch(6, set_index=s)
        for _ in range(copies):
            bufs.append(tuple(torch.from_numpy(x).to(dev) for x in arrs))
    draft = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
    nv = torch.empty((w.B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    k = [0]

    def one():
        b = bufs[k[0] % len(bufs)]
        d.propose(b[0], b[1], b[2], draft, nv, stream)
        k[0] += 1

    event_ms(torch, stream, one, len(bufs))
    ms = event_ms(torch, stream, one, calls)
    d.close()
    c = W.join_docs(docs)
    H = W.hot_gram(w.V)
    occ = int(((c[:-4] == H[0]) & (c[1:-3] == H[1]) & (c[2:-2] == H[2]) & (c[3:-1] == H[3]) &
               (c[4:] >= 0)).sum())
    return {"workload": w.name, "us_per_call": round(ms * 1e3, 1),
            "calls_per_s": round(1e3 / ms, 1), "tail_4gram_occurrences": occ,
            "rotating_buffers": len(bufs)}


def ingest_under_load(torch, sfx, W, dev, warm_steps=16, steps=6, calls=10):
    """The ingest-and-rebuild workload: a ring of 2^22 tokens seeded with the template corpus;
    every step harvests 256 finished rows of U[512,2048] tokens; propose runs at B=512, S=32768,
    k=32.  After warm_steps (ring full and evicting), per step: the harvest (HIP events on the
    calling stream), propose with that step's documents still in the delta, propose while the
    asynchronous rebuild of the whole ring runs on the side stream (and the wall time of that
    overlapped block), and propose once it is live (no delta).  Then five synchronous rebuilds
    alone (median wall time).  Then the whole corpus is saved to a host file and
    loaded into a fresh context (wall time of each), and in-flight ingest is timed on it.
    Outside the headline timed region."""
    w = W.WORKLOADS[5]
    t0 = time.time()
    n, tok, samp = W.make_batch(5)
    dn, dt, ds = (torch.from_numpy(x).to(dev) for x in (n, tok, samp))
    batches = []
    sync_reps = 5  # synchronous rebuilds, each after a harvest of new documents
    for st in range(warm_steps + steps + sync_reps):
        itok, rows, lens = W.ingest_batch(5, st)
        batches.append((torch.from_numpy(rows).to(dev), torch.from_numpy(lens).to(dev),
                        torch.from_numpy(itok).to(dev), int(lens.sum())))
    log(f"[bench] ingest workload inputs in {time.time() - t0:.1f}s")
    cfg = sfx.Config(max_batch=w.B, max_seq=w.S, max_sampled=w.T,
                     corpus_capacity=w.ring_capacity, **w.knobs())
    d = sfx.Drafter(cfg)
    d.ingest_docs(W.corpus_docs(5))
    d.rebuild()
    stream = torch.cuda.current_stream()
    draft = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
    nv = torch.empty((w.B,), dtype=torch.int32, device=dev)
    for st in range(warm_steps):
        rows, lens, itok, _ = batches[st]
        d.harvest_finished(rows, lens, itok, stream)
        d.rebuild(stream)
    torch.cuda.synchronize()

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    def prop():
        d.propose(dn, dt, ds, draft, nv, stream)

    ing_ms, ing_tok, p_delta, p_during, p_live, reb_ms, step_ms = [], 0, [], [], [], [], []
    delta_tok = []  # tokens in the delta when the delta proposes run (documents plus separators)
    sync_ms = []
    for st in range(warm_steps, warm_steps + steps):
        rows, lens, itok, ntok = batches[st]
        ts = time.time()
        ing_ms.append(timed(lambda: d.harvest_finished(rows, lens, itok, stream), 1))
        ing_tok += ntok
        delta_tok.append(ntok + int(rows.numel()))
        p_delta.append(timed(prop, calls))
        tr = time.time()
        d.rebuild_async(stream)
        p_during.append(timed(prop, calls))
        d.wait_rebuild(stream)
        torch.cuda.synchronize()
        reb_ms.append((time.time() - tr) * 1e3)
        step_ms.append((time.time() - ts) * 1e3)
        p_live.append(timed(prop, calls))
    # the rebuild alone: synchronous, nothing else on the GPU, after one more harvest each
    reb_rounds, reb_tokens = [], []
    for st in range(sync_reps):
        rows, lens, itok, _ = batches[warm_steps + steps + st]
        d.harvest_finished(rows, lens, itok, stream)
        torch.cuda.synchronize()
        tr = time.time()
        d.rebuild(stream)
        torch.cuda.synchronize()
        sync_ms.append((time.time() - tr) * 1e3)
        r, ntok = d.rebuild_stats()
        reb_rounds.append(r)
        reb_tokens.append(ntok)
    # save and restore of the whole corpus (host file; a fresh context of the same capacity)
    import tempfile

    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "corpus.sfx")
        torch.cuda.synchronize()
        t1 = time.time()
        d.save(path, stream)
        save_ms = (time.time() - t1) * 1e3
        file_mb = os.path.getsize(path) / 1e6
        d2 = sfx.Drafter(cfg)
        torch.cuda.synchronize()
        t1 = time.time()
        d2.load(path, stream)
        load_ms = (time.time() - t1) * 1e3
    # in-flight ingest on the restored context: B rows of responses growing by k + 1 tokens per
    # step, chunks of at least 64 tokens (one 66-token chunk per row every second step)
    rows = torch.arange(w.B, dtype=torch.int32, device=dev)
    resp = torch.from_numpy(np.concatenate(
        [batches[i % len(batches)][2].cpu().numpy() for i in range(2)])).to(dev)[: w.B]
    lens = torch.zeros(w.B, dtype=torch.int32, device=dev)
    fl_ms = []
    for st in range(16):
        lens += w.k + 1
        fl_ms.append(timed(lambda: d2.ingest_inflight(rows, lens, resp, min_chunk=64,
                                                      stream=stream), 1))
    d2.close()
    d.close()
    # what the delta adds to a call: the per-call pair index (its passes over the delta) and
    # each request's extension of its own pair's occurrences
    extra_us = (float(np.mean(p_delta)) - float(np.mean(p_live))) * 1e3
    out = {
        "workload": f"ingest-B{w.B}-S{w.S}-ring{w.ring_capacity}",
        "steps": steps, "warm_steps": warm_steps,
        "harvest_ms": round(float(np.mean(ing_ms)), 3),
        "harvest_tokens_per_s": round(ing_tok / (sum(ing_ms) * 1e-3), 1),
        "propose_us_with_delta": round(float(np.mean(p_delta)) * 1e3, 1),
        "propose_us_during_rebuild": round(float(np.mean(p_during)) * 1e3, 1),
        "propose_us_no_delta": round(float(np.mean(p_live)) * 1e3, 1),
        "delta_tokens": int(np.mean(delta_tok)),
        "delta_extra_us": round(extra_us, 1),
        "rebuild_ms": round(float(np.median(sync_ms)), 2),
        "rebuild_tokens_per_s": round(w.ring_capacity / (float(np.median(sync_ms)) * 1e-3), 1),
        "rebuild_snapshot_tokens": int(np.median(reb_tokens)),
        "rebuild_rounds": int(np.median(reb_rounds)),
        # prefix doubling's bytes per token and round: key build 8, four radix passes of key and
        # value read and written plus their histogram 4 x 32, re-rank 16
        "rebuild_bytes_per_round": int(np.median(reb_tokens)) * REBUILD_BYTES_PER_TOKEN_ROUND,
        "rebuild_GBps": round(np.median(reb_rounds) * np.median(reb_tokens) *
                              REBUILD_BYTES_PER_TOKEN_ROUND / (np.median(sync_ms) * 1e-3) / 1e9,
                              1),
        "rebuild_roofline_frac": round(np.median(reb_rounds) * np.median(reb_tokens) *
                                       REBUILD_BYTES_PER_TOKEN_ROUND /
                                       (np.median(sync_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "async_rebuild_with_proposes_ms": round(float(np.mean(reb_ms)), 2),
        "step_ms": round(float(np.mean(step_ms)), 2),
        "save_ms": round(save_ms, 1),
        "load_ms": round(load_ms, 1),
        "corpus_file_MB": round(file_mb, 1),
        "inflight_ingest_ms": round(float(np.mean(fl_ms)), 3),
        "inflight_tokens_per_s": round(8 * w.B * 66 / (sum(fl_ms) * 1e-3), 1),
    }
    log(f"[bench] ingest workload: {out}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--distinct-sets", type=int, default=4)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-ingest-load", action="store_true",
                    help="skip the ingest-and-rebuild measurement after the timed region")
    ap.add_argument("--ingest-load-only", action="store_true",
                    help="run only the ingest-and-rebuild measurement (for profiling)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain copy of this many MiB before the timed region (counter "
                         "calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the drafter path has no multi-GPU mode in this "
              "build (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import suffix_match_drafter_amd as sfx
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.ingest_load_only:
        print(json.dumps({"ingest_under_load": ingest_under_load(torch, sfx, W, dev)}), flush=True)
        return
    w = W.WORKLOADS[args.config]
    log(f"[bench] workload {w.name}: B={w.B} S={w.S} V={w.V} k={w.k} mode={w.mode}")

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    sets = [W.make_batch(args.config, set_index=i) for i in range(args.distinct_sets)]
    docs = W.corpus_docs(args.config)
    log(f"[bench] generated {len(sets)} input sets and {len(docs)} corpus docs "
        f"in {time.time() - t0:.1f}s")
    cfg = sfx.Config(max_batch=w.B, max_seq=w.S, max_sampled=w.T,
                     corpus_capacity=(1 << 20) if w.corpus else 0, **w.knobs())
    d = sfx.Drafter(cfg)
    rebuild_s = None
    rebuild_rounds = None
    corpus_n = 0
    if w.corpus:
        d.ingest_docs(docs)
        torch.cuda.synchronize()
        t1 = time.time()
        d.rebuild()
        torch.cuda.synchronize()
        rebuild_s = time.time() - t1
        corpus_n = int(d.corpus_snapshot().numel())
        rebuild_rounds = d.rebuild_stats()[0]
        log(f"[bench] corpus {corpus_n} tokens indexed in {rebuild_s * 1e3:.1f} ms, "
            f"{rebuild_rounds} doubling rounds")
    bufs = []
    for c in range(args.copies):
        for (n, tok, samp) in sets:
            bufs.append((torch.from_numpy(n).to(dev), torch.from_numpy(tok).to(dev),
                         torch.from_numpy(samp).to(dev)))
    nbuf = len(bufs)
    resident_mb = sum(b[1].numel() * 4 for b in bufs) / 1e6
    alg = [algorithmic_bytes(n, samp, w.B, w.T, w.k) for (n, tok, samp) in sets]
    alg_floor = float(np.mean([a[0] for a in alg]))
    alg_exact = exact_alg_bytes(w.name, len(sets))
    alg_bytes = alg_exact["total"] if alg_exact else alg_floor
    ctx_tokens = float(np.mean([a[1] for a in alg]))
    draft = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
    nv = torch.empty((w.B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib > 0:
        copy_calibration(torch, dev, args.copy_calibration_mib, 5)

    # ---------------------------------------------------------------- timed region
    for i in range(args.warmup):
        b = bufs[i % nbuf]
        d.propose(b[0], b[1], b[2], draft, nv, stream)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    # the rotation goes on where the warm-up left it, so a timed call does not reread a buffer
    # the warm-up touched last (it could still sit in the last-level cache)
    for i in range(args.warmup, args.warmup + args.steps):
        b = bufs[i % nbuf]
        d.propose(b[0], b[1], b[2], draft, nv, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    calls_s = 1e3 / ms
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps over {nbuf} rotating buffers ({resident_mb:.0f} MB): "
        f"{ms * 1e3:.2f} us/step, {calls_s:.0f} calls/s, {achieved:.0f} GB/s algorithmic")

    # ---------------------------------------------------------------- outside the timed region
    # acceptance estimate [B, k] and verifier feedback, each right after a propose
    est = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
    acc = torch.full((w.B,), w.k // 2, dtype=torch.int32, device=dev)
    est_ms, fb_ms = [], []
    for i in range(20):
        b = bufs[i % nbuf]
        d.propose(b[0], b[1], b[2], draft, nv, stream)
        for fn, lst in ((lambda: d.accept_estimate(w.B, est, stream), est_ms),
                        (lambda: d.accept_feedback(acc, stream), fb_ms)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            lst.append(e0.elapsed_time(e1))
    graph_cps = graph_calls_per_s(torch, d, bufs, draft, nv)
    buckets = [w.B // 4, w.B // 2, 3 * w.B // 4, w.B]
    bucket_cps, bucket_replayed = bucketed_graph_calls_per_s(torch, d, bufs, draft, nv, w.B,
                                                             buckets)
    pad_b = w.B - 6
    bucket_pad_cps, _ = bucketed_graph_calls_per_s(torch, d, bufs, draft, nv, pad_b, buckets)
    log(f"[bench] bucketed graphs {buckets}: B={w.B} {bucket_cps:.0f} calls/s "
        f"(replayed {bucket_replayed:.2f}), B={pad_b} padded to {w.B} {bucket_pad_cps:.0f}")
    single = 1e3 / event_ms(torch, stream, lambda: d.propose(bufs[0][0], bufs[0][1], bufs[0][2],
                                                             draft, nv, stream), 500)
    others = other_workloads(torch, sfx, W, dev)
    hot = hot_gram_workload(torch, sfx, W, dev)
    log(f"[bench] hot 4-gram workload: {hot['us_per_call']} us/call "
        f"({hot['tail_4gram_occurrences']} occurrences of the tail 4-gram)")
    copy_gbs = copy_bandwidth_gbs(torch, dev, stream)
    log(f"[bench] graph-captured {graph_cps:.0f} calls/s; one resident buffer {single:.0f} "
        f"calls/s; {others}")
    load = None if args.no_ingest_load else ingest_under_load(torch, sfx, W, dev)

    # ---------------------------------------------------------------- oracle baseline
    cpu = None
    cpu_extra = None
    if not args.no_cpu_baseline:
        import oracle as O

        cores = len(os.sched_getaffinity(0))
        corpus = W.join_docs(docs) if w.corpus else None
        p = O.params_from(w.knobs())
        calls, t2 = 0, time.time()
        while True:
            n, tok, samp = sets[calls % len(sets)]
            O.propose(p, n, tok, samp, corpus=corpus, num_threads=cores)
            calls += 1
            dt = time.time() - t2
            if dt >= args.cpu_seconds:
                break
        cpu = {"value": round(calls / dt, 3), "unit": "propose calls/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{calls} full B={w.B} calls of the same workload over the "
                         f"{len(sets)} input sets, {dt:.1f}s wall, OpenMP over rows, "
                         f"{O.BUILD_FLAGS}"}
        log(f"[bench] oracle: {calls} calls in {dt:.1f}s on {cores} cores")
        # one core, on the first 32 rows of one input set (scaled to whole calls), and the
        # oracle's suffix array (single-threaded comparison sort) of the same corpus
        n, tok, samp = sets[0]
        t3 = time.time()
        O.propose(p, n[:32], tok[:32], samp[:32], corpus=corpus, num_threads=1)
        one_core = (32 / w.B) / (time.time() - t3)
        cpu_sa = None
        if corpus is not None:
            t3 = time.time()
            O.suffix_array(corpus)
            cpu_sa = len(corpus) / (time.time() - t3)
        cpu_extra = {"oracle_calls_per_s_1core": round(one_core, 4),
                     "oracle_1core_sample": f"rows 0-31 of one input set, scaled to B={w.B}",
                     "oracle_suffix_array_tokens_per_s":
                         None if cpu_sa is None else round(cpu_sa, 1)}

    out = {
        "metric": "propose calls/s at B=256,S=16K,1M-token corpus; % of HBM roofline",
        "value": round(calls_s, 1),
        "unit": "propose calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "T": w.T, "V": w.V, "k": w.k,
                   "max_tree_depth": w.max_tree_depth, "num_backoff": w.num_backoff,
                   "max_occurrences": w.max_occurrences,
                   "mode": "scored" if w.mode == 1 else "longest_fill",
                   "corpus_tokens": corpus_n, "rotating_buffers": nbuf,
                   "resident_input_MB": round(resident_mb, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name)},
        "cpu_baseline": cpu,
        "extra": {"tokens_scanned_per_s": round(ctx_tokens * calls_s, 1),
                  "algorithmic_bytes_per_call": int(alg_bytes),
                  "algorithmic_bytes_source": "oracle counter (oracle/alg_bytes.json)"
                  if alg_exact else "floor: context and I/O words only",
                  "algorithmic_bytes_by_category":
                      None if not alg_exact else {k: int(v) for k, v in alg_exact.items()},
                  "algorithmic_bytes_floor": int(alg_floor),
                  "index_rebuild_ms": None if rebuild_s is None else round(rebuild_s * 1e3, 2),
                  "index_rebuild_rounds": rebuild_rounds,
                  "index_rebuild_tokens_per_s":
                      None if not rebuild_s else round(corpus_n / rebuild_s, 1),
                  "measured_copy_GBps": round(copy_gbs, 1),
                  "frac_of_measured_copy": round(achieved / copy_gbs, 4),
                  "graph_captured_calls_per_s": round(graph_cps, 1),
                  "bucketed_graph": {"buckets": buckets, "calls_per_s": round(bucket_cps, 1),
                                     "replayed_fraction": round(bucket_replayed, 3),
                                     "padded_B": pad_b,
                                     "padded_calls_per_s": round(bucket_pad_cps, 1)},
                  "single_buffer_calls_per_s": round(single, 1),
                  "workloads_calls_per_s": others,
                  "hot_4gram": hot,
                  "accept_estimate_us": round(float(np.mean(est_ms)) * 1e3, 2),
                  "accept_feedback_us": round(float(np.mean(fb_ms)) * 1e3, 2),
                  "ingest_under_load": load,
                  "cpu_oracle_more": cpu_extra},
    }
    print(json.dumps(out), flush=True)
    d.close()


if __name__ == "__main__":
    main()
