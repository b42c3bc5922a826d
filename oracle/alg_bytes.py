"""Writes oracle/alg_bytes.json: the exact algorithmic bytes of one propose call (alg_bytes.c's
word counts times 4, by category) for each workload's benchmark input sets.

Run:  python oracle/alg_bytes.py [--sets 4]

The benchmark reads the file; it never calls the oracle for this.  Inputs are the seeded
synthetic sets of workloads/ (the same ones the benchmark rotates through); each entry records
the workload name and set index it was computed on."""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(ROOT, "oracle", "alg_bytes.json")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--workloads", default="1,2,3,4")
    args = ap.parse_args()
    O.build(force=False)
    threads = min(16, len(os.sched_getaffinity(0)))
    res = {"about": __doc__.strip().splitlines()[0], "unit": "bytes per call",
           "categories": list(O.ALG_CATEGORIES), "workloads": {}}
    for cid in [int(x) for x in args.workloads.split(",")]:
        w = W.WORKLOADS[cid]
        p = O.params_from(w.knobs())
        C = W.join_docs(W.corpus_docs(cid)) if w.corpus else None
        sa = O.suffix_array(C) if C is not None else None
        sets = []
        for i in range(args.sets):
            n, tok, samp = W.make_batch(cid, set_index=i)
            words = O.alg_words(p, n, tok, samp, corpus=C, sa=sa, num_threads=threads)
            b = {k: 4 * v for k, v in words.items()}
            b["total"] = sum(b.values())
            sets.append({"set_index": i, "bytes": b})
            print(f"workload {w.name} set {i}: {b}", flush=True)
        mean = {k: float(np.mean([s["bytes"][k] for s in sets])) for k in sets[0]["bytes"]}
        res["workloads"][w.name] = {"sets": sets, "mean": mean}
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
