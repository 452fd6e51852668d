"""Timing of the oracle on the host cores, for the benchmark's CPU-baseline leg.

TEST INFRASTRUCTURE ONLY: started as a child process by bench.py's cpu_baseline leg (a separate
process, so that the affinity it sets and the memory it uses never touch the GPU process). The
oracle is timed as it stands: single-threaded C, -O2, no fast-math.

Input: files written by the parent under one path prefix: the bf16 bits of a prefix of the
workload's key rows (`_x.npy`, [n, D] uint16, memory-mapped), of its queries (`_q.npy`, [Hq, D]
uint16, one batch row) and the codec's parameters (`_codec.json`). The child pins itself to the cores it is given, encodes and decodes its shard of the
rows, then scores pairs (query head, token) of its shard against the shard's own records (the
oracle's score decodes the record once per pair: it is the plain definition q . decode(record)).
Prints one JSON line: rows, seconds for encode+decode, pairs, seconds for the scores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--input", required=True, help="path prefix of the input files")
    ap.add_argument("--core", type=int, required=True, help="the one core this process runs on")
    ap.add_argument("--shard", type=int, default=0)
    ap.add_argument("--shards", type=int, default=1)
    ap.add_argument("--group", type=int, default=4, help="query heads per KV head")
    ap.add_argument("--score-tokens", type=int, default=0, help="tokens of the shard scored")
    args = ap.parse_args()
    os.sched_setaffinity(0, {args.core})
    x = np.load(args.input + "_x.npy", mmap_mode="r", allow_pickle=False)
    q = np.load(args.input + "_q.npy", allow_pickle=False)
    with open(args.input + "_codec.json") as f:
        cfg = json.load(f)
    D, bits, seed = int(cfg["D"]), int(cfg["bits"]), int(cfg["seed"])
    n = x.shape[0]
    lo, hi = n * args.shard // args.shards, n * (args.shard + 1) // args.shards
    xs = np.ascontiguousarray(x[lo:hi])
    cd = oracle.Codec(D, bits, seed=seed)
    oracle.lib()
    t0 = time.perf_counter()
    rec = oracle.encode_records(cd, xs)
    oracle.decode(cd, rec)
    t_ed = time.perf_counter() - t0
    # score: every query head of the group against each of the first score_tokens records
    nt = min(args.score_tokens, rec.shape[0])
    pairs, t_sc = 0, 0.0
    if nt > 0:
        G = args.group
        qq = np.repeat(q[:G], nt, axis=0)                  # [G * nt, D]
        rr = np.tile(rec[:nt], (G, 1))                     # [G * nt, rec_bytes]
        t0 = time.perf_counter()
        oracle.score(cd, qq, rr)
        t_sc = time.perf_counter() - t0
        pairs = G * nt
    print(json.dumps({"rows": int(hi - lo), "encdec_s": t_ed, "pairs": pairs, "score_s": t_sc,
                      "core": args.core}), flush=True)


if __name__ == "__main__":
    main()
