"""Benchmark of the indexer hot path on one MI355X.

A step is one pass of the whole path over one batch already resident in HBM:
score (decode scorer) -> top-k -> expand/translate.  The default workload is
the uncompressed (c = 1) DSA-style decode: 16 requests x 1 row at L = 81,920
tokens, an independent 81,920 x 128 bf16 key set per request (320 MiB),
top-2048, translation through 64-token pages.

Prints one JSON line.  `value` is rows/s over the timed steps; `roofline`
covers the dominant kernel (the decode scorer, HBM bound) with its average
launch time taken from HIP events recorded around each launch on the stream
it runs on; `cpu_baseline` is the CPU oracle timed on the host on repeated
full batches of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def scorer_bytes(inp) -> int:
    """Algorithmic HBM bytes of one scorer launch: each visible key of each
    request read once (256 B), each row's q (1 KiB), the page-table entries of
    the visible range (4 B per page), one FP32 score written per visible
    (row, block)."""
    import numpy as np
    per_page = 64 // inp.c
    keys = pages = 0
    for b in range(inp.num_req):
        rows = inp.row_pos[inp.req_row_ptr[b]:inp.req_row_ptr[b + 1]]
        if rows.size == 0:
            continue
        nmax = int(((rows.astype(np.int64) + 1) // inp.c).max())
        keys += nmax
        pages += -(-nmax // per_page)
    nvis = ((inp.row_pos.astype(np.int64) + 1) // inp.c).sum()
    return int(keys * 256 + inp.num_rows * 1024 + pages * 4 + nvis * 4)


def prefill_flops(inp) -> int:
    import numpy as np
    nvis = ((inp.row_pos.astype(np.int64) + 1) // inp.c).sum()
    return int(nvis) * 4 * 128 * 2


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_scoring_top_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, min_seconds: float):
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.pipeline(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 5000:
            break
    return {"value": inp.num_rows * reps / el, "unit": "rows/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{reps} full batches of the timed workload ({inp.num_rows} rows each) through "
                      f"score + top-k (full sort) + expand/translate, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsa_decode_16x80k")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): every call of this path runs on one "
              "GPU with no collectives; see the sharding note in DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = synth.WORKLOADS[args.workload]
    log(f"generating {args.workload}")
    inp = gen()
    scorer = "prefill" if args.workload == "qsa_prefill_8k" else "decode"
    dinp = upload(inp, dev)
    path = IndexerPath(dinp, scorer)
    log(f"rows={inp.num_rows} max_vis={inp.max_vis} k={inp.k} c={inp.c} scorer={scorer}")

    for _ in range(args.warmup):
        path.run()
    torch.cuda.synchronize()
    log("warmup done")

    stream = torch.cuda.current_stream(dev)
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        path.score()
        e[1].record(stream)
        path.select()
        e[2].record(stream)
        path.expand()
        e[3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    t_score = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_topk = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    t_expand = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    log(f"timed {K} steps: {ms_step * 1e3:.1f} us/step (host wall {wall * 1e6 / K:.1f} us/step); "
        f"score {t_score * 1e3:.1f} us, top-k {t_topk * 1e3:.1f} us, expand {t_expand * 1e3:.1f} us")

    rows_per_s = inp.num_rows / (ms_step * 1e-3)
    if scorer == "decode":
        alg = scorer_bytes(inp)
        achieved = alg / (t_score * 1e-3) / 1e9
        kname = "score_decode"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kname, source_digest("score_decode.hip", "device.h")),
                "kernel": "score_decode_kernel", "algorithmic_bytes": alg, "avg_us": round(t_score * 1e3, 2)}
    else:
        fl = prefill_flops(inp)
        achieved = fl / (t_score * 1e-3) / 1e12
        kname = "score_prefill"
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(kname, source_digest("score_prefill.hip", "device.h")),
                "kernel": "score_prefill_kernel", "algorithmic_flops": fl, "avg_us": round(t_score * 1e3, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    line = {
        "metric": "indexer rows/s (score+top-k) at L=80k; achieved HBM GB/s and % of peak",
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q ~N(0,1), keys ~N(0,1) L2-normalised, bf16; random page permutation)",
        "config": {"workload": args.workload, "rows": inp.num_rows, "requests": inp.num_req,
                   "max_visible_blocks": inp.max_vis, "k": inp.k, "c": inp.c, "scorer": scorer,
                   "page_tokens": 64},
        "kernels_us": {"score": round(t_score * 1e3, 2), "topk": round(t_topk * 1e3, 2),
                       "expand": round(t_expand * 1e3, 2)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
