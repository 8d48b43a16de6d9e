"""Benchmark of the indexer hot path on one MI355X.

A step is one pass of the whole path over one batch already resident in HBM:
score (decode scorer) -> top-k -> expand/translate, the last two fused in one
kernel (idx_select_translate; --unfused times the separate calls).  The
default workload is
the uncompressed (c = 1) DSA-style decode: 16 requests x 1 row at L = 81,920
tokens, an independent 81,920 x 128 bf16 key set per request (320 MiB),
top-2048, translation through 64-token pages.

Prints one JSON line.  `value` is rows/s over the timed steps (two HIP
events around K steps).  `roofline` covers the dominant kernel (the decode
scorer, HBM bound): its average launch duration comes from HIP events on its
stream around back-to-back launches right after the timed region (the figure
a kernel trace reports), its bytes count its own output (the scores); the
committed kernel trace's average and the fraction it gives are reported
beside it when the trace was taken on the current source.  `step_roofline`
is the whole step against HBM peak, counting the algorithmic bytes of the
path (keys once, q, page-table entries, the selection; scores are an
intermediate).  `cpu_baseline` is the CPU oracle timed on the host on
repeated full batches of the same workload.
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


def measured_traffic(kernel: str, digest: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source and on this workload; else
    None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != digest or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, min_seconds: float):
    import oracle
    import synth
    topk_only = isinstance(inp, synth.ScoreRows)
    select_only = isinstance(inp, synth.SelectBatch)
    reps, t0 = 0, time.perf_counter()
    while True:
        if topk_only:
            oracle.topk(inp.scores, inp.row_len, inp.k)
        elif select_only:
            sel, cnt = oracle.topk(inp.scores, inp.row_len, inp.inp.k)
            oracle.expand_translate(inp.inp, sel, cnt)
        else:
            oracle.pipeline(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= 5000:
            break
    what = ("top-k (full sort)" if topk_only else "top-k (full sort) + expand/translate" if select_only
            else "score + top-k (full sort) + expand/translate")
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(inp.num_rows * reps / el, 2), "unit": "rows/s", "cores": oracle.threads(),
            "cpu_model": model, "kind": "oracle",
            "sample": f"{reps} full batches of the timed workload ({inp.num_rows} rows each) through {what}, "
                      f"{el:.1f} s"}


def bound(fns, stream):
    """Prepared calls with the stream fixed once (each call is then a single C
    call: looking up torch's current stream costs ~2.7 us of host time per
    call, which made the small steps host-bound)."""
    import block_scoring_top_amd as bst
    return [f.bind(stream) if isinstance(f, bst.PreparedCall) else f for f in fns]


def time_steps(fns, K, warmup, stream, probe=0, probe_every=10, burst=20):
    """Runs the callables of a step K times after `warmup` untimed steps and
    returns (ms per step, dict of dominant-kernel timings).

    The step time comes from two HIP events around the K steps, with nothing
    else recorded in between.  The dominant callable fns[probe] is then timed
    twice, every event recorded on `stream`, the stream all calls are
    launched on:
      * burst_ms: events around `burst` back-to-back launches of it alone,
        divided by `burst` -- its average launch duration, the figure a
        kernel trace reports (the launches queue behind each other, so the
        dispatch latency is paid once);
      * in_steps_ms: events around it inside `probe_every`-th steps of a
        second run of K steps (each bracket also holds the launch latency of
        a kernel queued behind an event marker, a few microseconds)."""
    import numpy as np
    import torch
    fns = bound(fns, stream)
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(K):
        for f in fns:
            f()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    probes = []
    for i in range(K):
        for j, f in enumerate(fns):
            if j == probe and i % probe_every == 0:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                f()
                b.record(stream)
                probes.append((a, b))
            else:
                f()
    torch.cuda.synchronize()
    in_steps = float(np.mean([a.elapsed_time(b) for a, b in probes]))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(burst):
        fns[probe]()
    b.record(stream)
    torch.cuda.synchronize()
    return ms, {"burst_ms": a.elapsed_time(b) / burst, "in_steps_ms": in_steps, "burst": burst}


def cold_steps(fns, reps, stream, flush_bytes=512 << 20):
    """Median step time with the 256 MB Infinity Cache flushed before every
    step: a `flush_bytes` scratch buffer is read (a reduction over it) between
    steps, outside the events that bracket each step.  Reading, not writing:
    a written buffer leaves the cache full of dirty lines, whose write-back
    would then run inside the timed step.  The scratch is written once and
    read twice before the first step, so the lines it leaves are clean."""
    import numpy as np
    import torch
    fns = bound(fns, stream)
    scratch = torch.zeros(flush_bytes // 8, dtype=torch.int64, device=torch.cuda.current_device())
    for _ in range(2):
        scratch.sum()
    torch.cuda.synchronize()
    times = []
    for i in range(reps):
        scratch.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for f in fns:
            f()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del scratch
    return float(np.median(times))


def kernel_trace_us(kernel_key: str, digest: str):
    """Average duration (us) of a kernel in the committed rocprofv3 kernel
    trace of this workload, if that trace was taken on the current source."""
    path = os.path.join(ROOT, "profiles", "kernel_trace.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel_key)
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent.get("avg_us")


def step_bytes(inp) -> int:
    """Algorithmic HBM bytes of one pass of the whole path (score -> top-k ->
    expand/translate): each request's visible keys once (256 B), each row's q
    (1 KiB), the page-table entries of the visible range (4 B), and the
    selection written (k int32 per row).  Scores are an intermediate (written
    by the scorer, read by the selection) and are not counted; neither are
    the translated slots and positions (8 B per expanded entry), reported
    separately."""
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
    return int(keys * 256 + inp.num_rows * 1024 + pages * 4 + inp.num_rows * inp.k * 4)


def kernel_breakdown(fns, K, stream):
    """Average time of each callable, each bracketed by HIP events, in a
    separate pass after the timed region (for the per-kernel report only)."""
    import numpy as np
    import torch
    fns = bound(fns, stream)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        e = ev[i]
        e[0].record(stream)
        for j, f in enumerate(fns):
            f()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    return [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) for j in range(len(fns))]


def run_workload(name, K, warmup, dev, fused=True, cold_reps=False):
    import torch

    import block_scoring_top_amd as bst
    import synth
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload

    log(f"generating {name}")
    inp = synth.WORKLOADS[name]()
    stream = torch.cuda.current_stream(dev)
    if isinstance(inp, synth.ScoreRows):
        # top-k only on given FP32 rows
        s = torch.from_numpy(inp.scores).to(dev)
        rl = torch.from_numpy(inp.row_len).to(dev)
        sel = torch.empty((inp.num_rows, inp.k), dtype=torch.int32, device=dev)
        cnt = torch.empty(inp.num_rows, dtype=torch.int32, device=dev)
        ws = bst.topk_workspace(inp.num_rows, inp.max_len, inp.k, dev)
        ms, kt = time_steps([bst.prepare_topk(s, rl, inp.max_len, inp.k, sel, cnt, ws)], K, warmup, stream)
        t_topk = kt["burst_ms"]
        alg = inp.num_rows * inp.max_len * 4 + inp.num_rows * inp.k * 4
        ach = alg / (t_topk * 1e-3) / 1e9
        log(f"{name}: {ms * 1e3:.1f} us/step (top-k {t_topk * 1e3:.1f} us)")
        return {"_inp": inp, "rows_per_s": round(inp.num_rows / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
                "config": {"workload": name, "rows": inp.num_rows, "row_len": inp.max_len, "k": inp.k,
                           "steps": "top-k only"},
                "kernels_us": {"topk": round(t_topk * 1e3, 2)},
                "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "topk (all launches)",
                             "algorithmic_bytes": alg, "avg_us": round(t_topk * 1e3, 2)}}
    if name == "qsa_indexshare_64req":
        return run_indexshare(name, inp, K, warmup, dev, stream)
    if isinstance(inp, synth.SelectBatch):
        return run_select_planned(name, inp, K, warmup, dev, stream)
    if isinstance(inp, synth.CompressInputs):
        return run_compress(name, inp, K, warmup, dev, stream)
    scorer = "prefill" if name == "qsa_prefill_8k" else "decode"
    path = IndexerPath(upload(inp, dev), scorer)
    if fused:
        fns, names = list(path.prepared()), ["score", "select_translate"]
    else:
        fns, names = [path.score, path.select, path.expand], ["score", "topk", "expand"]
    ms, kt = time_steps(fns, K, warmup, stream, probe=0)
    t_score = kt["burst_ms"]
    br = kernel_breakdown(fns, K, stream)
    cold = cold_steps(fns, 20, stream) if cold_reps else None
    log(f"{name}: {ms * 1e3:.1f} us/step; score {t_score * 1e3:.1f} us ({kt['burst']} back-to-back), "
        f"{kt['in_steps_ms'] * 1e3:.1f} us inside steps; separate pass: " +
        ", ".join(f"{n} {t * 1e3:.1f} us" for n, t in zip(names, br)) +
        (f"; cold (Infinity Cache flushed) {cold * 1e3:.1f} us/step" if cold else ""))
    method = (f"HIP events on the launch stream around {kt['burst']} back-to-back launches, right after the "
              "timed region")
    if scorer == "decode":
        # More than two rows per request (rounded up) go to the matrix-core
        # rows kernel (its own trace and traffic records).
        mfma_rows = -(-inp.num_rows // inp.num_req) > 2
        kname = "score_rows_mfma_kernel" if mfma_rows else "score_decode_kernel"
        dig = source_digest("score_decode.hip", "device.h")
        alg = scorer_bytes(inp)
        ach = alg / (t_score * 1e-3) / 1e9
        tr = kernel_trace_us(f"{name}:{kname}", dig)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("score_rows_mfma" if mfma_rows else "score_decode", dig, name),
                "kernel": kname, "algorithmic_bytes": alg, "avg_us": round(t_score * 1e3, 2), "avg_us_method": method,
                "avg_us_in_steps": round(kt["in_steps_ms"] * 1e3, 2),
                "kernel_trace_avg_us": tr,
                "frac_kernel_trace": round(alg / (tr * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if tr else None}
    else:
        kname, dig = "score_prefill_kernel", source_digest("score_prefill.hip", "device.h")
        fl = prefill_flops(inp)
        ach = fl / (t_score * 1e-3) / 1e12
        tr = kernel_trace_us(f"{name}:{kname}", dig)
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("score_prefill", dig, name),
                "kernel": kname, "algorithmic_flops": fl, "avg_us": round(t_score * 1e3, 2), "avg_us_method": method,
                "avg_us_in_steps": round(kt["in_steps_ms"] * 1e3, 2),
                "kernel_trace_avg_us": tr,
                "frac_kernel_trace": round(fl / (tr * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4) if tr else None}
    sb = step_bytes(inp)
    step_roof = {"bound": "hbm", "algorithmic_bytes": sb, "achieved": round(sb / (ms * 1e-3) / 1e9, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(sb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "bytes": "keys once per request + q + page-table entries + selection written; scores are an "
                          "intermediate, not counted"}
    out = {"_inp": inp, "rows_per_s": round(inp.num_rows / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
           "config": {"workload": name, "rows": inp.num_rows, "requests": inp.num_req,
                      "max_visible_blocks": inp.max_vis, "k": inp.k, "c": inp.c, "scorer": scorer,
                      "page_tokens": 64,
                      "steps": "score -> select+translate (one kernel)" if fused else
                               "score -> top-k -> expand/translate"},
           "kernels_us": {**{n: round(t * 1e3, 2) for n, t in zip(names, br)},
                          "note": "separate pass after the timed region, every call bracketed by HIP events"},
           "roofline": roof, "step_roofline": step_roof}
    if cold:
        out["cold_ms_per_step"] = round(cold, 5)
        out["cold_rows_per_s"] = round(inp.num_rows / (cold * 1e-3), 1)
        out["cold_note"] = ("median of 20 steps, each after a reduction over a 512 MiB scratch buffer (reads "
                            "evict the 256 MB Infinity Cache and leave it clean), outside the events")
    return out


def run_select_planned(name, w, K, warmup, dev, stream):
    """Selection + translation of a mixed batch on given FP32 rows, as the
    layers of one step would run it: a step is two select+translate calls on
    the same lengths (two layers).  Planned: topk_plan_rows once per step,
    then two idx_select_translate_planned calls on its work list.  Unplanned
    (reported beside it): two idx_select_translate calls, which size their
    launch from max_len alone."""
    import torch

    import block_scoring_top_amd as bst
    from synth.device import upload

    inp = w.inp
    d = upload(inp, dev)
    R, L, k = w.num_rows, w.max_len, inp.k
    s = torch.from_numpy(w.scores).to(dev)
    rl = torch.from_numpy(w.row_len).to(dev)
    sel = torch.empty((R, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(R, dtype=torch.int32, device=dev)
    slots = torch.empty((R, inp.ld_out), dtype=torch.int32, device=dev)
    pos = torch.empty((R, inp.ld_out), dtype=torch.int32, device=dev)
    oc = torch.empty(R, dtype=torch.int32, device=dev)
    plan = bst.topk_plan(R, L, dev)
    ws_p = bst.topk_planned_workspace(R, L, k, dev)
    ws_u = bst.topk_workspace(R, L, k, dev)
    mk_plan = bst.prepare_plan(rl, L, plan)
    sel_p = bst.prepare_select_translate_planned(s, L, k, d.req_row_ptr, d.row_pos, inp.c, d.page_table, sel, cnt,
                                                 slots, oc, plan, out_pos=pos, workspace=ws_p)
    sel_u = bst.prepare_select_translate(s, rl, L, k, d.req_row_ptr, d.row_pos, inp.c, d.page_table, sel, cnt,
                                         slots, oc, out_pos=pos, workspace=ws_u)
    ms_p, kt_p = time_steps([mk_plan, sel_p, sel_p], K, warmup, stream, probe=1)
    _, kt_plan = time_steps([mk_plan], max(K // 5, 2), 2, stream, probe=0)
    ms_u, kt_u = time_steps([sel_u, sel_u], K, warmup, stream, probe=0)
    torch.cuda.synchronize()
    items = int(plan[0].item())
    split = int(plan[1].item())
    n_out = int(oc.sum().item())
    t_sel = kt_p["burst_ms"]
    # one launch: every row read once up to its length, the selection, the
    # slots and positions written
    alg = int(w.row_len.astype("int64").sum()) * 4 + R * k * 4 + n_out * 8 + R * 8
    ach = alg / (t_sel * 1e-3) / 1e9
    log(f"{name}: planned {ms_p * 1e3:.1f} us/step (plan {kt_plan['burst_ms'] * 1e3:.1f} us, select "
        f"{t_sel * 1e3:.1f} us x 2; {items} items, split from {split}); unplanned {ms_u * 1e3:.1f} us/step "
        f"(select {kt_u['burst_ms'] * 1e3:.1f} us x 2)")
    return {"_inp": w, "rows_per_s": round(2 * R / (ms_p * 1e-3), 1), "ms_per_step": round(ms_p, 5),
            "unplanned_ms_per_step": round(ms_u, 5),
            "config": {"workload": name, "rows": R, "long_rows": int((w.row_len >= 32769).sum()),
                       "max_len": L, "k": k, "c": inp.c, "page_tokens": 64, "plan_items": items,
                       "split_from": split,
                       "steps": "plan once, then select+translate twice (two layers on the same lengths); "
                                "rows/s counts both calls' rows"},
            "kernels_us": {"plan": round(kt_plan["burst_ms"] * 1e3, 2), "select_planned": round(t_sel * 1e3, 2),
                           "select_unplanned": round(kt_u["burst_ms"] * 1e3, 2)},
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "topk_planned_kernel", "algorithmic_bytes": alg, "avg_us": round(t_sel * 1e3, 2)}}


def run_indexshare(name, inp, K, warmup, dev, stream):
    """A draft step under IndexShare: the selection made at each row's captured
    position (score + select on the GPU, once, outside the timed region) is
    expanded at the last draft position, captured + max_advance.  The step is
    the one idx_expand_translate_shared call."""
    import torch

    import block_scoring_top_amd as bst
    import synth
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload

    d = upload(inp, dev)
    path = IndexerPath(d, "decode")
    path.run()
    adv = synth.INDEXSHARE_MAX_ADVANCE
    now = (d.row_pos + adv).contiguous()
    R = d.num_rows
    ld_out = d.ld_out + adv
    slots = torch.empty((R, ld_out), dtype=torch.int32, device=dev)
    pos = torch.empty((R, ld_out), dtype=torch.int32, device=dev)
    cnt = torch.empty(R, dtype=torch.int32, device=dev)
    call = bst.prepare_expand_shared(path.sel, path.sel_count, d.k, d.req_row_ptr, d.row_pos, now, d.c, adv,
                                     d.page_table, slots, cnt, out_pos=pos)
    ms, kt = time_steps([call], K, warmup, stream)
    t_call = kt["burst_ms"]
    torch.cuda.synchronize()
    n_out = int(cnt.sum().item())
    alg = int(path.sel_count.sum().item()) * 4 + n_out * (4 + 4) + R * 16  # selection in, slots + positions out
    ach = alg / (t_call * 1e-3) / 1e9
    log(f"{name}: {ms * 1e3:.1f} us/step (expand of the captured selection at +{adv} positions)")
    return {"_inp": inp, "rows_per_s": round(R / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "config": {"workload": name, "rows": R, "requests": inp.num_req, "k": inp.k, "c": inp.c,
                       "max_advance": adv, "page_tokens": 64,
                       "steps": "expand/translate of a captured selection (the draft step's whole indexer work)"},
            "kernels_us": {"expand_shared": round(t_call * 1e3, 2)},
            "roofline": {"bound": "latency", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "expand_kernel",
                         "algorithmic_bytes": alg, "avg_us": round(t_call * 1e3, 2)}}


def run_compress(name, ci, K, warmup, dev, stream):
    """Key compression into the c = 4 cache: one idx_compress_store call over
    the batch's new raw keys (each step recomputes the same blocks)."""
    import numpy as np

    import block_scoring_top_amd as bst
    from synth.device import upload_compress

    d = upload_compress(ci, dev)
    call = bst.prepare_compress_store(*d.args())
    ms, kt = time_steps([call], K, warmup, stream)
    t_call = kt["burst_ms"]
    counts = np.diff(ci.req_tok_ptr).astype(np.int64)
    starts = ci.tok_start.astype(np.int64)
    blocks = (starts + counts) // 4 - starts // 4
    straddle = np.where((blocks > 0) & (starts % 4 > 0), starts % 4, 0)
    T = ci.num_tok
    alg = (T * 256 + (T * 12 if ci.mrope_pos is not None else 0)      # raw keys and MRoPE positions in
           + int(straddle.sum()) * 256 + ci.num_req * 8                  # ring entries of straddling blocks
           + int(blocks.sum()) * (256 + 4)                               # compressed keys out, page ids in
           + int(np.minimum(counts, 4).sum()) * 256 + ci.num_req * 12)   # ring and ring positions out
    ach = alg / (t_call * 1e-3) / 1e9
    log(f"{name}: {ms * 1e3:.1f} us/step ({int(blocks.sum())} compressed keys from {T} new tokens)")
    return {"_inp": ci, "rows_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "config": {"workload": name, "requests": ci.num_req, "new_tokens": T,
                       "compressed_keys": int(blocks.sum()), "rotary_dim": ci.rotary_dim,
                       "mrope_sections": list(ci.sections), "theta": ci.theta,
                       "mrope": "explicit" if ci.mrope_pos is not None else "text positions",
                       "steps": "key compression and store (rows = new tokens)"},
            "kernels_us": {"compress": round(t_call * 1e3, 2)},
            "roofline": {"bound": "latency", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "compress_kernel",
                         "algorithmic_bytes": alg, "avg_us": round(t_call * 1e3, 2)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsa_decode_16x80k")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="also time every other workload (extra field)")
    ap.add_argument("--unfused", action="store_true", help="separate top-k and expand calls")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the steps timed with the Infinity Cache flushed before each")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): every call of this path runs on one "
              "GPU with no collectives, and no multi-GPU form is built", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return
    res = run_workload(args.workload, args.steps, args.warmup, dev, fused=not args.unfused,
                       cold_reps=not args.no_cold)
    inp = res.pop("_inp")
    extra = {}
    if args.all:
        for name in synth.WORKLOADS:
            if name == args.workload:
                continue
            r = run_workload(name, args.steps, args.warmup, dev, fused=not args.unfused,
                             cold_reps=not args.no_cold)
            r.pop("_inp")
            extra[name] = r
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    line = {
        "metric": "indexer rows/s (score+top-k) at L=80k; achieved HBM GB/s and % of peak",
        "value": res["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q ~N(0,1), keys ~N(0,1) L2-normalised, bf16; random page permutation)",
        "config": res["config"],
        "kernels_us": res["kernels_us"],
        "roofline": res["roofline"],
        "step_roofline": res.get("step_roofline"),
        "cpu_baseline": cpu,
    }
    for key in ("cold_ms_per_step", "cold_rows_per_s", "cold_note"):
        if key in res:
            line[key] = res[key]
    if extra:
        line["other_workloads"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
