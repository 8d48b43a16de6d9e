"""Helpers for GPU tests: run the HIP path on seeded inputs and bring results
back as numpy arrays."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_scoring_top_amd as bst
from block_scoring_top_amd.pipeline import IndexerPath
from synth.device import upload, upload_compress


def say(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def run_path(inp, scorer: str = "decode", fused: bool = True, planned: bool = False):
    say(f"path {scorer} fused={fused} planned={planned}: {getattr(inp, 'name', '?')} rows={inp.num_rows} "
        f"max_vis={inp.max_vis} k={inp.k} c={inp.c}")
    dev = upload(inp, "cuda")
    p = IndexerPath(dev, scorer)
    p.run(fused=fused, planned=planned)
    torch.cuda.synchronize()
    return dict(scores=p.scores.cpu().numpy(), row_len=p.row_len.cpu().numpy(), sel=p.sel.cpu().numpy(),
                sel_count=p.sel_count.cpu().numpy(), slots=p.slots.cpu().numpy(), pos=p.pos.cpu().numpy(),
                out_count=p.out_count.cpu().numpy())


def gpu_topk(scores: np.ndarray, row_len: np.ndarray, k: int, max_len: int | None = None, reps: int = 1,
             workspace=None):
    """Runs topk_select_rows on given FP32 rows; returns a list of (sel, count)
    per repetition (same workspace each time)."""
    R, ld = scores.shape
    max_len = ld if max_len is None else max_len
    say(f"topk rows={R} ld={ld} max_len={max_len} k={k} reps={reps}")
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).cuda()
    rl = torch.from_numpy(np.ascontiguousarray(row_len, dtype=np.int32)).cuda()
    ws = workspace if workspace is not None else bst.topk_workspace(R, max_len, k, "cuda")
    outs = []
    for _ in range(reps):
        sel = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
        bst.topk_select_rows(s, rl, max_len, k, sel, cnt, ws)
        torch.cuda.synchronize()
        outs.append((sel.cpu().numpy(), cnt.cpu().numpy()))
    return outs, ws


def gpu_expand(inp, sel: np.ndarray, count: np.ndarray):
    say(f"expand rows={inp.num_rows} k={inp.k} c={inp.c}")
    dev = upload(inp, "cuda")
    R = inp.num_rows
    s = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(count, dtype=np.int32)).cuda()
    slots = torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda")
    oc = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    bst.idx_expand_translate(s, c, inp.k, dev.req_row_ptr, dev.row_pos, inp.c, dev.page_table, slots, oc,
                             out_pos=pos)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), pos.cpu().numpy(), oc.cpu().numpy()


def gpu_expand_shared(inp, sel: np.ndarray, count: np.ndarray, row_pos_now: np.ndarray, max_advance: int):
    say(f"expand shared rows={inp.num_rows} k={inp.k} c={inp.c} max_advance={max_advance}")
    dev = upload(inp, "cuda")
    R = inp.num_rows
    ld_out = inp.ld_out + max_advance
    s = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(count, dtype=np.int32)).cuda()
    now = torch.from_numpy(np.ascontiguousarray(row_pos_now, dtype=np.int32)).cuda()
    slots = torch.full((R, ld_out), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((R, ld_out), -7, dtype=torch.int32, device="cuda")
    oc = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    bst.idx_expand_translate_shared(s, c, inp.k, dev.req_row_ptr, dev.row_pos, now, inp.c, max_advance,
                                    dev.page_table, slots, oc, out_pos=pos)
    torch.cuda.synchronize()
    return slots.cpu().numpy(), pos.cpu().numpy(), oc.cpu().numpy()


def gpu_scores(inp, scorer: str = "decode", ld: int | None = None):
    say(f"score {scorer}: rows={inp.num_rows} max_vis={inp.max_vis} c={inp.c}")
    dev = upload(inp, "cuda")
    R = inp.num_rows
    ld = max(inp.max_vis, 1) if ld is None else ld
    scores = torch.full((R, ld), float("nan"), dtype=torch.float32, device="cuda")
    row_len = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    fn = bst.idx_score_decode if scorer == "decode" else bst.idx_score_prefill
    fn(dev.q, dev.kcache, dev.num_pages, dev.page_table, dev.req_row_ptr, dev.row_pos, inp.c, inp.max_vis,
       scores, row_len)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), row_len.cpu().numpy()


def pending_counts(inp) -> np.ndarray:
    t = inp.row_pos.astype(np.int64)
    return (t + 1 - inp.c * ((t + 1) // inp.c)).astype(np.int32)


def gpu_compress(ci, kcache=None, ring=None, ring_pos=None, max_tok=None):
    """Runs idx_compress_store on ``ci`` starting from the given (default:
    ci's) cache and ring state; returns dict(kcache, ring, ring_pos)."""
    say(f"compress {getattr(ci, 'name', '?')} requests={ci.num_req} tokens={ci.num_tok} max_tok={ci.max_tok} "
        f"rot={ci.rotary_dim} sections={ci.sections} mrope={'yes' if ci.mrope_pos is not None else 'text'}")
    d = upload_compress(ci, "cuda")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    if kcache is not None:
        d.kcache = bf(kcache)
    if ring is not None:
        d.ring = bf(ring)
    if ring_pos is not None:
        d.ring_pos = torch.from_numpy(np.ascontiguousarray(ring_pos, dtype=np.int32)).cuda()
    if max_tok is not None:
        d.max_tok = int(max_tok)
    bst.idx_compress_store(*d.args())
    torch.cuda.synchronize()
    return dict(kcache=d.kcache.cpu().numpy().view(np.uint16), ring=d.ring.cpu().numpy().view(np.uint16),
                ring_pos=d.ring_pos.cpu().numpy())

