"""idx_select_translate_noalloc (long-row records in a static device array)
against idx_select_translate (records in the caller's workspace): the same
selections and translations, on two calls in a row, the second smaller, plus
a batch of short rows (no records) and a request too large for the array."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scoring_top_amd as bst
import oracle
import synth
from checkers import canonical_expand, canonical_sel, check_topk_exact

pytestmark = pytest.mark.gpu


def _batch(rng, lens, c, k):
    """One row per request at the last position of an n_vis-block context,
    a seeded page permutation, FP32 score rows (nothing is scored)."""
    ctx = [int(c * (n + 1)) for n in lens]
    pages = [-(-t // 64) for t in ctx]
    perm = rng.permutation(int(sum(pages)))
    pt = np.full((len(ctx), max(pages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[off:off + n]
        off += n
    R = len(lens)
    row_pos = np.array([t - 1 for t in ctx], dtype=np.int32)
    inp = synth.IndexerInputs(name="noalloc", c=c, k=k, q=np.zeros((R, 4, 128), np.uint16),
                              kcache=np.zeros((64 // c, 128), np.uint16), num_pages=int(off), page_table=pt,
                              req_row_ptr=np.arange(R + 1, dtype=np.int32), row_pos=row_pos,
                              max_vis=int(((row_pos.astype(np.int64) + 1) // c).max()), seed=0)
    rows = rng.standard_normal((R, int(max(lens)))).astype(np.float32)
    return inp, rows, np.asarray(lens, dtype=np.int32)


def _run(inp, rows, lens, noalloc):
    from synth.device import upload
    d = upload(inp, "cuda")
    R, ld = rows.shape
    s = torch.from_numpy(rows).cuda()
    rl = torch.from_numpy(lens).cuda()
    out = dict(sel=torch.full((R, inp.k), -7, dtype=torch.int32, device="cuda"),
               cnt=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
               slots=torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda"),
               pos=torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda"),
               oc=torch.full((R,), -7, dtype=torch.int32, device="cuda"))
    args = (s, rl, ld, inp.k, d.req_row_ptr, d.row_pos, inp.c, d.page_table, out["sel"], out["cnt"], out["slots"],
            out["oc"])
    if noalloc:
        print(f"[no-alloc] noalloc call rows={R} max_len={ld} k={inp.k} c={inp.c}", flush=True)
        bst.idx_select_translate_noalloc(*args, out_pos=out["pos"])
    else:
        print(f"[no-alloc] workspace call rows={R} max_len={ld} k={inp.k} c={inp.c}", flush=True)
        ws = bst.topk_workspace(R, ld, inp.k, "cuda")
        bst.idx_select_translate(*args, out_pos=out["pos"], workspace=ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _same(a, b, inp):
    assert np.array_equal(a["cnt"], b["cnt"]) and np.array_equal(a["oc"], b["oc"])
    for x, y in zip(canonical_sel(a["sel"], a["cnt"]), canonical_sel(b["sel"], b["cnt"])):
        assert np.array_equal(x, y)
    t = inp.row_pos.astype(np.int64)
    pend = (t + 1 - inp.c * ((t + 1) // inp.c)).astype(np.int32)
    for (p1, s1), (p2, s2) in zip(canonical_expand(a["slots"], a["pos"], a["oc"], pend),
                                  canonical_expand(b["slots"], b["pos"], b["oc"], pend)):
        assert np.array_equal(p1, p2) and np.array_equal(s1, s2)


def test_noalloc_matches_the_workspace_call():
    rng = np.random.default_rng(4242)
    # 1: sixteen rows of 81,920 entries (every row split over chunk workgroups)
    inp, rows, lens = _batch(rng, [81920] * 16, 1, 2048)
    a, b = _run(inp, rows, lens, True), _run(inp, rows, lens, False)
    _same(a, b, inp)
    check_topk_exact(a["sel"], a["cnt"], *oracle.topk(rows, lens, inp.k))
    # 2: a smaller batch right after, other lengths, k and c (the array keeps
    # the first call's contents; that call left them zero-filled)
    inp, rows, lens = _batch(rng, [40000, 33000, 50001], 4, 512)
    rows[1] = np.float32(0.75)  # a tie storm: the whole-row fallback
    a, b = _run(inp, rows, lens, True), _run(inp, rows, lens, False)
    _same(a, b, inp)
    check_topk_exact(a["sel"], a["cnt"], *oracle.topk(rows, lens, inp.k))
    # 3: short rows only (no records needed)
    inp, rows, lens = _batch(rng, [3000, 16384, 20000], 4, 512)
    a, b = _run(inp, rows, lens, True), _run(inp, rows, lens, False)
    _same(a, b, inp)


def test_noalloc_rejects_more_than_its_scratch():
    rng = np.random.default_rng(4343)
    per_row = bst.topk_workspace_bytes(1, 81920, 2048)
    R = bst.NOALLOC_SCRATCH_BYTES // per_row + 1
    inp, rows, lens = _batch(rng, [81920] * R, 1, 2048)
    with pytest.raises(bst.BlockScoreError):
        _run(inp, rows, lens, True)
