"""HIP path vs the CPU oracle, through the C ABI, on seeded inputs.

Bars: scores within 1e-4*(1+|s|); top-k on given FP32 rows identical; top-k
on the GPU's own scores identical to the oracle's top-k of those same scores;
end-to-end selections differing only within 2e-4 of the k-th oracle score;
expand/translate of a given selection identical in canonical form.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from checkers import (check_expand_exact, check_scores, check_topk_e2e, check_topk_exact)

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def _full_check(inp, scorer="decode", fused=True, planned=False):
    """Every stage against the oracle: scores (tolerance), top-k of the GPU
    scores (exact), end-to-end selection (band), expand of the GPU selection
    (exact).  fused: select + translate in one kernel, else separate calls;
    planned: the selection over a plan built from the scorer's row lengths."""
    g = gu.run_path(inp, scorer, fused, planned)
    ref = oracle.pipeline(inp)
    assert np.array_equal(g["row_len"], ref["row_len"])
    check_scores(g["scores"], ref["scores"], ref["row_len"])
    ld = max(inp.max_vis, 1)
    sel_on_gpu_scores, cnt_on_gpu_scores = oracle.topk(np.ascontiguousarray(g["scores"][:, :ld]), g["row_len"], inp.k)
    check_topk_exact(g["sel"], g["sel_count"], sel_on_gpu_scores, cnt_on_gpu_scores)
    swaps = check_topk_e2e(g["sel"], g["sel_count"], ref["scores"], ref["sel"], ref["sel_count"], ref["row_len"])
    slots, pos, oc = oracle.expand_translate(inp, g["sel"], g["sel_count"])
    check_expand_exact(g["slots"], g["pos"], g["out_count"], slots, pos, oc, gu.pending_counts(inp))
    return swaps


# ---------------------------------------------------------------------------
# Decode scorer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fused", [True, False])
def test_decode_cfg_qsa_1x8k_end_to_end(fused):
    _full_check(synth.qsa_decode_1x8k(), fused=fused)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_verify_small_ragged(fused):
    _full_check(synth.qsa_verify_64req(B=8, lo=300, hi=20000), fused=fused)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_dsa_small(fused):
    _full_check(synth.dsa_decode_16x80k(B=3, L=5000), fused=fused)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_dsa_long_rows_small_batch(fused):
    # few long rows: the multi-workgroup selection (and its fused translation)
    _full_check(synth.dsa_decode_16x80k(B=3, L=50000), fused=fused)


def test_decode_edge_rows():
    # rows with 0 visible blocks, 1 block, page boundaries; a request with no
    # rows; a request with 11 rows (more than one row group).
    rng = np.random.default_rng(101)
    rows = [[0, 1, 2], [3, 4, 5, 62, 63, 64, 65, 66, 67], [], [400 + i for i in range(11)]]
    inp = synth.build_paged_batch("edge", 101, c=4, k=8, ctx_tokens=[3, 68, 1, 411], row_pos_per_req=rows, rng=rng)
    _full_check(inp)
    inp1 = synth.build_paged_batch("edge1", 102, c=1, k=8, ctx_tokens=[3, 68, 1, 411], row_pos_per_req=rows, rng=rng)
    _full_check(inp1)


@pytest.mark.parametrize("c", [4, 1])
def test_decode_many_rows_per_request(c):
    # 11 rows per request on average: the matrix-core multi-row scorer with
    # 16 rows per pass (a 20-row request takes two passes); a 1-row request
    # and rows near page boundaries in the same batch.
    rng = np.random.default_rng(303 + c)
    rows = [list(range(2000, 2020)), [63], list(range(4090, 4103)), list(range(900, 911))]
    inp = synth.build_paged_batch("many", 303 + c, c=c, k=64, ctx_tokens=[2020, 64, 4103, 911],
                                  row_pos_per_req=rows, rng=rng)
    _full_check(inp)


def _rows_per_request_batch(seed, c, rpr, k):
    """Requests of exactly ``rpr`` query rows each (the row count per request
    picks the decode kernel: 1-2 the VALU kernel with that many rows per pass,
    3-4 the matrix-core kernel with 4 rows per pass).  Rows end at the last
    context token; one request sits at the start of the context (n_vis = 0
    for t <= 2 at c = 4) and one straddles a page boundary."""
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(200, 12000, 6)]
    rows = [list(range(t - rpr, t)) for t in ctx]
    ctx.append(rpr)
    rows.append(list(range(rpr)))
    b0 = 64 if c == 1 else 256  # first token of page 1 (c = 1) / block 64 (c = 4)
    first = b0 - (rpr + 1) // 2
    ctx.append(first + rpr + 1)
    rows.append(list(range(first, first + rpr)))
    return synth.build_paged_batch(f"rpr{rpr}", seed, c=c, k=k, ctx_tokens=ctx, row_pos_per_req=rows, rng=rng)


@pytest.mark.parametrize("c", [4, 1])
@pytest.mark.parametrize("rpr", [1, 2, 3, 4])
def test_decode_each_rows_per_request_kernel(rpr, c):
    inp = _rows_per_request_batch(500 + 10 * rpr + c, c, rpr, k=64)
    assert np.all(np.diff(inp.req_row_ptr) == rpr)
    _full_check(inp)


def test_decode_verify_with_few_drafts():
    # speculative verify with 1-3 draft tokens (2-4 rows per request)
    for rows in (2, 3, 4):
        _full_check(synth.qsa_verify_64req(B=12, verify_rows=rows, lo=300, hi=40000))


def test_decode_power_of_two_scaling_exact():
    # s(2q) == 2*s(q) bit for bit in any fixed accumulation order.
    inp = synth.qsa_verify_64req(B=4, lo=1000, hi=9000)
    s1, l1 = gu.gpu_scores(inp)
    q2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.q) * np.float32(2.0))
    s2, l2 = gu.gpu_scores(synth.IndexerInputs(**{**inp.__dict__, "q": q2}))
    for r in range(inp.num_rows):
        n = l1[r]
        assert np.array_equal(s2[r, :n], np.float32(2.0) * s1[r, :n])


@pytest.mark.parametrize("wl", ["verify", "dsa"])
def test_decode_planned_end_to_end(wl):
    # score -> plan (from the scorer's row lengths) -> planned select+translate:
    # the ragged verify batch (rows of 75-5,000 blocks) and long DSA rows
    # (split into chunk items).
    inp = (synth.qsa_verify_64req(B=8, lo=300, hi=20000) if wl == "verify"
           else synth.dsa_decode_16x80k(B=3, L=40000))
    _full_check(inp, planned=True)


def test_bound_calls_match_prepared():
    # The step through calls bound to a stream gives the same outputs as the
    # prepared calls on the current stream (and as the oracle).
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload
    inp = synth.qsa_verify_64req(B=4, lo=300, hi=9000)
    gu.say("bound calls vs prepared calls")
    p = IndexerPath(upload(inp, "cuda"), "decode")
    p.run()
    torch.cuda.synchronize()
    want = [t.cpu().numpy().copy() for t in (p.scores, p.row_len, p.sel_count, p.out_count)]
    sel_w = np.sort(p.sel.cpu().numpy(), 1)
    for t in (p.scores, p.sel, p.sel_count, p.slots, p.out_count):
        t.fill_(-3)
    stream = torch.cuda.Stream()
    score, select = p.bound(stream)
    score()
    select()
    stream.synchronize()
    got = [t.cpu().numpy() for t in (p.scores, p.row_len, p.sel_count, p.out_count)]
    rl = want[1]
    for r in range(inp.num_rows):
        assert np.array_equal(got[0][r, :rl[r]].view(np.uint32), want[0][r, :rl[r]].view(np.uint32))
    for a, b in zip(got[1:], want[1:]):
        assert np.array_equal(a, b)
    assert np.array_equal(np.sort(p.sel.cpu().numpy(), 1), sel_w)


def test_decode_leaves_invisible_entries_untouched():
    inp = synth.qsa_verify_64req(B=5, lo=500, hi=6000)
    s, rl = gu.gpu_scores(inp, ld=inp.max_vis + 40)
    for r in range(inp.num_rows):
        assert np.all(np.isfinite(s[r, :rl[r]]))
        assert np.all(np.isnan(s[r, rl[r]:]))


def _ws_clean(ws) -> bool:
    """What every call must leave in a workspace for the next: the first
    4 bytes of every 64 KiB block zero."""
    return int(ws.view(torch.int32)[::16384].count_nonzero().item()) == 0 if ws is not None else True


# ---------------------------------------------------------------------------
# Top-k on given FP32 rows: bit-exact
# ---------------------------------------------------------------------------

def test_topk_cfg_8x80k_exact():
    w = synth.topk_8x80k()
    (out,), _ = gu.gpu_topk(w.scores, w.row_len, w.k)
    ref_sel, ref_cnt = oracle.topk(w.scores, w.row_len, w.k)
    check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


def test_topk_1x1m_exact():
    # The one-million-entry row that bench.py times (123 chunks, one launch).
    w = synth.topk_1x1m()
    (out,), _ = gu.gpu_topk(w.scores, w.row_len, w.k)
    ref_sel, ref_cnt = oracle.topk(w.scores, w.row_len, w.k)
    check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


@pytest.mark.parametrize("n", [1, 7, 511, 512, 513, 2047, 2048, 2049, 4096, 16383, 16384, 16385, 32768, 32769,
                               50000])
def test_topk_lengths_and_tie_storms(n):
    rows = synth.tie_storm_rows(1000 + n, 8, n)
    rng = np.random.default_rng(n)
    rows = np.concatenate([rows, rng.standard_normal((2, n)).astype(np.float32)])
    lens = np.full(rows.shape[0], n, dtype=np.int32)
    for k in (1, 512, 2048):
        (out,), _ = gu.gpu_topk(rows, lens, k)
        ref_sel, ref_cnt = oracle.topk(rows, lens, k)
        check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


def test_topk_many_rows_exact():
    # A batch of >= 1,024 rows of at most 16,384 entries takes the many-rows
    # shape (several rows per CU); mixed lengths, tie storms and rows whose
    # boundary bin overflows the LDS candidate list.
    n = 16384
    R = 1100
    rng = np.random.default_rng(1100)
    rows = rng.standard_normal((R, n)).astype(np.float32)
    rows[:64] = synth.tie_storm_rows(1101, 64, n)
    rows[64:80] = np.float32(1.0) + rng.integers(0, 3, (16, n)).astype(np.float32) * np.float32(2.0 ** -20)
    lens = rng.integers(0, n + 1, R).astype(np.int32)
    special = [0, 1, 511, 512, 513, 2047, 2048, 2049, 16383, 16384]
    lens[:len(special)] = special
    lens[64:80] = n
    for k in (512, 2048):
        (out,), _ = gu.gpu_topk(rows, lens, k)
        ref_sel, ref_cnt = oracle.topk(rows, lens, k)
        check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


def test_topk_mixed_lengths_one_launch():
    # one launch mixing every path: take-all, register, streaming, multi-workgroup
    rng = np.random.default_rng(7)
    ld = 90000
    lens = np.array([0, 1, 100, 511, 512, 600, 5000, 16384, 16385, 30000, 32768, 32769, 45000, 81920, 90000],
                    dtype=np.int32)
    rows = rng.standard_normal((lens.shape[0], ld)).astype(np.float32)
    rows[3] = 1.0
    rows[9, ::3] = 0.25
    for k in (512, 2048):
        (out,), _ = gu.gpu_topk(rows, lens, k)
        ref_sel, ref_cnt = oracle.topk(rows, lens, k)
        check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


@pytest.mark.parametrize("R", [256, 257])
def test_topk_long_rows_many(R):
    # Hundreds of rows of >= 32,769 entries, each split over chunk workgroups
    # (workspace, device-scope hand-off), with a few short rows selected whole
    # in the same launch.  Odd k values, ragged lengths, tie storms.
    n = 33000
    rng = np.random.default_rng(R)
    rows = rng.standard_normal((R, n)).astype(np.float32)
    rows[:16] = synth.tie_storm_rows(R + 5, 16, n)
    lens = rng.integers(32769, n + 1, R).astype(np.int32)
    lens[-4:] = [0, 1, 2048, 32768]
    for k in (3, 1000, 2047):
        (out,), _ = gu.gpu_topk(rows, lens, k)
        ref_sel, ref_cnt = oracle.topk(rows, lens, k)
        check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


@pytest.mark.parametrize("fused", [False, True])
def test_topk_very_long_rows(fused):
    # Rows far past the headline length, through every form of the long-row
    # resolution: at 200,000 entries and k = 2,048 the resolving workgroup
    # holds 16 candidate slots per lane (4,800 slots), at 1,000,000 entries 32
    # (11,808 slots); a 1,000,000-entry row whose winners cluster in one chunk
    # fails the exactness check and is selected whole by streaming, and so is
    # a 2,000,000-entry row, whose candidate slots (23,520) exceed what the
    # resolving workgroup holds; a short row rides along.
    rng = np.random.default_rng(2100)
    n = 2_000_000
    lens = np.array([200_000, 1_000_000, 1_000_000, n, 5000], dtype=np.int32)
    rows = rng.standard_normal((lens.size, n)).astype(np.float32)
    rows[2, 500_000:510_000] += np.float32(3.0)  # winners clustered in one chunk
    for k in (2048, 512):
        if fused:
            inp = _given_rows_batch(rng, [int(x) + 1 for x in lens], 1, k)
            _check_given(inp, rows, lens, _select_translate_given(inp, rows, lens, n))
        else:
            (out,), _ = gu.gpu_topk(rows, lens, k)
            ref_sel, ref_cnt = oracle.topk(rows, lens, k)
            check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


def test_topk_overflowing_boundary_bin():
    # more than 4,096 entries tie in the boundary bin: exercises the re-scan refinement
    rng = np.random.default_rng(8)
    for n in (12000, 30000, 70000):
        rows = np.empty((3, n), dtype=np.float32)
        rows[0] = np.float32(1.0) + rng.integers(0, 16, n).astype(np.float32) * np.float32(2.0 ** -20)
        rows[1] = np.float32(3.0)
        rows[2] = rng.choice(np.array([0.5, 0.5000001, 0.50000006], dtype=np.float32), n)
        lens = np.full(3, n, dtype=np.int32)
        for k in (1, 2048):
            (out,), _ = gu.gpu_topk(rows, lens, k)
            ref_sel, ref_cnt = oracle.topk(rows, lens, k)
            check_topk_exact(out[0], out[1], ref_sel, ref_cnt)


def test_topk_repeat_determinism_and_workspace_reset():
    w = synth.topk_8x80k(seed=77)
    outs, ws = gu.gpu_topk(w.scores, w.row_len, w.k, reps=20)
    ref_sel, ref_cnt = oracle.topk(w.scores, w.row_len, w.k)
    for sel, cnt in outs:
        check_topk_exact(sel, cnt, ref_sel, ref_cnt)
    assert _ws_clean(ws), "the first word of every 64 KiB block of the workspace must be left zero"
    # another batch through the same workspace
    w2 = synth.topk_8x80k(seed=78)
    (out,), _ = gu.gpu_topk(w2.scores, w2.row_len, w2.k, workspace=ws)
    r2 = oracle.topk(w2.scores, w2.row_len, w2.k)
    check_topk_exact(out[0], out[1], *r2)


def test_topk_workspace_reused_across_shapes():
    # One zero-filled workspace, sized for the largest call, used by calls of
    # other row counts, lengths and k in turn: each leaves it zero-filled, so
    # the next call's layout over it starts from zeros.
    rng = np.random.default_rng(2024)
    shapes = [(16, 81920, 2048), (3, 50000, 512), (40, 33000, 100), (16, 81920, 2048), (7, 70000, 2047)]
    import block_scoring_top_amd as bst
    big = max(bst.topk_workspace_bytes(R, n, k) for R, n, k in shapes)
    import torch
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for R, n, k in shapes:
        rows = rng.standard_normal((R, n)).astype(np.float32)
        lens = rng.integers(32769, n + 1, R).astype(np.int32)
        (out,), _ = gu.gpu_topk(rows, lens, k, workspace=ws)
        check_topk_exact(out[0], out[1], *oracle.topk(rows, lens, k))
        assert _ws_clean(ws)


def test_topk_qsa_score_rows():
    # real QSA-shaped score rows (non-negative, many exact zeros)
    inp = synth.qsa_verify_64req(B=6, lo=20000, hi=131072)
    scores, rl = oracle.score(inp)
    scores = np.nan_to_num(scores, nan=-1.0)
    (out,), _ = gu.gpu_topk(scores, rl, 512, max_len=inp.max_vis)
    ref = oracle.topk(scores, rl, 512)
    check_topk_exact(out[0], out[1], *ref)


# ---------------------------------------------------------------------------
# Expand / translate: exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("c", [1, 4])
def test_expand_exact_on_oracle_selection(c):
    inp = (synth.qsa_verify_64req(B=7, lo=200, hi=30000) if c == 4 else synth.dsa_decode_16x80k(B=2, L=6000))
    ref = oracle.pipeline(inp)
    # scramble the order within each selection: the output order is free
    sel = ref["sel"].copy()
    rng = np.random.default_rng(5)
    for r in range(sel.shape[0]):
        m = ref["sel_count"][r]
        sel[r, :m] = rng.permutation(sel[r, :m])
    slots, pos, oc = gu.gpu_expand(inp, sel, ref["sel_count"])
    check_expand_exact(slots, pos, oc, ref["slots"], ref["pos"], ref["out_count"], gu.pending_counts(inp))


def _many_rows_batch(rng, n_req, rows_per_req, c, k, long_ctx=200_000, n_long=6):
    """A batch of many rows for the expansion alone (no keys are read): most
    requests hold 2-9K tokens, n_long of them long_ctx tokens (more than the
    2,048 pages the row kernel caches), pages a seeded permutation."""
    ctx = [int(x) for x in rng.integers(2000, 9000, n_req)]
    for i in rng.choice(n_req, n_long, replace=False):
        ctx[i] = long_ctx
    pages = [-(-t // 64) for t in ctx]
    perm = rng.permutation(int(sum(pages)))
    pt = np.full((n_req, max(pages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[off:off + n]
        off += n
    rows = [ctx[b] - 1 - np.sort(rng.choice(min(ctx[b], 500), rows_per_req, replace=False))[::-1]
            for b in range(n_req)]
    row_pos = np.concatenate(rows).astype(np.int32)
    ptr = np.arange(0, n_req * rows_per_req + 1, rows_per_req, dtype=np.int32)
    per_page = 64 // c
    return synth.IndexerInputs(name="many", c=c, k=k, q=np.zeros((row_pos.shape[0], 4, 128), np.uint16),
                               kcache=np.zeros((per_page, 128), np.uint16), num_pages=int(off),
                               page_table=pt, req_row_ptr=ptr, row_pos=row_pos,
                               max_vis=int(((row_pos.astype(np.int64) + 1) // c).max()), seed=0)


def _random_selection(rng, inp):
    """min(k, n_vis) distinct visible blocks per row, in random order."""
    R = inp.num_rows
    sel = np.full((R, inp.k), -1, dtype=np.int32)
    cnt = np.zeros(R, dtype=np.int32)
    for r in range(R):
        nv = (int(inp.row_pos[r]) + 1) // inp.c
        m = min(inp.k, nv)
        sel[r, :m] = rng.choice(nv, m, replace=False)
        cnt[r] = m
    return sel, cnt


@pytest.mark.parametrize("c", [1, 4])
def test_expand_many_rows_exact(c):
    # >= 1,024 rows: the one-workgroup-per-row expansion, including rows whose
    # pages exceed its LDS page cache
    rng = np.random.default_rng(80 + c)
    inp = _many_rows_batch(rng, 180, 6, c, 512 if c == 4 else 2048)
    assert inp.num_rows >= 1024 and int(inp.row_pos.max()) // 64 >= 2048
    sel, cnt = _random_selection(rng, inp)
    rs, rp, rc = oracle.expand_translate(inp, sel, cnt)
    slots, pos, oc = gu.gpu_expand(inp, sel, cnt)
    check_expand_exact(slots, pos, oc, rs, rp, rc, gu.pending_counts(inp))


def test_expand_shared_many_rows_exact():
    rng = np.random.default_rng(90)
    N = 5
    inp = _many_rows_batch(rng, 180, 6, 4, 512)
    sel, cnt = _random_selection(rng, inp)
    now = inp.row_pos + rng.integers(0, N + 1, inp.num_rows).astype(np.int32)
    rs, rp, rc = oracle.expand_translate_shared(inp, sel, cnt, now, N)
    slots, pos, oc = gu.gpu_expand_shared(inp, sel, cnt, now, N)
    tail = now + 1 - 4 * ((inp.row_pos + 1) // 4)
    check_expand_exact(slots, pos, oc, rs, rp, rc, tail)


def test_expand_many_rows_invalid_entries_become_sentinels():
    rng = np.random.default_rng(91)
    inp = _many_rows_batch(rng, 180, 6, 4, 512, n_long=2)
    sel, cnt = _random_selection(rng, inp)
    bad = rng.random(sel.shape) < 0.01
    live = np.arange(inp.k)[None, :] < cnt[:, None]
    nv = (inp.row_pos.astype(np.int64) + 1) // 4
    sel[bad & live] = np.where(rng.random(int((bad & live).sum())) < 0.5, -1,
                               np.repeat(nv, inp.k).reshape(sel.shape)[bad & live])
    slots, pos, oc = gu.gpu_expand(inp, sel, cnt)
    assert np.array_equal(oc, 4 * cnt + gu.pending_counts(inp))
    R, k = sel.shape
    live = np.arange(k)[None, :] < cnt[:, None]
    ok = live & (sel >= 0) & (sel < nv[:, None])
    assert (live & ~ok).sum() > 100
    b = np.searchsorted(inp.req_row_ptr, np.arange(R), side="right") - 1
    want_pos = np.where(ok[..., None], 4 * sel[..., None] + np.arange(4), -1)
    page = inp.page_table[b[:, None], np.clip(4 * sel // 64, 0, inp.pt_stride - 1)]
    want_slot = np.where(ok[..., None], page[..., None] * 64 + want_pos % 64, -1)
    got_pos = pos[:, :4 * k].reshape(R, k, 4)
    got_slot = slots[:, :4 * k].reshape(R, k, 4)
    assert np.array_equal(got_pos[live], want_pos[live])
    assert np.array_equal(got_slot[live], want_slot[live])


def test_expand_invalid_entries_become_sentinels():
    inp = synth.qsa_decode_1x8k()
    sel = np.full((1, inp.k), -1, dtype=np.int32)
    sel[0, :4] = [5, -1, 2048, 7]  # -1 and the unfinished block 2048 are invalid
    slots, pos, oc = gu.gpu_expand(inp, sel, np.array([4], dtype=np.int32))
    assert oc[0] == 4 * 4 + 2
    assert np.all(slots[0, 4:12] == -1) and np.all(pos[0, 4:12] == -1)
    assert pos[0, :4].tolist() == [20, 21, 22, 23] and pos[0, 12:16].tolist() == [28, 29, 30, 31]
    assert pos[0, 16:18].tolist() == [8192, 8193]
    assert np.all(slots[0, 18:] == -1)


def _advancing_batch(rng, c, k, n_req, max_advance):
    # rows whose contexts hold max_advance more tokens past the rows' positions
    rows = [[int(x) for x in np.sort(rng.choice(np.arange(8, 20000), int(rng.integers(1, 4)), replace=False))]
            for _ in range(n_req)]
    ctx = [max(r) + max_advance + 1 for r in rows]
    return synth.build_paged_batch("adv", 9, c=c, k=k, ctx_tokens=ctx, row_pos_per_req=rows, rng=rng)


@pytest.mark.parametrize("c", [1, 4])
def test_expand_shared_exact_on_oracle_selection(c):
    # IndexShare: a selection captured at row_pos, expanded at row_pos + advance
    rng = np.random.default_rng(60 + c)
    N = 7
    inp = _advancing_batch(rng, c, 512 if c == 4 else 2048, 9, N)
    ref = oracle.pipeline(inp)
    sel = ref["sel"].copy()
    for r in range(sel.shape[0]):
        m = ref["sel_count"][r]
        sel[r, :m] = rng.permutation(sel[r, :m])
    adv = rng.integers(0, N + 1, inp.num_rows).astype(np.int32)
    adv[0], adv[-1] = 0, N
    now = inp.row_pos + adv
    rs, rp, rc = oracle.expand_translate_shared(inp, ref["sel"], ref["sel_count"], now, N)
    slots, pos, oc = gu.gpu_expand_shared(inp, sel, ref["sel_count"], now, N)
    tail = now + 1 - c * ((inp.row_pos + 1) // c)
    check_expand_exact(slots, pos, oc, rs, rp, rc, tail)


def test_expand_shared_clamps_the_advance():
    # a current position behind the captured one, or too far ahead, is clamped
    rng = np.random.default_rng(70)
    N = 3
    inp = _advancing_batch(rng, 4, 64, 4, N)
    ref = oracle.pipeline(inp)
    now = inp.row_pos.copy()
    now[0] -= 5           # behind: treated as the captured position
    now[1:] += N + 9      # too far: treated as the captured position + N
    clamped = np.clip(now, inp.row_pos, inp.row_pos + N)
    rs, rp, rc = oracle.expand_translate_shared(inp, ref["sel"], ref["sel_count"], clamped, N)
    slots, pos, oc = gu.gpu_expand_shared(inp, ref["sel"], ref["sel_count"], now, N)
    tail = clamped + 1 - 4 * ((inp.row_pos + 1) // 4)
    check_expand_exact(slots, pos, oc, rs, rp, rc, tail)


def test_expand_shared_full_indexshare_workload():
    # the benchmark's IndexShare workload: selection by the GPU path at the
    # captured rows, then the draft step's expansion at +max_advance, exact
    # against the oracle expanding the same selection
    import torch
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload
    inp = synth.qsa_indexshare_64req()
    adv = synth.INDEXSHARE_MAX_ADVANCE
    p = IndexerPath(upload(inp, "cuda"), "decode")
    p.run()
    torch.cuda.synchronize()
    sel, cnt = p.sel.cpu().numpy(), p.sel_count.cpu().numpy()
    now = inp.row_pos + adv
    rs, rp, rc = oracle.expand_translate_shared(inp, sel, cnt, now, adv)
    slots, pos, oc = gu.gpu_expand_shared(inp, sel, cnt, now, adv)
    tail = now + 1 - 4 * ((inp.row_pos + 1) // 4)
    check_expand_exact(slots, pos, oc, rs, rp, rc, tail)


# ---------------------------------------------------------------------------
# End to end at the full workload sizes
# ---------------------------------------------------------------------------

def test_e2e_verify_64req_full():
    _full_check(synth.qsa_verify_64req())


@pytest.mark.parametrize("fused", [True, False])
def test_e2e_dsa_16x80k_full(fused):
    _full_check(synth.dsa_decode_16x80k(), fused=fused)


def test_prepared_calls_match_the_public_calls():
    # The pipeline launches through prepared calls; the public functions check
    # and marshal on every call.  Both run the same kernels on the same inputs.
    import torch
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload
    inp = synth.qsa_verify_64req(B=5, lo=300, hi=40000)
    d = upload(inp, "cuda")
    a = IndexerPath(d, "decode")
    a.run()
    b = IndexerPath(d, "decode")
    b.score()
    b.select_translate()
    torch.cuda.synchronize()
    for x, y in ((a.row_len, b.row_len), (a.sel_count, b.sel_count), (a.out_count, b.out_count)):
        assert torch.equal(x, y)
    for r in range(d.num_rows):
        v = int(a.row_len[r])  # entries past the visible range are left untouched (uninitialised here)
        assert torch.equal(a.scores[r, :v].isnan(), b.scores[r, :v].isnan())
        assert torch.equal(a.scores[r, :v].nan_to_num(), b.scores[r, :v].nan_to_num())
        n = int(a.sel_count[r])
        assert torch.equal(a.sel[r, :n].sort().values, b.sel[r, :n].sort().values)
        m = int(a.out_count[r])
        pa, pb = a.pos[r, :m], b.pos[r, :m]
        oa, ob = pa.argsort(), pb.argsort()
        assert torch.equal(pa[oa], pb[ob]) and torch.equal(a.slots[r, :m][oa], b.slots[r, :m][ob])


def test_fused_select_translate_on_given_rows():
    # idx_select_translate on given FP32 rows (tie storms, long and short rows
    # in one batch) against the oracle's top-k and expand of the same rows
    import torch
    import block_scoring_top_amd as bst
    from synth.device import upload
    rng = np.random.default_rng(41)
    ctx = [90000, 70000, 3000, 40000]
    inp = synth.build_paged_batch("fs", 41, c=1, k=2048, ctx_tokens=ctx, row_pos_per_req=[[t - 1] for t in ctx],
                                  rng=rng)
    lens = ((inp.row_pos + 1) // inp.c).astype(np.int32)
    ld = int(lens.max())
    rows = synth.tie_storm_rows(42, 4, ld)
    rows[0] = rng.standard_normal(ld).astype(np.float32)
    dev = upload(inp, "cuda")
    s = torch.from_numpy(rows).cuda()
    rl = torch.from_numpy(lens).cuda()
    R = inp.num_rows
    sel = torch.empty((R, inp.k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")
    slots = torch.empty((R, inp.ld_out), dtype=torch.int32, device="cuda")
    pos = torch.empty((R, inp.ld_out), dtype=torch.int32, device="cuda")
    oc = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = bst.topk_workspace(R, ld, inp.k, "cuda")
    for rep in range(3):
        gu.say(f"select_translate rep {rep}")
        bst.idx_select_translate(s, rl, ld, inp.k, dev.req_row_ptr, dev.row_pos, inp.c, dev.page_table, sel, cnt,
                                 slots, oc, out_pos=pos, workspace=ws)
        torch.cuda.synchronize()
        ref_sel, ref_cnt = oracle.topk(rows, lens, inp.k)
        check_topk_exact(sel.cpu().numpy(), cnt.cpu().numpy(), ref_sel, ref_cnt)
        rs, rp, rc = oracle.expand_translate(inp, sel.cpu().numpy(), cnt.cpu().numpy())
        check_expand_exact(slots.cpu().numpy(), pos.cpu().numpy(), oc.cpu().numpy(), rs, rp, rc,
                           gu.pending_counts(inp))


def _given_rows_batch(rng, ctx, c, k, row_pos=None):
    return synth.given_rows_batch(rng, ctx, c, k, row_pos)


def _select_translate_given(inp, rows, lens, max_len, reps=1):
    """idx_select_translate on given FP32 rows; returns numpy outputs per rep."""
    import torch
    import block_scoring_top_amd as bst
    from synth.device import upload
    dev = upload(inp, "cuda")
    R = inp.num_rows
    s = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32)).cuda()
    rl = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    ws = bst.topk_workspace(R, max_len, inp.k, "cuda")
    outs = []
    for rep in range(reps):
        gu.say(f"select_translate rows={R} max_len={max_len} k={inp.k} c={inp.c} rep={rep}")
        sel = torch.full((R, inp.k), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
        slots = torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda")
        pos = torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda")
        oc = torch.full((R,), -7, dtype=torch.int32, device="cuda")
        bst.idx_select_translate(s, rl, max_len, inp.k, dev.req_row_ptr, dev.row_pos, inp.c, dev.page_table, sel,
                                 cnt, slots, oc, out_pos=pos, workspace=ws)
        torch.cuda.synchronize()
        outs.append(tuple(t.cpu().numpy() for t in (sel, cnt, slots, pos, oc)))
        if ws is not None:
            assert _ws_clean(ws), "the first word of every 64 KiB block of the workspace must be left zero"
    return outs


def _check_given(inp, rows, lens, outs):
    ref_sel, ref_cnt = oracle.topk(np.ascontiguousarray(rows, dtype=np.float32), lens, inp.k)
    for sel, cnt, slots, pos, oc in outs:
        check_topk_exact(sel, cnt, ref_sel, ref_cnt)
        rs, rp, rc = oracle.expand_translate(inp, sel, cnt)
        check_expand_exact(slots, pos, oc, rs, rp, rc, gu.pending_counts(inp))


@pytest.mark.parametrize("c", [4, 1])
def test_fused_many_rows_exact(c):
    # >= 1,024 rows of at most 16,384 entries: the many-rows shape of the fused
    # kernel (256 lanes x 64 values, several rows per CU), bit-exact; tie
    # storms, ragged lengths, rows whose boundary bin overflows the LDS list,
    # and rows at positions past the 1,024 pages the kernel caches in LDS.
    rng = np.random.default_rng(1200 + c)
    R, n = 1040, 16384
    k = 512 if c == 4 else 2048
    ctx = [int(x) for x in rng.integers(2, 4 * n if c == 4 else n, R)]
    ctx[:16] = [int(x) for x in rng.integers(70000, 90000, 16)]  # t/64 >= 1,024 pages
    inp = _given_rows_batch(rng, ctx, c, k)
    nv = (inp.row_pos.astype(np.int64) + 1) // c
    lens = np.minimum(nv, n).astype(np.int32)
    lens[16:20] = [0, 1, k, k + 1]
    lens[16:20] = np.minimum(lens[16:20], nv[16:20])
    rows = rng.standard_normal((R, n)).astype(np.float32)
    rows[20:84] = synth.tie_storm_rows(1203, 64, n)
    rows[84:100] = np.float32(1.0) + rng.integers(0, 3, (16, n)).astype(np.float32) * np.float32(2.0 ** -20)
    assert inp.num_rows >= 1024 and int(lens.max()) <= n
    _check_given(inp, rows, lens, _select_translate_given(inp, rows, lens, n))


@pytest.mark.parametrize("layout", ["aligned", "odd_ld", "offset_base"])
def test_mid_rows_read_layouts(layout):
    # Rows of 16,385-32,768 entries in a small batch take the 512-lane x
    # 64-entry shape.  Rows that start 16-byte aligned are read 16 bytes per
    # lane, the quad holding entry n-1 whole; other layouts one entry per
    # lane.  Every entry past a row's length holds +inf, so a read past n that
    # is not masked would be selected.  Fused and unfused, against the oracle.
    import block_scoring_top_amd as bst
    from synth.device import upload
    rng = np.random.default_rng(1300)
    R, max_len, k, c = 40, 30000, 2048, 1
    ld = max_len + (1 if layout == "odd_ld" else 0)
    off = 1 if layout == "offset_base" else 0
    lens = rng.integers(16385, max_len + 1, R).astype(np.int32)
    lens[:12] = [0, 1, k, k + 1, 16385, 16386, 16387, 16388, 29997, 29998, 29999, 30000]
    rows = rng.standard_normal((R, max_len)).astype(np.float32)
    rows[12:20] = synth.tie_storm_rows(1301, 8, max_len)
    host = np.full(R * ld + off + 4, np.inf, dtype=np.float32)
    for r in range(R):
        host[off + r * ld: off + r * ld + lens[r]] = rows[r, :lens[r]]
    flat = torch.from_numpy(host).cuda()
    s = flat[off:off + R * ld].view(R, ld)
    assert (s.data_ptr() % 16 == 0) == (layout != "offset_base") and s.stride(0) == ld
    rl = torch.from_numpy(lens).cuda()
    inp = _given_rows_batch(rng, [max(1, int(x)) for x in lens], c, k)
    dev = upload(inp, "cuda")
    ws = bst.topk_workspace(R, max_len, k, "cuda")
    ref_sel, ref_cnt = oracle.topk(rows, lens, k)
    gu.say(f"mid rows {layout}: unfused")
    sel = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    bst.topk_select_rows(s, rl, max_len, k, sel, cnt, ws)
    torch.cuda.synchronize()
    check_topk_exact(sel.cpu().numpy(), cnt.cpu().numpy(), ref_sel, ref_cnt)
    gu.say(f"mid rows {layout}: fused")
    sel.fill_(-7)
    cnt.fill_(-7)
    slots = torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda")
    pos = torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda")
    oc = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    bst.idx_select_translate(s, rl, max_len, k, dev.req_row_ptr, dev.row_pos, c, dev.page_table, sel, cnt, slots,
                             oc, out_pos=pos, workspace=ws)
    torch.cuda.synchronize()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    check_topk_exact(sel_h, cnt_h, ref_sel, ref_cnt)
    rs, rp, rc = oracle.expand_translate(inp, sel_h, cnt_h)
    check_expand_exact(slots.cpu().numpy(), pos.cpu().numpy(), oc.cpu().numpy(), rs, rp, rc, gu.pending_counts(inp))


@pytest.mark.parametrize("c", [1, 4])
def test_long_rows_fused_exact(c):
    # rows of >= 32,769 entries (one workgroup per 8,192-entry chunk, the last
    # to arrive resolving the row): random rows (candidate filter), tie storms
    # and a row whose winners sit in one chunk (the whole-row fallback), row
    # lengths that are not a multiple of the chunk, 3 calls on one workspace.
    rng = np.random.default_rng(1300 + c)
    k = 2048 if c == 1 else 512
    lens = np.array([32769, 40000, 81920, 81920, 65537, 50001, 98304, 81920], dtype=np.int32)
    ctx = [int(c * (n + 1)) for n in lens]
    inp = _given_rows_batch(rng, ctx, c, k)
    nv = (inp.row_pos.astype(np.int64) + 1) // c
    assert np.all(nv >= lens)
    ld = int(lens.max())
    rows = rng.standard_normal((lens.size, ld)).astype(np.float32)
    rows[1] = synth.tie_storm_rows(1301, 8, ld)[7]
    rows[2] = synth.tie_storm_rows(1302, 8, ld)[1]
    rows[3, 20000:23000] += np.float32(5.0)   # winners clustered in one chunk
    rows[5] = np.abs(rows[5]) * np.float32(0.01)
    _check_given(inp, rows, lens, _select_translate_given(inp, rows, lens, ld, reps=3))


def test_long_rows_row_len_past_visible_blocks():
    # row_len > n_vis on rows of >= 32,769 entries: chosen blocks at or past
    # n_vis expand to -1 slots and positions (the -1 sentinel), the rest as
    # usual, and the count is still c*m + p.
    rng = np.random.default_rng(1400)
    c, k = 4, 512
    ctx = [90001, 140003, 70002]
    inp = _given_rows_batch(rng, ctx, c, k, row_pos=[20000, 150, 70001])
    nv = (inp.row_pos.astype(np.int64) + 1) // c
    lens = np.array([40000, 33000, 34000], dtype=np.int32)
    rows = rng.standard_normal((3, 40000)).astype(np.float32)
    rows[0, 6000:] += np.float32(3.0)   # the top lies past n_vis = 5000
    (sel, cnt, slots, pos, oc), = _select_translate_given(inp, rows, lens, 40000)
    ref_sel, ref_cnt = oracle.topk(rows, lens, k)
    check_topk_exact(sel, cnt, ref_sel, ref_cnt)
    assert np.array_equal(oc, c * cnt + gu.pending_counts(inp))
    for r in range(3):
        m = int(cnt[r])
        j = sel[r, :m].astype(np.int64)
        ok = (j >= 0) & (j < nv[r])
        want_pos = np.where(ok[:, None], c * j[:, None] + np.arange(c), -1)
        page = inp.page_table[r, np.clip(c * j // 64, 0, inp.pt_stride - 1)]
        want_slot = np.where(ok[:, None], page[:, None] * 64 + want_pos % 64, -1)
        assert np.array_equal(pos[r, :c * m].reshape(m, c), want_pos)
        assert np.array_equal(slots[r, :c * m].reshape(m, c), want_slot)
        p = int(gu.pending_counts(inp)[r])
        tail = c * int(nv[r]) + np.arange(p)
        assert np.array_equal(pos[r, c * m:c * m + p], tail)
        assert np.array_equal(slots[r, c * m:c * m + p], inp.page_table[r, tail // 64] * 64 + tail % 64)
        assert np.all(slots[r, c * m + p:] == -1) and np.all(pos[r, c * m + p:] == -1)
    assert (sel[0, :k] >= nv[0]).sum() > 100


def test_mixed_batch_long_rows_among_many():
    # 300 rows, 16 of them at 81,920 entries and the rest at 2,000-8,000: each
    # long row is split over chunk workgroups and the others are selected whole,
    # in one launch, whatever the row count.
    rng = np.random.default_rng(1500)
    R, c, k = 300, 1, 2048
    lens = rng.integers(2000, 8001, R).astype(np.int32)
    lens[rng.choice(R, 16, replace=False)] = 81920
    inp = _given_rows_batch(rng, [int(n) for n in lens], c, k)
    rows = rng.standard_normal((R, 81920)).astype(np.float32)
    _check_given(inp, rows, lens, _select_translate_given(inp, rows, lens, 81920, reps=2))


def _items_of(lens, cut):
    return int(sum(-(-int(n) // 8192) if n >= cut else 1 for n in lens))


def _planned_given(inp, rows, lens, max_len, ks=None, reps=2):
    """topk_plan_rows once, then idx_select_translate_planned on that plan
    `reps` times for each k in ks (default inp.k), one workspace sized for the
    largest k; returns the plan's header and [(inp for that k, outputs)]."""
    import dataclasses
    import block_scoring_top_amd as bst
    from synth.device import upload
    dev = upload(inp, "cuda")
    R = inp.num_rows
    ks = ks or [inp.k]
    s = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32)).cuda()
    rl = torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    plan = bst.topk_plan(R, max_len, "cuda")
    ws = bst.topk_planned_workspace(R, max_len, max(ks), "cuda")
    gu.say(f"plan rows={R} max_len={max_len}")
    bst.topk_plan_rows(rl, max_len, plan)
    rl.fill_(-5)  # the selection must take the lengths from the plan
    torch.cuda.synchronize()
    header = plan[:8].cpu().numpy()
    outs = []
    for k in ks:
        ik = dataclasses.replace(inp, k=k)
        for rep in range(reps):
            gu.say(f"planned select_translate rows={R} max_len={max_len} k={k} c={inp.c} rep={rep}")
            sel = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
            cnt = torch.full((R,), -7, dtype=torch.int32, device="cuda")
            slots = torch.full((R, ik.ld_out), -7, dtype=torch.int32, device="cuda")
            pos = torch.full((R, ik.ld_out), -7, dtype=torch.int32, device="cuda")
            oc = torch.full((R,), -7, dtype=torch.int32, device="cuda")
            bst.idx_select_translate_planned(s, max_len, k, dev.req_row_ptr, dev.row_pos, inp.c, dev.page_table,
                                             sel, cnt, slots, oc, plan, out_pos=pos, workspace=ws)
            torch.cuda.synchronize()
            outs.append((ik, tuple(t.cpu().numpy() for t in (sel, cnt, slots, pos, oc))))
            if ws is not None:
                assert _ws_clean(ws), "the first word of every 64 KiB block of the workspace must be left zero"
    return header, outs


def _check_planned(rows, lens, max_len, header, outs):
    assert header[2] == len(lens) and header[3] == max_len
    cut = int(header[1])
    assert cut in (16385, 32769)
    n = np.minimum(lens, max_len)
    assert int(header[0]) == _items_of(n, cut)
    assert int(header[4]) == int(sum(-(-int(x) // 8192) for x in n if x >= cut))  # the chunk items, listed first
    for ik, o in outs:
        _check_given(ik, rows, lens, [o])
    return cut


@pytest.mark.parametrize("c", [1, 4])
def test_planned_mixed_batch_exact(c):
    # 300 rows, 16 of them at 81,920 entries and the rest at 2,000-8,000: the
    # plan is built once and serves two selections; each long row is split
    # into 10 chunk items and every other row is one whole-row item, read
    # only up to its length.
    rng = np.random.default_rng(1600 + c)
    R = 300
    k = 2048 if c == 1 else 512
    lens = rng.integers(2000, 8001, R).astype(np.int32)
    lens[rng.choice(R, 16, replace=False)] = 81920
    ctx = [int(c * (n + 1)) for n in lens]
    inp = _given_rows_batch(rng, ctx, c, k)
    rows = rng.standard_normal((R, 81920)).astype(np.float32)
    rows[3] = synth.tie_storm_rows(1601, 4, 81920)[2]
    header, outs = _planned_given(inp, rows, lens, 81920, reps=2)
    _check_planned(rows, lens, 81920, header, outs)


def test_planned_plan_reused_across_k():
    # One plan (it depends on the lengths only) serving selections with
    # different k, as the layers of one step would; one workspace sized for
    # the largest k.
    rng = np.random.default_rng(1700)
    c = 4
    lens = np.array([81920, 40000, 32769, 20000, 16385, 16384, 9000, 8192, 2048, 100, 1, 0], dtype=np.int32)
    ctx = [int(c * (n + 1)) for n in lens]
    inp = _given_rows_batch(rng, ctx, c, 512)
    rows = rng.standard_normal((lens.size, 81920)).astype(np.float32)
    rows[1, 30000:31000] += np.float32(4.0)  # winners clustered in one chunk (the whole-row fallback)
    header, outs = _planned_given(inp, rows, lens, 81920, ks=[512, 2048, 64], reps=1)
    cut = _check_planned(rows, lens, 81920, header, outs)
    assert cut == 16385  # 12 rows fit on the device at once, so rows from 16,385 entries on are split


@pytest.mark.parametrize("extra_ld", [0, 1])
def test_planned_many_rows_keep_medium_rows_whole(extra_ld):
    # More items at the low split length than the device holds at once: the
    # plan splits only rows of 32,769 entries or more, and the 16,385-32,768
    # rows are selected whole (512 lanes x 64 entries); at an aligned and at
    # an odd row stride.
    rng = np.random.default_rng(1800)
    R, c, k = 1100, 1, 2048
    lens = rng.integers(16385, 32769, R).astype(np.int32)
    lens[:4] = [16385, 24576, 32768, 2]
    lens[4:8] = [32769, 40000, 65536, 49152]
    lens[16:20] = [16386, 16387, 32767, 30001]  # ends inside a 16-byte quad
    ctx = [int(c * (n + 1)) for n in lens]
    inp = _given_rows_batch(rng, ctx, c, k)
    rows = rng.standard_normal((R, 65536 + extra_ld)).astype(np.float32)
    rows[8:16, :65536] = synth.tie_storm_rows(1801, 8, 65536)
    header, outs = _planned_given(inp, rows, lens, 65536, reps=1)
    assert _check_planned(rows, lens, 65536, header, outs) == 32769


def test_planned_rows_past_the_register_blocks():
    # 5,000 rows: the planner keeps 4,096 rows' lengths in registers between
    # its passes and reads the rest again; many rows, so only rows of 32,769
    # entries or more are split (three here, in the middle of the batch).
    rng = np.random.default_rng(2000)
    R, c, k = 5000, 1, 256
    lens = rng.integers(0, 3001, R).astype(np.int32)
    lens[[0, 2500, 4500]] = [40000, 32769, 36000]
    lens[4096:4100] = [0, 1, 256, 257]
    ctx = [int(c * (n + 1)) for n in lens]
    inp = _given_rows_batch(rng, ctx, c, k)
    rows = np.zeros((R, 40000), dtype=np.float32)
    for r in np.flatnonzero(lens):
        rows[r, :lens[r]] = rng.standard_normal(int(lens[r])).astype(np.float32)
    header, outs = _planned_given(inp, rows, lens, 40000, reps=1)
    assert _check_planned(rows, lens, 40000, header, outs) == 32769


def test_planned_very_long_rows():
    # The planned launch on rows whose candidate slots need the resolver's
    # larger forms: 1,000,000 entries (11,808 slots at k = 2,048: 32 per
    # lane), 200,000 (16 per lane) and 16,385 (split into 3 chunks, 16 per
    # lane), with a whole-row item beside them.
    rng = np.random.default_rng(2200)
    n = 1_000_000
    lens = np.array([n, 200_000, 16_385, 5000], dtype=np.int32)
    rows = rng.standard_normal((lens.size, n)).astype(np.float32)
    ctx = [int(x) + 1 for x in lens]
    inp = _given_rows_batch(rng, ctx, 1, 2048)
    header, outs = _planned_given(inp, rows, lens, n, ks=[2048, 512], reps=1)
    assert _check_planned(rows, lens, n, header, outs) == 16385


def test_planned_short_rows_only():
    # max_len below 16,385: no workspace, one whole-row item per row, every
    # length edge (0, 1, k - 1, k, k + 1, a full register tile, past it).
    rng = np.random.default_rng(1900)
    c, k = 1, 512
    lens = np.array([0, 1, 511, 512, 513, 8192, 8193, 12000, 16384] + [3000] * 40, dtype=np.int32)
    ctx = [int(c * (n + 1)) for n in lens]
    inp = _given_rows_batch(rng, ctx, c, k)
    rows = rng.standard_normal((lens.size, 16384)).astype(np.float32)
    rows[9:20] = synth.tie_storm_rows(1901, 11, 16384)
    header, outs = _planned_given(inp, rows, lens, 16384, reps=2)
    _check_planned(rows, lens, 16384, header, outs)
    assert int(header[0]) == lens.size


# ---------------------------------------------------------------------------
# Prefill scorer (matrix cores)
# ---------------------------------------------------------------------------

def test_prefill_small_vs_oracle():
    _full_check(synth.qsa_prefill_8k(rows=200, ctx=3001), scorer="prefill")


def test_prefill_multi_request_ragged():
    rng = np.random.default_rng(55)
    rows = [list(range(900, 1000)), [5, 6, 7], list(range(2000, 2077)), []]
    inp = synth.build_paged_batch("pf", 55, c=4, k=64, ctx_tokens=[1000, 8, 2077, 10], row_pos_per_req=rows,
                                  rng=rng)
    _full_check(inp, scorer="prefill")


def test_prefill_full_size_all_rows():
    # The full 8,192-row prefill chunk in the benchmark's launch shape (the
    # fused many-rows selection): every row's scores against the oracle, the
    # exact top-k of the GPU's scores, the end-to-end band, the exact expansion.
    _full_check(synth.qsa_prefill_8k(), scorer="prefill")


def test_prefill_agrees_with_decode_scorer():
    inp = synth.qsa_prefill_8k(rows=130, ctx=5000)
    a, la = gu.gpu_scores(inp, "prefill")
    b, lb = gu.gpu_scores(inp, "decode")
    assert np.array_equal(la, lb)
    check_scores(a, b.astype(np.float64), la, what="prefill vs decode")


@pytest.mark.parametrize("extra_ld", [0, 3])
def test_prefill_c1_ragged_and_row_stride(extra_ld):
    # c = 1 (one key per token, 64 per page), requests of several 64-row
    # blocks with ragged tails; extra_ld = 3 gives a row stride that is not a
    # multiple of 4 floats (the kernel's per-float store path).  Entries past
    # each row's visible range stay untouched.
    rng = np.random.default_rng(77)
    rows = [list(range(1500, 1630)), [0, 1, 2, 63, 64], list(range(3000, 3071)), []]
    inp = synth.build_paged_batch("pf1", 77, c=1, k=256, ctx_tokens=[1630, 65, 3071, 9], row_pos_per_req=rows,
                                  rng=rng)
    s, rl = gu.gpu_scores(inp, "prefill", ld=inp.max_vis + extra_ld)
    ref = oracle.pipeline(inp)
    assert np.array_equal(rl, ref["row_len"])
    check_scores(s[:, :inp.max_vis], ref["scores"], ref["row_len"])
    for r in range(inp.num_rows):
        assert np.all(np.isnan(s[r, rl[r]:]))
