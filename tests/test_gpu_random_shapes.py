"""Seeded random batches across every selection shape, checked bit-exact
against the oracle: the fused select+translate call and the planned pair on
the same rows.  Each case draws a row count and a max_len that land in one
shape (short rows, 1,024 x 16, 512 x 64, many rows, long rows over chunk
workgroups), a value mix (normal, small alphabet, FP16-snapped, heavy tail),
k, c, ragged lengths and a row stride that is or is not a multiple of 4."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from checkers import check_expand_exact, check_topk_exact
from gpu_util import pending_counts, say

pytestmark = pytest.mark.gpu

SHAPES = {  # (rows lo, rows hi, max_len lo, max_len hi)
    "short": (1, 8, 1, 2048),
    "row16": (1, 48, 2049, 16384),
    "mid": (1, 96, 16385, 32768),
    "many": (1024, 1200, 512, 16384),
    "long": (1, 12, 32769, 150000),
}
CASES = [(shape, i) for shape in SHAPES for i in range(8)]


def _values(rng, R, n, kind):
    if kind == 0:
        return rng.standard_normal((R, n)).astype(np.float32)
    if kind == 1:  # small alphabet: ties everywhere
        return rng.choice(np.array([-1.0, 0.0, 0.5, 0.5000001, 2.0], dtype=np.float32), size=(R, n))
    if kind == 2:  # FP16-snapped: many entries share bins
        return rng.standard_normal((R, n)).astype(np.float16).astype(np.float32)
    x = rng.standard_normal((R, n)).astype(np.float32)  # heavy tail
    m = rng.random((R, n)) < 0.01
    x[m] *= np.float32(50.0)
    return x


@pytest.mark.parametrize("shape,i", CASES)
def test_random_batch_exact(shape, i):
    import torch
    import block_scoring_top_amd as bst
    from synth.device import upload
    rng = np.random.default_rng(4000 + 37 * list(SHAPES).index(shape) + i)
    rlo, rhi, nlo, nhi = SHAPES[shape]
    R = int(rng.integers(rlo, rhi + 1))
    max_len = int(rng.integers(nlo, nhi + 1))
    k = int(rng.choice([1, 7, 64, 512, 2048]))
    c = int(rng.choice([1, 4]))
    ld = max_len + int(rng.choice([0, 1, 3, 4]))
    kind = int(rng.integers(0, 4))
    lens = rng.integers(0, max_len + 1, R).astype(np.int32)
    lens[rng.random(R) < 0.3] = max_len
    say(f"random case {shape}/{i}: rows={R} max_len={max_len} ld={ld} k={k} c={c} values={kind}")
    rows = np.full((R, ld), np.inf, dtype=np.float32)  # past each row's length: +inf, never selected
    vals = _values(rng, R, max_len, kind)
    for r in range(R):
        rows[r, :lens[r]] = vals[r, :lens[r]]
    inp = synth.given_rows_batch(rng, [int(c * (n + 1)) for n in lens], c, k)
    dev = upload(inp, "cuda")
    s = torch.from_numpy(rows).cuda()
    rl = torch.from_numpy(lens).cuda()
    ref_sel, ref_cnt = oracle.topk(np.ascontiguousarray(vals), lens, k)

    def outputs():
        return (torch.full((R, k), -7, dtype=torch.int32, device="cuda"),
                torch.full((R,), -7, dtype=torch.int32, device="cuda"),
                torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda"),
                torch.full((R, inp.ld_out), -7, dtype=torch.int32, device="cuda"),
                torch.full((R,), -7, dtype=torch.int32, device="cuda"))

    def check(o):
        sel, cnt, slots, pos, oc = (t.cpu().numpy() for t in o)
        check_topk_exact(sel, cnt, ref_sel, ref_cnt)
        rs, rp, rc = oracle.expand_translate(inp, sel, cnt)
        check_expand_exact(slots, pos, oc, rs, rp, rc, pending_counts(inp))

    ws = bst.topk_workspace(R, max_len, k, "cuda")
    o = outputs()
    bst.idx_select_translate(s, rl, max_len, k, dev.req_row_ptr, dev.row_pos, c, dev.page_table, o[0], o[1], o[2],
                             o[4], out_pos=o[3], workspace=ws)
    torch.cuda.synchronize()
    check(o)

    plan = bst.topk_plan(R, max_len, "cuda")
    pws = bst.topk_planned_workspace(R, max_len, k, "cuda")
    bst.topk_plan_rows(rl, max_len, plan)
    o = outputs()
    bst.idx_select_translate_planned(s, max_len, k, dev.req_row_ptr, dev.row_pos, c, dev.page_table, o[0], o[1],
                                     o[2], o[4], plan, out_pos=o[3], workspace=pws)
    torch.cuda.synchronize()
    check(o)


SCORER_CASES = [(scorer, i) for scorer in ("decode", "prefill") for i in range(6)]


@pytest.mark.parametrize("scorer,i", SCORER_CASES)
def test_random_indexer_batch(scorer, i):
    # Score -> select+translate on a random paged batch: 1-16 requests with
    # log-uniform contexts; decode rows at arbitrary positions of their
    # request (1-8 per request, unsorted, repeats allowed), prefill rows a
    # consecutive chunk ending at the context's end.  Scores within the
    # tolerance, top-k of the GPU's scores exact, end-to-end selection inside
    # the tie band, expansion exact.
    import gpu_util as gu
    from checkers import check_scores, check_topk_e2e
    rng = np.random.default_rng(5000 + 11 * i + (0 if scorer == "decode" else 500))
    c = int(rng.choice([1, 4]))
    k = int(rng.choice([16, 512, 2048]))
    B = int(rng.integers(1, 17))
    hi = 40000 if c == 4 else 12000
    ctx = [int(np.exp(rng.uniform(0.0, np.log(hi)))) + 1 for _ in range(B)]
    if scorer == "decode":
        rows = [sorted(rng.integers(0, t, int(rng.integers(1, 9))).tolist(), key=lambda _: rng.random())
                for t in ctx]
    else:
        rows = []
        for t in ctx:
            m = int(rng.integers(1, min(t, 200) + 1))
            rows.append(list(range(t - m, t)))
    inp = synth.build_paged_batch(f"random_{scorer}", 0, c=c, k=k, ctx_tokens=ctx, row_pos_per_req=rows, rng=rng)
    say(f"random indexer case {scorer}/{i}: requests={B} rows={inp.num_rows} max_vis={inp.max_vis} c={c} k={k}")
    g = gu.run_path(inp, scorer, True, False)
    ref = oracle.pipeline(inp)
    assert np.array_equal(g["row_len"], ref["row_len"])
    check_scores(g["scores"], ref["scores"], ref["row_len"])
    ld = max(inp.max_vis, 1)
    s_gpu, c_gpu = oracle.topk(np.ascontiguousarray(g["scores"][:, :ld]), g["row_len"], inp.k)
    check_topk_exact(g["sel"], g["sel_count"], s_gpu, c_gpu)
    check_topk_e2e(g["sel"], g["sel_count"], ref["scores"], ref["sel"], ref["sel_count"], ref["row_len"])
    rs, rp, rc = oracle.expand_translate(inp, g["sel"], g["sel_count"])
    check_expand_exact(g["slots"], g["pos"], g["out_count"], rs, rp, rc, pending_counts(inp))
