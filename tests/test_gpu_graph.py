"""The step captured in a HIP graph (torch.cuda.CUDAGraph): every call only
enqueues kernels on the current stream (no allocation, no memset, no
synchronisation), and the long-row selection leaves its workspace zeroed, so a
captured step replays correctly.  Each replay follows eager work (new query
values copied in) and a synchronisation, and is compared bit for bit with the
same step run eagerly."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def _outputs(p):
    return [t.cpu().numpy().copy() for t in (p.scores, p.row_len, p.sel, p.sel_count, p.slots, p.pos, p.out_count)]


@pytest.mark.parametrize("case", ["dsa_long_rows", "qsa_verify", "qsa_prefill"])
def test_captured_step_replays_like_eager(case):
    import torch
    from block_scoring_top_amd.pipeline import IndexerPath
    from synth.device import upload
    if case == "dsa_long_rows":
        inp, scorer = synth.dsa_decode_16x80k(B=3, L=50000), "decode"
    elif case == "qsa_verify":
        inp, scorer = synth.qsa_verify_64req(B=8, lo=300, hi=20000), "decode"
    else:
        inp, scorer = synth.qsa_prefill_8k(rows=300, ctx=6001), "prefill"
    say(f"graph capture: {case} rows={inp.num_rows} max_vis={inp.max_vis} k={inp.k} c={inp.c}")
    dev = upload(inp, "cuda")
    p = IndexerPath(dev, scorer)
    rng = np.random.default_rng(3)
    qs = [dev.q.clone()] + [torch.from_numpy(synth.draw_q(rng, inp.num_rows).view(np.int16)).cuda() for _ in range(3)]

    # eager references, one per query set
    want = []
    for q in qs:
        dev.q.copy_(q)
        p.run()
        torch.cuda.synchronize()
        want.append(_outputs(p))

    # capture (after a warm-up on a side stream, as torch requires)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        p.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.run()
    torch.cuda.synchronize()

    for rep in range(2):
        for i, q in enumerate(qs):
            dev.q.copy_(q)                   # eager work between replays
            torch.cuda.synchronize()
            for t in (p.scores, p.sel, p.slots, p.pos):
                t.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = _outputs(p)
            assert np.array_equal(got[1], want[i][1]) and np.array_equal(got[3], want[i][3])
            assert np.array_equal(got[6], want[i][6]), (rep, i, "out_count")
            n = want[i][1]
            for r in range(inp.num_rows):
                assert np.array_equal(got[0][r, :n[r]], want[i][0][r, :n[r]]), (rep, i, "scores", r)
                # the order of a selection is unspecified (the long-row path
                # emits in device-atomic order): compare canonical forms
                assert np.array_equal(np.sort(got[2][r]), np.sort(want[i][2][r])), (rep, i, "sel", r)
                og, ow = np.argsort(got[5][r], kind="stable"), np.argsort(want[i][5][r], kind="stable")
                assert np.array_equal(got[5][r][og], want[i][5][r][ow]), (rep, i, "pos", r)
                assert np.array_equal(got[4][r][og], want[i][4][r][ow]), (rep, i, "slots", r)
        say(f"replay round {rep}: {len(qs)} replays match eager (canonical form)")
