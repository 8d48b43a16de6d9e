"""The comparison rules the GPU tests rest on (tests/checkers.py) catch planted
mistakes: an oracle result, altered the way a kernel bug would alter it, must
raise Mismatch, and the unaltered result (or a reordering the rules allow) must
pass.  CPU only: the "GPU outputs" here are edited copies of the oracle's."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from checkers import (Mismatch, check_expand_exact, check_scores, check_topk_e2e, check_topk_exact)


@pytest.fixture(scope="module")
def ref():
    inp = synth.qsa_verify_64req(B=6, lo=300, hi=9000)
    out = oracle.pipeline(inp)
    t = inp.row_pos.astype(np.int64)
    pend = (t + 1 - inp.c * ((t + 1) // inp.c)).astype(np.int32)
    return inp, out, pend


def _row_with_choice(out):
    """A row whose selection leaves unselected blocks."""
    for r in range(out["sel"].shape[0]):
        if out["row_len"][r] > out["sel_count"][r] + 2:
            return r
    raise AssertionError("no row with unselected blocks")


def test_unaltered_results_pass(ref):
    inp, out, pend = ref
    check_scores(out["scores"].astype(np.float32), out["scores"], out["row_len"])
    check_topk_exact(out["sel"], out["sel_count"], out["sel"], out["sel_count"])
    assert check_topk_e2e(out["sel"], out["sel_count"], out["scores"], out["sel"], out["sel_count"],
                          out["row_len"]) == 0
    check_expand_exact(out["slots"], out["pos"], out["out_count"], out["slots"], out["pos"], out["out_count"], pend)


def test_reordered_selection_and_expansion_pass(ref):
    # the output order is free: a permuted selection and its expansion, with
    # the pending tail permuted among itself, still pass
    inp, out, pend = ref
    rng = np.random.default_rng(1)
    sel = out["sel"].copy()
    for r in range(sel.shape[0]):
        m = out["sel_count"][r]
        sel[r, :m] = rng.permutation(sel[r, :m])
    check_topk_exact(sel, out["sel_count"], out["sel"], out["sel_count"])
    slots, pos, oc = oracle.expand_translate(inp, sel, out["sel_count"])
    for r in range(pos.shape[0]):
        n, p = int(oc[r]), int(pend[r])
        perm = rng.permutation(p)
        pos[r, n - p:n] = pos[r, n - p:n][perm]
        slots[r, n - p:n] = slots[r, n - p:n][perm]
    check_expand_exact(slots, pos, oc, out["slots"], out["pos"], out["out_count"], pend)


def test_flipped_selected_index_is_caught(ref):
    inp, out, pend = ref
    r = _row_with_choice(out)
    sel = out["sel"].copy()
    m = int(out["sel_count"][r])
    unselected = np.setdiff1d(np.arange(out["row_len"][r]), sel[r, :m])
    sel[r, 0] = unselected[0]
    with pytest.raises(Mismatch):
        check_topk_exact(sel, out["sel_count"], out["sel"], out["sel_count"])


def test_duplicate_count_and_padding_mistakes_are_caught(ref):
    inp, out, pend = ref
    r = _row_with_choice(out)
    m = int(out["sel_count"][r])
    dup = out["sel"].copy()
    dup[r, 1] = dup[r, 0]
    with pytest.raises(Mismatch):
        check_topk_exact(dup, out["sel_count"], out["sel"], out["sel_count"])
    cnt = out["sel_count"].copy()
    cnt[r] -= 1
    with pytest.raises(Mismatch):
        check_topk_exact(out["sel"], cnt, out["sel"], out["sel_count"])
    if m < out["sel"].shape[1]:
        pad = out["sel"].copy()
        pad[r, m] = 0
        with pytest.raises(Mismatch):
            check_topk_exact(pad, out["sel_count"], out["sel"], out["sel_count"])


def test_swap_outside_the_band_is_caught_inside_it_passes(ref):
    inp, out, pend = ref
    r = _row_with_choice(out)
    m = int(out["sel_count"][r])
    s = out["scores"][r].astype(np.float64)
    chosen = out["sel"][r, :m]
    kth = s[chosen].min()
    unselected = np.setdiff1d(np.arange(out["row_len"][r]), chosen)
    far_out = unselected[np.argmin(s[unselected])]          # the lowest unselected score
    far_in = chosen[np.argmax(s[chosen])]                    # the highest selected score
    assert kth - s[far_out] > 2e-4 and s[far_in] - kth > 2e-4
    sel = out["sel"].copy()
    sel[r, list(chosen).index(far_in)] = far_out
    with pytest.raises(Mismatch):
        check_topk_e2e(sel, out["sel_count"], out["scores"], out["sel"], out["sel_count"], out["row_len"])
    # the same swap between blocks within the band passes (scores tied to 2e-4)
    scores = out["scores"].copy()
    kth_blk = chosen[np.argmin(s[chosen])]
    near = unselected[0]
    scores[r, near] = scores[r, kth_blk] - np.float32(1e-5)
    sel = out["sel"].copy()
    sel[r, list(chosen).index(kth_blk)] = near
    assert check_topk_e2e(sel, out["sel_count"], scores, out["sel"], out["sel_count"], out["row_len"]) == 1


def test_expansion_mistakes_are_caught(ref):
    inp, out, pend = ref
    r = int(np.argmax(pend))  # a row with pending tokens
    assert pend[r] > 0
    n = int(out["out_count"][r])
    args = (out["slots"], out["pos"], out["out_count"])
    # a dropped pending token
    oc = out["out_count"].copy()
    oc[r] -= 1
    slots, pos = out["slots"].copy(), out["pos"].copy()
    slots[r, n - 1] = pos[r, n - 1] = -1
    with pytest.raises(Mismatch):
        check_expand_exact(slots, pos, oc, *args, pend)
    # a perturbed slot (one page off)
    slots = out["slots"].copy()
    slots[r, 0] += 64
    with pytest.raises(Mismatch):
        check_expand_exact(slots, out["pos"], out["out_count"], *args, pend)
    # a position moved to the neighbouring token, slot consistent with it
    pos, slots = out["pos"].copy(), out["slots"].copy()
    pos[r, 0] ^= 1
    slots[r, 0] ^= 1
    with pytest.raises(Mismatch):
        check_expand_exact(slots, pos, out["out_count"], *args, pend)
    # a block's positions expanded in the wrong order inside the block pass
    # canonicalisation only if they are the same set; a duplicated token fails
    pos, slots = out["pos"].copy(), out["slots"].copy()
    pos[r, 1], slots[r, 1] = pos[r, 0], slots[r, 0]
    with pytest.raises(Mismatch):
        check_expand_exact(slots, pos, out["out_count"], *args, pend)


def test_score_mistakes_are_caught(ref):
    inp, out, pend = ref
    r = 0
    s = out["scores"].astype(np.float32).copy()
    j = int(out["row_len"][r]) // 2
    lim = 1e-4 * (1 + abs(float(out["scores"][r, j])))
    ok = s.copy()
    ok[r, j] = np.float32(float(out["scores"][r, j]) + 0.5 * lim)
    check_scores(ok, out["scores"], out["row_len"])
    bad = s.copy()
    bad[r, j] = np.float32(float(out["scores"][r, j]) + 2.0 * lim)
    with pytest.raises(Mismatch):
        check_scores(bad, out["scores"], out["row_len"])
    nan = s.copy()
    nan[r, j] = np.nan
    with pytest.raises(Mismatch):
        check_scores(nan, out["scores"], out["row_len"])
