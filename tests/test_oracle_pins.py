"""Pins the CPU oracle to things other than itself: hand-worked examples,
closed forms, exhaustive checks, brute force and library routines.

Every function the oracle exports is covered; a plausible slip (a dropped head,
a wrong sign, a swapped index, a wrong page) fails at least one test here.
"""
from __future__ import annotations

import itertools
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f32_round_of_decimal(text: str) -> np.float32:
    """Correctly rounded FP32 of a decimal string (via exact Fractions)."""
    x = Fraction(Decimal(text))
    lo = np.float32(float(x))
    cands = [np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))


# ---------------------------------------------------------------------------
# FP16 conversion and order-preserving keys
# ---------------------------------------------------------------------------

@pytest.mark.slow
def test_f16_conversion_exhaustive_vs_host_f16c():
    # all 2^32 FP32 patterns against the host's hardware FP32->FP16 conversion
    assert oracle.check_f16_all() == 0


def test_f16_conversion_vs_numpy_sample():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # every exponent, with boundary mantissas
    e = np.arange(256, dtype=np.uint32) << 23
    m = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x2000, 0x3000, 0x7FFFFF, 0x400000], dtype=np.uint32)
    u = np.concatenate([u, (e[:, None] | m[None, :]).ravel(), (e[:, None] | m[None, :]).ravel() | 0x80000000])
    f = u.view(np.float32)
    keep = ~np.isnan(f)
    u, f = u[keep], f[keep]
    with np.errstate(over="ignore"):
        want = f.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16_bits(f)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(u[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:5]]


def test_key16_order_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    keep = ~np.isnan(v)
    h, v = h[keep], v[keep]
    assert h.size == 65536 - 2 * 1023  # 63,490 non-NaN patterns
    keys = np.array([oracle.key16(int(x)) for x in h], dtype=np.int64)
    o = np.argsort(v, kind="stable")
    vs, ks = v[o], keys[o]
    dv, dk = np.diff(vs), np.diff(ks)
    assert np.all(dk[dv > 0] > 0), "strictly larger value must get a strictly larger key"
    assert np.all(dk[dv == 0] == 0), "equal values (+0/-0) must get equal keys"


@pytest.mark.slow
def test_key32_order_exhaustive_chain():
    bad, visited = oracle.check_key32_chain()
    assert visited == 2**32 - 2 * (2**23 - 1)
    assert bad == 0


def test_bins_golden():
    g = _gold("topk_bins.json")
    for case in g["cases"]:
        v = np.float32(float(case["value"]))
        h = int(oracle.f32_to_f16_bits(np.array([v]))[0])
        assert h == int(case["f16"], 16), case
        assert oracle.key16(h) == int(case["key16"], 16), case
        assert oracle.bin_of(float(v)) == case["bin"], case


def test_key32_small_cases():
    # bit inversion for negatives, top bit for non-negatives, -0 folded
    assert oracle.key32(0x00000000) == 0x80000000
    assert oracle.key32(0x80000000) == 0x80000000
    assert oracle.key32(0x3F800000) == 0xBF800000
    assert oracle.key32(0xBF800000) == 0x407FFFFF
    assert oracle.key32(0x7F800000) == 0xFF800000
    assert oracle.key32(0xFF800000) == 0x007FFFFF


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------

def _rank_brute(row: np.ndarray, k: int) -> np.ndarray:
    """The rank definition, O(n^2): rank(j) = #{i: s_i > s_j} + #{i: s_i == s_j, i < j}."""
    n = row.shape[0]
    s = row.astype(np.float64)
    gt = (s[None, :] > s[:, None]).sum(axis=1)
    eq_lower = np.array([np.sum((s[:j] == s[j])) for j in range(n)])
    rank = gt + eq_lower
    return np.nonzero(rank < min(k, n))[0].astype(np.int32)


def _oracle_sel(rows: np.ndarray, k: int, lens=None):
    R, n = rows.shape
    lens = np.full(R, n, dtype=np.int32) if lens is None else lens
    sel, cnt = oracle.topk(rows, lens, k)
    return [sel[r, :cnt[r]] for r in range(R)], sel, cnt


def test_topk_vs_rank_definition_random():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(1, 90))
        alphabet = rng.standard_normal(int(rng.integers(1, 12))).astype(np.float32)
        row = rng.choice(alphabet, size=n)
        row[rng.random(n) < 0.1] = -0.0
        k = int(rng.integers(1, n + 3))
        got, _, cnt = _oracle_sel(row[None, :], k)
        assert cnt[0] == min(k, n)
        assert np.array_equal(got[0], _rank_brute(row, k)), (trial, n, k)


def test_topk_exhaustive_small_alphabet():
    # every row of length 7 over {-1, -0, +0, 1}, every k in 1..8
    alphabet = np.array([-1.0, -0.0, 0.0, 1.0], dtype=np.float32)
    idx = np.array(list(itertools.product(range(4), repeat=7)), dtype=np.int64)
    rows = alphabet[idx]
    n = rows.shape[1]
    s = rows.astype(np.float64)
    gt = (s[:, None, :] > s[:, :, None]).sum(axis=2)
    lower = np.tril(np.ones((n, n), dtype=bool), k=-1)  # [j, i]: i < j
    eq_lower = ((s[:, None, :] == s[:, :, None]) & lower[None]).sum(axis=2)
    rank = gt + eq_lower
    for k in range(1, n + 2):
        want = rank < min(k, n)
        sel, cnt = oracle.topk(rows, np.full(rows.shape[0], n, dtype=np.int32), k)
        got = np.zeros_like(want)
        for r in range(rows.shape[0]):
            got[r, sel[r, :cnt[r]]] = True
        assert np.array_equal(got, want), k


def test_topk_vs_numpy_lexsort():
    rng = np.random.default_rng(12)
    rows = []
    for n in (1, 2, 3, 17, 100, 511, 512, 513, 1000, 2000):
        rows.append(rng.standard_normal(n).astype(np.float32))
    for r in synth.tie_storm_rows(13, 16, 1500):
        rows.append(r)
    for row in rows:
        n = row.shape[0]
        for k in (1, 7, 512, 2048):
            order = np.lexsort((np.arange(n), -row.astype(np.float64)))
            want = np.sort(order[:min(k, n)])
            got, _, _ = _oracle_sel(row[None, :], k)
            assert np.array_equal(got[0], want), (n, k)


def _invariants(row, sel, k):
    n = row.shape[0]
    m = min(k, n)
    assert sel.shape[0] == m
    assert np.unique(sel).shape[0] == m
    if 0 < m < n:
        mask = np.zeros(n, dtype=bool)
        mask[sel] = True
        lo_in, hi_out = row[mask].min(), row[~mask].max()
        assert lo_in >= hi_out
        tied_in = np.nonzero(mask & (row == lo_in))[0]
        tied_out = np.nonzero(~mask & (row == lo_in))[0]
        if tied_out.size:
            assert tied_in.max() < tied_out.min(), "ties must go to the lower index"


def test_topk_hist_algorithm_equals_sort():
    rng = np.random.default_rng(14)
    rows = list(synth.tie_storm_rows(15, 16, 5000))
    cfg1 = synth.topk_8x80k(rows=2)
    rows += [cfg1.scores[0], cfg1.scores[1]]
    rows += [rng.standard_normal(3000).astype(np.float32) * np.float32(1e-3)]
    for row in rows:
        for k in (1, 5, 512, 2048):
            sel_h, hist = oracle.topk_hist(row, k)
            assert int(hist.sum()) == row.shape[0]
            got, _, _ = _oracle_sel(row[None, :], k)
            assert np.array_equal(sel_h, got[0]), k
            _invariants(row, got[0], k)


def test_topk_respects_row_len_and_pads():
    rng = np.random.default_rng(16)
    rows = rng.standard_normal((4, 64)).astype(np.float32)
    rows[:, 40:] = 100.0  # beyond row_len: must be ignored
    lens = np.array([0, 3, 40, 10], dtype=np.int32)
    sel, cnt = oracle.topk(rows, lens, 8)
    assert cnt.tolist() == [0, 3, 8, 8]
    assert np.all(sel[0] == -1)
    assert sel[1, :3].tolist() == [0, 1, 2] and np.all(sel[1, 3:] == -1)
    for r in (2, 3):
        assert sel[r, :8].max() < lens[r]


def test_topk_rejects_nan():
    rows = np.array([[1.0, np.nan, 0.0]], dtype=np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.topk(rows, np.array([3], dtype=np.int32), 1)


# ---------------------------------------------------------------------------
# Scoring
# ---------------------------------------------------------------------------

def _one_page_inputs(c, q_f32, keys_f32, t, page=0, num_pages=1, k=4):
    """Single request, single row; logical page 0 maps to physical ``page``."""
    per_page = 64 // c
    kc = np.zeros((num_pages * per_page, 128), dtype=np.float32)
    kc[:] = 1000.0  # garbage everywhere else: a wrong slot shows up
    for j, v in enumerate(keys_f32):
        kc[page * per_page + j] = v
    pt = np.array([[page]], dtype=np.int32)
    return synth.IndexerInputs(name="t", c=c, k=k, q=synth.f32_to_bf16_bits(q_f32[None]),
                               kcache=synth.f32_to_bf16_bits(kc), num_pages=num_pages, page_table=pt,
                               req_row_ptr=np.array([0, 1], dtype=np.int32),
                               row_pos=np.array([t], dtype=np.int32), max_vis=max((t + 1) // c, 1), seed=0)


def _sparse(spec):
    v = np.zeros(128, dtype=np.float32)
    for d, x in spec:
        v[int(d)] += np.float32(x)
    return v


def test_score_golden_worked_examples():
    g = _gold("score_worked.json")
    qh = np.stack([_sparse(h) for h in g["q_heads"]])
    for case in g["cases"]:
        c, t = case["c"], case["t"]
        keys = [_sparse(case["block_keys"][str(j)]) for j in range(len(case["block_keys"]))]
        inp = _one_page_inputs(c, qh, keys, t, page=case["physical_page_of_logical_page_0"],
                               num_pages=case["num_pages"], k=case["k"])
        scores, row_len = oracle.score(inp, ld=max(len(keys), 1))
        assert row_len[0] == case["n_vis"], case["name"]
        want = [_f32_round_of_decimal(s) for s in case["scores_decimal"]]
        assert scores[0, :case["n_vis"]].tolist() == [float(w) for w in want], case["name"]
        assert np.all(np.isnan(scores[0, case["n_vis"]:])), "invisible blocks must stay unwritten"
        sel, cnt = oracle.topk(scores, row_len, case["k"])
        assert sel[0, :cnt[0]].tolist() == case["topk"], case["name"]
        slots, pos, oc = oracle.expand_translate(inp, sel, cnt)
        assert pos[0, :oc[0]].tolist() == case["positions"], case["name"]
        assert slots[0, :oc[0]].tolist() == case["slots"], case["name"]
        assert pos[0, oc[0] - len(case["pending"]):oc[0]].tolist() == case["pending"]


def test_score_unit_vectors_closed_form():
    # q_h = e_{i_h}, key = e_j  ->  s = #{h : i_h = j} / sqrt(128)
    rng = np.random.default_rng(21)
    for _ in range(20):
        ih = rng.integers(0, 4, size=4)
        q = np.zeros((4, 128), dtype=np.float32)
        q[np.arange(4), ih] = 1.0
        keys = [np.eye(128, dtype=np.float32)[j] for j in range(4)]
        inp = _one_page_inputs(4, q, keys, t=15)
        s, _ = oracle.score(inp)
        for j in range(4):
            cnt = int(np.sum(ih == j))
            assert s[0, j] == _f32_round_of_decimal(str(Decimal(cnt) / Decimal(128).sqrt())), (ih, j)


def test_score_relu_is_per_head():
    # flipping a head's sign switches exactly that head off
    rng = np.random.default_rng(22)
    q = np.abs(rng.standard_normal((4, 128))).astype(np.float32)
    key = np.abs(rng.standard_normal(128)).astype(np.float32)
    key /= np.linalg.norm(key)
    base = oracle.score(_one_page_inputs(4, q, [key], t=3))[0][0, 0]
    for h in range(4):
        qf = q.copy()
        qf[h] = -qf[h]
        s = oracle.score(_one_page_inputs(4, qf, [key], t=3))[0][0, 0]
        qz = q.copy()
        qz[h] = 0.0
        z = oracle.score(_one_page_inputs(4, qz, [key], t=3))[0][0, 0]
        assert s == z and s < base
    allneg = oracle.score(_one_page_inputs(4, -q, [key], t=3))[0][0, 0]
    assert allneg == 0.0


def test_score_power_of_two_scaling_exact():
    inp = synth.qsa_decode_1x8k()
    s1, _ = oracle.score(inp)
    q2 = synth.bf16_bits_to_f32(inp.q) * np.float32(2.0)
    inp2 = synth.IndexerInputs(**{**inp.__dict__, "q": synth.f32_to_bf16_bits(q2)})
    s2, _ = oracle.score(inp2)
    assert np.array_equal(s2, s1 * np.float32(2.0))


def test_score_exact_rational():
    # The exact value of the equation, from the bf16 inputs as rationals:
    # s = N * sqrt(2) / 16 with N = sum_h max(0, sum_d q_hd k_d).  The oracle's
    # FP32 must be the correctly rounded value (or its neighbour).
    getcontext().prec = 60
    rng = np.random.default_rng(23)
    inp = synth.build_paged_batch("t", 5, c=4, k=8, ctx_tokens=[300], row_pos_per_req=[[299]], rng=rng)
    s, row_len = oracle.score(inp)
    qf = synth.bf16_bits_to_f32(inp.q[0]).astype(np.float64)
    for j in rng.choice(int(row_len[0]), size=12, replace=False):
        page = int(inp.page_table[0, (4 * j) // 64])
        key = synth.bf16_bits_to_f32(inp.kcache[page * 16 + j % 16]).astype(np.float64)
        N = Fraction(0)
        for h in range(4):
            dot = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qf[h], key))
            N += max(dot, Fraction(0))
        exact = Decimal(N.numerator) / Decimal(N.denominator) * Decimal(2).sqrt() / Decimal(16)
        want = _f32_round_of_decimal(str(exact))
        got = s[0, j]
        ulps = abs(int(np.float32(got).view(np.int32)) - int(np.float32(want).view(np.int32)))
        assert ulps <= 1, (j, got, want)


def test_score_page_table_permutation_invariance():
    # Moving whole physical pages (and updating the table) leaves scores unchanged.
    inp = synth.qsa_verify_64req(B=3, lo=300, hi=2000)
    s1, l1 = oracle.score(inp)
    rng = np.random.default_rng(24)
    perm = rng.permutation(inp.num_pages)            # new physical id of old page p
    per = 64 // inp.c
    kc = np.empty_like(inp.kcache)
    for p in range(inp.num_pages):
        kc[perm[p] * per:(perm[p] + 1) * per] = inp.kcache[p * per:(p + 1) * per]
    pt = np.where(inp.page_table >= 0, perm[np.maximum(inp.page_table, 0)], -1).astype(np.int32)
    inp2 = synth.IndexerInputs(**{**inp.__dict__, "kcache": kc, "page_table": pt})
    s2, l2 = oracle.score(inp2)
    assert np.array_equal(l1, l2)
    assert np.array_equal(s1, s2, equal_nan=True)


def test_score_identity_table_reads_slot_j():
    # With the identity page table, block j's key is compressed slot j.
    rng = np.random.default_rng(25)
    for c in (1, 4):
        inp = synth.build_paged_batch("t", 6, c=c, k=8, ctx_tokens=[200], row_pos_per_req=[[199]],
                                      rng=rng, identity_pages=True)
        s, rl = oracle.score(inp)
        q = synth.bf16_bits_to_f32(inp.q[0]).astype(np.float64)
        K = synth.bf16_bits_to_f32(inp.kcache[:rl[0]]).astype(np.float64)
        ref = np.maximum(q @ K.T, 0).sum(axis=0) / np.sqrt(128.0)
        assert np.allclose(s[0, :rl[0]], ref, rtol=1e-6, atol=1e-7)


def test_visibility_closed_form():
    for c in (1, 4):
        for t in range(0, 140):
            assert oracle.n_vis(t, c) == (t + 1) // c
    inp = synth.qsa_verify_64req(B=4, lo=100, hi=700)
    s, rl = oracle.score(inp)
    assert np.array_equal(rl, (inp.row_pos + 1) // 4)
    for r in range(inp.num_rows):
        assert np.all(np.isfinite(s[r, :rl[r]])) and np.all(np.isnan(s[r, rl[r]:]))


# ---------------------------------------------------------------------------
# Expand / append / translate
# ---------------------------------------------------------------------------

def test_expand_qsa_counts_golden():
    g = _gold("qsa_counts.json")
    rng = np.random.default_rng(31)
    for case in g["cases"]:
        p = case["pending"]
        t = 4 * 4000 + p - 1
        inp = synth.build_paged_batch("t", 7, c=g["c"], k=g["k"], ctx_tokens=[t + 1], row_pos_per_req=[[t]], rng=rng)
        nv = (t + 1) // 4
        sel = np.sort(rng.choice(nv, size=g["k"], replace=False)).astype(np.int32)[None]
        slots, pos, oc = oracle.expand_translate(inp, sel, np.array([g["k"]], dtype=np.int32))
        assert oc[0] == case["positions"] <= g["max_positions"]
        assert inp.ld_out == g["max_positions"]


def test_expand_invariants_and_inverse_translation():
    inp = synth.qsa_verify_64req(B=5, lo=200, hi=5000)
    out = oracle.pipeline(inp)
    inv = {}
    for b in range(inp.num_req):
        for lp, pp in enumerate(inp.page_table[b]):
            if pp >= 0:
                inv[int(pp)] = (b, lp)
    for b in range(inp.num_req):
        for r in range(inp.req_row_ptr[b], inp.req_row_ptr[b + 1]):
            t = int(inp.row_pos[r])
            nv = (t + 1) // 4
            m = min(inp.k, nv)
            p = t + 1 - 4 * nv
            n = int(out["out_count"][r])
            assert n == 4 * m + p <= 2051
            pos = out["pos"][r, :n]
            assert np.unique(pos).size == n and pos.max() <= t and pos.min() >= 0
            assert pos[n - p:].tolist() == list(range(4 * nv, t + 1))
            blocks = out["sel"][r, :m]
            assert pos[:n - p].tolist() == [4 * j + u for j in blocks for u in range(4)]
            for s_, q_ in zip(out["slots"][r, :n], pos):
                bb, lp = inv[int(s_) // 64]
                assert bb == b and lp * 64 + int(s_) % 64 == q_
            assert np.all(out["slots"][r, n:] == -1)


def test_expand_identity_table_slot_is_position():
    rng = np.random.default_rng(32)
    inp = synth.build_paged_batch("t", 8, c=4, k=16, ctx_tokens=[999], row_pos_per_req=[[990, 997, 998]],
                                  rng=rng, identity_pages=True)
    out = oracle.pipeline(inp)
    for r in range(3):
        n = out["out_count"][r]
        assert np.array_equal(out["slots"][r, :n], out["pos"][r, :n])


def test_expand_rejects_invisible_block():
    inp = synth.qsa_decode_1x8k()
    sel = np.full((1, inp.k), -1, dtype=np.int32)
    sel[0, 0] = 2048  # n_vis = 2048: block 2048 is the unfinished one
    with pytest.raises(oracle.OracleError):
        oracle.expand_translate(inp, sel, np.array([1], dtype=np.int32))


def test_pipeline_config_shapes():
    inp = synth.qsa_decode_1x8k()
    assert inp.row_pos.tolist() == [8193] and inp.num_pages == 129
    out = oracle.pipeline(inp)
    assert out["row_len"].tolist() == [2048]
    assert out["sel_count"].tolist() == [512]
    assert out["out_count"].tolist() == [2050]


# ---------------------------------------------------------------------------
# IndexShare expansion (QSA page, section IndexShare MTP): a selection
# captured at t0 is reused while the row advances to t1; the tail holds the
# captured pending tokens and every position since.
# ---------------------------------------------------------------------------

def _shared_batch(rng, c, k, rows_per_req, advance_room):
    # contexts long enough that every position up to t0 + advance_room has a page
    ctx, row_pos = [], []
    for rows in rows_per_req:
        ctx.append(max(rows) + advance_room + 1)
        row_pos.append(rows)
    return synth.build_paged_batch("shared", 5, c=c, k=k, ctx_tokens=ctx, row_pos_per_req=row_pos, rng=rng)


def test_shared_expand_worked_example():
    # c = 4, captured at t0 = 10: blocks 0 and 1 are visible (tokens 0..7),
    # tokens 8, 9, 10 are pending.  Chosen block: 1 (tokens 4..7).  At t1 = 13
    # the tail is 8..13, so the positions are 4 5 6 7 8 9 10 11 12 13.
    rng = np.random.default_rng(41)
    inp = synth.build_paged_batch("ex", 6, c=4, k=4, ctx_tokens=[64], row_pos_per_req=[[10]], rng=rng,
                                  identity_pages=True)
    sel = np.array([[1, -1, -1, -1]], dtype=np.int32)
    slots, pos, oc = oracle.expand_translate_shared(inp, sel, np.array([1], dtype=np.int32), [13], 3)
    assert oc[0] == 10
    assert pos[0, :10].tolist() == [4, 5, 6, 7, 8, 9, 10, 11, 12, 13]
    assert slots[0, :10].tolist() == pos[0, :10].tolist()  # identity pages
    assert np.all(pos[0, 10:] == -1) and np.all(slots[0, 10:] == -1)


def test_shared_expand_without_advance_is_the_plain_expansion():
    rng = np.random.default_rng(42)
    for c in (1, 4):
        inp = _shared_batch(rng, c, 64, [[300, 301, 302], [517], [1000, 1003]], advance_room=8)
        out = oracle.pipeline(inp)
        for adv_room in (0, 5):
            s2, p2, o2 = oracle.expand_translate_shared(inp, out["sel"], out["sel_count"], inp.row_pos, adv_room)
            assert np.array_equal(o2, out["out_count"])
            w = inp.ld_out
            assert np.array_equal(p2[:, :w], out["pos"]) and np.array_equal(s2[:, :w], out["slots"])
            assert np.all(p2[:, w:] == -1) and np.all(s2[:, w:] == -1)


def test_shared_expand_invariants_and_inverse_translation():
    rng = np.random.default_rng(43)
    N = 6
    for c in (1, 4):
        rows = [[int(x)] for x in rng.integers(8, 5000, 12)]
        inp = _shared_batch(rng, c, 128, rows, advance_room=N)
        out = oracle.pipeline(inp)
        adv = rng.integers(0, N + 1, inp.num_rows)
        now = inp.row_pos + adv.astype(np.int32)
        slots, pos, oc = oracle.expand_translate_shared(inp, out["sel"], out["sel_count"], now, N)
        inv = {}
        for b in range(inp.num_req):
            for lp, pp in enumerate(inp.page_table[b]):
                if pp >= 0:
                    inv[int(pp)] = (b, lp)
        for b in range(inp.num_req):
            for r in range(inp.req_row_ptr[b], inp.req_row_ptr[b + 1]):
                t0, t1 = int(inp.row_pos[r]), int(now[r])
                nv = (t0 + 1) // c
                m = int(out["sel_count"][r])
                n = int(oc[r])
                assert n == c * m + (t1 - c * nv + 1) <= inp.ld_out + N
                pr = pos[r, :n]
                assert np.unique(pr).size == n and pr.min() >= 0 and pr.max() <= t1
                assert pr[c * m:].tolist() == list(range(c * nv, t1 + 1))
                assert pr[:c * m].tolist() == out["pos"][r, :c * m].tolist()
                for s_, q_ in zip(slots[r, :n], pr):
                    bb, lp = inv[int(s_) // 64]
                    assert bb == b and lp * 64 + int(s_) % 64 == q_
                assert np.all(slots[r, n:] == -1) and np.all(pos[r, n:] == -1)


def test_shared_expand_rejects_bad_advances():
    rng = np.random.default_rng(44)
    inp = _shared_batch(rng, 4, 16, [[200]], advance_room=4)
    out = oracle.pipeline(inp)
    for now, room in (([199], 4), ([205], 4), ([203], 2)):  # behind t0; beyond t0 + room
        with pytest.raises(oracle.OracleError):
            oracle.expand_translate_shared(inp, out["sel"], out["sel_count"], now, room)
    with pytest.raises(oracle.OracleError):  # ld_out below k*c + c - 1 + max_advance
        oracle.expand_translate_shared(inp, out["sel"], out["sel_count"], [201], 4, ld_out=inp.ld_out + 3)
