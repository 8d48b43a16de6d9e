"""Comparison rules between the HIP path and the oracle.

  * scores:        |s_gpu - s_ref| <= 1e-4 * (1 + |s_ref|) on every visible entry;
  * top-k on given FP32 rows: identical sets (order of output unspecified);
  * end to end:    selections may differ only on blocks whose oracle score lies
                   within 2e-4 of the row's k-th oracle score;
  * expand/translate of a given selection: identical in canonical form
                   (block positions ascending, then pending ascending).
"""
from __future__ import annotations

import numpy as np

SCORE_RTOL = 1e-4
E2E_BAND = 2e-4


class Mismatch(AssertionError):
    pass


def check_scores(gpu: np.ndarray, ref: np.ndarray, row_len: np.ndarray, what: str = "scores"):
    R = ref.shape[0]
    for r in range(R):
        n = int(row_len[r])
        g = gpu[r, :n].astype(np.float64)
        s = ref[r, :n].astype(np.float64)
        if not np.all(np.isfinite(g)):
            bad = np.nonzero(~np.isfinite(g))[0][:5]
            raise Mismatch(f"{what}: row {r}: non-finite GPU score at {bad.tolist()}")
        err = np.abs(g - s)
        lim = SCORE_RTOL * (1.0 + np.abs(s))
        if np.any(err > lim):
            j = int(np.argmax(err - lim))
            raise Mismatch(f"{what}: row {r} block {j}: gpu {g[j]!r} ref {s[j]!r} (|d|={err[j]:.3g} > {lim[j]:.3g})")


def canonical_sel(sel: np.ndarray, count: np.ndarray):
    """Sorted selected indices per row, as a list of arrays; checks padding."""
    out = []
    for r in range(sel.shape[0]):
        m = int(count[r])
        if m < 0 or m > sel.shape[1]:
            raise Mismatch(f"row {r}: count {m} out of range")
        row = sel[r]
        if np.any(row[m:] != -1):
            raise Mismatch(f"row {r}: padding after {m} entries is not -1")
        s = np.sort(row[:m])
        if m > 1 and np.any(s[1:] == s[:-1]):
            raise Mismatch(f"row {r}: duplicate selected index")
        out.append(s)
    return out


def check_topk_exact(gpu_sel, gpu_cnt, ref_sel, ref_cnt):
    g = canonical_sel(np.asarray(gpu_sel), np.asarray(gpu_cnt))
    for r in range(len(g)):
        m = int(ref_cnt[r])
        if int(gpu_cnt[r]) != m:
            raise Mismatch(f"top-k row {r}: count {int(gpu_cnt[r])} != {m}")
        if not np.array_equal(g[r], ref_sel[r, :m]):
            d = np.setxor1d(g[r], ref_sel[r, :m])[:8]
            raise Mismatch(f"top-k row {r}: sets differ, e.g. {d.tolist()}")


def check_topk_e2e(gpu_sel, gpu_cnt, ref_scores, ref_sel, ref_cnt, row_len, band: float = E2E_BAND):
    """GPU selection vs oracle selection when the GPU ranked its own scores:
    every difference must be a block whose oracle score is within ``band`` of
    the row's k-th oracle score.  Returns the number of swapped blocks."""
    g = canonical_sel(np.asarray(gpu_sel), np.asarray(gpu_cnt))
    swaps = 0
    for r in range(len(g)):
        m = int(ref_cnt[r])
        if int(gpu_cnt[r]) != m:
            raise Mismatch(f"e2e row {r}: count {int(gpu_cnt[r])} != {m}")
        ref = ref_sel[r, :m]
        diff = np.setxor1d(g[r], ref)
        if diff.size == 0:
            continue
        n = int(row_len[r])
        if np.any(diff < 0) or np.any(diff >= n):
            raise Mismatch(f"e2e row {r}: index out of range {diff.tolist()[:5]}")
        kth = float(ref_scores[r, ref].min())
        far = np.abs(ref_scores[r, diff].astype(np.float64) - kth) > band
        if np.any(far):
            j = int(diff[np.argmax(far)])
            raise Mismatch(f"e2e row {r}: block {j} (score {ref_scores[r, j]!r}) differs but kth={kth!r}")
        swaps += int(diff.size) // 2
    return swaps


def canonical_expand(slots: np.ndarray, pos: np.ndarray, count: np.ndarray, n_pending: np.ndarray):
    """Canonical form of an expanded row: block part sorted by position (slots
    carried along), then the pending tail sorted the same way."""
    out = []
    for r in range(slots.shape[0]):
        n = int(count[r])
        if n < 0 or n > slots.shape[1]:
            raise Mismatch(f"expand row {r}: count {n} out of range")
        if np.any(slots[r, n:] != -1):
            raise Mismatch(f"expand row {r}: slot padding is not -1")
        p = int(n_pending[r])
        blk_pos, blk_slot = pos[r, :n - p], slots[r, :n - p]
        o = np.argsort(blk_pos, kind="stable")
        tail_pos, tail_slot = pos[r, n - p:n], slots[r, n - p:n]
        o2 = np.argsort(tail_pos, kind="stable")
        out.append((np.concatenate([blk_pos[o], tail_pos[o2]]), np.concatenate([blk_slot[o], tail_slot[o2]])))
    return out


def check_expand_exact(gpu_slots, gpu_pos, gpu_cnt, ref_slots, ref_pos, ref_cnt, n_pending):
    g = canonical_expand(np.asarray(gpu_slots), np.asarray(gpu_pos), np.asarray(gpu_cnt), n_pending)
    for r in range(len(g)):
        n = int(ref_cnt[r])
        if int(gpu_cnt[r]) != n:
            raise Mismatch(f"expand row {r}: count {int(gpu_cnt[r])} != {n}")
        gp, gs = g[r]
        if not np.array_equal(gp, ref_pos[r, :n]):
            raise Mismatch(f"expand row {r}: positions differ")
        if not np.array_equal(gs, ref_slots[r, :n]):
            raise Mismatch(f"expand row {r}: slots differ")
