"""CPU oracle for the sparse-attention indexer hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP path never
imports, links or calls it, and it imports nothing from the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only marshals numpy arrays into it and assembles the three steps.  Every
function is pinned by ``tests/test_oracle_pins.py`` to closed forms, brute
force, exhaustive checks or library routines.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """The oracle library; ``ORACLE_LIB`` may name another build of the same
    source (the sanitizer build in ``tests/test_oracle_sanitized.py``)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB") or _build.LIB
        if path == _build.LIB and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        L = C.CDLL(path)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.oracle_score.argtypes = [P, P, i64, P, i32, P, i32, P, i32, i32, P, i64, P]
        L.oracle_score.restype = C.c_int
        L.oracle_topk.argtypes = [P, i64, P, i32, i32, P, P]
        L.oracle_topk.restype = C.c_int
        L.oracle_expand_translate.argtypes = [P, P, i32, P, i32, P, i32, i32, P, i32, P, P, P, i32]
        L.oracle_expand_translate.restype = C.c_int
        L.oracle_expand_translate_shared.argtypes = [P, P, i32, P, i32, P, P, i32, i32, i32, P, i32, P, P, P, i32]
        L.oracle_expand_translate_shared.restype = C.c_int
        L.oracle_compress_store.argtypes = [P, P, P, P, i32, i32, P, C.c_double, P, P, P, i32, P, i64, P]
        L.oracle_compress_store.restype = C.c_int
        L.oracle_f64_to_bf16.argtypes = [C.c_double]
        L.oracle_f64_to_bf16.restype = C.c_uint16
        L.oracle_f32_to_f16.argtypes = [C.c_uint32]
        L.oracle_f32_to_f16.restype = C.c_uint16
        L.oracle_key16.argtypes = [C.c_uint16]
        L.oracle_key16.restype = C.c_uint16
        L.oracle_key32.argtypes = [C.c_uint32]
        L.oracle_key32.restype = C.c_uint32
        L.oracle_bin.argtypes = [C.c_float]
        L.oracle_bin.restype = C.c_int32
        L.oracle_topk_hist.argtypes = [P, i32, i32, P, P]
        L.oracle_topk_hist.restype = C.c_int32
        L.oracle_check_f16_all.argtypes = []
        L.oracle_check_f16_all.restype = C.c_int64
        L.oracle_check_key32_chain.argtypes = [C.POINTER(C.c_int64)]
        L.oracle_check_key32_chain.restype = C.c_int64
        L.oracle_n_vis.argtypes = [i32, i32]
        L.oracle_n_vis.restype = C.c_int32
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


class OracleError(RuntimeError):
    pass


def threads() -> int:
    return int(lib().oracle_threads())


def n_vis(t: int, c: int) -> int:
    return int(lib().oracle_n_vis(int(t), int(c)))


def score(inp, ld: int | None = None, fill=np.nan):
    """QSA score of every visible block of every row.  Returns (scores
    float32 [R][ld], row_len int32 [R]); entries at j >= row_len keep ``fill``."""
    ld = int(inp.max_vis if ld is None else ld)
    R = inp.num_rows
    scores = np.full((R, max(ld, 1)), fill, dtype=np.float32)
    row_len = np.full(R, -1, dtype=np.int32)
    q = np.ascontiguousarray(inp.q, dtype=np.uint16)
    kc = np.ascontiguousarray(inp.kcache, dtype=np.uint16)
    pt = np.ascontiguousarray(inp.page_table, dtype=np.int32)
    ptr = np.ascontiguousarray(inp.req_row_ptr, dtype=np.int32)
    pos = np.ascontiguousarray(inp.row_pos, dtype=np.int32)
    st = lib().oracle_score(_p(q), _p(kc), int(inp.num_pages), _p(pt), pt.shape[1],
                            _p(ptr), ptr.shape[0] - 1, _p(pos), R, int(inp.c),
                            _p(scores), scores.shape[1], _p(row_len))
    if st != 0:
        raise OracleError("oracle_score failed: %d" % st)
    return scores, row_len


def topk(scores: np.ndarray, row_len: np.ndarray, k: int):
    """Top-k by full sort.  Returns (sel int32 [R][k] ascending, -1 padded;
    count int32 [R])."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    rl = np.ascontiguousarray(row_len, dtype=np.int32)
    R = s.shape[0]
    sel = np.empty((R, k), dtype=np.int32)
    cnt = np.empty(R, dtype=np.int32)
    st = lib().oracle_topk(_p(s), s.shape[1], _p(rl), R, int(k), _p(sel), _p(cnt))
    if st != 0:
        raise OracleError("oracle_topk failed: %d" % st)
    return sel, cnt


def expand_translate(inp, sel: np.ndarray, count: np.ndarray, ld_out: int | None = None):
    """Expand chosen blocks to positions, append pending, translate to slots.
    Returns (slots, positions, count), canonical order, -1 padded."""
    ld_out = int(inp.ld_out if ld_out is None else ld_out)
    R = inp.num_rows
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    cnt = np.ascontiguousarray(count, dtype=np.int32)
    k = sel.shape[1]
    slots = np.empty((R, ld_out), dtype=np.int32)
    pos = np.empty((R, ld_out), dtype=np.int32)
    oc = np.empty(R, dtype=np.int32)
    pt = np.ascontiguousarray(inp.page_table, dtype=np.int32)
    ptr = np.ascontiguousarray(inp.req_row_ptr, dtype=np.int32)
    rp = np.ascontiguousarray(inp.row_pos, dtype=np.int32)
    st = lib().oracle_expand_translate(_p(sel), _p(cnt), k, _p(ptr), ptr.shape[0] - 1, _p(rp), R,
                                       int(inp.c), _p(pt), pt.shape[1], _p(slots), _p(pos), _p(oc), ld_out)
    if st != 0:
        raise OracleError("oracle_expand_translate failed: %d" % st)
    return slots, pos, oc


def expand_translate_shared(inp, sel: np.ndarray, count: np.ndarray, row_pos_now, max_advance: int,
                            ld_out: int | None = None):
    """IndexShare expansion (QSA page, section IndexShare MTP): the selection
    captured at each row's inp.row_pos is expanded as by expand_translate, and
    the tail runs from the captured pending tokens through row_pos_now.
    Returns (slots, positions, count), canonical order, -1 padded."""
    ld_out = int(inp.ld_out + max_advance if ld_out is None else ld_out)
    R = inp.num_rows
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    cnt = np.ascontiguousarray(count, dtype=np.int32)
    now = np.ascontiguousarray(row_pos_now, dtype=np.int32)
    k = sel.shape[1]
    slots = np.empty((R, ld_out), dtype=np.int32)
    pos = np.empty((R, ld_out), dtype=np.int32)
    oc = np.empty(R, dtype=np.int32)
    pt = np.ascontiguousarray(inp.page_table, dtype=np.int32)
    ptr = np.ascontiguousarray(inp.req_row_ptr, dtype=np.int32)
    rp = np.ascontiguousarray(inp.row_pos, dtype=np.int32)
    st = lib().oracle_expand_translate_shared(_p(sel), _p(cnt), k, _p(ptr), ptr.shape[0] - 1, _p(rp), _p(now), R,
                                              int(inp.c), int(max_advance), _p(pt), pt.shape[1], _p(slots),
                                              _p(pos), _p(oc), ld_out)
    if st != 0:
        raise OracleError("oracle_expand_translate_shared failed: %d" % st)
    return slots, pos, oc


def compress_store(ci, kcache=None, ring=None, ring_pos=None, mrope_pos="inputs", strict=True):
    """Key compression and store (QSA page, section on Qwen sparse attention:
    4 raw index keys averaged in FP32, normalised, MRoPE-rotated at the
    block's first token, one bf16 key per block at full_slot/4; the
    unfinished block's raw keys kept in a 4-slot ring per request).

    Starts from copies of ``kcache`` / ``ring`` / ``ring_pos`` (default: the
    state held by ``ci``) and returns dict(kcache, ring, ring_pos, exact):
    the state after the call and, for every cache entry written, its value
    before bf16 rounding (NaN elsewhere).  With ``strict=False`` blocks whose
    page id is out of range (or requests with a negative start) are skipped
    instead of raising."""
    kc = np.array(ci.kcache if kcache is None else kcache, dtype=np.uint16, copy=True, order="C")
    rg = np.array(ci.ring if ring is None else ring, dtype=np.uint16, copy=True, order="C")
    rp = np.array(ci.ring_pos if ring_pos is None else ring_pos, dtype=np.int32, copy=True, order="C")
    mp = ci.mrope_pos if isinstance(mrope_pos, str) else mrope_pos
    mp = None if mp is None else np.ascontiguousarray(mp, dtype=np.int32)
    exact = np.full(kc.shape, np.nan, dtype=np.float64)
    k_raw = np.ascontiguousarray(ci.k_raw, dtype=np.uint16)
    ptr = np.ascontiguousarray(ci.req_tok_ptr, dtype=np.int32)
    st0 = np.ascontiguousarray(ci.tok_start, dtype=np.int32)
    pt = np.ascontiguousarray(ci.page_table, dtype=np.int32)
    sec = np.ascontiguousarray(ci.sections, dtype=np.int32)
    st = lib().oracle_compress_store(_p(k_raw) if k_raw.size else None, _p(ptr), _p(st0),
                                     None if mp is None else _p(mp), ptr.shape[0] - 1,
                                     int(ci.rotary_dim), _p(sec), float(ci.theta), _p(rg), _p(rp),
                                     _p(pt), pt.shape[1], _p(kc), int(ci.num_pages), _p(exact))
    if st != 0 and (strict or st != -5):
        raise OracleError("oracle_compress_store failed: %d" % st)
    return dict(kcache=kc, ring=rg, ring_pos=rp, exact=exact)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Elementwise double -> bf16 (round to nearest even, one rounding)."""
    v = np.asarray(x, dtype=np.float64).ravel()
    f = lib().oracle_f64_to_bf16
    return np.fromiter((f(float(a)) for a in v), dtype=np.uint16, count=v.size)


def pipeline(inp):
    """The whole hot path on the CPU: score -> top-k -> expand/translate."""
    scores, row_len = score(inp)
    sel, cnt = topk(scores, row_len, inp.k)
    slots, pos, oc = expand_translate(inp, sel, cnt)
    return dict(scores=scores, row_len=row_len, sel=sel, sel_count=cnt,
                slots=slots, pos=pos, out_count=oc)


def f32_to_f16_bits(x) -> np.ndarray:
    """Elementwise oracle FP32 -> FP16 conversion (bit patterns)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).ravel()
    f = lib().oracle_f32_to_f16
    return np.fromiter((f(int(v)) for v in u), dtype=np.uint16, count=u.size)


def key16(h: int) -> int:
    return int(lib().oracle_key16(int(h)))


def key32(u: int) -> int:
    return int(lib().oracle_key32(int(u)))


def bin_of(v: float) -> int:
    return int(lib().oracle_bin(float(v)))


def topk_hist(row: np.ndarray, k: int):
    """The blog's histogram/threshold/refine steps on one row.  Returns
    (selected ascending, hist[1024])."""
    row = np.ascontiguousarray(row, dtype=np.float32)
    n = row.shape[0]
    sel = np.empty(max(min(k, n), 1), dtype=np.int32)
    hist = np.empty(1024, dtype=np.uint32)
    m = lib().oracle_topk_hist(_p(row), n, int(k), _p(sel), _p(hist))
    return sel[:m].copy(), hist


def check_f16_all() -> int:
    return int(lib().oracle_check_f16_all())


def check_key32_chain():
    visited = C.c_int64(0)
    bad = lib().oracle_check_key32_chain(C.byref(visited))
    return int(bad), int(visited.value)
