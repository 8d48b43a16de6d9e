"""MI355X-native sparse-attention indexer hot path.

Thin Python binding over ``libblockscore.so`` (C ABI in ``include/blockscore.h``).
Every function here only marshals torch tensors into the C call: it checks
dtypes, devices and contiguity, takes raw device pointers and the current HIP
stream, and raises if the library returns an error.  All computation runs in
the HIP kernels; there is no CPU fallback.  If the library is not built this
module raises on first use.

Steps (same names as the C ABI):
  idx_score_decode / idx_score_prefill  ->  topk_select_rows  ->  idx_expand_translate
  (idx_select_translate: the last two in one kernel; topk_plan_rows +
  idx_select_translate_planned: the same over a work list built once per step
  from the row lengths; idx_expand_translate_shared: the expansion of a
  selection reused across speculative draft steps)
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libblockscore.so")

HEADS = 4
DIM = 128
PAGE_TOKENS = 64
KMAX = 2048
NOALLOC_SCRATCH_BYTES = 8 << 20  # BS_NOALLOC_SCRATCH_BYTES

_lib = None


class BlockScoreError(RuntimeError):
    pass


def lib():
    """Loads the HIP library (built by ``block_scoring_top_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BlockScoreError(
                f"{LIB_PATH} is missing: build it with `python -m block_scoring_top_amd.build` "
                "(or __graft_entry__.build()); there is no CPU fallback")
        L = C.CDLL(LIB_PATH)
        P, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        score_args = [P, P, i64, P, i32, P, i32, P, i32, i32, i32, P, i64, P, P]
        for name in ("idx_score_decode", "idx_score_prefill"):
            f = getattr(L, name)
            f.argtypes = score_args
            f.restype = C.c_int
        L.topk_workspace_bytes.argtypes = [i32, i32, i32]
        L.topk_workspace_bytes.restype = C.c_size_t
        L.topk_select_rows.argtypes = [P, i64, P, i32, i32, i32, P, P, P, C.c_size_t, P]
        L.topk_select_rows.restype = C.c_int
        L.idx_expand_translate.argtypes = [P, P, i32, P, i32, P, i32, i32, P, i32, P, P, P, i32, P]
        L.idx_expand_translate.restype = C.c_int
        L.idx_expand_translate_shared.argtypes = [P, P, i32, P, i32, P, P, i32, i32, i32, P, i32, P, P, P, i32, P]
        L.idx_expand_translate_shared.restype = C.c_int
        L.idx_select_translate.argtypes = [P, i64, P, i32, i32, i32, P, i32, P, i32, P, i32, P, P, P, P, P, i32,
                                           P, C.c_size_t, P]
        L.idx_select_translate.restype = C.c_int
        L.idx_select_translate_noalloc.argtypes = [P, i64, P, i32, i32, i32, P, i32, P, i32, P, i32, P, P, P, P, P,
                                                   i32, P]
        L.idx_select_translate_noalloc.restype = C.c_int
        L.topk_plan_bytes.argtypes = [i32, i32]
        L.topk_plan_bytes.restype = C.c_size_t
        L.topk_planned_workspace_bytes.argtypes = [i32, i32, i32]
        L.topk_planned_workspace_bytes.restype = C.c_size_t
        L.topk_plan_rows.argtypes = [P, i32, i32, P, C.c_size_t, P]
        L.topk_plan_rows.restype = C.c_int
        L.idx_select_translate_planned.argtypes = [P, i64, i32, i32, i32, P, i32, P, i32, P, i32, P, P, P, P, P,
                                                   i32, P, C.c_size_t, P, C.c_size_t, P]
        L.idx_select_translate_planned.restype = C.c_int
        L.idx_compress_store.argtypes = [P, i32, P, P, P, i32, i32, i32, i32, i32, i32, C.c_double, P, P, P, i32,
                                         P, i64, P]
        L.idx_compress_store.restype = C.c_int
        L.bs_status_string.argtypes = [C.c_int]
        L.bs_status_string.restype = C.c_char_p
        L.bs_abi_version.argtypes = []
        L.bs_abi_version.restype = C.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bs_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise BlockScoreError(f"{what}: {status_string(status)} ({status})")


def _ptr(t: Optional[torch.Tensor], dtypes, name: str, device: Optional[torch.device] = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream, device) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _score_args(q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis, scores, row_len=None):
    """Checked argument tuple of a scorer call (all but the stream)."""
    dev = q.device
    num_rows = int(row_pos.shape[0])
    num_req = int(req_row_ptr.shape[0]) - 1
    if q.numel() != num_rows * HEADS * DIM:
        raise ValueError("q must hold num_rows x 4 x 128 values")
    if scores.dim() != 2 or scores.shape[0] != num_rows:
        raise ValueError("scores must be [num_rows, ld]")
    if row_len is not None and row_len.numel() != num_rows:
        raise ValueError("row_len must hold num_rows entries")
    per_page = PAGE_TOKENS // int(c) if int(c) in (1, 4) else 1
    if kcache.numel() < int(num_pages) * per_page * DIM:
        raise ValueError("kcache holds fewer than num_pages pages")
    return (_ptr(q, _BF16, "q", dev), _ptr(kcache, _BF16, "kcache", dev), int(num_pages),
            _ptr(page_table, _I32, "page_table", dev), int(page_table.shape[1]),
            _ptr(req_row_ptr, _I32, "req_row_ptr", dev), num_req,
            _ptr(row_pos, _I32, "row_pos", dev), num_rows, int(c), int(max_vis),
            _ptr(scores, _F32, "scores", dev), int(scores.stride(0)),
            _ptr(row_len, _I32, "row_len", dev))


def _score(fn: str, q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis, scores,
           row_len=None, stream=None):
    args = _score_args(q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis, scores, row_len)
    _check(getattr(lib(), fn)(*args, _stream(stream, q.device)), fn)


def idx_score_decode(q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis, scores,
                     row_len=None, stream=None):
    """Paged decode/verify scorer.  See ``idx_score_decode`` in blockscore.h."""
    _score("idx_score_decode", q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis,
           scores, row_len, stream)


def idx_score_prefill(q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis, scores,
                      row_len=None, stream=None):
    """Prefill scorer on the matrix cores.  See ``idx_score_prefill`` in blockscore.h."""
    _score("idx_score_prefill", q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis,
           scores, row_len, stream)


def topk_workspace_bytes(num_rows: int, max_len: int, k: int) -> int:
    return int(lib().topk_workspace_bytes(int(num_rows), int(max_len), int(k)))


def topk_workspace(num_rows: int, max_len: int, k: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace of the size the call needs (None if none)."""
    n = topk_workspace_bytes(num_rows, max_len, k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _topk_args(scores, row_len, max_len, k, sel, sel_count, workspace=None):
    """Checked argument tuple of a ``topk_select_rows`` call (all but the stream)."""
    dev = scores.device
    R = int(scores.shape[0])
    if sel.dim() != 2 or sel.shape[0] != R or sel.shape[1] != k:
        raise ValueError("sel must be [num_rows, k]")
    if sel_count.numel() != R or row_len.numel() != R:
        raise ValueError("row_len and sel_count must hold num_rows entries")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(scores, _F32, "scores", dev), int(scores.stride(0)), _ptr(row_len, _I32, "row_len", dev), R,
            int(max_len), int(k), _ptr(sel, _I32, "sel", dev), _ptr(sel_count, _I32, "sel_count", dev),
            _ptr(workspace, (torch.uint8,), "workspace", dev), ws_bytes)


def topk_select_rows(scores, row_len, max_len, k, sel, sel_count, workspace=None, stream=None):
    """Exact top-k per FP32 row.  See ``topk_select_rows`` in blockscore.h."""
    args = _topk_args(scores, row_len, max_len, k, sel, sel_count, workspace)
    _check(lib().topk_select_rows(*args, _stream(stream, scores.device)), "topk_select_rows")


def idx_expand_translate(sel, sel_count, k, req_row_ptr, row_pos, c, page_table, out_slots, out_count,
                         out_pos=None, stream=None):
    """Expand, append pending, translate.  See ``idx_expand_translate`` in blockscore.h."""
    dev = sel.device
    R = int(row_pos.shape[0])
    if sel.dim() != 2 or sel.shape[0] != R or sel.shape[1] != k:
        raise ValueError("sel must be [num_rows, k]")
    if out_slots.dim() != 2 or out_slots.shape[0] != R:
        raise ValueError("out_slots must be [num_rows, ld_out]")
    if out_pos is not None and out_pos.shape != out_slots.shape:
        raise ValueError("out_pos must match out_slots")
    st = lib().idx_expand_translate(
        _ptr(sel, _I32, "sel", dev), _ptr(sel_count, _I32, "sel_count", dev), int(k),
        _ptr(req_row_ptr, _I32, "req_row_ptr", dev), int(req_row_ptr.shape[0]) - 1,
        _ptr(row_pos, _I32, "row_pos", dev), R, int(c),
        _ptr(page_table, _I32, "page_table", dev), int(page_table.shape[1]),
        _ptr(out_slots, _I32, "out_slots", dev), _ptr(out_pos, _I32, "out_pos", dev),
        _ptr(out_count, _I32, "out_count", dev), int(out_slots.stride(0)), _stream(stream, dev))
    _check(st, "idx_expand_translate")


def _expand_shared_args(sel, sel_count, k, req_row_ptr, row_pos, row_pos_now, c, max_advance, page_table,
                        out_slots, out_count, out_pos=None):
    """Checked argument tuple of an ``idx_expand_translate_shared`` call (all but the stream)."""
    dev = sel.device
    R = int(row_pos.shape[0])
    if sel.dim() != 2 or sel.shape[0] != R or sel.shape[1] != k:
        raise ValueError("sel must be [num_rows, k]")
    if row_pos_now.numel() != R or sel_count.numel() != R:
        raise ValueError("row_pos_now and sel_count must hold num_rows entries")
    if out_slots.dim() != 2 or out_slots.shape[0] != R:
        raise ValueError("out_slots must be [num_rows, ld_out]")
    if out_pos is not None and out_pos.shape != out_slots.shape:
        raise ValueError("out_pos must match out_slots")
    return (_ptr(sel, _I32, "sel", dev), _ptr(sel_count, _I32, "sel_count", dev), int(k),
            _ptr(req_row_ptr, _I32, "req_row_ptr", dev), int(req_row_ptr.shape[0]) - 1,
            _ptr(row_pos, _I32, "row_pos", dev), _ptr(row_pos_now, _I32, "row_pos_now", dev), R, int(c),
            int(max_advance), _ptr(page_table, _I32, "page_table", dev), int(page_table.shape[1]),
            _ptr(out_slots, _I32, "out_slots", dev), _ptr(out_pos, _I32, "out_pos", dev),
            _ptr(out_count, _I32, "out_count", dev), int(out_slots.stride(0)))


def idx_expand_translate_shared(sel, sel_count, k, req_row_ptr, row_pos, row_pos_now, c, max_advance, page_table,
                                out_slots, out_count, out_pos=None, stream=None):
    """Expansion of a selection reused across draft steps (IndexShare).  See
    ``idx_expand_translate_shared`` in blockscore.h."""
    args = _expand_shared_args(sel, sel_count, k, req_row_ptr, row_pos, row_pos_now, c, max_advance, page_table,
                               out_slots, out_count, out_pos)
    _check(lib().idx_expand_translate_shared(*args, _stream(stream, sel.device)), "idx_expand_translate_shared")


def _select_translate_args(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                           out_slots, out_count, out_pos=None, workspace=None):
    """Checked argument tuple of an ``idx_select_translate`` call (all but the stream)."""
    dev = scores.device
    R = int(scores.shape[0])
    if sel.dim() != 2 or sel.shape[0] != R or sel.shape[1] != k:
        raise ValueError("sel must be [num_rows, k]")
    if sel_count.numel() != R or row_pos.numel() != R or (row_len is not None and row_len.numel() != R):
        raise ValueError("row_len, row_pos and sel_count must hold num_rows entries")
    if out_slots.dim() != 2 or out_slots.shape[0] != R:
        raise ValueError("out_slots must be [num_rows, ld_out]")
    if out_pos is not None and out_pos.shape != out_slots.shape:
        raise ValueError("out_pos must match out_slots")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(scores, _F32, "scores", dev), int(scores.stride(0)), _ptr(row_len, _I32, "row_len", dev), R,
            int(max_len), int(k), _ptr(req_row_ptr, _I32, "req_row_ptr", dev), int(req_row_ptr.shape[0]) - 1,
            _ptr(row_pos, _I32, "row_pos", dev), int(c), _ptr(page_table, _I32, "page_table", dev),
            int(page_table.shape[1]), _ptr(sel, _I32, "sel", dev), _ptr(sel_count, _I32, "sel_count", dev),
            _ptr(out_slots, _I32, "out_slots", dev), _ptr(out_pos, _I32, "out_pos", dev),
            _ptr(out_count, _I32, "out_count", dev), int(out_slots.stride(0)),
            _ptr(workspace, (torch.uint8,), "workspace", dev), ws_bytes)


def idx_select_translate(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                         out_slots, out_count, out_pos=None, workspace=None, stream=None):
    """Top-k and expand/translate in one kernel.  See ``idx_select_translate`` in blockscore.h."""
    args = _select_translate_args(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table, sel,
                                  sel_count, out_slots, out_count, out_pos, workspace)
    _check(lib().idx_select_translate(*args, _stream(stream, scores.device)), "idx_select_translate")


def idx_select_translate_noalloc(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                                 out_slots, out_count, out_pos=None, stream=None):
    """``idx_select_translate`` without a workspace (static device scratch of
    NOALLOC_SCRATCH_BYTES per GPU).  See ``idx_select_translate_noalloc`` in
    blockscore.h."""
    args = _select_translate_args(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table, sel,
                                  sel_count, out_slots, out_count, out_pos, None)[:-2]
    _check(lib().idx_select_translate_noalloc(*args, _stream(stream, scores.device)), "idx_select_translate_noalloc")


def topk_plan_bytes(num_rows: int, max_len: int) -> int:
    return int(lib().topk_plan_bytes(int(num_rows), int(max_len)))


def topk_planned_workspace_bytes(num_rows: int, max_len: int, k: int) -> int:
    return int(lib().topk_planned_workspace_bytes(int(num_rows), int(max_len), int(k)))


def topk_plan(num_rows: int, max_len: int, device) -> torch.Tensor:
    """Storage for a plan (int32, uninitialised: ``topk_plan_rows`` fills it)."""
    n = topk_plan_bytes(num_rows, max_len)
    return torch.empty(max(1, (n + 3) // 4), dtype=torch.int32, device=device)


def topk_planned_workspace(num_rows: int, max_len: int, k: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace for ``idx_select_translate_planned`` (None if none)."""
    n = topk_planned_workspace_bytes(num_rows, max_len, k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _plan_args(row_len, max_len, plan):
    dev = row_len.device
    return (_ptr(row_len, _I32, "row_len", dev), int(row_len.numel()), int(max_len), _ptr(plan, _I32, "plan", dev),
            plan.numel() * plan.element_size())


def topk_plan_rows(row_len, max_len, plan, stream=None):
    """Build the selection's work list from the row lengths.  See
    ``topk_plan_rows`` in blockscore.h."""
    _check(lib().topk_plan_rows(*_plan_args(row_len, max_len, plan), _stream(stream, row_len.device)),
           "topk_plan_rows")


def _select_translate_planned_args(scores, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                                   out_slots, out_count, plan, out_pos=None, workspace=None):
    # The argument tuple of idx_select_translate with row_len taken out and the
    # plan put before the workspace.
    a = _select_translate_args(scores, None, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                               out_slots, out_count, out_pos, workspace)
    return (*a[:2], *a[3:18], _ptr(plan, _I32, "plan", scores.device), plan.numel() * plan.element_size(), *a[18:])


def idx_select_translate_planned(scores, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                                 out_slots, out_count, plan, out_pos=None, workspace=None, stream=None):
    """``idx_select_translate`` over the work list of a plan (the plan's row
    lengths).  See ``idx_select_translate_planned`` in blockscore.h."""
    args = _select_translate_planned_args(scores, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                                          out_slots, out_count, plan, out_pos, workspace)
    _check(lib().idx_select_translate_planned(*args, _stream(stream, scores.device)), "idx_select_translate_planned")


def _compress_args(k_raw, req_tok_ptr, tok_start, mrope_pos, max_tok, rotary_dim, sections, theta, ring,
                   ring_pos, page_table, kcache, num_pages):
    """Checked argument tuple of an ``idx_compress_store`` call (all but the stream)."""
    dev = k_raw.device
    T = int(k_raw.shape[0])
    B = int(req_tok_ptr.shape[0]) - 1
    if k_raw.dim() != 2 or k_raw.shape[1] != 128:
        raise ValueError("k_raw must be [num_tok, 128]")
    if tok_start.numel() != B or ring.shape != (B, 4, 128):
        raise ValueError("tok_start must hold num_req entries and ring be [num_req, 4, 128]")
    if mrope_pos is not None and mrope_pos.shape != (T, 3):
        raise ValueError("mrope_pos must be [num_tok, 3]")
    if ring_pos is not None and ring_pos.shape != (B, 3):
        raise ValueError("ring_pos must be [num_req, 3]")
    if kcache.dim() != 2 or kcache.shape[1] != 128 or kcache.shape[0] < 16 * int(num_pages):
        raise ValueError("kcache must be [>= num_pages * 16, 128]")
    sec = [int(v) for v in sections]
    if len(sec) != 3:
        raise ValueError("sections must hold 3 entries (t, h, w)")
    return (_ptr(k_raw, _BF16, "k_raw", dev), T, _ptr(req_tok_ptr, _I32, "req_tok_ptr", dev),
            _ptr(tok_start, _I32, "tok_start", dev), _ptr(mrope_pos, _I32, "mrope_pos", dev), B, int(max_tok),
            int(rotary_dim), sec[0], sec[1], sec[2], float(theta), _ptr(ring, _BF16, "ring", dev),
            _ptr(ring_pos, _I32, "ring_pos", dev), _ptr(page_table, _I32, "page_table", dev),
            int(page_table.shape[1]), _ptr(kcache, _BF16, "kcache", dev), int(num_pages))


def idx_compress_store(k_raw, req_tok_ptr, tok_start, mrope_pos, max_tok, rotary_dim, sections, theta, ring,
                       ring_pos, page_table, kcache, num_pages, stream=None):
    """Compress new raw index keys into the c = 4 key cache (and update the
    rings).  See ``idx_compress_store`` in blockscore.h."""
    args = _compress_args(k_raw, req_tok_ptr, tok_start, mrope_pos, max_tok, rotary_dim, sections, theta, ring,
                          ring_pos, page_table, kcache, num_pages)
    _check(lib().idx_compress_store(*args, _stream(stream, k_raw.device)), "idx_compress_store")


class PreparedCall:
    """One C call with its arguments checked and marshalled once (the tensors
    behind the pointers must outlive it); ``__call__`` adds the stream and
    checks the status.  For loops that issue the same call many times."""

    def __init__(self, fn: str, args: tuple, device):
        self.fn = fn
        self.args = args
        self.device = device
        self._f = getattr(lib(), fn)

    def __call__(self, stream=None):
        st = self._f(*self.args, _stream(stream, self.device))
        if st != 0:
            _check(st, self.fn)

    def bind(self, stream=None) -> "BoundCall":
        """The same call with the stream resolved now (default: the current
        stream): each call is then one C call with nothing looked up."""
        return BoundCall(self, _stream(stream, self.device))


class BoundCall:
    """A PreparedCall with its stream fixed; ``__call__`` takes no arguments."""

    __slots__ = ("fn", "_f", "_args")

    def __init__(self, prepared: PreparedCall, stream_ptr):
        self.fn = prepared.fn
        self._f = prepared._f
        # Arguments as instances of their declared C types, so that a call
        # converts nothing.
        args = (*prepared.args, stream_ptr)
        self._args = tuple(a if isinstance(a, t) else t(a) for a, t in zip(args, self._f.argtypes))

    def __call__(self):
        st = self._f(*self._args)
        if st != 0:
            _check(st, self.fn)


def prepare_score(fn: str, q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis, scores,
                  row_len=None) -> PreparedCall:
    """``idx_score_decode`` or ``idx_score_prefill`` with fixed arguments."""
    if fn not in ("idx_score_decode", "idx_score_prefill"):
        raise ValueError("fn must be idx_score_decode or idx_score_prefill")
    return PreparedCall(fn, _score_args(q, kcache, num_pages, page_table, req_row_ptr, row_pos, c, max_vis,
                                        scores, row_len), q.device)


def prepare_topk(scores, row_len, max_len, k, sel, sel_count, workspace=None) -> PreparedCall:
    """``topk_select_rows`` with fixed arguments."""
    return PreparedCall("topk_select_rows", _topk_args(scores, row_len, max_len, k, sel, sel_count, workspace),
                        scores.device)


def prepare_expand_shared(sel, sel_count, k, req_row_ptr, row_pos, row_pos_now, c, max_advance, page_table,
                          out_slots, out_count, out_pos=None) -> PreparedCall:
    """``idx_expand_translate_shared`` with fixed arguments."""
    return PreparedCall("idx_expand_translate_shared",
                        _expand_shared_args(sel, sel_count, k, req_row_ptr, row_pos, row_pos_now, c, max_advance,
                                            page_table, out_slots, out_count, out_pos), sel.device)


def prepare_select_translate(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                             out_slots, out_count, out_pos=None, workspace=None) -> PreparedCall:
    """``idx_select_translate`` with fixed arguments."""
    return PreparedCall("idx_select_translate",
                        _select_translate_args(scores, row_len, max_len, k, req_row_ptr, row_pos, c, page_table,
                                               sel, sel_count, out_slots, out_count, out_pos, workspace),
                        scores.device)


def prepare_plan(row_len, max_len, plan) -> PreparedCall:
    """``topk_plan_rows`` with fixed arguments."""
    return PreparedCall("topk_plan_rows", _plan_args(row_len, max_len, plan), row_len.device)


def prepare_select_translate_planned(scores, max_len, k, req_row_ptr, row_pos, c, page_table, sel, sel_count,
                                     out_slots, out_count, plan, out_pos=None, workspace=None) -> PreparedCall:
    """``idx_select_translate_planned`` with fixed arguments."""
    return PreparedCall("idx_select_translate_planned",
                        _select_translate_planned_args(scores, max_len, k, req_row_ptr, row_pos, c, page_table, sel,
                                                       sel_count, out_slots, out_count, plan, out_pos, workspace),
                        scores.device)


__all__ = [
    "idx_score_decode", "idx_score_prefill", "topk_workspace_bytes", "topk_workspace",
    "topk_select_rows", "idx_expand_translate", "idx_expand_translate_shared", "idx_select_translate",
    "idx_select_translate_noalloc", "NOALLOC_SCRATCH_BYTES", "idx_compress_store", "status_string", "BlockScoreError",
    "lib", "PreparedCall", "BoundCall", "prepare_score", "prepare_topk", "prepare_select_translate", "prepare_expand_shared",
    "prepare_compress_store", "topk_plan_bytes", "topk_planned_workspace_bytes", "topk_plan",
    "topk_planned_workspace", "topk_plan_rows", "idx_select_translate_planned", "prepare_plan",
    "prepare_select_translate_planned",
]


def prepare_compress_store(k_raw, req_tok_ptr, tok_start, mrope_pos, max_tok, rotary_dim, sections, theta, ring,
                           ring_pos, page_table, kcache, num_pages) -> PreparedCall:
    """``idx_compress_store`` with fixed arguments."""
    return PreparedCall("idx_compress_store",
                        _compress_args(k_raw, req_tok_ptr, tok_start, mrope_pos, max_tok, rotary_dim, sections,
                                       theta, ring, ring_pos, page_table, kcache, num_pages), k_raw.device)
