"""The whole hot path on one GPU: score -> top-k -> expand/translate.

Allocates the output and workspace tensors once (torch, device memory) and
then enqueues the three C-ABI calls on the current stream.  No host
synchronisation happens inside :meth:`IndexerPath.run`.
"""
from __future__ import annotations

import torch

from . import (idx_expand_translate, idx_score_decode, idx_score_prefill, idx_select_translate,
               idx_select_translate_planned, prepare_score, prepare_select_translate, topk_plan, topk_plan_rows,
               topk_planned_workspace, topk_select_rows, topk_workspace)


class IndexerPath:
    """Buffers for one batch shape plus the three calls.

    ``inp`` is any object with the device-input fields (c, k, q, kcache,
    num_pages, page_table, req_row_ptr, row_pos, max_vis), e.g.
    ``synth.device.DeviceInputs``.  ``scorer`` is "decode" or "prefill".
    """

    def __init__(self, inp, scorer: str = "decode"):
        if scorer not in ("decode", "prefill"):
            raise ValueError("scorer must be 'decode' or 'prefill'")
        self.inp = inp
        self.scorer = scorer
        dev = inp.q.device
        R = int(inp.row_pos.shape[0])
        ld = max(int(inp.max_vis), 1)
        ld = (ld + 3) // 4 * 4  # 16-byte aligned rows
        self.scores = torch.empty((R, ld), dtype=torch.float32, device=dev)
        self.row_len = torch.empty(R, dtype=torch.int32, device=dev)
        self.sel = torch.empty((R, inp.k), dtype=torch.int32, device=dev)
        self.sel_count = torch.empty(R, dtype=torch.int32, device=dev)
        ld_out = inp.k * inp.c + inp.c - 1
        self.slots = torch.empty((R, ld_out), dtype=torch.int32, device=dev)
        self.pos = torch.empty((R, ld_out), dtype=torch.int32, device=dev)
        self.out_count = torch.empty(R, dtype=torch.int32, device=dev)
        self.workspace = topk_workspace(R, int(inp.max_vis), inp.k, dev)
        self.plan_buf = None          # planned selection: allocated on first use
        self.planned_workspace = None
        self._prepared = None

    def _prepare(self):
        """The two calls of the fused path with their arguments checked and
        marshalled once (``run`` then costs two plain C calls on the host)."""
        i = self.inp
        fn = "idx_score_decode" if self.scorer == "decode" else "idx_score_prefill"
        self._prepared = (
            prepare_score(fn, i.q, i.kcache, i.num_pages, i.page_table, i.req_row_ptr, i.row_pos, i.c, i.max_vis,
                          self.scores, self.row_len),
            prepare_select_translate(self.scores, self.row_len, int(i.max_vis), i.k, i.req_row_ptr, i.row_pos,
                                     i.c, i.page_table, self.sel, self.sel_count, self.slots, self.out_count,
                                     out_pos=self.pos, workspace=self.workspace))

    def score(self, stream=None):
        i = self.inp
        fn = idx_score_decode if self.scorer == "decode" else idx_score_prefill
        fn(i.q, i.kcache, i.num_pages, i.page_table, i.req_row_ptr, i.row_pos, i.c, i.max_vis,
           self.scores, self.row_len, stream=stream)

    def select(self, stream=None):
        topk_select_rows(self.scores, self.row_len, int(self.inp.max_vis), self.inp.k, self.sel,
                         self.sel_count, self.workspace, stream=stream)

    def expand(self, stream=None):
        i = self.inp
        idx_expand_translate(self.sel, self.sel_count, i.k, i.req_row_ptr, i.row_pos, i.c, i.page_table,
                             self.slots, self.out_count, out_pos=self.pos, stream=stream)

    def select_translate(self, stream=None):
        """Top-k and expand/translate fused in one kernel."""
        i = self.inp
        idx_select_translate(self.scores, self.row_len, int(i.max_vis), i.k, i.req_row_ptr, i.row_pos, i.c,
                             i.page_table, self.sel, self.sel_count, self.slots, self.out_count, out_pos=self.pos,
                             workspace=self.workspace, stream=stream)

    def plan(self, stream=None):
        """Builds the selection's work list from ``row_len`` (as the scorer
        wrote it); every later ``select_translate_planned`` uses it, until the
        next call here (the lengths change only with the row positions)."""
        i = self.inp
        if self.plan_buf is None:
            R, dev = int(i.row_pos.shape[0]), i.q.device
            self.plan_buf = topk_plan(R, int(i.max_vis), dev)
            self.planned_workspace = topk_planned_workspace(R, int(i.max_vis), i.k, dev)
        topk_plan_rows(self.row_len, int(i.max_vis), self.plan_buf, stream=stream)

    def select_translate_planned(self, stream=None):
        """``select_translate`` over the work list of the last ``plan``."""
        if self.plan_buf is None:
            raise RuntimeError("plan() must be called first")
        i = self.inp
        idx_select_translate_planned(self.scores, int(i.max_vis), i.k, i.req_row_ptr, i.row_pos, i.c, i.page_table,
                                     self.sel, self.sel_count, self.slots, self.out_count, self.plan_buf,
                                     out_pos=self.pos, workspace=self.planned_workspace, stream=stream)

    def bound(self, stream=None):
        """(score, select_translate) with arguments and stream fixed: each is
        one C call taking no arguments (for loops that run the step many
        times on one stream)."""
        return tuple(c.bind(stream) for c in self.prepared())

    def prepared(self):
        """(score, select_translate) as prepared calls: each takes an optional
        stream and launches with no per-call argument checking."""
        if self._prepared is None:
            self._prepare()
        return self._prepared

    def run(self, stream=None, fused: bool = True, planned: bool = False):
        """One pass of the path: score, then select + translate (fused into one
        kernel, the default) or the separate select and expand calls.
        planned: score, plan, then the planned select + translate."""
        if planned:
            self.score(stream)
            self.plan(stream)
            self.select_translate_planned(stream)
        elif fused:
            score, select_translate = self.prepared()
            score(stream)
            select_translate(stream)
        else:
            self.score(stream)
            self.select(stream)
            self.expand(stream)
