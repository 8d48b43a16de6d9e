"""The C-ABI library loads, exports every symbol include/*.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""
from __future__ import annotations

import ctypes as C
import glob
import os
import re

import pytest

import block_scoring_top_amd as bst

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

BS_OK, BS_ERR_NULL, BS_ERR_ARG, BS_ERR_WORKSPACE = 0, -1, -2, -3


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for want in ("idx_score_decode", "idx_score_prefill", "topk_select_rows", "idx_expand_translate",
                 "topk_workspace_bytes", "bs_status_string", "bs_abi_version"):
        assert want in names, names


def test_library_exports_every_declared_symbol():
    L = bst.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    assert bst.lib().bs_abi_version() == 1
    assert bst.status_string(BS_OK) == "BS_OK"
    for s in (BS_ERR_NULL, BS_ERR_ARG, BS_ERR_WORKSPACE, -4):
        assert bst.status_string(s).startswith("BS_ERR")
    assert bst.status_string(12345) == "unknown status"


P = C.c_void_p
NULL = None
FAKE = C.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _score(fn, **kw):
    a = dict(q=FAKE, kc=FAKE, num_pages=1, pt=FAKE, pt_stride=1, ptr=FAKE, num_req=1, pos=FAKE, num_rows=1,
             c=4, max_vis=16, scores=FAKE, ld=16, row_len=NULL, stream=NULL)
    a.update(kw)
    return getattr(bst.lib(), fn)(a["q"], a["kc"], a["num_pages"], a["pt"], a["pt_stride"], a["ptr"], a["num_req"],
                                  a["pos"], a["num_rows"], a["c"], a["max_vis"], a["scores"], a["ld"],
                                  a["row_len"], a["stream"])


@pytest.mark.parametrize("fn", ["idx_score_decode", "idx_score_prefill"])
def test_score_validation(fn):
    assert _score(fn, num_rows=0) == BS_OK          # no-op, nothing launched
    assert _score(fn, num_req=0) == BS_OK
    assert _score(fn, c=3) == BS_ERR_ARG
    assert _score(fn, c=2) == BS_ERR_ARG
    assert _score(fn, num_rows=-1) == BS_ERR_ARG
    assert _score(fn, max_vis=-1) == BS_ERR_ARG
    assert _score(fn, ld=15) == BS_ERR_ARG          # ld < max_vis
    assert _score(fn, pt_stride=0) == BS_ERR_ARG
    assert _score(fn, max_vis=17) == BS_ERR_ARG     # 4*17 tokens > one 64-token page
    assert _score(fn, c=1, max_vis=65, ld=65) == BS_ERR_ARG
    for k in ("q", "kc", "pt", "ptr", "pos", "scores"):
        assert _score(fn, **{k: NULL}) == BS_ERR_NULL, k


def test_score_decode_row_bound():
    # rows beyond 65,535 * 4,096 blocks are refused before any launch (every
    # other argument valid for that size)
    big = 65535 * 4096 + 1
    assert _score("idx_score_decode", c=1, max_vis=big, ld=big, pt_stride=(big + 63) // 64) == BS_ERR_ARG


def _topk(**kw):
    a = dict(scores=FAKE, ld=100000, row_len=FAKE, num_rows=2, max_len=100000, k=2048, sel=FAKE, cnt=FAKE,
             ws=FAKE, ws_bytes=1 << 30, stream=NULL)
    a.update(kw)
    return bst.lib().topk_select_rows(a["scores"], a["ld"], a["row_len"], a["num_rows"], a["max_len"], a["k"],
                                      a["sel"], a["cnt"], a["ws"], a["ws_bytes"], a["stream"])


def test_topk_validation():
    assert _topk(num_rows=0) == BS_OK
    assert _topk(k=0) == BS_ERR_ARG
    assert _topk(k=2049) == BS_ERR_ARG
    assert _topk(max_len=-1) == BS_ERR_ARG
    assert _topk(ld=99999) == BS_ERR_ARG
    for k in ("scores", "row_len", "sel", "cnt"):
        assert _topk(**{k: NULL}) == BS_ERR_NULL, k
    need = bst.topk_workspace_bytes(2, 100000, 2048)
    assert need > 0
    assert _topk(ws=NULL) == BS_ERR_WORKSPACE
    assert _topk(ws_bytes=need - 1) == BS_ERR_WORKSPACE


def test_topk_workspace_sizes():
    assert bst.topk_workspace_bytes(0, 100000, 2048) == 0
    assert bst.topk_workspace_bytes(8192, 16384, 512) == 0       # single-workgroup rows need none
    a = bst.topk_workspace_bytes(8, 81920, 2048)
    b = bst.topk_workspace_bytes(16, 81920, 2048)
    assert a > 0 and b == 2 * a


def _expand(**kw):
    a = dict(sel=FAKE, cnt=FAKE, k=512, ptr=FAKE, num_req=1, pos=FAKE, num_rows=1, c=4, pt=FAKE, pt_stride=1,
             slots=FAKE, opos=NULL, ocnt=FAKE, ld_out=2051, stream=NULL)
    a.update(kw)
    return bst.lib().idx_expand_translate(a["sel"], a["cnt"], a["k"], a["ptr"], a["num_req"], a["pos"],
                                          a["num_rows"], a["c"], a["pt"], a["pt_stride"], a["slots"], a["opos"],
                                          a["ocnt"], a["ld_out"], a["stream"])


def test_expand_validation():
    assert _expand(num_rows=0) == BS_OK
    assert _expand(ld_out=2050) == BS_ERR_ARG           # needs k*c + c - 1 = 2051
    assert _expand(c=1, ld_out=2047, k=2048) == BS_ERR_ARG
    assert _expand(k=0) == BS_ERR_ARG
    assert _expand(k=2049, ld_out=10000) == BS_ERR_ARG
    assert _expand(c=2) == BS_ERR_ARG
    assert _expand(num_req=0) == BS_ERR_ARG
    assert _expand(pt_stride=0) == BS_ERR_ARG
    for k in ("sel", "cnt", "ptr", "pos", "pt", "slots", "ocnt"):
        assert _expand(**{k: NULL}) == BS_ERR_NULL, k


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bst, "_lib", None)
    monkeypatch.setattr(bst, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(bst.BlockScoreError):
        bst.lib()


def test_product_path_does_not_import_the_oracle():
    # The HIP path must never route through the CPU oracle.
    for path in glob.glob(os.path.join(ROOT, "block_scoring_top_amd", "**", "*"), recursive=True):
        if path.endswith((".py", ".hip", ".h", ".cpp")):
            text = open(path).read()
            assert "import oracle" not in text and "from oracle" not in text, path
            assert "liboracle" not in text, path


def test_prepared_calls_check_their_arguments_when_prepared():
    # Argument checking happens once, when the call is prepared (CPU tensors,
    # wrong dtypes and wrong shapes are rejected there, before any HIP call).
    import torch
    q = torch.zeros((2, 4, 128), dtype=torch.int16)
    i32 = torch.zeros(3, dtype=torch.int32)
    f32 = torch.zeros((2, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        bst.prepare_score("idx_score_decode", q, q, 1, i32.view(1, 3), i32[:2], i32[:2], 4, 8, f32)
    with pytest.raises(ValueError):
        bst.prepare_score("idx_score_sideways", q, q, 1, i32.view(1, 3), i32[:2], i32[:2], 4, 8, f32)
    with pytest.raises((TypeError, ValueError)):
        bst.prepare_topk(f32, i32[:2], 8, 4, torch.zeros((2, 4), dtype=torch.int64), i32[:2])
    with pytest.raises(ValueError):
        bst.prepare_topk(f32, i32[:2], 8, 4, torch.zeros((2, 5), dtype=torch.int32), i32[:2])


def _expand_shared(**kw):
    a = dict(sel=FAKE, cnt=FAKE, k=512, ptr=FAKE, num_req=1, pos=FAKE, now=FAKE, num_rows=1, c=4, adv=4,
             pt=FAKE, pt_stride=1, slots=FAKE, opos=NULL, ocnt=FAKE, ld_out=2055, stream=NULL)
    a.update(kw)
    return bst.lib().idx_expand_translate_shared(a["sel"], a["cnt"], a["k"], a["ptr"], a["num_req"], a["pos"],
                                                 a["now"], a["num_rows"], a["c"], a["adv"], a["pt"],
                                                 a["pt_stride"], a["slots"], a["opos"], a["ocnt"], a["ld_out"],
                                                 a["stream"])


def test_expand_shared_validation():
    assert _expand_shared(num_rows=0) == BS_OK
    assert _expand_shared(ld_out=2054) == BS_ERR_ARG       # needs k*c + c - 1 + max_advance = 2055
    assert _expand_shared(adv=-1) == BS_ERR_ARG
    assert _expand_shared(adv=1025, ld_out=10000) == BS_ERR_ARG
    assert _expand_shared(k=0) == BS_ERR_ARG
    assert _expand_shared(c=2) == BS_ERR_ARG
    assert _expand_shared(num_req=0) == BS_ERR_ARG
    assert _expand_shared(pt_stride=0) == BS_ERR_ARG
    for k in ("sel", "cnt", "ptr", "pos", "now", "pt", "slots", "ocnt"):
        assert _expand_shared(**{k: NULL}) == BS_ERR_NULL, k


def _compress(**kw):
    a = dict(k_raw=FAKE, num_tok=8, ptr=FAKE, start=FAKE, mpos=NULL, num_req=1, max_tok=8, rot=128, st=16, sh=24,
             sw=24, theta=1.0e6, ring=FAKE, ring_pos=NULL, pt=FAKE, pt_stride=1, kc=FAKE, num_pages=1, stream=NULL)
    a.update(kw)
    return bst.lib().idx_compress_store(a["k_raw"], a["num_tok"], a["ptr"], a["start"], a["mpos"], a["num_req"],
                                        a["max_tok"], a["rot"], a["st"], a["sh"], a["sw"], a["theta"], a["ring"],
                                        a["ring_pos"], a["pt"], a["pt_stride"], a["kc"], a["num_pages"],
                                        a["stream"])


def test_compress_validation():
    assert _compress(num_req=0) == BS_OK
    assert _compress(num_tok=0, max_tok=0) == BS_OK
    assert _compress(max_tok=0) == BS_OK
    assert _compress(max_tok=9) == BS_ERR_ARG              # more than num_tok
    assert _compress(num_req=-1) == BS_ERR_ARG
    assert _compress(num_req=65536) == BS_ERR_ARG
    assert _compress(rot=127, st=63, sh=0, sw=0) == BS_ERR_ARG
    assert _compress(rot=130, st=65, sh=0, sw=0) == BS_ERR_ARG
    assert _compress(rot=64) == BS_ERR_ARG                  # sections sum to 64, not 32
    assert _compress(st=-1, sh=41) == BS_ERR_ARG
    assert _compress(theta=0.0) == BS_ERR_ARG
    assert _compress(theta=float("inf")) == BS_ERR_ARG
    assert _compress(theta=float("nan")) == BS_ERR_ARG
    assert _compress(pt_stride=0) == BS_ERR_ARG
    assert _compress(num_pages=0) == BS_ERR_ARG
    for k in ("k_raw", "ptr", "start", "ring", "pt", "kc"):
        assert _compress(**{k: NULL}) == BS_ERR_NULL, k
    assert _compress(mpos=FAKE) == BS_ERR_NULL              # MRoPE positions need ring_pos


def _noalloc(**kw):
    a = dict(scores=FAKE, ld=81920, row_len=FAKE, num_rows=1, max_len=81920, k=2048, ptr=FAKE, num_req=1, pos=FAKE,
             c=1, pt=FAKE, pt_stride=1280, sel=FAKE, cnt=FAKE, slots=FAKE, opos=NULL, ocnt=FAKE, ld_out=2048,
             stream=NULL)
    a.update(kw)
    return bst.lib().idx_select_translate_noalloc(a["scores"], a["ld"], a["row_len"], a["num_rows"], a["max_len"],
                                                  a["k"], a["ptr"], a["num_req"], a["pos"], a["c"], a["pt"],
                                                  a["pt_stride"], a["sel"], a["cnt"], a["slots"], a["opos"],
                                                  a["ocnt"], a["ld_out"], a["stream"])


def test_noalloc_validation():
    # host-side checks only: every case fails (or is a no-op) before anything is launched
    assert _noalloc(num_rows=0) == BS_OK
    assert _noalloc(k=0) == BS_ERR_ARG
    assert _noalloc(c=2) == BS_ERR_ARG
    assert _noalloc(ld_out=2047) == BS_ERR_ARG
    assert _noalloc(ld=81919) == BS_ERR_ARG
    assert _noalloc(num_req=0) == BS_ERR_ARG
    for k in ("scores", "row_len", "sel", "cnt", "ptr", "pos", "pt", "slots", "ocnt"):
        assert _noalloc(**{k: NULL}) == BS_ERR_NULL, k
    # more long rows than the static scratch holds: rejected with the workspace status
    per_row = bst.topk_workspace_bytes(1, 81920, 2048)
    assert per_row > 0
    too_many = bst.NOALLOC_SCRATCH_BYTES // per_row + 1
    assert _noalloc(num_rows=too_many) == BS_ERR_WORKSPACE
    assert "static scratch" in bst.status_string(BS_ERR_WORKSPACE)


def test_plan_sizes():
    assert bst.topk_plan_bytes(0, 81920) == 0
    # one 16-byte slot per row below 16,385 entries, one per 8,192-entry chunk from there on
    assert bst.topk_plan_bytes(300, 8192) == 32 + 16 * 300
    assert bst.topk_plan_bytes(300, 16384) == 32 + 16 * 300
    assert bst.topk_plan_bytes(300, 16385) == 32 + 16 * 300 * 3
    assert bst.topk_plan_bytes(300, 81920) == 32 + 16 * 300 * 10
    assert bst.topk_planned_workspace_bytes(300, 16384, 2048) == 0
    w = bst.topk_planned_workspace_bytes(8, 20000, 2048)
    assert w > 0 and w % (64 << 10) == 0
    assert bst.topk_planned_workspace_bytes(16, 20000, 2048) == 2 * w
    # records sized for rows split from 16,385 entries on cover the unplanned launch's
    assert bst.topk_planned_workspace_bytes(16, 81920, 2048) >= bst.topk_workspace_bytes(16, 81920, 2048)


def _plan(**kw):
    a = dict(row_len=FAKE, num_rows=300, max_len=81920, plan=FAKE, plan_bytes=32 + 16 * 3000, stream=NULL)
    a.update(kw)
    return bst.lib().topk_plan_rows(a["row_len"], a["num_rows"], a["max_len"], a["plan"], a["plan_bytes"],
                                    a["stream"])


def _planned(**kw):
    a = dict(scores=FAKE, ld=81920, num_rows=300, max_len=81920, k=2048, ptr=FAKE, num_req=300, pos=FAKE, c=1,
             pt=FAKE, pt_stride=1280, sel=FAKE, cnt=FAKE, slots=FAKE, opos=NULL, ocnt=FAKE, ld_out=2048, plan=FAKE,
             plan_bytes=32 + 16 * 3000, ws=FAKE, ws_bytes=0, stream=NULL)
    a.update(kw)
    return bst.lib().idx_select_translate_planned(a["scores"], a["ld"], a["num_rows"], a["max_len"], a["k"],
                                                  a["ptr"], a["num_req"], a["pos"], a["c"], a["pt"], a["pt_stride"],
                                                  a["sel"], a["cnt"], a["slots"], a["opos"], a["ocnt"], a["ld_out"],
                                                  a["plan"], a["plan_bytes"], a["ws"], a["ws_bytes"], a["stream"])


def test_plan_validation():
    # host-side checks only: every case fails (or is a no-op) before anything is launched
    assert _plan(num_rows=0) == BS_OK
    assert _plan(num_rows=-1) == BS_ERR_ARG
    assert _plan(max_len=-1) == BS_ERR_ARG
    assert _plan(max_len=65535 * 4096 + 1, num_rows=1, plan_bytes=1 << 40) == BS_ERR_ARG
    assert _plan(num_rows=(1 << 22) // 10 + 1, plan_bytes=1 << 40) == BS_ERR_ARG  # more than 2^22 slots
    assert _plan(row_len=NULL) == BS_ERR_NULL
    assert _plan(plan=NULL) == BS_ERR_NULL
    assert _plan(plan_bytes=32 + 16 * 3000 - 1) == BS_ERR_WORKSPACE


def test_planned_select_validation():
    need = bst.topk_planned_workspace_bytes(300, 81920, 2048)
    assert _planned(num_rows=0) == BS_OK
    assert _planned(k=0, ws_bytes=need) == BS_ERR_ARG
    assert _planned(k=2049, ws_bytes=need) == BS_ERR_ARG
    assert _planned(c=2, ws_bytes=need) == BS_ERR_ARG
    assert _planned(ld_out=2047, ws_bytes=need) == BS_ERR_ARG
    assert _planned(ld=81919, ws_bytes=need) == BS_ERR_ARG
    assert _planned(num_req=0, ws_bytes=need) == BS_ERR_ARG
    for k in ("scores", "plan", "sel", "cnt", "ptr", "pos", "pt", "slots", "ocnt"):
        assert _planned(**{k: NULL}, ws_bytes=need) == BS_ERR_NULL, k
    assert _planned(plan_bytes=32 + 16 * 3000 - 1, ws_bytes=need) == BS_ERR_WORKSPACE
    assert _planned(ws_bytes=need - 1) == BS_ERR_WORKSPACE
    assert _planned(ws=NULL, ws_bytes=need) == BS_ERR_WORKSPACE
