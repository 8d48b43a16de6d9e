"""Seeded synthetic inputs for the indexer hot path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no scoring, no selection, no expansion).  Both the CPU
oracle (under ``oracle/``) and the HIP path are fed from here, so the two see
identical bits.

Workload shapes follow the indexer described in "Qwen3.8-Flash-Next Day-0 in
SGLang" (theainews.cc, section on Qwen sparse attention, QSA): 4 query heads of
128 dims, one bf16 compressed index key per 4 tokens, top-512 blocks; and the
DSA indexer of the GLM-5.2 SGLang blog (aihot.virxact.com, Kernel Optimization
> TopK-V2): FP32 score rows near 80K long with k = 2048.  The pages publish no
datasets for this path; the value distributions below are synthetic.

Layout conventions (shared with the C-ABI):
  * ``q``: uint16 bf16 bit patterns, ``[rows][4][128]``.
  * ``kcache``: uint16 bf16 bit patterns, ``[num_pages * (64 // c)][128]``;
    physical page ``p`` holds compressed slots ``p*(64//c) ... p*(64//c)+64//c-1``.
  * ``page_table``: int32 ``[requests][pt_stride]``, logical 64-token page ->
    physical page, -1 beyond a request's pages.
  * ``req_row_ptr``: int32 ``[requests + 1]``; rows of a request are contiguous.
  * ``row_pos``: int32 ``[rows]``, 0-based token position of each query row.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

HEADS = 4
DIM = 128
PAGE_TOKENS = 64

# One fixed seed per named workload.
SEEDS = {
    "qsa_decode_1x8k": 1001,
    "topk_8x80k": 1002,
    "qsa_verify_64req": 1003,
    "dsa_decode_16x80k": 1004,
    "qsa_prefill_8k": 1005,
    "qsa_indexshare_64req": 1006,
    "qsa_compress_prefill_8k": 1007,
    "qsa_compress_decode_64req": 1008,
    "select_mixed_300rows": 1009,
    "topk_1x1m": 1010,
}

# Rotary parameters of the compressed index key.  The pages name an MRoPE
# rotation at the block's first token and nothing more; the values taken are
# Qwen2-VL's: the whole 128-dim key rotated, its 64 frequency pairs split
# 16 / 24 / 24 over the temporal / height / width position components, base
# 1,000,000.
ROPE_DIM = 128
MROPE_SECTIONS = (16, 24, 24)
ROPE_THETA = 1.0e6

# Draft steps of the IndexShare workload; a draft step at most this many
# positions past the captured row is served by the captured selection.
INDEXSHARE_DRAFT_STEPS = 3
INDEXSHARE_MAX_ADVANCE = INDEXSHARE_DRAFT_STEPS + 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns
    the uint16 bit patterns.  Inputs here are finite, so no NaN handling."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class IndexerInputs:
    """One batch of indexer inputs (decode or prefill)."""

    name: str
    c: int                      # compression ratio: 4 (QSA c4) or 1 (DSA)
    k: int                      # blocks to keep per row
    q: np.ndarray               # uint16 [R][4][128]
    kcache: np.ndarray          # uint16 [num_pages*(64//c)][128]
    num_pages: int
    page_table: np.ndarray      # int32 [B][pt_stride]
    req_row_ptr: np.ndarray     # int32 [B+1]
    row_pos: np.ndarray         # int32 [R]
    max_vis: int                # host-side bound on visible blocks per row
    seed: int

    @property
    def num_rows(self) -> int:
        return int(self.row_pos.shape[0])

    @property
    def num_req(self) -> int:
        return int(self.req_row_ptr.shape[0] - 1)

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def ld_out(self) -> int:
        """Smallest legal row stride of the expanded slot list."""
        return self.k * self.c + self.c - 1


@dataclasses.dataclass
class ScoreRows:
    """Given FP32 score rows for the top-k-only workload."""

    name: str
    k: int
    scores: np.ndarray          # float32 [R][ld]
    row_len: np.ndarray         # int32 [R]
    seed: int

    @property
    def num_rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def max_len(self) -> int:
        return int(self.scores.shape[1])


@dataclasses.dataclass
class SelectBatch:
    """Given FP32 score rows of a paged batch, for the fused selection and
    translation on its own (nothing is scored: `inp` carries the paging,
    with zero queries and keys)."""

    inp: "IndexerInputs"
    scores: np.ndarray          # float32 [R][max_len]
    row_len: np.ndarray         # int32 [R]

    @property
    def name(self) -> str:
        return self.inp.name

    @property
    def num_rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def max_len(self) -> int:
        return int(self.scores.shape[1])


@dataclasses.dataclass
class CompressInputs:
    """New raw index keys of a batch of requests, to be compressed into the
    c = 4 index cache, with the cache and ring state before the call."""

    name: str
    k_raw: np.ndarray                 # uint16 [T][128] bf16, tokens of a request contiguous
    req_tok_ptr: np.ndarray           # int32 [B+1]
    tok_start: np.ndarray             # int32 [B], position of each request's first new token
    mrope_pos: Optional[np.ndarray]   # int32 [T][3] (t, h, w) or None for text positions
    ring: np.ndarray                  # uint16 [B][4][128] bf16
    ring_pos: np.ndarray              # int32 [B][3]
    page_table: np.ndarray            # int32 [B][pt_stride]
    kcache: np.ndarray                # uint16 [num_pages*16][128] bf16
    num_pages: int
    rotary_dim: int
    sections: tuple
    theta: float
    seed: int

    @property
    def num_req(self) -> int:
        return int(self.req_tok_ptr.shape[0] - 1)

    @property
    def num_tok(self) -> int:
        return int(self.k_raw.shape[0])

    @property
    def max_tok(self) -> int:
        """Host-side bound on new tokens per request."""
        return int(np.max(np.diff(self.req_tok_ptr), initial=0))

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])


def mrope_positions(tokens: np.ndarray, images=()) -> np.ndarray:
    """(t, h, w) position components of token indices ``tokens`` for a
    sequence whose image spans are ``images`` = [(first token, grid g), ...]
    in order.  Text tokens carry t = h = w; an image of g x g tokens shares
    one t, its rows and columns add to h and w, and the text after it resumes
    g positions later."""
    x = np.asarray(tokens, dtype=np.int64)
    out = np.empty((x.shape[0], 3), dtype=np.int64)
    shift = np.zeros_like(x)
    in_img = np.zeros(x.shape[0], dtype=bool)
    for a, g in images:
        inside = (x >= a) & (x < a + g * g)
        base = a - shift[inside]
        off = x[inside] - a
        out[inside, 0] = base
        out[inside, 1] = base + off // g
        out[inside, 2] = base + off % g
        in_img |= inside
        shift[x >= a + g * g] += g * g - g
    text = ~in_img
    out[text, :] = (x[text] - shift[text])[:, None]
    return out.astype(np.int32)


def build_compress_batch(name: str, seed: int, starts, counts, ctx_tokens,
                         images=None, text_positions: bool = False,
                         rng: Optional[np.random.Generator] = None,
                         identity_pages: bool = False,
                         rotary_dim: int = ROPE_DIM, sections=MROPE_SECTIONS,
                         theta: float = ROPE_THETA) -> CompressInputs:
    """Lay out one compression call: request ``b`` appends ``counts[b]`` new
    tokens at positions ``starts[b]`` ... and owns ``ceil(ctx_tokens[b]/64)``
    pages (a seeded permutation of all pages).  Raw keys ~N(0,1) rounded to
    bf16.  The ring holds raw keys of the tokens of the block the first new
    token falls in (random keys in its stale slots) and the MRoPE position of
    that block's first token; the cache starts filled with normalised random
    keys.  ``images[b]`` lists request ``b``'s image spans; with
    ``text_positions`` the call passes no MRoPE positions at all."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    B = len(starts)
    images = images if images is not None else [()] * B
    pages = [max(1, -(-int(t) // PAGE_TOKENS)) for t in ctx_tokens]
    total = int(sum(pages))
    perm = np.arange(total, dtype=np.int64) if identity_pages else rng.permutation(total)
    pt = np.full((B, max(pages)), -1, dtype=np.int32)
    off = 0
    for b, np_b in enumerate(pages):
        pt[b, :np_b] = perm[off:off + np_b]
        off += np_b
    ptr = np.zeros(B + 1, dtype=np.int32)
    ptr[1:] = np.cumsum(counts)
    T = int(ptr[-1])
    k_raw = f32_to_bf16_bits(_normal_f32(rng, (max(T, 1), DIM)))[:T]
    mpos = np.zeros((T, 3), dtype=np.int32)
    ring_pos = rng.integers(0, 1 << 20, size=(B, 3)).astype(np.int32)
    for b in range(B):
        s, n = int(starts[b]), int(counts[b])
        mpos[ptr[b]:ptr[b + 1]] = mrope_positions(np.arange(s, s + n), images[b])
        ring_pos[b] = mrope_positions(np.array([s - s % 4]), images[b])[0]
    ring = f32_to_bf16_bits(_normal_f32(rng, (B * 4, DIM))).reshape(B, 4, DIM)
    kcache = draw_normalised_keys(rng, total * (PAGE_TOKENS // 4))
    return CompressInputs(name=name, k_raw=k_raw, req_tok_ptr=ptr,
                          tok_start=np.asarray(starts, dtype=np.int32),
                          mrope_pos=None if text_positions else mpos,
                          ring=ring, ring_pos=ring_pos, page_table=pt, kcache=kcache,
                          num_pages=total, rotary_dim=int(rotary_dim),
                          sections=tuple(int(v) for v in sections), theta=float(theta), seed=seed)


def _normal_f32(rng: np.random.Generator, shape, chunk_rows: int = 1 << 16) -> np.ndarray:
    """N(0,1) float32 of ``shape``, drawn row-chunk by row-chunk to bound memory."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = rng.standard_normal(size=(r1 - r0, flat.shape[1]), dtype=np.float32)
    return out


def draw_q(rng: np.random.Generator, rows: int) -> np.ndarray:
    """Query heads ~N(0,1) in FP32, rounded to bf16."""
    return f32_to_bf16_bits(_normal_f32(rng, (rows, HEADS, DIM)))


def draw_normalised_keys(rng: np.random.Generator, n: int, chunk: int = 1 << 16) -> np.ndarray:
    """Keys ~N(0,1) in FP32, L2-normalised in FP32, then rounded to bf16."""
    out = np.empty((n, DIM), dtype=np.uint16)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        x = rng.standard_normal(size=(r1 - r0, DIM), dtype=np.float32)
        nrm = np.sqrt(np.einsum("ij,ij->i", x, x, dtype=np.float32)).astype(np.float32)
        x /= nrm[:, None]
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def build_paged_batch(name: str, seed: int, c: int, k: int, ctx_tokens: list[int],
                      row_pos_per_req: list[list[int]],
                      rng: Optional[np.random.Generator] = None,
                      extra_pages: int = 0,
                      identity_pages: bool = False) -> IndexerInputs:
    """Lay out a paged batch.

    ``ctx_tokens[b]`` is the number of tokens request ``b`` holds (its pages are
    ``ceil(ctx/64)``); ``row_pos_per_req[b]`` lists its query positions.  Physical
    pages are a seeded permutation of all pages (disjoint across requests), or
    the identity when ``identity_pages``.  Keys are drawn directly in physical
    order, so each physical page holds independent keys.
    """
    assert c in (1, 4)
    rng = rng if rng is not None else np.random.default_rng(seed)
    pages = [max(1, -(-t // PAGE_TOKENS)) for t in ctx_tokens]
    total = int(sum(pages)) + extra_pages
    perm = np.arange(total, dtype=np.int64) if identity_pages else rng.permutation(total)
    pt_stride = max(pages)
    pt = np.full((len(pages), pt_stride), -1, dtype=np.int32)
    off = 0
    for b, np_b in enumerate(pages):
        pt[b, :np_b] = perm[off:off + np_b]
        off += np_b
    rows = [p for lst in row_pos_per_req for p in lst]
    ptr = np.zeros(len(pages) + 1, dtype=np.int32)
    ptr[1:] = np.cumsum([len(lst) for lst in row_pos_per_req])
    row_pos = np.asarray(rows, dtype=np.int32)
    q = draw_q(rng, len(rows))
    kcache = draw_normalised_keys(rng, total * (PAGE_TOKENS // c))
    max_vis = max([(p + 1) // c for p in rows], default=0)
    return IndexerInputs(name=name, c=c, k=k, q=q, kcache=kcache, num_pages=total,
                         page_table=pt, req_row_ptr=ptr, row_pos=row_pos,
                         max_vis=max_vis, seed=seed)


# ----------------------------------------------------------------------------
# The five named workloads.
# ----------------------------------------------------------------------------

def qsa_decode_1x8k(seed: int = SEEDS["qsa_decode_1x8k"]) -> IndexerInputs:
    """QSA c4 decode: 1 request, 1 query row, L = 8192 tokens in complete
    blocks (2048 compressed blocks) plus 2 pending tokens; top-512."""
    L, p = 8192, 2
    t = L + p - 1
    return build_paged_batch("qsa_decode_1x8k", seed, c=4, k=512,
                             ctx_tokens=[L + p], row_pos_per_req=[[t]])


def topk_8x80k(seed: int = SEEDS["topk_8x80k"], rows: int = 8, n: int = 81920,
               k: int = 2048) -> ScoreRows:
    """Top-k only: FP32 rows ~N(0,1); 1% of entries replaced by N(0,1)*20
    (heavy tail); an independent 5% snapped to FP16-representable values so
    many entries share the boundary bin."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(rows, n), dtype=np.float32)
    for r in range(rows):
        heavy = rng.choice(n, size=n // 100, replace=False)
        x[r, heavy] = rng.standard_normal(size=heavy.shape[0], dtype=np.float32) * np.float32(20.0)
        snap = rng.choice(n, size=n // 20, replace=False)
        x[r, snap] = x[r, snap].astype(np.float16).astype(np.float32)
    return ScoreRows(name="topk_8x80k", k=k, scores=x,
                     row_len=np.full(rows, n, dtype=np.int32), seed=seed)


def topk_1x1m(seed: int = SEEDS["topk_1x1m"], rows: int = 1, n: int = 1_000_000, k: int = 2048) -> ScoreRows:
    """Top-k only on one row of a million entries (the pages' 1M-token ISL
    case of TopK-V2), with the value recipe of topk_8x80k."""
    w = topk_8x80k(seed=seed, rows=rows, n=n, k=k)
    return ScoreRows(name="topk_1x1m", k=k, scores=w.scores, row_len=w.row_len, seed=seed)


def verify_lengths(rng: np.random.Generator, B: int, lo: int = 4096, hi: int = 131072):
    """Context lengths log-uniform in [lo, hi], rounded to a multiple of 4,
    and 0-3 pending tokens per request."""
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    L = (4 * np.round(np.exp(u) / 4)).astype(np.int64)
    L = np.clip(L, lo, hi)
    p = rng.integers(0, 4, size=B)
    return L, p


def qsa_verify_64req(seed: int = SEEDS["qsa_verify_64req"], B: int = 64, verify_rows: int = 6,
                     lo: int = 4096, hi: int = 131072) -> IndexerInputs:
    """QSA c4 speculative verify: B requests, L log-uniform in [lo, hi] tokens,
    0-3 pending tokens each; 6 query rows per request (1 accepted + 5 drafts)
    at consecutive positions ending at the last context token."""
    rng = np.random.default_rng(seed)
    L, p = verify_lengths(rng, B, lo, hi)
    ctx = [int(L[b] + p[b]) for b in range(B)]
    rows = [[ctx[b] - verify_rows + i for i in range(verify_rows)] for b in range(B)]
    return build_paged_batch("qsa_verify_64req", seed, c=4, k=512,
                             ctx_tokens=ctx, row_pos_per_req=rows, rng=rng)


def dsa_decode_16x80k(seed: int = SEEDS["dsa_decode_16x80k"], B: int = 16, L: int = 81920) -> IndexerInputs:
    """Uncompressed (c = 1) DSA-style decode: B requests x 1 row at L tokens,
    an independent 81920 x 128 key set per request, top-2048 tokens."""
    return build_paged_batch("dsa_decode_16x80k", seed, c=1, k=2048,
                             ctx_tokens=[L] * B, row_pos_per_req=[[L - 1]] * B)


def qsa_prefill_8k(seed: int = SEEDS["qsa_prefill_8k"], rows: int = 8192, ctx: int = 65536) -> IndexerInputs:
    """QSA c4 prefill: 1 request, query rows at the last ``rows`` positions of a
    ``ctx``-token context, causal visibility per row, top-512 blocks."""
    first = ctx - rows
    return build_paged_batch("qsa_prefill_8k", seed, c=4, k=512,
                             ctx_tokens=[ctx], row_pos_per_req=[list(range(first, ctx))])


def qsa_indexshare_64req(seed: int = SEEDS["qsa_indexshare_64req"], B: int = 64,
                         draft_steps: int = INDEXSHARE_DRAFT_STEPS) -> IndexerInputs:
    """IndexShare draft step (QSA page, section IndexShare MTP): B requests
    with contexts drawn as for qsa_verify_64req; one row per request at its
    last accepted token t0 (the draft-extend row whose selection the draft
    loop reuses); the cache also holds the draft_steps + 1 positions drafted
    since, so a draft step at t1 <= t0 + draft_steps + 1 has pages for all of
    them.  k = 512, c = 4."""
    rng = np.random.default_rng(seed)
    L, p = verify_lengths(rng, B)
    t0 = [int(L[b] + p[b]) - 1 for b in range(B)]
    ctx = [t + 1 + draft_steps + 1 for t in t0]
    return build_paged_batch("qsa_indexshare_64req", seed, c=4, k=512,
                             ctx_tokens=ctx, row_pos_per_req=[[t] for t in t0], rng=rng)


def qsa_compress_prefill_8k(seed: int = SEEDS["qsa_compress_prefill_8k"], chunk: int = 8192,
                            ctx: int = 65536) -> CompressInputs:
    """Key compression for the prefill chunk of qsa_prefill_8k: 1 request,
    ``chunk`` new tokens at positions ctx - chunk ... ctx - 1 (2048 complete
    blocks), explicit MRoPE positions with one 64 x 64 image early in the
    context and one 32 x 32 image inside the chunk."""
    first = ctx - chunk
    images = [((ctx // 4, 64), (first + chunk // 4 + 2, 32))]
    return build_compress_batch("qsa_compress_prefill_8k", seed, [first], [chunk], [ctx],
                                images=images)


def qsa_compress_decode_64req(seed: int = SEEDS["qsa_compress_decode_64req"], B: int = 64) -> CompressInputs:
    """Key compression in a decode step: B requests with contexts drawn as for
    qsa_verify_64req, each appending the key of its newest token (about a
    quarter of them complete a block); text positions."""
    rng = np.random.default_rng(seed)
    L, p = verify_lengths(rng, B)
    ctx = [int(L[b] + p[b]) for b in range(B)]
    return build_compress_batch("qsa_compress_decode_64req", seed, [c - 1 for c in ctx], [1] * B, ctx,
                                text_positions=True, rng=rng)


def given_rows_batch(rng: np.random.Generator, ctx, c: int, k: int, row_pos=None,
                     name: str = "given") -> IndexerInputs:
    """A paged batch of one row per request (positions row_pos, default the
    last context token) for selection on given FP32 rows: a seeded page
    permutation, no keys (nothing is scored)."""
    pages = [max(1, -(-t // 64)) for t in ctx]
    perm = rng.permutation(int(sum(pages)))
    pt = np.full((len(ctx), max(pages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[off:off + n]
        off += n
    t = np.array([x - 1 for x in ctx] if row_pos is None else row_pos, dtype=np.int32)
    R = t.size
    return IndexerInputs(name=name, c=c, k=k, q=np.zeros((R, 4, 128), np.uint16),
                         kcache=np.zeros((64 // c, 128), np.uint16), num_pages=int(off), page_table=pt,
                         req_row_ptr=np.arange(R + 1, dtype=np.int32), row_pos=t,
                         max_vis=int(((t.astype(np.int64) + 1) // c).max()), seed=0)


def select_mixed_300rows(seed: int = SEEDS["select_mixed_300rows"], R: int = 300, n_long: int = 16,
                         L: int = 81920, k: int = 2048) -> SelectBatch:
    """A mixed decode batch for the selection alone: 300 rows (one per
    request, c = 1), 16 of them at 81,920 entries and the rest uniform in
    2,000-8,000; FP32 scores ~N(0,1); top-2048 translated through 64-token
    pages."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(2000, 8001, R).astype(np.int32)
    lens[rng.choice(R, n_long, replace=False)] = L
    inp = given_rows_batch(rng, [int(n) + 1 for n in lens], 1, k, name="select_mixed_300rows")
    x = _normal_f32(rng, (R, L))
    return SelectBatch(inp=inp, scores=x, row_len=lens)


WORKLOADS = {
    "qsa_decode_1x8k": qsa_decode_1x8k,
    "topk_8x80k": topk_8x80k,
    "qsa_verify_64req": qsa_verify_64req,
    "dsa_decode_16x80k": dsa_decode_16x80k,
    "qsa_prefill_8k": qsa_prefill_8k,
    "qsa_indexshare_64req": qsa_indexshare_64req,
    "qsa_compress_prefill_8k": qsa_compress_prefill_8k,
    "qsa_compress_decode_64req": qsa_compress_decode_64req,
    "select_mixed_300rows": select_mixed_300rows,
    "topk_1x1m": topk_1x1m,
}


# ----------------------------------------------------------------------------
# Adversarial score rows for top-k tests (not timed).
# ----------------------------------------------------------------------------

def tie_storm_rows(seed: int, rows: int, n: int) -> np.ndarray:
    """A mix of tie-heavy FP32 rows: all equal, a small alphabet, +-0 mixes,
    +-inf, subnormals, FP16-snapped values and values that overflow FP16."""
    rng = np.random.default_rng(seed)
    out = np.empty((rows, n), dtype=np.float32)
    kinds = 8
    for r in range(rows):
        kind = r % kinds
        if kind == 0:
            out[r] = np.float32(0.75)
        elif kind == 1:
            out[r] = rng.choice(np.array([-1.0, 0.5, 2.0], dtype=np.float32), size=n)
        elif kind == 2:
            out[r] = rng.choice(np.array([-0.0, 0.0, 1e-3], dtype=np.float32), size=n)
        elif kind == 3:
            out[r] = rng.choice(np.array([-np.inf, np.inf, 0.0, 1.0], dtype=np.float32), size=n)
        elif kind == 4:
            out[r] = (rng.standard_normal(n).astype(np.float32) * np.float32(1e-40)).astype(np.float32)
        elif kind == 5:
            out[r] = rng.standard_normal(n).astype(np.float16).astype(np.float32)
        elif kind == 6:
            out[r] = (rng.standard_normal(n) * 1e5).astype(np.float32)
        else:
            v = rng.standard_normal(n).astype(np.float32)
            v[rng.random(n) < 0.5] = np.float32(1.0009765625)   # one FP16 bin, many ties
            out[r] = v
    return out
