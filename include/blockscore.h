/*
 * blockscore.h - C ABI of the MI355X (gfx950) sparse-attention indexer hot path.
 *
 * The path has three steps, each one call:
 *   1. score   - idx_score_decode / idx_score_prefill
 *   2. select  - topk_select_rows
 *   3. expand  - idx_expand_translate
 * plus idx_select_translate (steps 2 and 3 in one kernel),
 * topk_plan_rows + idx_select_translate_planned (the same over a work list
 * built once per step from the row lengths),
 * idx_expand_translate_shared (step 3 for a selection reused across
 * speculative draft steps) and idx_compress_store (the step before 1: raw
 * index keys compressed into the c = 4 key cache).
 *
 * Sources (pages on the subject):
 *   [QSA]   "Qwen3.8-Flash-Next Day-0 in SGLang" (theainews.cc), section on Qwen
 *           sparse attention (QSA): 4 indexer query heads of 128 dims and one
 *           shared key head; one bf16 compressed index key per 4 tokens; the
 *           score equation s_{t,b}; top-512 blocks expanded to 2048 positions
 *           plus the 0-3 tokens of the unfinished block (at most 2051); page-
 *           aligned full_slot/4 addressing of the compressed cache; a paged
 *           version of the same scorer for decode and a custom kernel for
 *           prefill.
 *   [TOPK]  GLM-5.2 on SGLang blog (aihot.virxact.com), Kernel Optimization >
 *           TopK-V2, text and Figures 2-4: top-k as selection rather than sort
 *           over FP32 score rows, runtime k up to 2048, exactly k results,
 *           selected logical positions translated to physical KV-cache slots.
 *   [MASK]  vllm-sparse-mla-blackwell (shadowgraph.io), Design notes: the only
 *           mask downstream is an index >= 0 sentinel, so padding is -1.
 *   [SYNC]  GLM-5.2 blog, Runtime Optimization: the indexer path carries no
 *           device-to-host synchronisation; [QSA]: the metadata path is graph-
 *           compatible and may run on a second stream.
 *
 * Conventions for every call:
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or synchronises; every call is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the default stream) and
 *     returns at once.  Outputs are valid once the stream reaches the call.
 *   - Arguments are validated on the host before anything is launched; on a
 *     failure the call returns a negative bs_status and launches nothing.
 *     HIP launch failures return BS_ERR_LAUNCH.
 *   - num_rows == 0 (or num_req == 0) is a no-op that returns BS_OK.
 *   - Device-resident data (positions, page ids, lengths, selections) is not
 *     read back to the host.  Its preconditions are stated per call; the
 *     kernels clamp every index so that a violation never reads or writes
 *     outside the buffers described by the host-side sizes, but the values
 *     produced for violating rows are then unspecified.
 *   - Calls are thread-safe.  The only library-wide state is the prefill
 *     scorer's resident-workgroups-per-CU figure, computed on first use and
 *     kept in an atomic.  Calls that share a workspace must not overlap in
 *     time (use one stream).
 *
 * Shapes and layouts:
 *   - bf16 values travel as their uint16 bit patterns.
 *   - q:          [num_rows][4][128] bf16, row-major (1 KiB per row).
 *   - kcache:     [num_pages * (64/c)][128] bf16.  Physical page p holds the
 *                 compressed slots p*(64/c) .. p*(64/c) + 64/c - 1.  Block j of
 *                 request b (covering tokens c*j .. c*j+c-1) lives at slot
 *                 page_table[b][(c*j)/64] * (64/c) + j mod (64/c), which is the
 *                 full slot of its first token divided by c [QSA].
 *   - page_table: [num_req][pt_stride] int32, logical 64-token page -> physical
 *                 page id in [0, num_pages); entries past a request's pages
 *                 may hold -1.
 *   - req_row_ptr:[num_req + 1] int32, non-decreasing, req_row_ptr[0] == 0 and
 *                 req_row_ptr[num_req] == num_rows; rows of request b are
 *                 req_row_ptr[b] .. req_row_ptr[b+1]-1.
 *   - row_pos:    [num_rows] int32, the 0-based token position t of each query
 *                 row.  The row sees tokens 0..t; its visible blocks are
 *                 j < n_vis(t) = floor((t+1)/c) and its pending (unfinished
 *                 block) tokens are c*n_vis .. t, 0 to c-1 of them.
 */
#ifndef BLOCKSCORE_H
#define BLOCKSCORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bs_status {
  BS_OK = 0,
  BS_ERR_NULL = -1,      /* a required pointer is NULL */
  BS_ERR_ARG = -2,       /* a size, stride, k or c is out of range */
  BS_ERR_WORKSPACE = -3, /* workspace missing or smaller than topk_workspace_bytes() */
  BS_ERR_LAUNCH = -4     /* the HIP runtime rejected a launch */
};

#define BS_HEADS 4        /* indexer query heads [QSA] */
#define BS_DIM 128        /* head dimension [QSA] */
#define BS_PAGE_TOKENS 64 /* tokens per KV page */
#define BS_KMAX 2048      /* largest runtime k [TOPK] */
#define BS_MAX_ADVANCE 1024 /* largest max_advance of idx_expand_translate_shared */

/*
 * idx_score_decode - paged block scores for decode / speculative-verify rows
 * [QSA: the paged scorer used in decode].
 *
 * For every row r of request b and every visible block j < n_vis(row_pos[r]):
 *   scores[r*ld_scores + j] =
 *       (1/sqrt(128)) * sum_{h=0..3} max(0, <q[r][h][:], kbar_b[j][:]>)
 * with kbar_b[j] read from kcache through the page table (layout above), bf16
 * products accumulated in FP32.  Keys are streamed once per request and scored
 * against all rows of that request.  Entries j >= n_vis(r) are not written.
 *
 *   c          compression ratio, 4 (QSA c4) or 1 (uncompressed, DSA style).
 *   num_pages  physical pages in kcache (page ids outside [0, num_pages) are
 *              not read; the scores of their blocks are unspecified).
 *   max_vis    host-side bound: every row must have n_vis <= max_vis; the
 *              kernels never score past it.  Requires max_vis <= ld_scores and
 *              c*max_vis <= 64*pt_stride.
 *   row_len    optional output [num_rows] int32: min(n_vis(r), max_vis), the
 *              length topk_select_rows takes.  May be NULL.
 * Device preconditions: row_pos[r] >= 0; page ids valid; rows of a request
 * contiguous as given by req_row_ptr.
 * Returns BS_OK, BS_ERR_NULL (q, kcache, page_table, req_row_ptr, row_pos or
 * scores NULL with num_rows > 0), BS_ERR_ARG (c not 1 or 4, negative counts,
 * pt_stride < 1, num_pages < 1, max_vis < 0, ld_scores < max_vis,
 * c*max_vis > 64*pt_stride; idx_score_decode also num_req > 65535, one
 * grid row per request, and max_vis > 65535*4096, the selection's bound on a
 * row) or BS_ERR_LAUNCH.
 */
int idx_score_decode(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                     const int32_t* page_table, int32_t pt_stride,
                     const int32_t* req_row_ptr, int32_t num_req,
                     const int32_t* row_pos, int32_t num_rows,
                     int32_t c, int32_t max_vis,
                     float* scores, int64_t ld_scores, int32_t* row_len,
                     void* stream);

/*
 * idx_score_prefill - the same scores for prefill chunks, computed as a dense
 * bf16 contraction on the matrix cores [QSA: the custom prefill index-score
 * kernel].  Same arguments, layouts, outputs and errors as idx_score_decode;
 * causal visibility per row (entries j >= n_vis(r) are not written).  Suited
 * to requests with many rows; any row count is correct.
 */
int idx_score_prefill(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                      const int32_t* page_table, int32_t pt_stride,
                      const int32_t* req_row_ptr, int32_t num_req,
                      const int32_t* row_pos, int32_t num_rows,
                      int32_t c, int32_t max_vis,
                      float* scores, int64_t ld_scores, int32_t* row_len,
                      void* stream);

/*
 * topk_workspace_bytes - device workspace topk_select_rows needs for
 * (num_rows, max_len, k): num_rows records of 64 KiB blocks (128 KiB per row
 * at max_len = 81,920) when max_len >= 32,769 (rows that long are split over
 * several workgroups), else 0, meaning no workspace is needed (NULL may be
 * passed).  The workspace must be zero-filled before its first use.  Every
 * call leaves the first 4 bytes of every 64 KiB block of it zero again, which
 * is all that a later call relies on (its per-row counters sit there;
 * everything else it reads it writes first), so one zero-fill at allocation
 * suffices, also when later calls use other shapes that fit it.  The rest of
 * its contents between calls is unspecified.
 */
size_t topk_workspace_bytes(int32_t num_rows, int32_t max_len, int32_t k);

/*
 * topk_select_rows - exact top-k per FP32 score row [TOPK].
 *
 * For each row r with n = min(row_len[r], max_len) entries scores[r*ld+0..n-1],
 * selects m = min(k, n) indices: those of the m largest scores, equal scores
 * going to the lower index (-0.0 equals +0.0).  The result is unique.
 *   sel        output [num_rows][k] int32: the m chosen indices in unspecified
 *              order, then -1 padding.
 *   sel_count  output [num_rows] int32: m.
 *   max_len    host-side bound on row_len (capacity); ld_scores >= max_len.
 *   k          1 .. 2048.
 * Method: a selection, not a sort.  FP32 scores are rounded to FP16, mapped
 * to an order-preserving 16-bit key whose upper 10 bits index a 1,024-bin
 * histogram; the bin holding the m-th largest is located, entries in higher
 * bins are emitted directly, and the boundary bin is resolved exactly on the
 * (FP32 key, index) pair by radix selection.  With max_len <= 32,768 every
 * row is done by one workgroup, in registers.  Otherwise a row shorter than
 * 32,769 entries is still done by one workgroup (streamed past 8,192
 * entries), and a longer row is split over one workgroup per 8,192 entries:
 * each keeps the entries at or above the
 * histogram bin of its local q-th largest (q a little above its share of the
 * row's top k) as candidates and publishes them; the last to arrive builds
 * the candidates' histogram, selects the threshold bin and resolves it, after
 * checking that the candidates hold every entry of the row at or above that
 * bin (when they do not, it selects the whole row itself).  The row's own
 * length decides on the device; the host only bounds it by max_len.
 * Device preconditions: row_len[r] >= 0 (negative counts as 0); no NaN
 * (a NaN is ordered above +inf or below -inf by its sign bit).
 * Returns BS_OK, BS_ERR_NULL, BS_ERR_ARG (k outside 1..2048, max_len < 0,
 * ld_scores < max_len), BS_ERR_WORKSPACE or BS_ERR_LAUNCH.
 */
int topk_select_rows(const float* scores, int64_t ld_scores, const int32_t* row_len,
                     int32_t num_rows, int32_t max_len, int32_t k,
                     int32_t* sel, int32_t* sel_count,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_expand_translate - expand chosen blocks to token positions, append the
 * pending tokens and translate to physical KV slots [QSA, TOPK, MASK].
 *
 * For row r of request b at position t with m = min(max(sel_count[r], 0), k):
 *   each chosen block j = sel[r*k + i] (i < m) becomes positions
 *   c*j .. c*j+c-1 (in that order, blocks in the order given), then the
 *   pending positions c*n_vis(t) .. t follow; out_count[r] = c*m + p.
 *   out_slots[r*ld_out + i] = page_table[b][pos/64] * 64 + pos mod 64.
 *   out_pos (optional, may be NULL) receives the logical positions.
 *   Entries past out_count[r] are -1.  A chosen index outside [0, n_vis) or a
 *   position whose page entry is negative yields -1 in its place.
 *   ld_out >= k*c + c - 1 (2051 for c = 4, k = 512).
 * Returns BS_OK, BS_ERR_NULL, BS_ERR_ARG (k outside 1..2048, c not 1 or 4,
 * ld_out too small, negative counts, pt_stride < 1, num_req == 0 while
 * num_rows > 0) or BS_ERR_LAUNCH.
 */
int idx_expand_translate(const int32_t* sel, const int32_t* sel_count, int32_t k,
                         const int32_t* req_row_ptr, int32_t num_req,
                         const int32_t* row_pos, int32_t num_rows, int32_t c,
                         const int32_t* page_table, int32_t pt_stride,
                         int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                         int32_t ld_out, void* stream);

/*
 * idx_expand_translate_shared - the expansion of a selection reused across
 * speculative draft steps [QSA, section IndexShare MTP: the selection made
 * for a request's last accepted row at draft-extend is kept for the whole
 * draft loop, and at each lookup the positions drafted since are appended so
 * that the draft still sees its own in-progress tokens].
 *
 * For row r of request b the selection sel/sel_count was made at position
 * t0 = row_pos[r]; the row is now at t1 = row_pos_now[r], t0 <= t1 <= t0 +
 * max_advance.  Output as idx_expand_translate for t0, except that the tail
 * runs through t1: chosen blocks become c*j .. c*j+c-1, then positions
 * c*n_vis(t0) .. t1 follow; out_count[r] = c*m + t1 + 1 - c*n_vis(t0).  With
 * t1 = t0 the output equals idx_expand_translate's.  out_pos may be NULL.
 * Positions whose page entry is negative or past pt_stride yield -1.
 *   max_advance  0 .. BS_MAX_ADVANCE (draft steps + 1, say).
 *   ld_out       >= k*c + c - 1 + max_advance.
 * Device precondition: t0 <= t1 <= t0 + max_advance (t1 is clamped into that
 * range otherwise).
 * Returns BS_OK, BS_ERR_NULL, BS_ERR_ARG (k outside 1..2048, c not 1 or 4,
 * max_advance out of range, ld_out too small, negative counts, pt_stride < 1,
 * num_req == 0 while num_rows > 0) or BS_ERR_LAUNCH.
 */
int idx_expand_translate_shared(const int32_t* sel, const int32_t* sel_count, int32_t k,
                                const int32_t* req_row_ptr, int32_t num_req,
                                const int32_t* row_pos, const int32_t* row_pos_now, int32_t num_rows,
                                int32_t c, int32_t max_advance,
                                const int32_t* page_table, int32_t pt_stride,
                                int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                                int32_t ld_out, void* stream);

/*
 * idx_select_translate - topk_select_rows and idx_expand_translate in one
 * kernel [TOPK: the selection and the page-table transform fused to cut
 * latency; QSA: expansion and pending append].
 *
 * Same selection as topk_select_rows (same arguments, workspace and
 * guarantees for scores .. sel_count) and, for each row, the same expansion,
 * append and translation of that selection as idx_expand_translate (same
 * arguments and guarantees for req_row_ptr .. ld_out); the slots follow the
 * order of the row's entries in sel.  Errors: the union of both calls'.
 */
int idx_select_translate(const float* scores, int64_t ld_scores, const int32_t* row_len,
                         int32_t num_rows, int32_t max_len, int32_t k,
                         const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos, int32_t c,
                         const int32_t* page_table, int32_t pt_stride,
                         int32_t* sel, int32_t* sel_count,
                         int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_select_translate_noalloc - idx_select_translate for callers that cannot
 * allocate device memory: code under HIP graph capture that must not
 * allocate, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, outputs, guarantees and errors as idx_select_translate,
 * without the workspace: the long-row records (rows of >= 32,769 entries)
 * live in a static device array of BS_NOALLOC_SCRATCH_BYTES per GPU, which
 * the library holds until the process ends.  A call whose
 * topk_workspace_bytes(num_rows, max_len, k) exceeds that size returns
 * BS_ERR_WORKSPACE and launches nothing (128 KiB per row at
 * max_len = 81,920, k = 2048: up to 64 such rows).  The call allocates and
 * frees nothing; its first call on a device looks the array's address up
 * (hipGetSymbolAddress) and keeps it.  The array is zero when the library is
 * loaded, and every call leaves it as topk_select_rows leaves a workspace
 * (the first word of every 64 KiB block zero), which is all the next call
 * needs.  All calls on one GPU share its array: calls that overlap in
 * time on one GPU (concurrent streams, threads) race and must not be made.
 */
#define BS_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int idx_select_translate_noalloc(const float* scores, int64_t ld_scores, const int32_t* row_len,
                                 int32_t num_rows, int32_t max_len, int32_t k,
                                 const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos, int32_t c,
                                 const int32_t* page_table, int32_t pt_stride,
                                 int32_t* sel, int32_t* sel_count,
                                 int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                                 void* stream);

/*
 * Planned selection [TOPK: a planning kernel reads the batch's length
 * distribution, picks the length from which rows are split over several
 * workgroups, and builds a work list that serves every DSA layer of the
 * forward pass].
 *
 * topk_plan_bytes - bytes of a plan for (num_rows, max_len): 32 + 16 per
 * work-list slot, one slot per row, or ceil(max_len / 8,192) per row when
 * max_len >= 16,385.  0 for num_rows <= 0.
 *
 * topk_planned_workspace_bytes - the workspace idx_select_translate_planned
 * needs: records as described at topk_workspace_bytes, sized for rows split
 * from 16,385 entries on, when max_len >= 16,385; else 0 (none needed).  The
 * same zero-fill-once contract: every call leaves the first 4 bytes of every
 * 64 KiB block zero.
 *
 * topk_plan_rows - one single-workgroup kernel that reads row_len[0 ..
 * num_rows-1] (clamped to 0 .. max_len) and writes the plan into `plan`
 * (device memory of at least topk_plan_bytes, owned by the caller; its
 * contents are internal).  The split length is 16,385 when the items that it
 * gives fit on the device at once (compute units times the selection's
 * resident workgroups per unit), else 32,769.  Every row shorter than the
 * split length is one item selected whole by one workgroup; a longer one is
 * one item per 8,192-entry chunk, resolved as in topk_select_rows.  The
 * chunk items come first in the list, so split rows start first.  The plan
 * depends on the lengths and max_len only (not on k, the scores or the
 * translation), so it is built once per step and passed to every
 * selection of that step.  Returns BS_OK, BS_ERR_NULL, BS_ERR_ARG (negative
 * counts, max_len > 65535*4096, more than 2^22 slots), BS_ERR_WORKSPACE
 * (plan_bytes too small) or BS_ERR_LAUNCH.
 *
 * idx_select_translate_planned - idx_select_translate with the row lengths
 * taken from a plan: same outputs and guarantees, for rows of the lengths
 * the plan was built from (row_len is not read).  It launches one workgroup
 * per plan slot; slots past the plan's item count exit at once, and rows
 * are never read past their length.  The plan must have been built on the
 * same stream (or be ordered before this call) by topk_plan_rows with the
 * same num_rows and max_len; a plan built from other lengths selects over
 * those lengths (the kernel still stays inside every buffer).  workspace: at
 * least topk_planned_workspace_bytes, zero-filled once (see above).
 * Errors: as idx_select_translate, plus BS_ERR_NULL for a NULL plan and
 * BS_ERR_WORKSPACE for plan_bytes < topk_plan_bytes(num_rows, max_len).
 */
size_t topk_plan_bytes(int32_t num_rows, int32_t max_len);
size_t topk_planned_workspace_bytes(int32_t num_rows, int32_t max_len, int32_t k);
int topk_plan_rows(const int32_t* row_len, int32_t num_rows, int32_t max_len, int32_t* plan, size_t plan_bytes,
                   void* stream);
int idx_select_translate_planned(const float* scores, int64_t ld_scores, int32_t num_rows, int32_t max_len,
                                 int32_t k, const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos,
                                 int32_t c, const int32_t* page_table, int32_t pt_stride,
                                 int32_t* sel, int32_t* sel_count,
                                 int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                                 const int32_t* plan, size_t plan_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * idx_compress_store - compression of new raw index keys into the c = 4 key
 * cache the scorers read [QSA: the indexer's one shared key head; each 4 raw
 * index keys are averaged in FP32, normalised and rotated with the MRoPE
 * position of their first token into one bf16 compressed key; the raw keys
 * of a request's unfinished block wait in a 4-slot ring; page-aligned
 * full_slot/4 addressing].
 *
 * Request b appends tokens req_tok_ptr[b] .. req_tok_ptr[b+1]-1 of k_raw at
 * consecutive positions tok_start[b], tok_start[b]+1, ...  The result is that
 * of taking the tokens in position order: the token at position p is written
 * to ring slot p mod 4 (and, when p mod 4 == 0, its MRoPE position to
 * ring_pos[b]); when p mod 4 == 3 the ring's 4 keys form block j = p/4:
 *   mean = ((k0 + k1) + k2) + k3 in FP32, times 0.25;
 *   y    = mean / ||mean||_2 (a zero mean gives zeros);
 *   rotate-half over the first rotary_dim dims: pair i < rotary_dim/2 joins
 *        dims i and i + rotary_dim/2 and turns by P * theta^(-2i/rotary_dim),
 *        P being the t, h or w component of the block position for i in the
 *        first sec_t, the next sec_h or the last sec_w pairs; other dims pass;
 *   the result, rounded to bf16 (nearest even), is stored at compressed slot
 *        page_table[b][(4j)/64] * 16 + j mod 16 (kcache layout above, c = 4).
 * The block position is the MRoPE position of token 4j (ring_pos[b] when that
 * token came in an earlier call).  Normalisation and rotation run in FP32 with
 * FP64 angles: each element is within 2^-17 of the exact value of these steps
 * before its bf16 rounding.
 *
 *   k_raw        [num_tok][128] bf16, the new raw keys.
 *   req_tok_ptr  [num_req + 1] int32, non-decreasing, last entry <= num_tok.
 *   tok_start    [num_req] int32 >= 0, position of each request's first new
 *                token; the ring must hold that request's tokens
 *                4*floor(tok_start/4) .. tok_start-1 from earlier calls.
 *   mrope_pos    [num_tok][3] int32 (t, h, w) of each new token, or NULL for
 *                text positions (t = h = w = the token position).
 *   max_tok      host-side bound on the new tokens of any request (sizes the
 *                grid; a request with more is cut to max_tok), <= num_tok.
 *   rotary_dim   0 .. 128, even; sec_t + sec_h + sec_w == rotary_dim / 2.
 *   theta        rotary base, finite and > 0.
 *   ring         [num_req][4][128] bf16, read and written.
 *   ring_pos     [num_req][3] int32, read and written; required when
 *                mrope_pos is given, may be NULL otherwise.
 *   page_table   as above; kcache [num_pages * 16][128] bf16, written only at
 *                the slots of completed blocks whose page id is in range.
 * Calls that share a ring or cache entries must not overlap in time.
 * Returns BS_OK (also when num_req, num_tok or max_tok is 0), BS_ERR_NULL,
 * BS_ERR_ARG (negative counts, num_req > 65535, max_tok > num_tok, bad
 * rotary_dim, sections or theta, pt_stride < 1, num_pages < 1) or
 * BS_ERR_LAUNCH.
 */
int idx_compress_store(const uint16_t* k_raw, int32_t num_tok, const int32_t* req_tok_ptr,
                       const int32_t* tok_start, const int32_t* mrope_pos, int32_t num_req, int32_t max_tok,
                       int32_t rotary_dim, int32_t sec_t, int32_t sec_h, int32_t sec_w, double theta,
                       uint16_t* ring, int32_t* ring_pos,
                       const int32_t* page_table, int32_t pt_stride, uint16_t* kcache, int64_t num_pages,
                       void* stream);

/* bs_status_string - a static, human-readable name for a status code. */
const char* bs_status_string(int status);

/* bs_abi_version - version of this ABI (1). */
int bs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKSCORE_H */
