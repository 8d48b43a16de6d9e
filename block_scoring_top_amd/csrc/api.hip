// api.hip - the extern "C" entry points: host-side validation, then launch.
//
// Nothing here allocates, frees or synchronises.  Every check below runs on
// host-side values only; device data is never read back.
#include <cmath>

#include "../../include/blockscore.h"
#include "kernels.h"

static_assert(BS_NOALLOC_SCRATCH_BYTES == bs::kNoAllocScratchBytes, "the header states the scratch size");

#define BS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

inline int check_score_args(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                            const int32_t* page_table, int32_t pt_stride, const int32_t* req_row_ptr,
                            int32_t num_req, const int32_t* row_pos, int32_t num_rows, int32_t c,
                            int32_t max_vis, const float* scores, int64_t ld_scores) {
  if (num_rows < 0 || num_req < 0 || max_vis < 0 || num_pages < 0) return BS_ERR_ARG;
  if (c != 1 && c != 4) return BS_ERR_ARG;
  if (num_rows == 0 || num_req == 0) return BS_OK;
  if (!q || !kcache || !page_table || !req_row_ptr || !row_pos || !scores) return BS_ERR_NULL;
  if (pt_stride < 1 || num_pages < 1 || ld_scores < (int64_t)max_vis) return BS_ERR_ARG;
  if ((int64_t)c * max_vis > (int64_t)BS_PAGE_TOKENS * pt_stride) return BS_ERR_ARG;
  return BS_OK;
}

}  // namespace

BS_EXPORT int idx_score_decode(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                               const int32_t* page_table, int32_t pt_stride,
                               const int32_t* req_row_ptr, int32_t num_req,
                               const int32_t* row_pos, int32_t num_rows,
                               int32_t c, int32_t max_vis,
                               float* scores, int64_t ld_scores, int32_t* row_len, void* stream) {
  const int st = check_score_args(q, kcache, num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos,
                                  num_rows, c, max_vis, scores, ld_scores);
  if (st != BS_OK || num_rows == 0 || num_req == 0) return st;
  if (num_req > 65535) return BS_ERR_ARG;  // one grid row per request
  // a row's scores are addressed through a buffer of 32-bit byte range; the
  // same bound as the selection's rows
  if ((int64_t)max_vis > (int64_t)65535 * 4096) return BS_ERR_ARG;
  return bs::launch_score_decode(q, kcache, num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos,
                                 num_rows, c, max_vis, scores, ld_scores, row_len,
                                 static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_score_prefill(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                                const int32_t* page_table, int32_t pt_stride,
                                const int32_t* req_row_ptr, int32_t num_req,
                                const int32_t* row_pos, int32_t num_rows,
                                int32_t c, int32_t max_vis,
                                float* scores, int64_t ld_scores, int32_t* row_len, void* stream) {
  const int st = check_score_args(q, kcache, num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos,
                                  num_rows, c, max_vis, scores, ld_scores);
  if (st != BS_OK || num_rows == 0 || num_req == 0) return st;
  return bs::launch_score_prefill(q, kcache, num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos,
                                  num_rows, c, max_vis, scores, ld_scores, row_len,
                                  static_cast<hipStream_t>(stream));
}

BS_EXPORT size_t topk_workspace_bytes(int32_t num_rows, int32_t max_len, int32_t k) {
  if (num_rows <= 0 || max_len <= 0) return 0;
  return bs::topk_workspace_size(num_rows, max_len, k);
}

BS_EXPORT int topk_select_rows(const float* scores, int64_t ld_scores, const int32_t* row_len,
                               int32_t num_rows, int32_t max_len, int32_t k,
                               int32_t* sel, int32_t* sel_count,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (num_rows < 0 || max_len < 0 || k < 1 || k > BS_KMAX) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (!scores || !row_len || !sel || !sel_count) return BS_ERR_NULL;
  if (ld_scores < (int64_t)max_len) return BS_ERR_ARG;
  if ((int64_t)max_len > (int64_t)65535 * 4096) return BS_ERR_ARG;  // grid y limit
  const size_t need = bs::topk_workspace_size(num_rows, max_len, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return BS_ERR_WORKSPACE;
  return bs::launch_topk(scores, ld_scores, row_len, num_rows, max_len, k, sel, sel_count, workspace,
                         static_cast<hipStream_t>(stream));
}

BS_EXPORT size_t topk_plan_bytes(int32_t num_rows, int32_t max_len) {
  if (num_rows <= 0 || max_len < 0) return 0;
  return bs::topk_plan_bytes(num_rows, max_len);
}

BS_EXPORT size_t topk_planned_workspace_bytes(int32_t num_rows, int32_t max_len, int32_t k) {
  if (num_rows <= 0 || max_len <= 0) return 0;
  return bs::topk_planned_workspace_size(num_rows, max_len, k);
}

namespace {
// The planned selection launches one 512-lane workgroup per plan slot (at
// most 2^22 slots keeps the grid under 2^31 lanes) and addresses a row with a
// buffer of 32-bit byte range.
inline bool plan_shape_ok(int32_t num_rows, int32_t max_len) {
  return (int64_t)max_len <= (int64_t)65535 * 4096 && bs::topk_plan_items(num_rows, max_len) <= ((size_t)1 << 22);
}
}  // namespace

BS_EXPORT int topk_plan_rows(const int32_t* row_len, int32_t num_rows, int32_t max_len, int32_t* plan,
                             size_t plan_bytes, void* stream) {
  if (num_rows < 0 || max_len < 0) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (!row_len || !plan) return BS_ERR_NULL;
  if (!plan_shape_ok(num_rows, max_len)) return BS_ERR_ARG;
  if (plan_bytes < bs::topk_plan_bytes(num_rows, max_len)) return BS_ERR_WORKSPACE;
  return bs::launch_topk_plan(row_len, num_rows, max_len, plan, static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_select_translate_planned(const float* scores, int64_t ld_scores, int32_t num_rows, int32_t max_len,
                                           int32_t k, const int32_t* req_row_ptr, int32_t num_req,
                                           const int32_t* row_pos, int32_t c, const int32_t* page_table,
                                           int32_t pt_stride, int32_t* sel, int32_t* sel_count, int32_t* out_slots,
                                           int32_t* out_pos, int32_t* out_count, int32_t ld_out, const int32_t* plan,
                                           size_t plan_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_rows < 0 || num_req < 0 || max_len < 0 || k < 1 || k > BS_KMAX) return BS_ERR_ARG;
  if (c != 1 && c != 4) return BS_ERR_ARG;
  if ((int64_t)ld_out < (int64_t)k * c + c - 1) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (num_req == 0) return BS_ERR_ARG;
  if (!scores || !plan || !sel || !sel_count || !req_row_ptr || !row_pos || !page_table || !out_slots || !out_count)
    return BS_ERR_NULL;
  if (ld_scores < (int64_t)max_len || pt_stride < 1) return BS_ERR_ARG;
  if (!plan_shape_ok(num_rows, max_len)) return BS_ERR_ARG;
  if (plan_bytes < bs::topk_plan_bytes(num_rows, max_len)) return BS_ERR_WORKSPACE;
  const size_t need = bs::topk_planned_workspace_size(num_rows, max_len, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return BS_ERR_WORKSPACE;
  return bs::launch_select_translate_planned(scores, ld_scores, num_rows, max_len, k, req_row_ptr, num_req, row_pos, c,
                                             page_table, pt_stride, sel, sel_count, out_slots, out_pos, out_count,
                                             ld_out, plan, workspace, static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_expand_translate(const int32_t* sel, const int32_t* sel_count, int32_t k,
                                   const int32_t* req_row_ptr, int32_t num_req,
                                   const int32_t* row_pos, int32_t num_rows, int32_t c,
                                   const int32_t* page_table, int32_t pt_stride,
                                   int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                                   int32_t ld_out, void* stream) {
  if (num_rows < 0 || num_req < 0 || k < 1 || k > BS_KMAX) return BS_ERR_ARG;
  if (c != 1 && c != 4) return BS_ERR_ARG;
  if ((int64_t)ld_out < (int64_t)k * c + c - 1) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (num_req == 0) return BS_ERR_ARG;  // rows need a request
  if (!sel || !sel_count || !req_row_ptr || !row_pos || !page_table || !out_slots || !out_count)
    return BS_ERR_NULL;
  if (pt_stride < 1) return BS_ERR_ARG;
  return bs::launch_expand(sel, sel_count, k, req_row_ptr, num_req, row_pos, nullptr, 0, num_rows, c, page_table,
                           pt_stride, out_slots, out_pos, out_count, ld_out, static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_expand_translate_shared(const int32_t* sel, const int32_t* sel_count, int32_t k,
                                          const int32_t* req_row_ptr, int32_t num_req,
                                          const int32_t* row_pos, const int32_t* row_pos_now, int32_t num_rows,
                                          int32_t c, int32_t max_advance,
                                          const int32_t* page_table, int32_t pt_stride,
                                          int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                                          int32_t ld_out, void* stream) {
  if (num_rows < 0 || num_req < 0 || k < 1 || k > BS_KMAX) return BS_ERR_ARG;
  if (c != 1 && c != 4) return BS_ERR_ARG;
  if (max_advance < 0 || max_advance > BS_MAX_ADVANCE) return BS_ERR_ARG;
  if ((int64_t)ld_out < (int64_t)k * c + c - 1 + max_advance) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (num_req == 0) return BS_ERR_ARG;  // rows need a request
  if (!sel || !sel_count || !req_row_ptr || !row_pos || !row_pos_now || !page_table || !out_slots || !out_count)
    return BS_ERR_NULL;
  if (pt_stride < 1) return BS_ERR_ARG;
  return bs::launch_expand(sel, sel_count, k, req_row_ptr, num_req, row_pos, row_pos_now, max_advance, num_rows, c,
                           page_table, pt_stride, out_slots, out_pos, out_count, ld_out,
                           static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_select_translate(const float* scores, int64_t ld_scores, const int32_t* row_len,
                                   int32_t num_rows, int32_t max_len, int32_t k,
                                   const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos, int32_t c,
                                   const int32_t* page_table, int32_t pt_stride,
                                   int32_t* sel, int32_t* sel_count,
                                   int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (num_rows < 0 || num_req < 0 || max_len < 0 || k < 1 || k > BS_KMAX) return BS_ERR_ARG;
  if (c != 1 && c != 4) return BS_ERR_ARG;
  if ((int64_t)ld_out < (int64_t)k * c + c - 1) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (num_req == 0) return BS_ERR_ARG;
  if (!scores || !row_len || !sel || !sel_count || !req_row_ptr || !row_pos || !page_table || !out_slots ||
      !out_count)
    return BS_ERR_NULL;
  if (ld_scores < (int64_t)max_len || pt_stride < 1) return BS_ERR_ARG;
  if ((int64_t)max_len > (int64_t)65535 * 4096) return BS_ERR_ARG;  // grid y limit
  const size_t need = bs::topk_workspace_size(num_rows, max_len, k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return BS_ERR_WORKSPACE;
  return bs::launch_select_translate(scores, ld_scores, row_len, num_rows, max_len, k, req_row_ptr, num_req,
                                     row_pos, c, page_table, pt_stride, sel, sel_count, out_slots, out_pos,
                                     out_count, ld_out, workspace, static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_select_translate_noalloc(const float* scores, int64_t ld_scores, const int32_t* row_len,
                                           int32_t num_rows, int32_t max_len, int32_t k,
                                           const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos,
                                           int32_t c, const int32_t* page_table, int32_t pt_stride,
                                           int32_t* sel, int32_t* sel_count,
                                           int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                                           void* stream) {
  if (num_rows < 0 || num_req < 0 || max_len < 0 || k < 1 || k > BS_KMAX) return BS_ERR_ARG;
  if (c != 1 && c != 4) return BS_ERR_ARG;
  if ((int64_t)ld_out < (int64_t)k * c + c - 1) return BS_ERR_ARG;
  if (num_rows == 0) return BS_OK;
  if (num_req == 0) return BS_ERR_ARG;
  if (!scores || !row_len || !sel || !sel_count || !req_row_ptr || !row_pos || !page_table || !out_slots ||
      !out_count)
    return BS_ERR_NULL;
  if (ld_scores < (int64_t)max_len || pt_stride < 1) return BS_ERR_ARG;
  if ((int64_t)max_len > (int64_t)65535 * 4096) return BS_ERR_ARG;  // grid y limit
  if (bs::topk_workspace_size(num_rows, max_len, k) > BS_NOALLOC_SCRATCH_BYTES) return BS_ERR_WORKSPACE;
  return bs::launch_select_translate_noalloc(scores, ld_scores, row_len, num_rows, max_len, k, req_row_ptr, num_req,
                                             row_pos, c, page_table, pt_stride, sel, sel_count, out_slots, out_pos,
                                             out_count, ld_out, static_cast<hipStream_t>(stream));
}

BS_EXPORT int idx_compress_store(const uint16_t* k_raw, int32_t num_tok, const int32_t* req_tok_ptr,
                                 const int32_t* tok_start, const int32_t* mrope_pos, int32_t num_req,
                                 int32_t max_tok, int32_t rotary_dim, int32_t sec_t, int32_t sec_h, int32_t sec_w,
                                 double theta, uint16_t* ring, int32_t* ring_pos, const int32_t* page_table,
                                 int32_t pt_stride, uint16_t* kcache, int64_t num_pages, void* stream) {
  if (num_req < 0 || num_tok < 0 || max_tok < 0 || num_pages < 0 || num_req > 65535) return BS_ERR_ARG;
  if (max_tok > num_tok) return BS_ERR_ARG;
  if (rotary_dim < 0 || rotary_dim > BS_DIM || (rotary_dim & 1)) return BS_ERR_ARG;
  if (sec_t < 0 || sec_h < 0 || sec_w < 0 || sec_t + sec_h + sec_w != rotary_dim / 2) return BS_ERR_ARG;
  if (!(theta > 0.0) || !std::isfinite(theta)) return BS_ERR_ARG;
  if (num_req == 0 || num_tok == 0 || max_tok == 0) return BS_OK;
  if (!k_raw || !req_tok_ptr || !tok_start || !ring || !page_table || !kcache) return BS_ERR_NULL;
  if (mrope_pos && !ring_pos) return BS_ERR_NULL;
  if (pt_stride < 1 || num_pages < 1) return BS_ERR_ARG;
  return bs::launch_compress(k_raw, num_tok, req_tok_ptr, tok_start, mrope_pos, num_req, max_tok, rotary_dim,
                             sec_t, sec_h, theta, ring, ring_pos, page_table, pt_stride, kcache, num_pages,
                             static_cast<hipStream_t>(stream));
}

BS_EXPORT const char* bs_status_string(int status) {
  switch (status) {
    case BS_OK: return "BS_OK";
    case BS_ERR_NULL: return "BS_ERR_NULL: a required pointer is NULL";
    case BS_ERR_ARG: return "BS_ERR_ARG: a size, stride, k or c is out of range";
    case BS_ERR_WORKSPACE:
      return "BS_ERR_WORKSPACE: workspace missing or too small (idx_select_translate_noalloc: the call needs more "
             "than its static scratch of BS_NOALLOC_SCRATCH_BYTES)";
    case BS_ERR_LAUNCH: return "BS_ERR_LAUNCH: the HIP runtime rejected a launch";
    default: return "unknown status";
  }
}

BS_EXPORT int bs_abi_version(void) { return 1; }
