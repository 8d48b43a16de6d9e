// kernels.h - internal launchers behind the C ABI (host side, validated inputs).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bs {

int launch_score_decode(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                        const int32_t* page_table, int32_t pt_stride,
                        const int32_t* req_row_ptr, int32_t num_req,
                        const int32_t* row_pos, int32_t num_rows,
                        int32_t c, int32_t max_vis,
                        float* scores, int64_t ld, int32_t* row_len, hipStream_t stream);

int launch_score_prefill(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                         const int32_t* page_table, int32_t pt_stride,
                         const int32_t* req_row_ptr, int32_t num_req,
                         const int32_t* row_pos, int32_t num_rows,
                         int32_t c, int32_t max_vis,
                         float* scores, int64_t ld, int32_t* row_len, hipStream_t stream);

size_t topk_workspace_size(int32_t num_rows, int32_t max_len, int32_t k);

int launch_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows,
                int32_t max_len, int32_t k, int32_t* sel, int32_t* sel_count,
                void* workspace, hipStream_t stream);

int launch_select_translate(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows,
                            int32_t max_len, int32_t k, const int32_t* req_row_ptr, int32_t num_req,
                            const int32_t* row_pos, int32_t c, const int32_t* page_table, int32_t pt_stride,
                            int32_t* sel, int32_t* sel_count, int32_t* out_slots, int32_t* out_pos,
                            int32_t* out_count, int32_t ld_out, void* workspace, hipStream_t stream);

// The same with the long-row records in a static device array of
// kNoAllocScratchBytes (per GPU); the caller checks the size first.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
int launch_select_translate_noalloc(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows,
                                    int32_t max_len, int32_t k, const int32_t* req_row_ptr, int32_t num_req,
                                    const int32_t* row_pos, int32_t c, const int32_t* page_table, int32_t pt_stride,
                                    int32_t* sel, int32_t* sel_count, int32_t* out_slots, int32_t* out_pos,
                                    int32_t* out_count, int32_t ld_out, hipStream_t stream);

// Planned selection: the plan's size and the workspace the planned launch
// needs, the planning launch, and the selection driven by a plan.
size_t topk_plan_items(int32_t num_rows, int32_t max_len);
size_t topk_plan_bytes(int32_t num_rows, int32_t max_len);
size_t topk_planned_workspace_size(int32_t num_rows, int32_t max_len, int32_t k);
int launch_topk_plan(const int32_t* row_len, int32_t num_rows, int32_t max_len, int32_t* plan, hipStream_t stream);
int launch_select_translate_planned(const float* scores, int64_t ld, int32_t num_rows, int32_t max_len, int32_t k,
                                    const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos, int32_t c,
                                    const int32_t* page_table, int32_t pt_stride, int32_t* sel, int32_t* sel_count,
                                    int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                                    const int32_t* plan, void* workspace, hipStream_t stream);

// row_pos_now == nullptr: the plain expansion; otherwise the IndexShare one
// (tail through row_pos_now[r], at most max_advance past row_pos[r]).
int launch_expand(const int32_t* sel, const int32_t* sel_count, int32_t k,
                  const int32_t* req_row_ptr, int32_t num_req,
                  const int32_t* row_pos, const int32_t* row_pos_now, int32_t max_advance,
                  int32_t num_rows, int32_t c,
                  const int32_t* page_table, int32_t pt_stride,
                  int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                  int32_t ld_out, hipStream_t stream);

// Key compression into the c = 4 cache; arguments validated by the caller.
int launch_compress(const uint16_t* k_raw, int32_t num_tok, const int32_t* req_tok_ptr, const int32_t* tok_start,
                    const int32_t* mrope_pos, int32_t num_req, int32_t max_tok, int32_t rotary_dim,
                    int32_t sec_t, int32_t sec_h, double theta, uint16_t* ring, int32_t* ring_pos,
                    const int32_t* page_table, int32_t pt_stride, uint16_t* kcache, int64_t num_pages,
                    hipStream_t stream);

}  // namespace bs
