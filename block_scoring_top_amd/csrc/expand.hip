// expand.hip - block -> token expansion, pending append, logical -> physical
// slot translation.
//
// Page "Qwen3.8-Flash-Next Day-0 in SGLang", QSA section: the kept blocks are
// expanded back to their token positions (512 blocks -> 2048 positions for
// c = 4) and the 0-3 tokens of the row's unfinished block are appended.
// GLM-5.2 on SGLang blog, TopK-V2 Figure 2 caption: the logical positions are
// then translated to physical KV-cache slots.  vllm-sparse-mla-blackwell,
// Design notes: -1 is the padding sentinel.
//
// One workgroup per row; lane i writes output entries i, i+256, ...  Each
// output entry is independent, so writes are coalesced and there is no
// cross-lane communication.
#include "device.h"
#include "kernels.h"

namespace bs {

__global__ __launch_bounds__(256) void expand_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int32_t k,
    const int32_t* __restrict__ req_row_ptr, int32_t num_req, const int32_t* __restrict__ row_pos,
    int32_t c, const int32_t* __restrict__ page_table, int32_t pt_stride,
    int32_t* __restrict__ out_slots, int32_t* __restrict__ out_pos, int32_t* __restrict__ out_count,
    int32_t ld_out) {
  const int r = blockIdx.x, tid = threadIdx.x;
  // Request of row r: the last b with req_row_ptr[b] <= r (binary search).
  int lo = 0, hi = num_req;  // invariant: req_row_ptr[lo] <= r < req_row_ptr[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (req_row_ptr[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int t = row_pos[r];
  const int nv = t >= 0 ? (t + 1) / c : 0;
  const int p = t >= 0 ? t + 1 - c * nv : 0;
  const int m = max(0, min(sel_count[r], k));
  const int nblk = c * m;
  const int total = nblk + p;
  const int32_t* pt = page_table + (int64_t)b * pt_stride;
  const int32_t* srow = sel + (int64_t)r * k;
  int32_t* orow = out_slots + (int64_t)r * ld_out;
  int32_t* prow = out_pos ? out_pos + (int64_t)r * ld_out : nullptr;
  for (int i = tid; i < ld_out; i += blockDim.x) {
    int pos = -1;
    if (i < nblk) {
      const int j = srow[i / c];
      pos = (j >= 0 && j < nv) ? c * j + (i - (i / c) * c) : -1;
    } else if (i < total) {
      pos = c * nv + (i - nblk);
    }
    int slot = -1;
    if (pos >= 0 && (pos >> 6) < pt_stride) {
      const int page = pt[pos >> 6];
      slot = page >= 0 ? page * kPage + (pos & (kPage - 1)) : -1;
    }
    orow[i] = slot;
    if (prow) prow[i] = pos;
  }
  if (tid == 0) out_count[r] = total;
}

int launch_expand(const int32_t* sel, const int32_t* sel_count, int32_t k, const int32_t* req_row_ptr,
                  int32_t num_req, const int32_t* row_pos, int32_t num_rows, int32_t c,
                  const int32_t* page_table, int32_t pt_stride, int32_t* out_slots, int32_t* out_pos,
                  int32_t* out_count, int32_t ld_out, hipStream_t stream) {
  hipLaunchKernelGGL(expand_kernel, dim3(num_rows), dim3(256), 0, stream, sel, sel_count, k, req_row_ptr,
                     num_req, row_pos, c, page_table, pt_stride, out_slots, out_pos, out_count, ld_out);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

}  // namespace bs
