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
// IndexShare (same QSA page, section IndexShare MTP): a selection captured
// for a row at position t0 is reused while the row advances; at position t1
// the tail holds the captured pending tokens and every position drafted
// since, c*n_vis(t0) .. t1 (row_pos_now != nullptr; t1 is clamped to
// [t0, t0 + max_advance]).
//
// Two kernels:
//   * batches of many rows (prefill): one workgroup per row.  The row's
//     selection and the page ids of its first 2,048 logical pages (every
//     position of the row lies at or before its tail end) are read into LDS
//     with coalesced loads, all issued at once; then each lane writes output
//     entries tid, tid + 256, ... (every store instruction covers 256
//     contiguous bytes) from LDS alone.  A row whose pages are not all
//     cached takes a separate path that may read page ids from global
//     memory: sharing one path would put a wait for global loads (which also
//     waits for all earlier stores, as vector memory operations retire in
//     order) before every store;
//   * few rows: one lane per output entry (a row spans ld_out / 256
//     workgroups), each lane a short chain of dependent loads (selection ->
//     page table) and one coalesced store.  With few rows this spreads the
//     work over more of the chip, and measured faster.
#include "device.h"
#include "kernels.h"

namespace bs {

constexpr int kExpandNT = 256;
constexpr int kExpandPages = 2048;
constexpr int kExpandRowsMin = 1024;  // batches with at least this many rows use the row kernel

template <bool CACHED>
__device__ __forceinline__ void expand_entries(const int32_t* s_sel, const int32_t* s_pages, int np,
                                               const int32_t* __restrict__ pt, int32_t pt_stride, int c, int nv,
                                               int nblk, int total, int32_t* __restrict__ orow,
                                               int32_t* __restrict__ prow, int32_t ld_out) {
  for (int i = (int)threadIdx.x; i < ld_out; i += kExpandNT) {
    int pos = -1;
    if (i < nblk) {
      const int q = i / c;
      const int j = s_sel[q];
      pos = (j >= 0 && j < nv) ? c * j + (i - q * c) : -1;
    } else if (i < total) {
      pos = c * nv + (i - nblk);
    }
    int slot = -1;
    if (pos >= 0) {
      const int lp = pos >> 6;
      int page = -1;
      if (CACHED) page = s_pages[lp];
      else if (lp < pt_stride) page = lp < np ? s_pages[lp] : pt[lp];
      slot = page >= 0 ? page * kPage + (pos & (kPage - 1)) : -1;
    }
    orow[i] = slot;
    if (prow) prow[i] = pos;
  }
}

__global__ __launch_bounds__(kExpandNT) void expand_row_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int32_t k,
    const int32_t* __restrict__ req_row_ptr, int32_t num_req, const int32_t* __restrict__ row_pos,
    const int32_t* __restrict__ row_pos_now, int32_t max_advance,
    int32_t c, const int32_t* __restrict__ page_table, int32_t pt_stride,
    int32_t* __restrict__ out_slots, int32_t* __restrict__ out_pos, int32_t* __restrict__ out_count,
    int32_t ld_out) {
  __shared__ int32_t s_sel[kKmax];
  __shared__ int32_t s_pages[kExpandPages];
  const int r = blockIdx.x, tid = threadIdx.x;
  // Request of row r: the number of requests starting at or before r, minus
  // one.  Each lane tests one request boundary; a ballot counts them.
  int b = -1;
  for (int base = 0; base < num_req; base += 64) {
    const int bi = base + (tid & 63);
    const bool started = bi < num_req && req_row_ptr[bi] <= r;
    b += __popcll(__ballot(started));
  }
  b = max(0, min(b, num_req - 1));
  const int t = row_pos[r];
  const int nv = t >= 0 ? (t + 1) / c : 0;
  const int te = (row_pos_now != nullptr && t >= 0) ? min(max(row_pos_now[r], t), t + max_advance) : t;
  const int p = t >= 0 ? te + 1 - c * nv : 0;  // the tail c*nv .. te
  const int m = max(0, min(sel_count[r], k));
  const int nblk = c * m;
  const int total = nblk + p;
  const int np = t >= 0 ? min((te >> 6) + 1, min(kExpandPages, pt_stride)) : 0;
  const int32_t* pt = page_table + (int64_t)b * pt_stride;
  const int32_t* srow = sel + (int64_t)r * k;
  for (int i = tid; i < m; i += kExpandNT) s_sel[i] = srow[i];
  for (int i = tid; i < np; i += kExpandNT) s_pages[i] = pt[i];
  __syncthreads();
  int32_t* orow = out_slots + (int64_t)r * ld_out;
  int32_t* prow = out_pos ? out_pos + (int64_t)r * ld_out : nullptr;
  if (t >= 0 && (te >> 6) < np)
    expand_entries<true>(s_sel, s_pages, np, pt, pt_stride, c, nv, nblk, total, orow, prow, ld_out);
  else
    expand_entries<false>(s_sel, s_pages, np, pt, pt_stride, c, nv, nblk, total, orow, prow, ld_out);
  if (tid == 0) out_count[r] = total;
}

__global__ __launch_bounds__(256) void expand_entry_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int32_t k,
    const int32_t* __restrict__ req_row_ptr, int32_t num_req, const int32_t* __restrict__ row_pos,
    const int32_t* __restrict__ row_pos_now, int32_t max_advance,
    int32_t c, const int32_t* __restrict__ page_table, int32_t pt_stride,
    int32_t* __restrict__ out_slots, int32_t* __restrict__ out_pos, int32_t* __restrict__ out_count,
    int32_t ld_out) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int i = blockIdx.y * blockDim.x + tid;  // one output entry per lane
  // Request of row r: the number of requests starting at or before r, minus
  // one.  Each lane tests one request boundary; a ballot counts them.
  int b = -1;
  for (int base = 0; base < num_req; base += 64) {
    const int bi = base + (tid & 63);
    const bool started = bi < num_req && req_row_ptr[bi] <= r;
    b += __popcll(__ballot(started));
  }
  b = max(0, min(b, num_req - 1));
  const int t = row_pos[r];
  const int nv = t >= 0 ? (t + 1) / c : 0;
  const int te = (row_pos_now != nullptr && t >= 0) ? min(max(row_pos_now[r], t), t + max_advance) : t;
  const int p = t >= 0 ? te + 1 - c * nv : 0;  // the tail c*nv .. te
  const int m = max(0, min(sel_count[r], k));
  const int nblk = c * m;
  const int total = nblk + p;
  if (i >= ld_out) return;
  int pos = -1;
  if (i < nblk) {
    const int q = i / c;
    const int j = sel[(int64_t)r * k + q];
    pos = (j >= 0 && j < nv) ? c * j + (i - q * c) : -1;
  } else if (i < total) {
    pos = c * nv + (i - nblk);
  }
  int slot = -1;
  if (pos >= 0 && (pos >> 6) < pt_stride) {
    const int page = page_table[(int64_t)b * pt_stride + (pos >> 6)];
    slot = page >= 0 ? page * kPage + (pos & (kPage - 1)) : -1;
  }
  out_slots[(int64_t)r * ld_out + i] = slot;
  if (out_pos) out_pos[(int64_t)r * ld_out + i] = pos;
  if (i == 0) out_count[r] = total;
}

int launch_expand(const int32_t* sel, const int32_t* sel_count, int32_t k, const int32_t* req_row_ptr,
                  int32_t num_req, const int32_t* row_pos, const int32_t* row_pos_now, int32_t max_advance,
                  int32_t num_rows, int32_t c, const int32_t* page_table, int32_t pt_stride, int32_t* out_slots,
                  int32_t* out_pos, int32_t* out_count, int32_t ld_out, hipStream_t stream) {
  if (num_rows >= kExpandRowsMin) {
    hipLaunchKernelGGL(expand_row_kernel, dim3(num_rows), dim3(kExpandNT), 0, stream, sel, sel_count, k,
                       req_row_ptr, num_req, row_pos, row_pos_now, max_advance, c, page_table, pt_stride,
                       out_slots, out_pos, out_count, ld_out);
  } else {
    const int chunks = (ld_out + 255) / 256;
    hipLaunchKernelGGL(expand_entry_kernel, dim3(num_rows, chunks), dim3(256), 0, stream, sel, sel_count, k,
                       req_row_ptr, num_req, row_pos, row_pos_now, max_advance, c, page_table, pt_stride,
                       out_slots, out_pos, out_count, ld_out);
  }
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

}  // namespace bs
