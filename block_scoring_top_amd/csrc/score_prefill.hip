// score_prefill.hip - block scores for prefill chunks on the matrix cores.
//
// Same equation as the decode scorer (page "Qwen3.8-Flash-Next Day-0 in
// SGLang", QSA section, score equation), for many query rows of one request
// at once: a dense bf16 contraction [rows*4 x 128] . [128 x keys] with FP32
// accumulation, which the same section handles with a custom prefill
// index-score kernel.
//
// Mapping on gfx950:
//   * v_mfma_f32_16x16x32_bf16.  The A operand holds query head-rows with the
//     4 heads of a query row on adjacent M rows, so in the 16x16 accumulator
//     (lane l holds rows 4*(l/16)+0..3 of column l%16) each lane owns all 4
//     heads of one (query row, key) pair: ReLU, head sum and scale stay in the
//     lane (fused epilogue), and 16 lanes store 64 contiguous bytes of a row;
//   * a workgroup (4 waves) owns 64 query rows of one request and a range of
//     key tiles; each wave keeps its 16 rows' q fragments in registers for the
//     whole loop;
//   * 64-key tiles are gathered through the page table into LDS (rows padded
//     to 272 bytes so 16-byte fragment reads are bank-conflict free), triple
//     buffered so tile t+2's global loads overlap tile t's MFMAs; the page
//     ids of the workgroup's key range are staged in LDS once, so no key load
//     waits on a page-table load;
//   * causal visibility: tiles past the block's last visible key are skipped,
//     and per-row masking happens at the store.
#include "device.h"
#include "kernels.h"

namespace bs {

constexpr int kPfRows = 64;         // query rows per workgroup, 16 per wave
constexpr int kPfKeys = 64;         // keys per tile
constexpr int kPfStride = 272;      // LDS bytes per key row (256 + 16 pad)
constexpr int kPfTileBytes = kPfKeys * kPfStride;
constexpr int kPfMaxTiles = 64;     // key tiles per workgroup (host sizing)
constexpr int kPfMaxPages = kPfMaxTiles * kPfKeys * 4 / kPage;  // logical pages they span (c = 4)

// Loads this lane's four 16-byte slices of a 64-key tile (keys j0 ..
// j0+63; slice e covers key (e*256 + lane) / 16, dims 8*((e*256 + lane) % 16)).
// Page ids come from the workgroup's LDS copy (lp0 = its first logical page).
__device__ __forceinline__ void pf_load_tile(const uint16_t* __restrict__ kcache, int64_t num_pages,
                                             const int32_t* pages, int lp0, int per_page, int c, int j0, int nmax,
                                             u32x4_t (&regs)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int flat = e * 256 + tid;
    const int n = flat >> 4, slice = flat & 15;
    const int j = j0 + n;
    regs[e] = u32x4_t{0u, 0u, 0u, 0u};
    if (j < nmax) {
      const int32_t page = pages[((c * j) >> 6) - lp0];
      if (page >= 0 && page < num_pages) {
        const int64_t slot = (int64_t)page * per_page + (j & (per_page - 1));
        regs[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kcache + slot * kDim) + slice);
      }
    }
  }
}

__device__ __forceinline__ void pf_store_tile(uint8_t* lds, const u32x4_t (&regs)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int flat = e * 256 + tid;
    const int n = flat >> 4, slice = flat & 15;
    *reinterpret_cast<u32x4_t*>(lds + n * kPfStride + slice * 16) = regs[e];
  }
}

__global__ __launch_bounds__(256) void score_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kcache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ req_row_ptr, int32_t num_req, const int32_t* __restrict__ row_pos,
    int32_t c, int32_t max_vis, float* __restrict__ scores, int64_t ld, int32_t* __restrict__ row_len) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[3][kPfTileBytes];
  __shared__ int32_t pages[kPfMaxPages];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Work item -> (request, block of 64 rows).
  int wg = blockIdx.x, b = -1, rb0 = 0, rb1 = 0;
  for (int i = 0; i < num_req; ++i) {
    const int r0 = req_row_ptr[i], r1 = req_row_ptr[i + 1];
    const int nblk = (r1 - r0 + kPfRows - 1) / kPfRows;
    if (wg < nblk) {
      b = i;
      rb0 = r0 + wg * kPfRows;
      rb1 = min(r1, rb0 + kPfRows);
      break;
    }
    wg -= nblk;
  }
  if (b < 0) return;
  if (blockIdx.y == 0 && row_len != nullptr && tid < rb1 - rb0)
    row_len[rb0 + tid] = max(0, min((row_pos[rb0 + tid] + 1) / c, max_vis));

  int nmax = 0;
  for (int r = rb0; r < rb1; ++r) nmax = max(nmax, min((row_pos[r] + 1) / c, max_vis));
  const int ntiles = (nmax + kPfKeys - 1) / kPfKeys;
  const int t0 = (int)((int64_t)ntiles * blockIdx.y / gridDim.y);
  const int t1 = (int)((int64_t)ntiles * (blockIdx.y + 1) / gridDim.y);
  if (t0 >= t1) return;

  const int per_page = kPage / c;
  const int32_t* pt = page_table + (int64_t)b * pt_stride;
  const int g = lane >> 4, i16 = lane & 15;

  // A fragments: M-subtile ms covers query rows 4*ms .. 4*ms+3 of this wave,
  // head-row i16 = 4*(row) + head; k-step ks covers dims 32*ks + 8*g .. +7.
  bf16x8_t afr[4][4];
  int nvis[4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    const int qr = rb0 + wave * 16 + ms * 4 + (i16 >> 2);
    const int head = i16 & 3;
    const bool ok = qr < rb1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (ok) v = *(reinterpret_cast<const u32x4_t*>(q + ((int64_t)qr * kHeads + head) * kDim + 32 * ks) + g);
      afr[ms][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
    // The accumulator row this lane stores: query row 4*ms + g.
    const int orow = rb0 + wave * 16 + ms * 4 + g;
    nvis[ms] = orow < rb1 ? min((row_pos[orow] + 1) / c, max_vis) : 0;
  }
  // Smallest visible length over the wave's 16 rows (rows past the block
  // count as 0, so a partial block always takes the masked path).
  int wave_min_vis = min(min(nvis[0], nvis[1]), min(nvis[2], nvis[3]));
  for (int off = 16; off < 64; off <<= 1) wave_min_vis = min(wave_min_vis, __shfl_xor(wave_min_vis, off));

  // The page ids of this workgroup's key range, once: key loads then depend
  // on LDS, not on a global page-table load.
  const int lp0 = (c * t0 * kPfKeys) >> 6;
  const int lp1 = min(pt_stride, ((c * (t1 * kPfKeys) - 1) >> 6) + 1);
  for (int i = tid; i < lp1 - lp0 && i < kPfMaxPages; i += 256) pages[i] = pt[lp0 + i];
  __syncthreads();

  // Three LDS buffers: tile t is computed while tile t+1 sits in LDS and the
  // loads of tile t+2 are in flight.
  u32x4_t pre[4];
  pf_load_tile(kcache, num_pages, pages, lp0, per_page, c, t0 * kPfKeys, nmax, pre);
  pf_store_tile(lds[0], pre);
  if (t0 + 1 < t1) pf_load_tile(kcache, num_pages, pages, lp0, per_page, c, (t0 + 1) * kPfKeys, nmax, pre);
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) % 3;
    u32x4_t nxt[4];
    if (t + 2 < t1) pf_load_tile(kcache, num_pages, pages, lp0, per_page, c, (t + 2) * kPfKeys, nmax, nxt);
    if (t + 1 < t1) pf_store_tile(lds[(t + 1 - t0) % 3], pre);
    const uint8_t* tile = lds[buf];
    f32x4_t acc[4][4];
    const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t bfr = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(tile + (ns * 16 + i16) * kPfStride + (32 * ks + 8 * g) * 2));
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)  // the first k-step starts from C = 0: no accumulator clearing
          acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[ms][ks], bfr, ks == 0 ? zero : acc[ms][ns], 0, 0, 0);
      }
    }
    // Epilogue: lane holds heads 0..3 of query row (4*ms + g) for key
    // (16*ns + i16).  Tiles wholly inside every row's visible range store
    // without masks (uniform branch); the causal boundary tile masks per row.
    const bool full = (t + 1) * kPfKeys <= wave_min_vis;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      float* dst = scores + (int64_t)(rb0 + wave * 16 + ms * 4 + g) * ld + t * kPfKeys + i16;
      const int lim = nvis[ms] - t * kPfKeys - i16;  // store column ns*16 iff ns*16 < lim
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const f32x4_t a = acc[ms][ns];
        const float sc = ((fmaxf(a.x, 0.f) + fmaxf(a.y, 0.f)) + (fmaxf(a.z, 0.f) + fmaxf(a.w, 0.f))) * kScale;
        if (full || ns * 16 < lim) dst[ns * 16] = sc;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) pre[e] = nxt[e];
    __syncthreads();
  }
}

int launch_score_prefill(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                         const int32_t* page_table, int32_t pt_stride,
                         const int32_t* req_row_ptr, int32_t num_req,
                         const int32_t* row_pos, int32_t num_rows,
                         int32_t c, int32_t max_vis,
                         float* scores, int64_t ld, int32_t* row_len, hipStream_t stream) {
  // Upper bound on (request, 64-row block) pairs; surplus workgroups exit.
  const int64_t blocks = (int64_t)(num_rows + kPfRows - 1) / kPfRows + num_req;
  const int64_t tiles = ((int64_t)max_vis + kPfKeys - 1) / kPfKeys;
  int64_t splits = (2048 + blocks - 1) / blocks;
  const int64_t min_splits = (tiles + kPfMaxTiles - 1) / kPfMaxTiles;  // at most kPfMaxTiles tiles each
  splits = splits < min_splits ? min_splits : splits;
  splits = splits < 1 ? 1 : splits;
  splits = splits > tiles ? (tiles > 0 ? tiles : 1) : splits;
  if (splits > 65535) return BS_ERR_ARG;
  if (blocks > 0x7FFFFFFF) return BS_ERR_ARG;
  hipLaunchKernelGGL(score_prefill_kernel, dim3((unsigned)blocks, (unsigned)splits), dim3(256), 0, stream, q,
                     kcache, num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos, c, max_vis, scores,
                     ld, row_len);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

}  // namespace bs
