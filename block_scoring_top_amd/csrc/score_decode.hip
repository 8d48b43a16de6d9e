// score_decode.hip - paged block scorer for decode and speculative-verify rows.
//
// Computes the QSA block score (page "Qwen3.8-Flash-Next Day-0 in SGLang",
// section on Qwen sparse attention, score equation): for a query row with
// 4 heads of 128 dims and a compressed key kbar,
//     s = (1/sqrt(128)) * sum_h max(0, <q_h, kbar>),
// over the row's visible blocks, reading keys through the page table (the
// section's paged decode scorer and full_slot/4 addressing).
//
// Mapping on gfx950 (64-lane waves, memory bound, no matrix cores):
//   * a workgroup of 256 lanes owns a chunk of one request's key range and
//     streams it once, 16 keys (4 KiB) per round, every lane loading one
//     16-byte slice (8 dims) of one key with a non-temporal load;
//   * 16 consecutive lanes (one DPP row) hold one key; each lane forms its
//     partial dot for the 4 heads with v_dot2_f32_bf16 (FP32 accumulate);
//   * a transposed butterfly over the row (mirror, half-mirror, two quad
//     swaps) reduces the 4 partial dots in 7 DPP adds, then ReLU per head and
//     two more DPP adds sum the heads;
//   * all rows of a request (up to RG at a time) are scored from the same
//     key registers, so keys leave HBM once per request.
//
// Requests with several rows (speculative verify: 1 accepted + drafts) make
// the VALU work per key byte grow with the row count; there the rows x keys
// product goes to the matrix cores instead (score_rows_mfma_kernel):
//   * v_mfma_f32_16x16x32_bf16 with A = the request's query head-rows (a
//     row's 4 heads on adjacent M rows, up to 4*NMS rows per pass), B = 16
//     keys: every wave holds all of the request's rows;
//   * each wave copies its 16-key subtiles (4 KiB, one page) from HBM
//     straight into LDS with 1 KiB contiguous transfers (buffer loads with the
//     LDS flag, full cache lines), then reads its B fragments from there
//     (swizzled, no bank conflicts).  Reading the fragments straight from HBM
//     made 64-byte requests, and was bound by the request rate at about half
//     the bandwidth.  Keys stay in LDS across row passes;
//   * in the 16x16 accumulator a lane holds the 4 heads of one (row, key):
//     ReLU, head sum and scale stay in the lane, 16 lanes store 64 contiguous
//     bytes of a row;
//   * a 16-key subtile lies in one page, so its page id is wave-uniform (the
//     chunk's page ids sit one per lane and are read with v_readlane).
#include "device.h"
#include "kernels.h"

namespace bs {

// Sum over the 16 lanes of a DPP row of four per-lane partial dots, ReLU per
// head, sum over heads.  Every lane of the row returns the unscaled score.
__device__ __forceinline__ float row_head_relu_sum(float h0, float h1, float h2, float h3, int sub) {
  const bool hi8 = (sub & 8) != 0;
  const float keep0 = hi8 ? h2 : h0, keep1 = hi8 ? h3 : h1;
  const float send0 = hi8 ? h0 : h2, send1 = hi8 ? h1 : h3;
  const float a0 = keep0 + dpp<kDppRowMirror>(send0);  // partner 15-i: other half
  const float a1 = keep1 + dpp<kDppRowMirror>(send1);
  const bool hi4 = (sub & 4) != 0;
  const float keep = hi4 ? a1 : a0, send = hi4 ? a0 : a1;
  float x = keep + dpp<kDppRowHalfMirror>(send);  // partner 7-i in the half: bit 2 flipped
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  // x: full dot of head 2*bit3(sub) + bit2(sub)
  float y = fmaxf(x, 0.0f);
  y += dpp<kDppRowHalfMirror>(y);
  y += dpp<kDppRowMirror>(y);
  return y;
}

__device__ __forceinline__ float slice_dot(const u32x4_t& k, const u32x4_t& q) {
  float acc = 0.0f;
  acc = dot2_bf16(k.x, q.x, acc);
  acc = dot2_bf16(k.y, q.y, acc);
  acc = dot2_bf16(k.z, q.z, acc);
  acc = dot2_bf16(k.w, q.w, acc);
  return acc;
}

template <int RG, int U>
__global__ __launch_bounds__(256) void score_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kcache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ req_row_ptr, const int32_t* __restrict__ row_pos,
    int32_t c, int32_t max_vis, int32_t chunk,
    float* __restrict__ scores, int64_t ld, int32_t* __restrict__ row_len) {
  const int b = blockIdx.y;
  const int r0 = req_row_ptr[b];
  const int r1 = req_row_ptr[b + 1];
  const int tid = threadIdx.x, lane = tid & 63;

  int nmax = 0;
  for (int r = r0; r < r1; ++r) nmax = max(nmax, visible_blocks(row_pos[r], c, max_vis));
  if (blockIdx.x == 0 && row_len != nullptr)
    for (int r = r0 + tid; r < r1; r += blockDim.x) row_len[r] = visible_blocks(row_pos[r], c, max_vis);

  const int j0 = blockIdx.x * chunk;
  if (j0 >= nmax) return;
  const int j1 = min(j0 + chunk, nmax);
  const int per_page = kPage / c;
  const int sub = tid & 15;  // 16-byte slice: dims 8*sub .. 8*sub+7
  const int kin = tid >> 4;  // key within a 16-key round
  // The chunk spans at most 64 pages (chunks are at most 1,024 keys): lane i
  // of every wave holds the chunk's i-th page id, read with v_readlane.
  const int32_t* pt = page_table + (int64_t)b * pt_stride;
  const int first_page = (c * j0) >> 6;
  const int npages = ((c * (j1 - 1)) >> 6) - first_page + 1;
  const int32_t my_page = lane < npages ? pt[first_page + lane] : -1;

  auto round_slot = [&](int jb, bool& ok) -> int64_t {
    // Keys past the chunk are clamped onto its last key (always a valid
    // read); their scores are never stored.  A 16-aligned round lies in one
    // page, so the page id is uniform.
    const int jc = min(jb, j1 - 1);
    const int page = __builtin_amdgcn_readlane(my_page, ((c * jc) >> 6) - first_page);
    ok = page >= 0 && page < num_pages;
    const int j = min(jb + kin, j1 - 1);
    return ok ? (int64_t)page * per_page + (j & (per_page - 1)) : 0;
  };

  for (int g0 = r0; g0 < r1; g0 += RG) {
    const int ng = min(RG, r1 - g0);
    u32x4_t qv[RG][kHeads];
    int nvis[RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = g0 + min(i, ng - 1);
      const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(q + (int64_t)r * kHeads * kDim) + sub;
#pragma unroll
      for (int h = 0; h < kHeads; ++h) qv[i][h] = qp[h * (kDim / 8)];
      nvis[i] = i < ng ? visible_blocks(row_pos[r], c, max_vis) : 0;
    }

    u32x4_t kv[U];
    bool ok[U];
    auto issue = [&](int jr) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t slot = round_slot(jr + 16 * u, ok[u]);
        kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kcache + slot * kDim) + sub);
      }
    };
    issue(j0);
    for (int jr = j0; jr < j1; jr += 16 * U) {
      u32x4_t cur[U];
      bool cok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cur[u] = kv[u];
        cok[u] = ok[u];
      }
      if (jr + 16 * U < j1) issue(jr + 16 * U);  // next group in flight during this one
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jr + 16 * u + kin;
#pragma unroll
        for (int i = 0; i < RG; ++i) {
          if (i < ng) {
            const float sc = row_head_relu_sum(slice_dot(cur[u], qv[i][0]), slice_dot(cur[u], qv[i][1]),
                                               slice_dot(cur[u], qv[i][2]), slice_dot(cur[u], qv[i][3]), sub);
            // j < j0 + chunk always holds here, so j < nvis[i] (the range
            // of the row's buffer) is the whole store condition; lanes other
            // than the key's first fall outside the range too.  No branch:
            // the wait for the next keys then leaves these stores in flight.
            const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
                scores + (int64_t)(g0 + i) * ld, (short)0, nvis[i] * 4, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cok[u] ? sc * kScale : __builtin_nanf("")), srs,
                                                  sub == 0 ? (uint32_t)j * 4u : 0x80000000u, 0, 0);
          }
        }
      }
    }
  }
}

template <int NMS, int NW, int KSUB>
__global__ __launch_bounds__(64 * NW) void score_rows_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kcache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ req_row_ptr, const int32_t* __restrict__ row_pos,
    int32_t c, int32_t max_vis, int32_t chunk, int32_t fold,
    float* __restrict__ scores, int64_t ld, int32_t* __restrict__ row_len) {
  // Per wave KSUB subtiles of 16 keys (4 KiB each), key n of a subtile at
  // bytes 256*n, its 16-byte slice s at slot s ^ n (the 16 lanes reading one
  // k-step slice of 16 keys then hit 16 different slots: no bank conflicts).
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NW][KSUB][4096];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int r0 = req_row_ptr[b];
  const int r1 = req_row_ptr[b + 1];
  if (blockIdx.x == 0 && row_len != nullptr)
    for (int r = r0 + tid; r < r1; r += blockDim.x) row_len[r] = visible_blocks(row_pos[r], c, max_vis);

  // The request's longest visible range bounds the chunk.
  int nmax = 0;
  for (int r = r0 + lane; r < r1; r += 64) nmax = max(nmax, visible_blocks(row_pos[r], c, max_vis));
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) nmax = max(nmax, __shfl_xor(nmax, off));
  nmax = __builtin_amdgcn_readfirstlane(nmax);
  // `fold` consecutive chunks per workgroup, one after the other (each
  // wave's LDS tiles are its own, so reusing them needs no barrier).
  for (int f = 0; f < fold; ++f) {
    const int j0 = (blockIdx.x * fold + f) * chunk;
    const int j1 = min(j0 + chunk, nmax);
    if (j0 >= j1) return;
    const int per_page = kPage / c;
    // The chunk spans at most 64 pages: lane i holds the chunk's i-th page id
    // (chunks are at most 16*NW*KSUB <= 1,024 keys).
    const int32_t* pt = page_table + (int64_t)b * pt_stride;
    const int first_page = (c * j0) >> 6;
    const int npages = ((c * (j1 - 1)) >> 6) - first_page + 1;
    const int32_t my_page = lane < npages ? pt[first_page + lane] : -1;
    const int nsub = (j1 - j0 + 15) / 16;

    // A fragments of rows g0 .. g0 + 4*NMS - 1: subtile ms holds rows
    // g0 + 4*ms .. +3, head-row i16 = 4*(row) + head; k-step ks covers dims
    // 32*ks + 8*g.
    bf16x8_t afr[NMS][4];
    int orow[NMS], nv[NMS];
    auto load_rows = [&](int g0) {
  #pragma unroll
      for (int ms = 0; ms < NMS; ++ms) {
        const int qr = g0 + 4 * ms + (i16 >> 2);
  #pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
          if (qr < r1) v = *(reinterpret_cast<const u32x4_t*>(q + ((int64_t)qr * kHeads + (i16 & 3)) * kDim + 32 * ks) + g);
          afr[ms][ks] = __builtin_bit_cast(bf16x8_t, v);
        }
        orow[ms] = g0 + 4 * ms + g;  // the accumulator row this lane stores
        nv[ms] = orow[ms] < r1 ? visible_blocks(row_pos[orow[ms]], c, max_vis) : 0;
      }
    };
    load_rows(r0);

    // This wave's subtiles s = wave + NW*p: their 16 keys lie in one page (a
    // 16-aligned run of keys, 64/c >= 16 keys per page), copied into LDS with
    // four 1 KiB transfers (lane l of transfer e fills slot l % 16 of key
    // 4*e + l/16, i.e. reads that key's slice (l % 16) ^ key).  Keys past the
    // chunk or behind an invalid page id read as zeros (buffer range check).
    bool valid[KSUB];
    const uint32_t lds_wave = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(&lds[wave][0][0]);
  #pragma unroll
    for (int p = 0; p < KSUB; ++p) {
      const int s = wave + NW * p;
      const int jb = j0 + 16 * s;
      const int page = __builtin_amdgcn_readlane(my_page, ((c * min(jb, j1 - 1)) >> 6) - first_page);
      valid[p] = s < nsub && page >= 0 && page < num_pages;
      uint64_t base = reinterpret_cast<uint64_t>(kcache);
      uint32_t bytes = 0;
      if (valid[p]) {
        base += (uint64_t)(((int64_t)page * per_page + (jb & (per_page - 1))) * kDim * 2);
        bytes = (uint32_t)(min(j1 - jb, 16) * kDim * 2);
      }
      const u32x4_t rs = u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, bytes, 0x00020000u};
  #pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = 4 * e + (lane >> 4);
        lds_dma_b128(rs, (uint32_t)(n * 256 + 16 * ((lane & 15) ^ n)), lds_wave + (uint32_t)(p * 4096 + e * 1024));
      }
    }
    wait_vmcnt<0>();  // this wave's keys (and rows) are in

    for (int g0 = r0;;) {
  #pragma unroll
      for (int p = 0; p < KSUB; ++p) {
        const int s = wave + NW * p;
        if (s >= nsub) break;
        const uint8_t* tile = lds[wave][p];
        bf16x8_t br[4];
  #pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          br[ks] = __builtin_bit_cast(bf16x8_t,
                                      *reinterpret_cast<const u32x4_t*>(tile + i16 * 256 + 16 * ((4 * ks + g) ^ i16)));
        f32x4_t acc[NMS];
        const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int ks = 0; ks < 4; ++ks)
  #pragma unroll
          for (int ms = 0; ms < NMS; ++ms)
            acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[ms][ks], br[ks], ks == 0 ? zero : acc[ms], 0, 0, 0);
        const int j = j0 + 16 * s + i16;
  #pragma unroll
        for (int ms = 0; ms < NMS; ++ms) {
          const f32x4_t a = acc[ms];
          const float sc = ((fmaxf(a.x, 0.f) + fmaxf(a.y, 0.f)) + (fmaxf(a.z, 0.f) + fmaxf(a.w, 0.f))) * kScale;
          if (j < j1 && j < nv[ms]) scores[(int64_t)orow[ms] * ld + j] = valid[p] ? sc : __builtin_nanf("");
        }
      }
      g0 += 4 * NMS;
      if (g0 >= r1) break;
      load_rows(g0);  // further rows reuse the keys held in LDS
    }
  }
}

constexpr int kRowsWaves = 4;  // waves per workgroup in the matrix-core kernel
constexpr int kRowsSub = 2;    // 16-key subtiles per wave there

// Rows per request (rounded up) pick the kernel: 1 or 2 -> the VALU kernel
// with that many rows per pass; more -> the matrix-core kernel.
static int rows_per_request(int num_rows, int num_req) { return (num_rows + num_req - 1) / num_req; }

int launch_score_decode(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                        const int32_t* page_table, int32_t pt_stride,
                        const int32_t* req_row_ptr, int32_t num_req,
                        const int32_t* row_pos, int32_t num_rows,
                        int32_t c, int32_t max_vis,
                        float* scores, int64_t ld, int32_t* row_len, hipStream_t stream) {
  constexpr int U = 4;
  // Chunk: many small workgroups stream best (measured on the 16 x 81,920
  // c = 1 batch: 128 keys per workgroup 6.4 TB/s, 640 keys 5.7 TB/s, 4,096
  // keys 3.9 TB/s); 64 keys for small batches, to spread them wider.
  const int64_t keys = (int64_t)max_vis * num_req;
  const int64_t chunk = keys >= (1 << 18) ? 128 : 64;
  const int nchunks = max_vis > 0 ? (int)((max_vis + chunk - 1) / chunk) : 1;
  dim3 grid(nchunks, num_req), block(256);
  const int avg = rows_per_request(num_rows, num_req);
  if (avg > 2) {
    // Several rows per request: the matrix-core kernel, 64*KSUB-key chunks.
    constexpr int P = kRowsSub, W = kRowsWaves, kChunkM = 16 * W * P;
    // Two chunks per workgroup: with ragged requests most workgroups of the
    // (chunk, request) grid find no keys, and halving their number measured
    // 37.3 -> 35.2 us on 64 requests x 6 rows of 1,022-32,768 blocks (four
    // chunks: 36.7 us).
    constexpr int kFold = 2;
    const int nch = max_vis > 0 ? ((max_vis + kChunkM - 1) / kChunkM + kFold - 1) / kFold : 1;
    dim3 gm(nch, num_req);
    if (avg <= 4)
      hipLaunchKernelGGL((score_rows_mfma_kernel<1, W, P>), gm, dim3(64 * W), 0, stream, q, kcache, num_pages, page_table,
                         pt_stride, req_row_ptr, row_pos, c, max_vis, kChunkM, kFold, scores, ld, row_len);
    else if (avg <= 8)
      hipLaunchKernelGGL((score_rows_mfma_kernel<2, W, P>), gm, dim3(64 * W), 0, stream, q, kcache, num_pages, page_table,
                         pt_stride, req_row_ptr, row_pos, c, max_vis, kChunkM, kFold, scores, ld, row_len);
    else
      hipLaunchKernelGGL((score_rows_mfma_kernel<4, W, P>), gm, dim3(64 * W), 0, stream, q, kcache, num_pages, page_table,
                         pt_stride, req_row_ptr, row_pos, c, max_vis, kChunkM, kFold, scores, ld, row_len);
    return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
  }
  if (avg <= 1)
    hipLaunchKernelGGL((score_decode_kernel<1, U>), grid, block, 0, stream, q, kcache, num_pages, page_table,
                       pt_stride, req_row_ptr, row_pos, c, max_vis, (int32_t)chunk, scores, ld, row_len);
  else
    hipLaunchKernelGGL((score_decode_kernel<2, U>), grid, block, 0, stream, q, kcache, num_pages, page_table,
                       pt_stride, req_row_ptr, row_pos, c, max_vis, (int32_t)chunk, scores, ld, row_len);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

}  // namespace bs
