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
//     lane (fused epilogue).  Column i of the n-th 16-key subtile is key 4*i+n
//     of the 64-key tile, so after the four subtiles a lane holds 4
//     consecutive keys of one row and stores them with one 16-byte store;
//   * a workgroup (4 waves) owns 64 query rows of one request at a time; each
//     wave keeps its 16 rows' q fragments in registers;
//   * 64-key tiles pass through LDS, double buffered: the next tile's global
//     loads are in flight while the current tile is multiplied.  Each wave
//     loads 16 consecutive keys of a tile, which lie in one page (a page holds
//     64/c >= 16 keys for c <= 4), so the page lookup and the bounds are
//     wave-uniform: one scalar page-table read and one buffer resource per
//     wave per tile, whose range check zero-fills keys past the visible range
//     or behind an invalid page id;
//   * the LDS tile is unpadded with an XOR swizzle (the 16-byte slice s of
//     key n sits at slot s ^ ((n / 4) mod 16)), so the fragment reads and the
//     tile writes are free of bank conflicts;
//   * work is the list of (64-row block, key tile) units, split into equal
//     contiguous ranges over a grid sized to the chip's resident workgroups;
//     tiles past a block's causal limit are skipped.
#include <atomic>

#include "device.h"
#include "kernels.h"

namespace bs {

constexpr int kPfRows = 64;                       // query rows per block, 16 per wave
constexpr int kPfKeys = 64;                       // keys per tile
constexpr int kPfTileBytes = kPfKeys * kDim * 2;  // 16 KiB
constexpr int kPfGroup = 16;                      // keys loaded per wave per tile

// Locates 64-row block `bi` (blocks are numbered request by request):
// returns false if there is no such block.
__device__ __forceinline__ bool pf_locate(int64_t bi, const int32_t* __restrict__ req_row_ptr, int num_req,
                                          int& b, int& r0, int& r1) {
  for (int i = 0; i < num_req; ++i) {
    const int a0 = req_row_ptr[i], a1 = req_row_ptr[i + 1];
    const int64_t nblk = (a1 - a0 + kPfRows - 1) / kPfRows;
    if (bi < nblk) {
      b = i;
      r0 = a0 + (int)bi * kPfRows;
      r1 = min(a1, r0 + kPfRows);
      return true;
    }
    bi -= nblk;
  }
  return false;
}

// max(x, 0) on the bit pattern: negative values (sign bit set) compare below
// 0 as signed integers.  One v_max_i32, no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float head_sum(const f32x4_t& a) {
  return ((relu_bits(a.x) + relu_bits(a.y)) + (relu_bits(a.z) + relu_bits(a.w))) * kScale;
}

template <bool VEC>
__global__ __launch_bounds__(256, 2) void score_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kcache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ req_row_ptr, int32_t num_req, const int32_t* __restrict__ row_pos,
    int32_t num_rows, int32_t c, int32_t max_vis, int32_t tiles_per_block, int64_t units,
    float* __restrict__ scores, int64_t ld, int32_t* __restrict__ row_len) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kPfTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;

  if (row_len != nullptr)
    for (int64_t r = (int64_t)blockIdx.x * 256 + tid; r < num_rows; r += (int64_t)gridDim.x * 256)
      row_len[r] = max(0, min((row_pos[r] + 1) / c, max_vis));

  // This workgroup's contiguous range of units.
  const int64_t u0 = units * blockIdx.x / gridDim.x;
  const int64_t u1 = units * (blockIdx.x + 1) / gridDim.x;
  const int per_page = kPage / c;
  // Page ids are int32: a bound above 2^31 - 1 admits every non-negative id.
  const int32_t num_pages32 = num_pages > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)num_pages;

  // Per-lane constant LDS offsets.  Tile write: slice lane % 16 of key
  // 16*wave + 4*e + lane/16 (whose key group E = 4*wave + e).  Fragment read
  // for k-step ks: key 4*i16 + ns (ns*256 added as an immediate), slice
  // 4*ks + g.
  uint32_t wofs[4], rofs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int E = 4 * wave + e;
    wofs[e] = (uint32_t)((16 * wave + 4 * e + (lane >> 4)) * 256 + 16 * ((lane & 15) ^ E));
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) rofs[ks] = (uint32_t)(i16 * 1024 + 16 * ((4 * ks + g) ^ i16));

  for (int64_t u = u0; u < u1;) {
    const int64_t bi = u / tiles_per_block;
    const int tb = (int)(u - bi * tiles_per_block);
    const int64_t next_block = (bi + 1) * tiles_per_block;
    const int te_range = (int)(min(u1, next_block) - bi * tiles_per_block);
    u = next_block;
    int b = 0, rb0 = 0, rb1 = 0;
    if (!pf_locate(bi, req_row_ptr, num_req, b, rb0, rb1)) break;  // past the last block

    // Visible lengths: the block's longest bounds its tiles; the wave's
    // shortest decides which tiles store without masks.
    int nmax = 0;
    if (lane < rb1 - rb0) nmax = max(0, min((row_pos[rb0 + lane] + 1) / c, max_vis));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) nmax = max(nmax, __shfl_xor(nmax, off));
    nmax = __builtin_amdgcn_readfirstlane(nmax);
    const int t0 = tb;
    const int t1 = min(te_range, (nmax + kPfKeys - 1) / kPfKeys);
    if (t0 >= t1) continue;

    // A fragments: M-subtile ms covers query rows 4*ms .. 4*ms+3 of this
    // wave, head-row i16 = 4*(row) + head; k-step ks covers dims 32*ks + 8*g.
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
      const int orow = rb0 + wave * 16 + ms * 4 + g;  // the accumulator row this lane stores
      nvis[ms] = orow < rb1 ? max(0, min((row_pos[orow] + 1) / c, max_vis)) : 0;
    }
    int wmin = min(min(nvis[0], nvis[1]), min(nvis[2], nvis[3]));
    wmin = min(wmin, __shfl_xor(wmin, 16));
    wmin = min(wmin, __shfl_xor(wmin, 32));
    wmin = __builtin_amdgcn_readfirstlane(wmin);  // rows past the block count as 0

    const int32_t* pt = page_table + (int64_t)b * pt_stride;
    // This wave's 16 keys of tile t start at key jw = 64*t + 16*wave: their
    // page id (-1 past the block's visible range), read one tile ahead.
    auto group_page = [&](int t) -> int32_t {
      const int jw = t * kPfKeys + kPfGroup * wave;
      return jw < nmax ? pt[(c * jw) >> 6] : -1;
    };
    // Buffer resource over those keys: based at the slot of key jw, covering
    // the keys below nmax, empty if the page id is invalid.
    auto load_group = [&](int t, int32_t page, u32x4_t(&regs)[4]) {
      const int jw = t * kPfKeys + kPfGroup * wave;
      const uint16_t* base = kcache;
      int bytes = 0;
      if (page >= 0 && page < num_pages32) {
        base = kcache + ((int64_t)page * per_page + (jw & (per_page - 1))) * kDim;
        bytes = min(nmax - jw, kPfGroup) * kDim * 2;
      }
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes, 0x00020000);
#pragma unroll
      for (int e = 0; e < 4; ++e) regs[e] = __builtin_amdgcn_raw_buffer_load_b128(rs, e * 1024 + lane * 16, 0, 0);
    };
    auto store_group = [&](uint8_t* buf, const u32x4_t(&regs)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4_t*>(buf + wofs[e]) = regs[e];
    };

    u32x4_t stage[4];
    load_group(t0, group_page(t0), stage);
    int32_t page_next = t0 + 1 < t1 ? group_page(t0 + 1) : -1;
    store_group(lds[0], stage);
    __syncthreads();

    for (int t = t0; t < t1; ++t) {
      const int cur = (t - t0) & 1;
      const bool more = t + 1 < t1;
      if (more) load_group(t + 1, page_next, stage);  // in flight during this tile
      const uint8_t* tile = lds[cur];
      f32x4_t acc[4][4];
      const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8_t bfr =
              __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(tile + rofs[ks] + ns * 256));
#pragma unroll
          for (int ms = 0; ms < 4; ++ms)  // the first k-step starts from C = 0
            acc[ms][ns] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[ms][ks], bfr, ks == 0 ? zero : acc[ms][ns], 0, 0, 0);
        }
      }
      // The page id for tile t+2 (a scalar load; waited on at the barrier).
      if (t + 2 < t1) page_next = group_page(t + 2);
      // Epilogue: lane holds heads 0..3 of query row 4*ms + g for keys
      // 4*i16 + ns, ns = 0..3.
      f32x4_t v[4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        v[ms] = f32x4_t{head_sum(acc[ms][0]), head_sum(acc[ms][1]), head_sum(acc[ms][2]), head_sum(acc[ms][3])};
      // The next tile goes to LDS before this tile's scores are stored, so
      // that waiting for its loads never waits for these stores.
      if (more) store_group(lds[cur ^ 1], stage);
      __builtin_amdgcn_sched_barrier(0);
      // Tiles inside the visible range of every row of the wave store
      // without masks.
      const bool full = (t + 1) * kPfKeys <= wmin;
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        float* dst = scores + (int64_t)(rb0 + wave * 16 + ms * 4 + g) * ld + t * kPfKeys + 4 * i16;
        if (VEC && full) {
          *reinterpret_cast<f32x4_t*>(dst) = v[ms];
        } else {
          const int lim = nvis[ms] - t * kPfKeys - 4 * i16;  // keys below lim are visible
          if (0 < lim) dst[0] = v[ms].x;
          if (1 < lim) dst[1] = v[ms].y;
          if (2 < lim) dst[2] = v[ms].z;
          if (3 < lim) dst[3] = v[ms].w;
        }
      }
      __syncthreads();
    }
  }
}

// Resident workgroups per CU for the kernel (a property of the code object;
// computed once).
static int pf_resident_per_cu(bool vec) {
  static std::atomic<int> cached[2] = {0, 0};
  int v = cached[vec].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    const hipError_t e =
        vec ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, score_prefill_kernel<true>, 256, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, score_prefill_kernel<false>, 256, 0);
    v = (e == hipSuccess && n > 0) ? n : 1;
    cached[vec].store(v, std::memory_order_relaxed);
  }
  return v;
}

int launch_score_prefill(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                         const int32_t* page_table, int32_t pt_stride,
                         const int32_t* req_row_ptr, int32_t num_req,
                         const int32_t* row_pos, int32_t num_rows,
                         int32_t c, int32_t max_vis,
                         float* scores, int64_t ld, int32_t* row_len, hipStream_t stream) {
  // Units: (64-row block, tile) over an upper bound on the block count.
  const int64_t blocks = (int64_t)(num_rows + kPfRows - 1) / kPfRows + num_req;
  const int64_t tpb = max_vis > 0 ? ((int64_t)max_vis + kPfKeys - 1) / kPfKeys : 1;
  const int64_t units = blocks * tpb;
  const bool vec = (ld % 4) == 0 && (reinterpret_cast<uintptr_t>(scores) % 16) == 0;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return BS_ERR_LAUNCH;
  int64_t grid = (int64_t)cus * pf_resident_per_cu(vec);
  grid = grid < units ? grid : units;
  grid = grid < 1 ? 1 : grid;
  if (tpb > 0x7FFFFFFF) return BS_ERR_ARG;
  if (vec)
    hipLaunchKernelGGL(score_prefill_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, q, kcache,
                       num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos, num_rows, c, max_vis,
                       (int32_t)tpb, units, scores, ld, row_len);
  else
    hipLaunchKernelGGL(score_prefill_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, q, kcache,
                       num_pages, page_table, pt_stride, req_row_ptr, num_req, row_pos, num_rows, c, max_vis,
                       (int32_t)tpb, units, scores, ld, row_len);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

}  // namespace bs
