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
//   * 64-key tiles are copied from HBM straight into LDS (buffer loads with
//     the LDS flag: no staging registers, no LDS write instructions), three
//     buffers, two tiles ahead.  Each wave copies 16 consecutive keys of a
//     tile, which lie in one page (a page holds 64/c >= 16 keys for c <= 4),
//     so the page lookup and the bounds are wave-uniform: one scalar
//     page-table read and one buffer resource per wave per tile, whose range
//     check zero-fills keys past the visible range or behind an invalid page
//     id.  A tile's 16 B fragments are read from LDS before its 64 MFMAs, so
//     the reads are in flight together;
//   * the LDS tile is unpadded with an XOR swizzle (the 16-byte slice s of
//     key n sits at slot s ^ ((n / 4) mod 16)), so the fragment reads are free
//     of bank conflicts;
//   * scores are written with non-temporal stores (they are read once, by the
//     selection, after the whole launch);
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
constexpr int kPfBufs = 3;                        // LDS tile buffers

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

// Workgroup barrier without a memory fence: __syncthreads() would also wait
// for this wave's outstanding global stores.  The asm is a compiler barrier
// for memory operations; LDS data written by the transfers above is published
// by the caller's vmcnt wait before it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool VEC>
__global__ __launch_bounds__(256, 2) void score_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kcache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int32_t pt_stride,
    const int32_t* __restrict__ req_row_ptr, int32_t num_req, const int32_t* __restrict__ row_pos,
    int32_t num_rows, int32_t c, int32_t max_vis, int32_t tiles_per_block, int64_t units,
    float* __restrict__ scores, int64_t ld, int32_t* __restrict__ row_len) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kPfBufs][kPfTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;

  if (row_len != nullptr)
    for (int64_t r = (int64_t)blockIdx.x * 256 + tid; r < num_rows; r += (int64_t)gridDim.x * 256)
      row_len[r] = visible_blocks(row_pos[r], c, max_vis);

  // This workgroup's contiguous range of units.
  const int64_t u0 = units * blockIdx.x / gridDim.x;
  const int64_t u1 = units * (blockIdx.x + 1) / gridDim.x;
  const int per_page = kPage / c;
  // Page ids are int32: a bound above 2^31 - 1 admits every non-negative id.
  const int32_t num_pages32 = num_pages > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)num_pages;

  // LDS tile layout: key n at bytes 256*n, its 16-byte slice s at slot
  // s ^ ((n / 4) mod 16).  Tile load: instruction e of a wave fills keys
  // 16*wave + 4*e .. +3 (1 KiB, key group E = 4*wave + e), lane i the slot
  // i % 16 of key 16*wave + 4*e + i/16, i.e. slice (i % 16) ^ E, read at this
  // byte offset from the wave's first key.  Fragment read for k-step ks: key
  // 4*i16 + ns (ns*256 added as an immediate), slice 4*ks + g.
  uint32_t vofs[4], rofs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vofs[e] = (uint32_t)(e * 1024 + (lane >> 4) * 256 + 16 * ((lane & 15) ^ (4 * wave + e)));
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) rofs[ks] = (uint32_t)(i16 * 1024 + 16 * ((4 * ks + g) ^ i16));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(&lds[0][0]);

  for (int64_t u = u0; u < u1;) {
    const int64_t bi = u / tiles_per_block;
    const int tb = (int)(u - bi * tiles_per_block);
    const int64_t next_block = (bi + 1) * tiles_per_block;
    const int te_range = (int)(min(u1, next_block) - bi * tiles_per_block);
    u = next_block;
    int b = 0, rb0 = 0, rb1 = 0;
    if (!pf_locate(bi, req_row_ptr, num_req, b, rb0, rb1)) break;  // past the last block

    // A fragments: M-subtile ms covers query rows 4*ms .. 4*ms+3 of this
    // wave, head-row i16 = 4*(row) + head; k-step ks covers dims 32*ks + 8*g.
    // All 16 reads are issued before anything waits on memory.
    bf16x8_t afr[4][4];
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
    }
    // Visible lengths, one read per row of the block (lane L: row rb0 + L,
    // 0 past the block): the block's longest bounds its tiles; each lane
    // takes those of the 4 rows it stores by shuffle; the wave's shortest
    // decides which tiles store without masks.
    const int nv_lane = lane < rb1 - rb0 ? visible_blocks(row_pos[rb0 + lane], c, max_vis) : 0;
    int nmax = nv_lane;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) nmax = max(nmax, __shfl_xor(nmax, off));
    nmax = __builtin_amdgcn_readfirstlane(nmax);
    const int t0 = tb;
    const int t1 = min(te_range, (nmax + kPfKeys - 1) / kPfKeys);
    if (t0 >= t1) continue;
    int nvis[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) nvis[ms] = __shfl(nv_lane, wave * 16 + ms * 4 + g);  // row stored by this lane
    int wmin = min(min(nvis[0], nvis[1]), min(nvis[2], nvis[3]));
    wmin = min(wmin, __shfl_xor(wmin, 16));
    wmin = min(wmin, __shfl_xor(wmin, 32));
    wmin = __builtin_amdgcn_readfirstlane(wmin);  // rows past the block count as 0

    const int32_t* pt = page_table + (int64_t)b * pt_stride;
    // This wave's 16 keys of tile t start at key jw = 64*t + 16*wave: their
    // page id, or -1 at or past the block's visible range.  The table index
    // is clamped so that the (scalar) read is unconditional.
    auto group_page = [&](int t) -> int32_t {
      const int jw = t * kPfKeys + kPfGroup * wave;
      const int32_t id = pt[min((c * jw) >> 6, pt_stride - 1)];
      return jw < nmax ? id : -1;
    };
    // Issues tile t's loads for this wave into LDS buffer `buf`: always 4
    // transfers (an invalid page or a tile past the range gives an empty
    // resource, so zeros), so the vmcnt arithmetic below is fixed.
    auto dma_group = [&](int t, int32_t page, int buf) {
      const int jw = t * kPfKeys + kPfGroup * wave;
      uint64_t base = reinterpret_cast<uint64_t>(kcache);
      uint32_t bytes = 0;
      if (page >= 0 && page < num_pages32 && jw < nmax) {
        base += (uint64_t)(((int64_t)page * per_page + (jw & (per_page - 1))) * kDim * 2);
        bytes = (uint32_t)(min(nmax - jw, kPfGroup) * kDim * 2);
      }
      const u32x4_t rs = u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, bytes, 0x00020000u};
      const uint32_t dst = lds0 + (uint32_t)(buf * kPfTileBytes + wave * 4096);
#pragma unroll
      for (int e = 0; e < 4; ++e) lds_dma_b128(rs, vofs[e], dst + e * 1024);
    };

    // Tile products from LDS buffer `buf`: the tile's 16 B fragments are
    // read first (all in flight at once), then the 64 MFMAs consume them in
    // order.
    auto mfma_tile = [&](f32x4_t(&acc)[4][4], int buf) {
      const uint8_t* tile = lds[buf];
      bf16x8_t bfr[4][4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          bfr[ns][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(tile + rofs[ks] + ns * 256));
      const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int ms = 0; ms < 4; ++ms)  // the first k-step starts from C = 0
            acc[ms][ns] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[ms][ks], bfr[ns][ks], ks == 0 ? zero : acc[ms][ns], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // the 16 LDS reads first
      __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);  // then the MFMAs
    };
    // Epilogue values: lane holds heads 0..3 of query row 4*ms + g for keys
    // 4*i16 + ns, ns = 0..3.
    auto head_sums = [&](const f32x4_t(&acc)[4][4], f32x4_t(&v)[4]) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        v[ms] = f32x4_t{head_sum(acc[ms][0]), head_sum(acc[ms][1]), head_sum(acc[ms][2]), head_sum(acc[ms][3])};
    };
    // Tiles inside the visible range of every row of the wave store without
    // masks.
    auto store_tile = [&](const f32x4_t(&v)[4], int t) {
      const bool full = (t + 1) * kPfKeys <= wmin;
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        float* dst = scores + (int64_t)(rb0 + wave * 16 + ms * 4 + g) * ld + t * kPfKeys + 4 * i16;
        if (VEC && full) {
          __builtin_nontemporal_store(v[ms], reinterpret_cast<f32x4_t*>(dst));
        } else {
          const int lim = nvis[ms] - t * kPfKeys - 4 * i16;  // keys below lim are visible
          if (0 < lim) __builtin_nontemporal_store(v[ms].x, dst);
          if (1 < lim) __builtin_nontemporal_store(v[ms].y, dst + 1);
          if (2 < lim) __builtin_nontemporal_store(v[ms].z, dst + 2);
          if (3 < lim) __builtin_nontemporal_store(v[ms].w, dst + 3);
        }
      }
    };

    // Pipeline over the block's tiles, three LDS buffers: in step t the
    // loads of tile t+2 are issued and tile t is multiplied; once tile t+1's
    // loads are complete the tile's scores are stored.
    dma_group(t0, group_page(t0), 0);
    dma_group(t0 + 1, group_page(t0 + 1), 1);
    int32_t page_ahead = group_page(t0 + 2);
    wait_vmcnt<4>();  // this wave's part of tile t0 is in LDS
    barrier_lds();
    for (int t = t0; t < t1; ++t) {
      const int i = t - t0;
      dma_group(t + 2, page_ahead, (i + 2) % kPfBufs);
      f32x4_t acc[4][4], v[4];
      mfma_tile(acc, i % kPfBufs);
      // Scheduling fences keep the order: the tile's MFMAs, then the next
      // page id (a scalar read issued earlier would make the fragment-read
      // waits above wait for it too), then the epilogue, and only then the
      // wait for tile t+1, which also waits for the previous tile's stores
      // (vector memory operations retire in issue order).
      __builtin_amdgcn_sched_barrier(0);
      page_ahead = group_page(t + 3);
      head_sums(acc, v);
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) asm volatile("" : "+v"(v[ms]));  // computed here, not in the store branches
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<4>();  // tile t+1 is in LDS (and every older store is done)
      store_tile(v, t);
      barrier_lds();
    }
    wait_vmcnt<0>();  // no transfer into LDS outlives the block
    __syncthreads();
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
