// topk.hip - exact top-k per FP32 score row, as a selection rather than a sort,
// optionally fused with expand / append / page translation.
//
// Follows the TopK-V2 description (GLM-5.2 on SGLang blog, Kernel Optimization
// > TopK-V2, text and Figures 2-3): each FP32 score is rounded to FP16 and
// mapped to an order-preserving 16-bit key whose upper 10 bits index a
// 1,024-bin histogram; the bin holding the m-th largest score is located;
// scores in higher bins are emitted directly; the boundary bin is resolved
// exactly.  The page leaves the exact tie rule open; here equal scores go to
// the lower index, so the boundary is resolved by radix selection on the
// 64-bit pair (FP32 key, inverted index), which makes every key unique and the
// result exactly m entries.  The same blog fuses the selection with the
// page-table transform; the TRANSLATE kernels do that (expand each chosen
// block to its token positions, append the pending tokens, translate to
// physical slots, as the QSA section of the Qwen3.8-Flash-Next SGLang page
// describes).
//
// CDNA4 has no thread-block clusters or distributed shared memory.  The
// blog's paths become:
//   * rows that are not few-and-long: one workgroup per row, the row held in
//     registers, 1,024 lanes x 16 values (longer rows streamed twice), or,
//     for batches of at least 1,024 rows of at most 16,384 entries, 256 lanes
//     x 64 values so that several rows share a CU.  The register path keeps
//     each entry's bin, not its value, and marks the entries above and in the
//     boundary bin with two bit masks;
//   * few long rows (>= 32,769 entries, at most 256 rows): one 256-lane
//     workgroup per 2,048-entry chunk (8 entries per lane, in registers).
//     A first launch merges the chunks' LDS histograms into the row's
//     histogram with device atomics.  In a second launch every chunk finds
//     the threshold bin, emits and translates its own above-threshold entries
//     and appends its boundary-bin entries to the row's candidate list; the
//     last chunk to arrive (a device-scope counter) resolves the boundary bin
//     from that list.  No workgroup waits on another (no co-residency
//     assumption) and no device-scope fence is issued: on gfx950 such a fence
//     writes back and invalidates the per-XCD L2, which measured far costlier
//     than the whole kernel.  Data crossing workgroups inside a launch (the
//     candidate list, the counters) moves only through device-scope atomic
//     loads and stores, performed at the device coherence point; each chunk
//     waits for its stores to complete before it arrives;
//   * emission is count, block scan, write (no per-entry atomics); the
//     threshold scan runs on one wave with DPP scans; the boundary
//     refinement costs one workgroup barrier per 8-bit radix pass.
#include "device.h"
#include "kernels.h"

namespace bs {

constexpr int kRowNT = 1024;                   // lanes per workgroup, one row per workgroup
constexpr int kRowVpt = 16;                    // register path: values per lane
constexpr int kRowCand = 2048;                 // boundary candidates held in LDS (row kernel)
constexpr int kMidNT = 512;                    // row kernel for rows of 16,385-32,768 entries: lanes per workgroup
constexpr int kMidVpt = 64;                    // ...values per lane in registers
constexpr int kMidCand = 2048;                 // ...boundary candidates in LDS
constexpr int kManyNT = 256;                   // row kernel for many rows: lanes per workgroup
constexpr int kManyVpt = 64;                   // ...values per lane in registers
constexpr int kManyCand = 1024;                // ...boundary candidates in LDS
constexpr int kManyMinRows = 1024;             // batches with at least this many rows
constexpr int kLongNT = 256;                   // lanes per workgroup on the long-row kernels
constexpr int kLongVpt = 16;                   // values per lane held at once there
constexpr int kLongCand = 4096;
constexpr int kLongMin = 32769;                // rows this long use several workgroups...
constexpr int kLongRowsMax = 256;              // ...when the batch has at most this many rows
constexpr int kChunk = 2048;                   // entries per workgroup on long rows (a sweep of 1,024-16,384 on 16 x 81,920 rows: 2,048 fastest)
constexpr int kPerLane = kChunk / kLongNT;     // 8
constexpr int kHistChunk = 4096;               // entries per workgroup in the long-row histogram launch (2,048-8,192 measured alike)
constexpr int kHistPerLane = kHistChunk / kLongNT;
static_assert(kHistChunk % (2 * kLongNT) == 0, "histogram chunks are whole lane pairs");
constexpr int kChunkPages = 4 * kChunk / kPage;  // logical pages a chunk's blocks span (c <= 4)
constexpr int kRowPages = 1024;                  // a row's first page ids, cached in LDS for its translation
static_assert(kChunk % kLongNT == 0, "a long-row chunk is a whole number of lanes");

// Workspace record per row (long rows only): merged histogram, counters
// ([0] arrivals, [1] emitted above the threshold, [2] boundary candidates),
// boundary candidate list.
constexpr size_t kWsHist = 0;
constexpr size_t kWsCtr = kBins * 4;
constexpr size_t kWsCand = kWsCtr + 64;
constexpr size_t kWsRow = kWsCand + (size_t)kLongCand * 8;

template <int CAP>
struct TopkShared {
  uint32_t hist[kBins];
  uint32_t digit[256];
  uint64_t cand[CAP];
  int32_t chosen[kKmax];  // the row's selection, for the fused translation
  uint32_t wave_tot[16];
  uint32_t emit;
  uint32_t T;
  uint32_t above;
  uint32_t last;
  uint32_t base_up, base_cand;
  uint64_t red_and[16], red_or[16];
  int32_t pages[kChunkPages];  // page ids of a long-row chunk's token range (fused translation)
  int32_t row_pages[kRowPages];  // page ids 0 .. row_npages-1 of a whole row's request (fused translation)
  uint32_t row_npages;
};

// Translation context (fused kernels only).
struct Translate {
  const int32_t* req_row_ptr;
  int32_t num_req;
  const int32_t* row_pos;
  int32_t c;
  const int32_t* page_table;
  int32_t pt_stride;
  int32_t* out_slots;
  int32_t* out_pos;
  int32_t* out_count;
  int32_t ld_out;
};

// The inverted index is formed by one opaque v_not_b32 at the point of use:
// left to itself the optimiser hoists it for every unrolled entry of a tile
// (64 live registers) and spills.
__device__ __forceinline__ uint32_t inverted_index(int idx) {
  uint32_t r;
  asm volatile("v_not_b32 %0, %1" : "=v"(r) : "v"(idx));
  return r;
}

// base + i*NT + lane, recomputed at each use: left to itself the compiler
// keeps all V of these (and their bounds tests) live across the kernel.
template <int NT>
__device__ __forceinline__ int entry_index(int base, int i) {
  int idx = base + i * NT + (int)threadIdx.x;
  asm volatile("" : "+v"(idx));
  return idx;
}

// Makes the compiler treat every value of x as newly produced here (no code
// is emitted), so that values derived from x earlier are recomputed rather
// than held in registers across a long stretch.
template <int V>
__device__ __forceinline__ void opaque(float (&x)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) asm volatile("" : "+v"(x[i]));
}

__device__ __forceinline__ uint64_t composite_key(float v, int idx) {
  return ((uint64_t)key32_of(v) << 32) | inverted_index(idx);
}

__device__ __forceinline__ int index_of(uint64_t key) { return (int)(~(uint32_t)key); }

// Reserves a slot per lane with `p` set, one atomic per wave.  All 64 lanes
// must call.  Returns the slot for lanes with `p` (undefined otherwise).
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, bool p) {
  const uint64_t mask = __ballot(p);
  const uint32_t n = (uint32_t)__popcll(mask);
  uint32_t base = 0;
  if (n != 0) {
    if (lane_id() == 0) base = atomicAdd(counter, n);
    base = readlane(base, 0);
  }
  return base + lanes_below(mask);
}

// One wave: over the NB counts h[0..NB) (NB a power of two <= 1024), the
// largest bin T whose suffix count reaches m, and the count strictly above
// T.  Lane L owns the L-th group of NB/64 bins from the top.  Returns T = 0,
// above = 0 if no bin qualifies (m above the total: a misuse).
template <int NB>
__device__ __forceinline__ void wave_threshold(const uint32_t* h, uint32_t m, uint32_t& T, uint32_t& above) {
  constexpr int PER = NB >= 64 ? NB / 64 : 1;
  const int lane = lane_id();
  const int top = NB - lane * PER;  // this lane's bins: top-PER .. top-1
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = top - 1 - i >= 0 ? h[top - 1 - i] : 0u;
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) t += c[i];
  const uint32_t incl = wave_incl_scan(t);
  const uint32_t excl = incl - t;
  const bool mine = top > 0 && excl < m && incl >= m;
  const uint64_t owners = __ballot(mine);
  uint32_t bt = 0, ba = 0, acc = excl;
  bool found = false;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool hit = !found && acc + c[i] >= m;
    bt = hit ? (uint32_t)(top - 1 - i) : bt;
    ba = hit ? acc : ba;
    found = found || hit;
    acc += c[i];
  }
  const int owner = owners ? (int)__ffsll((unsigned long long)owners) - 1 : 0;
  T = owners ? readlane(bt, owner) : 0u;
  above = owners ? readlane(ba, owner) : 0u;
}

// Block-wide exclusive prefix sum of one value per lane (all lanes call);
// `total` gets the block's sum.  Two barriers.
template <int NT, int CAP>
__device__ __forceinline__ uint32_t block_excl_scan(TopkShared<CAP>& s, uint32_t x, uint32_t& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(x);
  if (lane == 63) s.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = s.wave_tot[w];
    off += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + incl - x;
}

// Translation of the refinement's winners as they are emitted: a winner at
// selection position q holding block j fills output entries q*c .. q*c+c-1
// (positions c*j + u, slots page*64 + (c*j + u) mod 64, page read from the
// request's page-table row; -1 for an invalid block or page).  pt == nullptr:
// no translation.
struct WinnerTr {
  const int32_t* pt;
  int c, nv, pt_stride;
  int32_t* orow;
  int32_t* prow;  // may be nullptr
};

// The whole workgroup resolves the boundary bin from s.cand[0..nc) (nc > need
// >= 1, nc <= CAP): each lane holds up to PER candidates in registers
// (candidate i*NT + lane).  An exact MSB-first radix selection on the 64-bit
// keys, 8-bit digits after the bits all candidates share: per pass every lane
// adds its matching candidates to an LDS digit histogram, one barrier, then
// every wave finds the same digit from that histogram by itself.  Three digit
// buffers rotate (in s.hist, free once the threshold bin is known), so one
// barrier per pass suffices: the buffer pass p + 1 fills was last read in
// pass p - 2 and is cleared during pass p.  The `need` winners are
// emitted by count, block scan, write at out[base ...] (and chosen[base ...]);
// with translation each lane reads the page ids of its own candidates before
// the passes and writes the winners' slots as it emits them.
template <int NT, int CAP, int PER>
__device__ __forceinline__ void block_refine_per(TopkShared<CAP>& s, uint32_t nc, uint32_t need,
                                                 int32_t* __restrict__ out, int32_t* chosen, uint32_t base, int limit,
                                                 const WinnerTr& wt) {
  static_assert(3 * 256 <= kBins, "three digit buffers fit in the histogram's storage");
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t* const dig = s.hist;
  uint64_t key[PER];
  int pg[PER];
  uint64_t a = ~0ull, o = 0ull;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t j = (uint32_t)(i * NT + tid);
    key[i] = j < nc ? s.cand[j] : 0ull;
    if (j < nc) {
      a &= key[i];
      o |= key[i];
    }
  }
  if (wt.pt) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = index_of(key[i]);
      const int p0 = wt.c * idx;
      pg[i] = -1;
      if ((uint32_t)(i * NT + tid) < nc && idx >= 0 && idx < wt.nv && (p0 >> 6) < wt.pt_stride) pg[i] = wt.pt[p0 >> 6];
    }
  }
  a = wave_and64(a);
  o = wave_or64(o);
  if (lane_id() == 0) {
    s.red_and[wave] = a;
    s.red_or[wave] = o;
  }
  for (int i = tid; i < 512; i += NT) dig[i] = 0;  // buffers 0 and 1
  __syncthreads();
  a = ~0ull;
  o = 0ull;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    a &= s.red_and[w];
    o |= s.red_or[w];
  }
  const uint64_t diff = a ^ o;
  int hb = diff ? 63 - __clzll((long long)diff) : 0;
  uint64_t mask = ~((2ull << hb) - 1ull);
  uint64_t prefix = o & mask;
  uint32_t remaining = need;
  for (int pass = 0;; ++pass) {
    const int width = hb + 1 < 8 ? hb + 1 : 8;
    const int shift = hb + 1 - width;
    const int nb = 1 << width;
    uint32_t* const cur = dig + 256 * (pass % 3);
    // The buffer the next pass fills was last read in pass - 2, before the
    // previous barrier; buffers 0 and 1 start cleared.
    uint32_t* const next = dig + 256 * ((pass + 1) % 3);
    if (pass >= 1)
      for (int i = tid; i < 256; i += NT) next[i] = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((uint32_t)(i * NT + tid) < nc && (key[i] & mask) == prefix)
        atomicAdd(&cur[(key[i] >> shift) & (uint64_t)(nb - 1)], 1u);
    __syncthreads();
    uint32_t d, ab;
    wave_threshold<256>(cur, remaining, d, ab);
    remaining -= ab;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)(nb - 1) << shift;
    if (cur[d] == remaining || shift == 0) break;
    hb = shift - 1;
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) cnt += ((uint32_t)(i * NT + tid) < nc && (key[i] & mask) >= prefix) ? 1u : 0u;
  uint32_t total;
  uint32_t pos = base + block_excl_scan<NT>(s, cnt, total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if ((uint32_t)(i * NT + tid) < nc && (key[i] & mask) >= prefix) {
      if (pos < (uint32_t)limit) {
        const int idx = index_of(key[i]);
        if (out) out[pos] = idx;
        if (chosen) chosen[pos] = idx;
        if (wt.pt) {
          const bool valid = idx >= 0 && idx < wt.nv;
          const int p0 = wt.c * idx;
          for (int u = 0; u < wt.c; ++u) {
            wt.orow[pos * wt.c + u] = pg[i] >= 0 ? pg[i] * kPage + ((p0 + u) & (kPage - 1)) : -1;
            if (wt.prow) wt.prow[pos * wt.c + u] = valid ? p0 + u : -1;
          }
        }
      }
      ++pos;
    }
  }
}

// Holds just as many candidates per lane as nc needs.  All lanes call.
// Small boundary lists: candidate j (lane j) counts the candidates whose
// composite key exceeds its own; keys are unique, so that rank is its exact
// place in the boundary bin's order, and the `need` best take the positions
// base + rank.  One pass over the list per lane, read from LDS as broadcasts;
// no barrier inside, no atomics.  The same set as the radix refinement.
// Used where a row's latency decides the launch (the 512- and 1,024-lane
// shapes: one 2,048-entry row 10.4 -> 8.1 us); in the many-rows shape, whose
// throughput is the limit, the radix passes measured slightly faster.
constexpr int kRankMax = 256;

template <int NT, int CAP>
__device__ __forceinline__ void rank_refine(TopkShared<CAP>& s, uint32_t nc, uint32_t need,
                                            int32_t* __restrict__ out, int32_t* chosen, uint32_t base) {
  const uint32_t tid = threadIdx.x;
  if (tid < nc) {
    const uint64_t kj = s.cand[tid];
    uint32_t rank = 0, i = 0;
    for (; i + 4 <= nc; i += 4)
      rank += (uint32_t)(s.cand[i] > kj) + (uint32_t)(s.cand[i + 1] > kj) + (uint32_t)(s.cand[i + 2] > kj) +
              (uint32_t)(s.cand[i + 3] > kj);
    for (; i < nc; ++i) rank += (uint32_t)(s.cand[i] > kj);
    if (rank < need) {
      const int idx = index_of(kj);
      if (out) out[base + rank] = idx;
      if (chosen) chosen[base + rank] = idx;
    }
  }
}

template <int NT, int CAP>
__device__ __forceinline__ void block_refine(TopkShared<CAP>& s, uint32_t nc, uint32_t need, int32_t* __restrict__ out,
                                             int32_t* chosen, uint32_t base, int limit,
                                             const WinnerTr& wt = WinnerTr{}) {
  constexpr int PMAX = (CAP + NT - 1) / NT;
  if (PMAX > 1 && nc <= (uint32_t)NT) block_refine_per<NT, CAP, 1>(s, nc, need, out, chosen, base, limit, wt);
  else if (PMAX > 2 && nc <= 2u * NT) block_refine_per<NT, CAP, 2>(s, nc, need, out, chosen, base, limit, wt);
  else if (PMAX > 4 && nc <= 4u * NT) block_refine_per<NT, CAP, 4>(s, nc, need, out, chosen, base, limit, wt);
  else block_refine_per<NT, CAP, PMAX>(s, nc, need, out, chosen, base, limit, wt);
}

// Block-wide fallback when the boundary bin overflows the LDS list: radix
// passes re-read the row (entries in bin T), the digit histogram is built by
// every lane, the decisions are taken by wave 0.  Rare (tie storms).
template <int NT, int CAP>
__device__ __forceinline__ void block_refine_from_row(TopkShared<CAP>& s, const float* __restrict__ row, int n, uint32_t T,
                                      uint32_t need, int32_t* __restrict__ out, int32_t* chosen, int limit) {
  __shared__ uint64_t red_and[NT / 64], red_or[NT / 64];
  const int tid = threadIdx.x, wave = tid >> 6;
  uint64_t a = ~0ull, o = 0ull;
  for (int i = tid; i < n; i += NT) {
    const float v = row[i];
    if (bin_of(v) == T) {
      const uint64_t key = composite_key(v, i);
      a &= key;
      o |= key;
    }
  }
  a = wave_and64(a);
  o = wave_or64(o);
  if (lane_id() == 0) {
    red_and[wave] = a;
    red_or[wave] = o;
  }
  __syncthreads();
  a = ~0ull;
  o = 0ull;
  for (int w = 0; w < NT / 64; ++w) {
    a &= red_and[w];
    o |= red_or[w];
  }
  const uint64_t diff = a ^ o;
  int hb = diff ? 63 - __clzll((long long)diff) : 0;
  uint64_t mask = ~((2ull << hb) - 1ull);
  uint64_t prefix = o & mask;
  uint32_t remaining = need;
  for (;;) {
    const int width = hb + 1 < 8 ? hb + 1 : 8;
    const int shift = hb + 1 - width;
    const int nb = 1 << width;
    for (int i = tid; i < 256; i += NT) s.digit[i] = 0;  // bins past nb stay 0
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const float v = row[i];
      if (bin_of(v) == T) {
        const uint64_t key = composite_key(v, i);
        if ((key & mask) == prefix) atomicAdd(&s.digit[(key >> shift) & (uint64_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t d, ab;
      wave_threshold<256>(s.digit, remaining, d, ab);
      if (lane_id() == 0) {
        s.T = d;
        s.above = ab;
      }
    }
    __syncthreads();
    const uint32_t d = s.T;
    remaining -= s.above;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)(nb - 1) << shift;
    const bool settled = s.digit[d] == remaining;
    __syncthreads();
    if (settled || shift == 0) break;
    hb = shift - 1;
  }
  for (int b0 = 0; b0 < n; b0 += NT) {
    const int i = b0 + tid;
    bool p = false;
    if (i < n) {
      const float v = row[i];
      p = bin_of(v) == T && (composite_key(v, i) & mask) >= prefix;
    }
    const uint32_t pos = wave_reserve(&s.emit, p);
    if (p && pos < (uint32_t)limit) {
      if (out) out[pos] = i;
      if (chosen) chosen[pos] = i;
    }
  }
  __syncthreads();
}

// Emits the V values this lane holds (entry i is row[base + i*NT + lane]):
// above-threshold indices go to out[] (and chosen[]), boundary-bin entries
// become composite keys in s.cand.  Each lane counts its own matches, one
// block scan of the packed counts (above << 20 | boundary) hands out the
// positions, then plain writes: no atomics.  up_pos / cand_pos carry the
// running totals across tiles.
template <int NT, int V, int CAP>
__device__ __forceinline__ void emit_tile(TopkShared<CAP>& s, float (&x)[V], int base, int n, uint32_t T,
                                          uint32_t& up_pos, uint32_t& cand_pos, int m, int32_t* __restrict__ out,
                                          bool keep) {
  uint32_t nup = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int idx = entry_index<NT>(base, i);
    const uint32_t b = bin_of(x[i]);
    nup += (idx < n && b > T) ? 1u : 0u;
    neq += (idx < n && b == T) ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<NT>(s, (nup << 20) | neq, total);
  uint32_t pu = up_pos + (excl >> 20), pe = cand_pos + (excl & 0xFFFFFu);
  opaque(x);  // the bins are recomputed below, not kept live across the scan
#pragma unroll
  for (int i = 0; i < V; ++i) {
    __builtin_amdgcn_sched_barrier(0);  // keep one entry's work live at a time
    const int idx = entry_index<NT>(base, i);
    if (idx < n) {
      const uint32_t b = bin_of(x[i]);
      if (b > T) {
        if (pu < (uint32_t)m) {
          if (out) out[pu] = idx;
          if (keep) s.chosen[pu] = idx;
        }
        ++pu;
      } else if (b == T) {
        if (pe < (uint32_t)CAP) s.cand[pe] = composite_key(x[i], idx);
        ++pe;
      }
    }
  }
  up_pos += total >> 20;
  cand_pos += total & 0xFFFFFu;
}

template <int CAP>
__device__ __forceinline__ void threshold_to_shared(TopkShared<CAP>& s, uint32_t m) {
  if ((threadIdx.x >> 6) == 0) {
    uint32_t T, ab;
    wave_threshold<kBins>(s.hist, m, T, ab);
    if (lane_id() == 0) {
      s.T = T;
      s.above = ab;
    }
  }
  __syncthreads();
}

// One workgroup selects a whole row with n > m.  Rows of up to NT*V entries
// are read once and held in registers; longer rows are streamed: once for
// the histogram (skipped when it is ready), once in NT*V-entry tiles for
// emission.  HIST_READY: s.hist
// already holds the row's histogram (long-row finisher).  All lanes call.
template <int NT, int V, int CAP, bool HIST_READY, bool STREAM, class PF>
__device__ __forceinline__ void select_row(TopkShared<CAP>& s, const float* __restrict__ row, int n, int m,
                                           int32_t* __restrict__ out, bool keep, PF& pf) {
  constexpr int kTile = V;
  const int tid = threadIdx.x;
  if (!HIST_READY)
    for (int i = tid; i < kBins; i += NT) s.hist[i] = 0;
  __syncthreads();
  uint32_t up_pos = 0, cand_pos = 0;
  uint32_t T, above;
  const RowReader rd(row, n);
  if (!STREAM || n <= NT * V) {  // !STREAM: the caller guarantees n <= NT*V
    static_assert(V <= 64, "one mask bit per register entry");
    // Register path.  The entries' bins are kept, two 16-bit codes per
    // register (code = bin + 1, 0 past the row), not the FP32 values: after
    // the threshold, two bit masks mark the entries above and in the
    // boundary bin, and only the marked entries are visited.  Boundary
    // entries are re-read by index when their exact keys are needed.
    // Entries are handled in pairs (x[2p], x[2p+1]) with packed 16-bit
    // arithmetic: two bins per conversion, and a pair is checked against
    // the row length once for the whole workgroup unless it straddles the
    // row's end.
    static_assert(V % 2 == 0, "entries are binned in pairs");
    constexpr int P = V / 2;
    uint32_t pb[P];
    float x[V];
#pragma unroll
    for (int i = 0; i < V; ++i) x[i] = rd.at(tid, i * NT);  // every load in flight at once
    pf.issue();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (p % 4 == 0) __builtin_amdgcn_sched_barrier(0);  // a few bins live at a time
      const uint32_t B = bin_pair(x[2 * p], x[2 * p + 1]);
      uint32_t code;
      if ((2 * p + 2) * NT <= n) {  // the whole pair lies inside the row, for every lane
        if (!HIST_READY) {
          atomicAdd(&s.hist[B & 0xFFFFu], 1u);
          atomicAdd(&s.hist[B >> 16], 1u);
        }
        code = B + 0x00010001u;
      } else {
        const bool ok0 = entry_index<NT>(0, 2 * p) < n, ok1 = entry_index<NT>(0, 2 * p + 1) < n;
        if (!HIST_READY && ok0) atomicAdd(&s.hist[B & 0xFFFFu], 1u);
        if (!HIST_READY && ok1) atomicAdd(&s.hist[B >> 16], 1u);
        code = (ok0 ? (B & 0xFFFFu) + 1u : 0u) | (ok1 ? (B & 0xFFFF0000u) + 0x00010000u : 0u);
      }
      asm volatile("" : "+v"(code));  // packed here, not sunk past the loop
      pb[p] = code;
    }
    pf.commit(s);
    __syncthreads();
    threshold_to_shared(s, (uint32_t)m);
    T = s.T;
    above = s.above;
    // Bit i of upm / eqm: entry i's code (bin + 1) above / equal to T + 1.
    // Per pair, the 0/1 flags of both halves are placed by one dot product
    // with the halves' bit weights, 16 bits (8 pairs) per word.
    const uint32_t tgt = (T + 1u) * 0x00010001u, tge = T * 0x00010001u;
    uint32_t upw[(P + 7) / 8], gew[(P + 7) / 8];
#pragma unroll
    for (int w = 0; w < (P + 7) / 8; ++w) upw[w] = gew[w] = 0u;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const bs_ushort2 wt = {(uint16_t)(1u << (2 * (p % 8))), (uint16_t)(2u << (2 * (p % 8)))};
      upw[p / 8] = __builtin_amdgcn_udot2(__builtin_bit_cast(bs_ushort2, pk_gt_flags(pb[p], tgt)), wt, upw[p / 8], false);
      gew[p / 8] = __builtin_amdgcn_udot2(__builtin_bit_cast(bs_ushort2, pk_gt_flags(pb[p], tge)), wt, gew[p / 8], false);
    }
    uint64_t upm = 0, eqm = 0;
#pragma unroll
    for (int w = 0; w < (P + 7) / 8; ++w) {
      upm |= (uint64_t)upw[w] << (16 * w);
      eqm |= (uint64_t)(gew[w] & ~upw[w]) << (16 * w);
    }
    const uint32_t nup = (uint32_t)__popcll(upm), neq = (uint32_t)__popcll(eqm);
    uint32_t total;
    const uint32_t excl = block_excl_scan<NT>(s, (nup << 20) | neq, total);
    uint32_t pu = excl >> 20, pe = excl & 0xFFFFFu;
    while (upm) {
      const int i = __builtin_ctzll(upm);
      upm &= upm - 1;
      if (pu < (uint32_t)m) {
        const int idx = i * NT + tid;
        if (out) out[pu] = idx;
        if (keep) s.chosen[pu] = idx;
      }
      ++pu;
    }
    while (eqm) {
      const int i = __builtin_ctzll(eqm);
      eqm &= eqm - 1;
      if (pe < (uint32_t)CAP) s.cand[pe] = (uint64_t)(uint32_t)(i * NT + tid);  // index only, for now
      ++pe;
    }
    up_pos = total >> 20;
    cand_pos = total & 0xFFFFFu;
    __syncthreads();
    // Exact keys of the listed boundary entries, when a refinement needs them.
    const uint32_t nc = cand_pos, need = (uint32_t)m - above;
    if (nc <= (uint32_t)CAP && need < nc) {
      for (uint32_t j = tid; j < nc; j += NT) {
        const int idx = (int)(uint32_t)s.cand[j];
        s.cand[j] = composite_key(rd[idx], idx);
      }
    } else if (nc <= (uint32_t)CAP) {
      for (uint32_t j = tid; j < nc; j += NT) {
        const int idx = (int)(uint32_t)s.cand[j];
        s.cand[j] = (uint64_t)inverted_index(idx);  // index_of() reads the low word
      }
    }
  } else {
    pf.issue();
    if (!HIST_READY) {
      for (int b0 = 0; b0 < n; b0 += NT * 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = rd[b0 + j * NT + tid];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (b0 + j * NT + tid < n) atomicAdd(&s.hist[bin_of(x[j])], 1u);
      }
    }
    pf.commit(s);
    __syncthreads();
    threshold_to_shared(s, (uint32_t)m);
    T = s.T;
    above = s.above;
    for (int b0 = 0; b0 < n; b0 += NT * kTile) {
      float x[kTile];
#pragma unroll
      for (int i = 0; i < kTile; ++i) x[i] = rd[b0 + i * NT + tid];
      emit_tile<NT, kTile>(s, x, b0, n, T, up_pos, cand_pos, m, out, keep);
    }
  }
  __syncthreads();
  const uint32_t nc = cand_pos, need = (uint32_t)m - above;
  if (need == 0 || need > (uint32_t)m) return;  // the latter only on misuse
  int32_t* chosen = keep ? s.chosen : nullptr;
  if (nc <= (uint32_t)CAP) {
    if (need >= nc) {
      for (uint32_t i = tid; i < nc; i += NT) {
        const uint32_t at = above + i;
        if (at < (uint32_t)m) {
          const int idx = index_of(s.cand[i]);
          if (out) out[at] = idx;
          if (keep) s.chosen[at] = idx;
        }
      }
    } else if (NT != kManyNT && nc <= (uint32_t)kRankMax && nc <= (uint32_t)NT) {
      rank_refine<NT, CAP>(s, nc, need, out, chosen, above);
    } else {
      block_refine<NT, CAP>(s, nc, need, out, chosen, above, m);
    }
    __syncthreads();
  } else {
    if (tid == 0) s.emit = above;
    __syncthreads();
    block_refine_from_row<NT, CAP>(s, row, n, T, need, out, chosen, m);
  }
}

// Request of row r: the number of request starts at or before r, minus one.
// All 64 lanes of the calling wave must call.
__device__ __forceinline__ int request_of(const int32_t* __restrict__ req_row_ptr, int num_req, int r) {
  int b = -1;
  for (int base = 0; base < num_req; base += 64) {
    const int bi = base + lane_id();
    const bool started = bi < num_req && req_row_ptr[bi] <= r;
    b += __popcll(__ballot(started));
  }
  return max(0, min(b, num_req - 1));
}

// Fused translation.  Selection position q of row r holding block j becomes
// output entries q*c .. q*c+c-1 (positions c*j .. c*j+c-1); after the m
// chosen blocks come the pending positions c*n_vis .. t, then -1.  slot =
// page_table[b][pos/64]*64 + pos mod 64 (-1 for an invalid block or page).
struct RowGeom {
  int b, t, nv, p;
};

__device__ __forceinline__ RowGeom row_geometry(const Translate& tr, int r) {
  RowGeom g;
  g.b = request_of(tr.req_row_ptr, tr.num_req, r);
  g.t = tr.row_pos[r];
  g.nv = g.t >= 0 ? (g.t + 1) / tr.c : 0;
  g.p = g.t >= 0 ? g.t + 1 - tr.c * g.nv : 0;
  return g;
}

// The same, split so that its reads can be issued long before the values
// are needed: start() reads the row's position and the first 64 request
// starts (one per lane), finish() turns them into the geometry (all 64
// lanes of each wave call both; requests past the first 64 are read there).
struct RowGeomReads {
  int t, start;
};

__device__ __forceinline__ RowGeomReads row_geometry_start(const Translate& tr, int r) {
  const int bi = lane_id();
  return RowGeomReads{tr.row_pos[r], bi < tr.num_req ? tr.req_row_ptr[bi] : 0x7FFFFFFF};
}

__device__ __forceinline__ RowGeom row_geometry_finish(const Translate& tr, int r, const RowGeomReads& rd) {
  int b = __popcll(__ballot(rd.start <= r)) - 1;
  for (int base = 64; base < tr.num_req; base += 64) {
    const int bi = base + lane_id();
    b += __popcll(__ballot(bi < tr.num_req && tr.req_row_ptr[bi] <= r));
  }
  RowGeom g;
  g.b = max(0, min(b, tr.num_req - 1));
  g.t = rd.t;
  g.nv = g.t >= 0 ? (g.t + 1) / tr.c : 0;
  g.p = g.t >= 0 ? g.t + 1 - tr.c * g.nv : 0;
  return g;
}

__device__ __forceinline__ void put_slot(const Translate& tr, const RowGeom& g, int r, int i, int pos) {
  int slot = -1;
  if (pos >= 0 && (pos >> 6) < tr.pt_stride) {
    const int page = tr.page_table[(int64_t)g.b * tr.pt_stride + (pos >> 6)];
    slot = page >= 0 ? page * kPage + (pos & (kPage - 1)) : -1;
  }
  tr.out_slots[(int64_t)r * tr.ld_out + i] = slot;
  if (tr.out_pos) tr.out_pos[(int64_t)r * tr.ld_out + i] = pos;
}

// Output entries of selection position q (block j): the block's c positions
// lie in one page, so one page-table read serves them all.
__device__ __forceinline__ void translate_block(const Translate& tr, const RowGeom& g, int r, int q, int j) {
  const int c = tr.c;
  const bool valid = j >= 0 && j < g.nv;
  const int p0 = c * j;
  int page = -1;
  if (valid && (p0 >> 6) < tr.pt_stride) page = tr.page_table[(int64_t)g.b * tr.pt_stride + (p0 >> 6)];
  int32_t* orow = tr.out_slots + (int64_t)r * tr.ld_out + q * c;
  int32_t* prow = tr.out_pos ? tr.out_pos + (int64_t)r * tr.ld_out + q * c : nullptr;
  for (int u = 0; u < c; ++u) {
    orow[u] = page >= 0 ? page * kPage + ((p0 + u) & (kPage - 1)) : -1;
    if (prow) prow[u] = valid ? p0 + u : -1;
  }
}

// Output entries from m*c on: the pending tail, then -1; and the count.
template <int NT>
__device__ __forceinline__ void translate_tail(const Translate& tr, const RowGeom& g, int r, int m) {
  const int nblk = tr.c * m, total = nblk + g.p;
  for (int i = nblk + (int)threadIdx.x; i < tr.ld_out; i += NT) put_slot(tr, g, r, i, i < total ? tr.c * g.nv + (i - nblk) : -1);
  if (threadIdx.x == 0) tr.out_count[r] = total;
}

// The whole row from chosen[0..m).  Element-major: lane l handles output
// entries l, l + NT, l + 2*NT, ..., so every store instruction of a wave
// covers 256 contiguous bytes; entry i < c*m belongs to selection position
// i / c (c is 1 or 4), entries from c*m on are the pending tail, then -1.
// Each round reads the page ids of its E entries per lane first (the c
// entries of a block share one address), then writes them.  CACHED: every
// page id comes from `cached` (LDS).  That path holds no global load at
// all: a load there, even one no lane takes, brings a wait that also waits
// for every store issued before it (vector memory operations retire in
// order), so the two cases are separate code down to the stores.
template <int NT, bool CACHED>
__device__ __forceinline__ void translate_rounds(const Translate& tr, const RowGeom& g, int r, int m,
                                                 const int32_t* chosen, const int32_t* cached, int ncached) {
  constexpr int E = 8;
  const int c = tr.c, sh = c == 4 ? 2 : 0;
  const int nblk = c * m, total = nblk + g.p;
  const int32_t* pt = tr.page_table + (int64_t)g.b * tr.pt_stride;
  int32_t* orow = tr.out_slots + (int64_t)r * tr.ld_out;
  int32_t* prow = tr.out_pos ? tr.out_pos + (int64_t)r * tr.ld_out : nullptr;
  for (int i0 = 0; i0 < tr.ld_out; i0 += E * NT) {
    int pos[E], page[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e * NT + (int)threadIdx.x;
      int ps = -1;
      if (i < nblk) {
        const int j = chosen[i >> sh];
        if (j >= 0 && j < g.nv) ps = c * j + (i & (c - 1));
      } else if (i < total) {
        ps = c * g.nv + (i - nblk);
      }
      int pg = -1;
      if (CACHED) {
        if (ps >= 0) pg = cached[ps >> 6];
      } else if (ps >= 0 && (ps >> 6) < tr.pt_stride) {
        pg = (ps >> 6) < ncached ? cached[ps >> 6] : pt[ps >> 6];
      }
      pos[e] = ps;
      page[e] = pg;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e * NT + (int)threadIdx.x;
      if (i < tr.ld_out) {
        orow[i] = page[e] >= 0 ? page[e] * kPage + (pos[e] & (kPage - 1)) : -1;
        if (prow) prow[i] = pos[e];
      }
    }
  }
  if (threadIdx.x == 0) tr.out_count[r] = total;
}

// Every position of the row lies at or before t, so when the cache holds
// page t/64 (which implies t/64 < pt_stride) no page id is read from global
// memory.  The branch is uniform.
template <int NT>
__device__ __forceinline__ void translate_row(const Translate& tr, const RowGeom& g, int r, int m,
                                              const int32_t* chosen, const int32_t* cached = nullptr,
                                              int ncached = 0) {
  if (g.t >= 0 && (g.t >> 6) < ncached)
    translate_rounds<NT, true>(tr, g, r, m, chosen, cached, ncached);
  else
    translate_rounds<NT, false>(tr, g, r, m, chosen, cached, ncached);
}

// Page ids of a row's first kRowPages logical pages, for its fused
// translation: read right after the row's scores are issued (so their
// latency hides behind the binning) and put in LDS before the barrier that
// follows it.  Without them the translation waited for page-table reads that
// also waited for the selection's stores (vector memory operations retire in
// order).  ON = false: does nothing.
template <int NT, bool ON>
struct RowPagePrefetch {
  static constexpr int PER = (kRowPages + NT - 1) / NT;
  const Translate& tr;
  int r;
  RowGeomReads gr;
  RowGeom g{};
  int np = 0;
  int32_t v[PER];
  __device__ __forceinline__ void issue() {
    if (!ON) return;
    g = row_geometry_finish(tr, r, gr);
    np = g.t >= 0 ? min((g.t >> 6) + 1, min(kRowPages, tr.pt_stride)) : 0;
    const int32_t* pt = tr.page_table + (int64_t)g.b * tr.pt_stride;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = i * NT + (int)threadIdx.x;
      v[i] = idx < np ? pt[idx] : -1;
    }
  }
  template <int CAP>
  __device__ __forceinline__ void commit(TopkShared<CAP>& s) {
    if (!ON) return;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = i * NT + (int)threadIdx.x;
      if (idx < kRowPages) s.row_pages[idx] = v[i];
    }
    if (threadIdx.x == 0) s.row_npages = (uint32_t)np;
  }
};

// The whole selection of one row by one workgroup, any n.
template <int NT, int VPT, int CAP, bool TRANSLATE, bool STREAM = true>
__device__ __forceinline__ void select_whole_row(TopkShared<CAP>& s, const float* __restrict__ row, int n, int m, int k,
                                 int32_t* __restrict__ out, int32_t* __restrict__ sel_count, int r,
                                 const Translate& tr) {
  const int tid = threadIdx.x;
  RowGeomReads gr{};
  if (TRANSLATE) gr = row_geometry_start(tr, r);  // in flight during the selection
  RowPagePrefetch<NT, TRANSLATE> pf{tr, r, gr};
  // The selection is staged in LDS and written out once it is complete: a
  // global store issued early would hold up every later wait for a load
  // (vector memory operations retire in order).
  if (m == n) {
    pf.issue();
    for (int i = tid; i < n; i += NT) s.chosen[i] = i;
    pf.commit(s);
  } else {
    select_row<NT, VPT, CAP, false, STREAM>(s, row, n, m, nullptr, true, pf);
  }
  __syncthreads();
  for (int i = tid; i < k; i += NT) out[i] = i < m ? s.chosen[i] : -1;
  if (tid == 0) sel_count[r] = m;
  if (TRANSLATE) translate_row<NT>(tr, pf.g, r, m, s.chosen, s.row_pages, (int)s.row_npages);
}

// One workgroup of NT lanes per row.  Three shapes: 1,024 lanes holding 16
// entries each when the batch has few rows (each row gets a whole CU; longer
// rows are streamed), 512 lanes holding 64 entries each for rows of up to
// 32,768 entries (two rows per CU, one pass), 256 lanes holding 64 entries
// each when it has many rows (several rows per CU, so one row's latency chain
// overlaps the others').
template <bool TRANSLATE, int NT, int VPT, int CAP>
__global__ __launch_bounds__(NT, NT == kManyNT ? 4 : NT == kMidNT ? 2 : 1) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, Translate tr) {
  __shared__ TopkShared<CAP> s;
  const int r = blockIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  const int m = min(k, n);
  // The many-rows and mid shapes are launched only for rows of at most
  // NT*VPT entries.
  select_whole_row<NT, VPT, CAP, TRANSLATE, NT == kRowNT>(s, scores + (int64_t)r * ld, n, m, k,
                                                          sel + (int64_t)r * k, sel_count, r, tr);
}

// Output entries of selection position q (block j of a long-row chunk),
// page ids from the chunk's LDS copy.
template <int C>
__device__ __forceinline__ void translate_block_lds(const Translate& tr, int r, int q, int j, const int32_t* pages,
                                                    int first_lp) {
  int32_t* orow = tr.out_slots + (int64_t)r * tr.ld_out + q * C;
  int32_t* prow = tr.out_pos ? tr.out_pos + (int64_t)r * tr.ld_out + q * C : nullptr;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int pos = C * j + u;
    const int page = pages[(pos >> 6) - first_lp];
    orow[u] = page >= 0 ? page * kPage + (pos & (kPage - 1)) : -1;
    if (prow) prow[u] = pos;
  }
}

// Few long rows, first launch: one 256-lane workgroup per 4,096-entry chunk
// merges its LDS histogram into the row's histogram with device atomics.
// Rows shorter than kLongMin are done whole by their first workgroup.
template <bool TRANSLATE>
__global__ __launch_bounds__(kLongNT) void topk_long_hist_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, uint8_t* __restrict__ ws,
    Translate tr) {
  __shared__ TopkShared<kLongCand> s;
  const int r = blockIdx.x, w = blockIdx.y, tid = threadIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  const int m = min(k, n);
  const float* row = scores + (int64_t)r * ld;
  if (n < kLongMin) {
    if (w == 0)
      select_whole_row<kLongNT, kLongVpt, kLongCand, TRANSLATE>(s, row, n, m, k, sel + (int64_t)r * k, sel_count,
                                                                 r, tr);
    return;
  }
  const int lo = w * kHistChunk;
  if (lo >= n) return;
  uint32_t* gh = reinterpret_cast<uint32_t*>(ws + (size_t)r * kWsRow + kWsHist);
  for (int i = tid; i < kBins; i += kLongNT) s.hist[i] = 0;
  const RowReader rd(row, n);
  float x[kHistPerLane];
#pragma unroll
  for (int i = 0; i < kHistPerLane; ++i) x[i] = rd.at(tid, lo + i * kLongNT);
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kHistPerLane / 2; ++p) {
    const uint32_t B = bin_pair(x[2 * p], x[2 * p + 1]);
    if (lo + (2 * p + 2) * kLongNT <= n) {  // both entries inside the row, for every lane
      atomicAdd(&s.hist[B & 0xFFFFu], 1u);
      atomicAdd(&s.hist[B >> 16], 1u);
    } else {
      if (lo + 2 * p * kLongNT + tid < n) atomicAdd(&s.hist[B & 0xFFFFu], 1u);
      if (lo + (2 * p + 1) * kLongNT + tid < n) atomicAdd(&s.hist[B >> 16], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < kBins; i += kLongNT) {
    const uint32_t cnt = s.hist[i];
    if (cnt != 0) __hip_atomic_fetch_add(&gh[i], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Few long rows, second launch.  Every chunk's workgroup reads the merged
// histogram, finds the threshold bin, emits (and translates) its own
// above-threshold entries through one device atomic per workgroup, and
// appends its boundary-bin entries to the row's candidate list with
// device-scope stores.  It waits for those stores to complete and arrives on
// the row's counter; the last to arrive resolves the boundary bin from the
// candidate list (read back with device-scope loads), writes the pending tail
// and leaves the row's workspace zero-filled.  No fence, no spin.
template <bool TRANSLATE>
__global__ __launch_bounds__(kLongNT) void topk_long_emit_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, uint8_t* __restrict__ ws,
    Translate tr) {
  __shared__ TopkShared<kLongCand> s;
  const int r = blockIdx.x, w = blockIdx.y, tid = threadIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  if (n < kLongMin) return;
  const int lo = w * kChunk;
  if (lo >= n) return;
  const int nchunk = (n + kChunk - 1) / kChunk;
  const int m = k;  // n > 2048 >= k
  const float* row = scores + (int64_t)r * ld;
  int32_t* out = sel + (int64_t)r * k;
  uint8_t* rec = ws + (size_t)r * kWsRow;
  uint32_t* gh = reinterpret_cast<uint32_t*>(rec + kWsHist);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(rec + kWsCtr);
  uint64_t* gcand = reinterpret_cast<uint64_t*>(rec + kWsCand);

  const RowReader rd(row, n);
  float x[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) x[i] = rd[lo + i * kLongNT + tid];
  for (int i = tid; i < kBins; i += kLongNT) s.hist[i] = gh[i];
  RowGeom g{};
  int first_lp = 0;
  if (TRANSLATE) {
    // The chunk's blocks [lo, lo + kChunk) cover at most kChunkPages logical pages.
    g = row_geometry(tr, r);
    first_lp = (tr.c * lo) >> 6;
    for (int i = tid; i < kChunkPages; i += kLongNT) {
      const int lp = first_lp + i;
      s.pages[i] = lp < tr.pt_stride ? tr.page_table[(int64_t)g.b * tr.pt_stride + lp] : -1;
    }
  }
  __syncthreads();
  threshold_to_shared(s, (uint32_t)m);
  const uint32_t T = s.T, above = s.above;

  // Count, block scan, one device atomic per list for the workgroup.
  uint32_t nup = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const bool valid = lo + i * kLongNT + tid < n;
    const uint32_t b = bin_of(x[i]);
    nup += (valid && b > T) ? 1u : 0u;
    neq += (valid && b == T) ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<kLongNT>(s, (nup << 20) | neq, total);
  // The list offsets are reserved first and published after the staging
  // below, so the atomics' round trip overlaps it.
  uint32_t bu, bc;  // read by lane 0 only
  if (tid == 0) {
    bu = __hip_atomic_fetch_add(&ctr[1], total >> 20, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bc = __hip_atomic_fetch_add(&ctr[2], total & 0xFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Stage this workgroup's picks in LDS at their scanned offsets (the
  // running per-lane counters keep each lane's picks in index order), then
  // write them out with all lanes: coalesced stores, no divergent loop.
  uint32_t lu = excl >> 20, le = excl & 0xFFFFFu;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int idx = lo + i * kLongNT + tid;
    if (idx < n) {
      const uint32_t b = bin_of(x[i]);
      if (b > T) {
        if (lu < (uint32_t)kKmax) s.chosen[lu] = idx;
        ++lu;
      } else if (b == T) {
        if (le < (uint32_t)kLongCand) s.cand[le] = composite_key(x[i], idx);
        ++le;
      }
    }
  }
  if (tid == 0) {
    s.base_up = bu;
    s.base_cand = bc;
  }
  __syncthreads();
  const uint32_t tot_up = min(total >> 20, (uint32_t)kKmax), tot_eq = min(total & 0xFFFFFu, (uint32_t)kLongCand);
  for (uint32_t j = tid; j < tot_up; j += kLongNT) {
    const uint32_t pos = s.base_up + j;
    if (pos < (uint32_t)m) {
      const int idx = s.chosen[j];
      out[pos] = idx;
      if (TRANSLATE) {
        if (tr.c == 1) translate_block_lds<1>(tr, r, (int)pos, idx, s.pages, first_lp);
        else translate_block_lds<4>(tr, r, (int)pos, idx, s.pages, first_lp);
      }
    }
  }
  for (uint32_t j = tid; j < tot_eq; j += kLongNT) {
    const uint32_t cpos = s.base_cand + j;
    if (cpos < (uint32_t)kLongCand)
      __hip_atomic_store(&gcand[cpos], s.cand[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Every lane's candidate stores have completed before the chunk arrives.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s.last = __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(nchunk - 1);
  __syncthreads();
  if (!s.last) return;

  // The last chunk to arrive resolves the boundary bin.  The head of the
  // candidate list is read together with its length (one round trip); the
  // list's storage holds kLongCand entries, those past the length are unused.
  constexpr int kSpec = 4;
  static_assert(kSpec * kLongNT <= kLongCand, "speculative reads stay inside the list");
  uint64_t head[kSpec];
#pragma unroll
  for (int t = 0; t < kSpec; ++t)
    head[t] = __hip_atomic_load(&gcand[t * kLongNT + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t nc = __hip_atomic_load(&ctr[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t need = (uint32_t)m - above;
  if (nc <= (uint32_t)kLongCand) {
#pragma unroll
    for (int t = 0; t < kSpec; ++t)
      if ((uint32_t)(t * kLongNT + tid) < nc) s.cand[t * kLongNT + tid] = head[t];
    for (int i = kSpec * kLongNT + tid; i < (int)nc; i += kLongNT)
      s.cand[i] = __hip_atomic_load(&gcand[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  bool translated = false;
  if (need >= 1 && need <= (uint32_t)m) {
    if (nc <= (uint32_t)kLongCand) {
      if (need >= nc) {
        for (uint32_t i = tid; i < nc; i += kLongNT) {
          const uint32_t at = above + i;
          if (at < (uint32_t)m) {
            const int idx = index_of(s.cand[i]);
            out[at] = idx;
            s.chosen[at] = idx;
          }
        }
      } else {
        WinnerTr wt{};
        if (TRANSLATE)
          wt = WinnerTr{tr.page_table + (int64_t)g.b * tr.pt_stride, tr.c, g.nv, tr.pt_stride,
                        tr.out_slots + (int64_t)r * tr.ld_out,
                        tr.out_pos ? tr.out_pos + (int64_t)r * tr.ld_out : nullptr};
        block_refine<kLongNT, kLongCand>(s, nc, need, out, s.chosen, above, m, wt);
        translated = TRANSLATE;
      }
      __syncthreads();
    } else {
      if (tid == 0) s.emit = above;
      __syncthreads();
      block_refine_from_row<kLongNT, kLongCand>(s, row, n, T, need, out, s.chosen, m);
    }
  }
  if (tid == 0) sel_count[r] = m;
  if (TRANSLATE) {
    if (!translated)
      for (int q = (int)above + tid; q < m; q += kLongNT) translate_block(tr, g, r, q, s.chosen[q]);
    translate_tail<kLongNT>(tr, g, r, m);
  }
  // Leave the row's workspace zero-filled for the next call.
  for (int i = tid; i < kBins; i += kLongNT) __hip_atomic_store(&gh[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid < 16) __hip_atomic_store(&ctr[tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int used = (int)min(nc, (uint32_t)kLongCand);
  for (int i = tid; i < used; i += kLongNT)
    __hip_atomic_store(&gcand[i], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static bool use_long_path(int32_t num_rows, int32_t max_len) {
  return max_len >= kLongMin && num_rows <= kLongRowsMax;
}

size_t topk_workspace_size(int32_t num_rows, int32_t max_len, int32_t /*k*/) {
  return use_long_path(num_rows, max_len) ? (size_t)num_rows * kWsRow : 0;
}

template <bool TRANSLATE>
static int launch_select(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows, int32_t max_len,
                         int32_t k, int32_t* sel, int32_t* sel_count, void* workspace, const Translate& tr,
                         hipStream_t stream) {
  if (use_long_path(num_rows, max_len)) {
    const int nchunk = (max_len + kChunk - 1) / kChunk;
    const int nhist = (max_len + kHistChunk - 1) / kHistChunk;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipLaunchKernelGGL(topk_long_hist_kernel<TRANSLATE>, dim3(num_rows, nhist), dim3(kLongNT), 0, stream, scores,
                       ld, row_len, max_len, k, sel, sel_count, ws, tr);
    if (hipGetLastError() != hipSuccess) return BS_ERR_LAUNCH;
    hipLaunchKernelGGL(topk_long_emit_kernel<TRANSLATE>, dim3(num_rows, nchunk), dim3(kLongNT), 0, stream, scores,
                       ld, row_len, max_len, k, sel, sel_count, ws, tr);
  } else if (num_rows >= kManyMinRows && max_len <= kManyNT * kManyVpt) {
    hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kManyNT, kManyVpt, kManyCand>), dim3(num_rows), dim3(kManyNT), 0,
                       stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  } else if (max_len > kRowNT * kRowVpt && max_len <= kMidNT * kMidVpt) {
    hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kMidNT, kMidVpt, kMidCand>), dim3(num_rows), dim3(kMidNT), 0,
                       stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  } else {
    hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kRowNT, kRowVpt, kRowCand>), dim3(num_rows), dim3(kRowNT), 0,
                       stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  }
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

int launch_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows, int32_t max_len,
                int32_t k, int32_t* sel, int32_t* sel_count, void* workspace, hipStream_t stream) {
  const Translate none{};
  return launch_select<false>(scores, ld, row_len, num_rows, max_len, k, sel, sel_count, workspace, none, stream);
}

int launch_select_translate(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows,
                            int32_t max_len, int32_t k, const int32_t* req_row_ptr, int32_t num_req,
                            const int32_t* row_pos, int32_t c, const int32_t* page_table, int32_t pt_stride,
                            int32_t* sel, int32_t* sel_count, int32_t* out_slots, int32_t* out_pos,
                            int32_t* out_count, int32_t ld_out, void* workspace, hipStream_t stream) {
  const Translate tr{req_row_ptr, num_req, row_pos, c, page_table, pt_stride, out_slots, out_pos, out_count, ld_out};
  return launch_select<true>(scores, ld, row_len, num_rows, max_len, k, sel, sel_count, workspace, tr, stream);
}

}  // namespace bs
