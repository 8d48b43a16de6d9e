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
//   * rows shorter than 32,769 entries: one workgroup per row, the row held
//     in registers: 512 lanes x 4 values for rows of up to 2,048 entries in
//     small batches, 1,024 lanes x 16 values (longer rows streamed twice),
//     512 lanes x 64 values for rows of up to 32,768 entries (read 16 bytes
//     per lane when the rows start aligned), or, for batches of at least
//     1,024 rows of at most 16,384 entries, 256 lanes x 64 values so that
//     several rows share a CU.  The register path keeps each entry's bin, not
//     its value, and marks the entries above and in the boundary bin with two
//     bit masks;
//   * long rows (>= 32,769 entries, any number of rows): one launch, one
//     512-lane workgroup per 8,192-entry chunk, the chunk in registers (the
//     launch's rows shorter than that are each selected whole by their first
//     workgroup).  In place of the cluster's merged histogram, each chunk
//     builds its own histogram and keeps as candidates every entry at or
//     above the bin of its local q-th largest, q a little above the chunk's
//     expected share of the row's top k; it publishes them with its
//     histogram and bin floor and arrives on the row's counter.  The last
//     chunk to arrive sums the published histograms, finds the threshold
//     bin, emits the candidates above it and refines the boundary bin
//     exactly.  The candidates are the whole row at and above the threshold
//     bin whenever that bin is not below any chunk's floor (checked;
//     otherwise the same workgroup selects the whole row by streaming it), so
//     the result is exact in every case.  No workgroup waits on another (no
//     co-residency assumption) and no device-scope fence is issued: on
//     gfx950 such a fence writes back and invalidates the per-XCD L2, which
//     measured far costlier than the whole kernel;
//   * planned (the blog's planning kernel): one small kernel turns the row
//     lengths into a work list of whole-row and chunk items and picks the
//     length from which rows are split; the selection then runs one
//     workgroup per item, reading each row only up to its length, and every
//     call on the same lengths reuses the list;
//   * emission is count, block scan, write (no per-entry atomics); the
//     threshold is found block-wide (each lane scans its share of the bins
//     with DPP, the wave totals meet in LDS); the boundary refinement costs
//     one workgroup barrier per 8-bit radix pass.
#include <algorithm>
#include <atomic>

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
constexpr int kSmallNT = 512;                  // row kernel for short rows in small batches: lanes per workgroup
constexpr int kSmallVpt = 4;                   // ...values per lane (rows of up to 2,048 entries)
constexpr int kLongMin = 32769;                // rows this long are split over several workgroups
constexpr int kCkNT = 512;                     // long rows: lanes per workgroup (1,024 measured slower)
constexpr int kCkVpt = 16;                     // ...values per lane
constexpr int kCkChunk = kCkNT * kCkVpt;       // ...entries per chunk (one workgroup each)
constexpr int kCkCand = 4096;                  // ...boundary-bin candidates the resolving workgroup holds
constexpr int kCkAll = 8192;                   // ...chunk candidates it holds in registers
constexpr int kCkMeta = 1024;                  // ...chunks per row it can track
constexpr int kRowPages = 1024;                // a row's first page ids, cached in LDS for its translation
constexpr int kCkPages = 4096;                 // the same on long rows

// Candidates a long-row chunk of CH entries keeps: e = its expected share of
// the row's top k (rounded up), plus 4 standard deviations of a binomial
// count and 16.  Non-increasing in n.  Host and device compute it alike
// (integers only; CH*k + n fits 32 bits for every admitted row).
__host__ __device__ __forceinline__ constexpr int ck_isqrt_ceil(int e) {
  int s = 0;
  while (s * s < e) ++s;
  return s;
}
template <int CH>
__host__ __device__ __forceinline__ constexpr int ck_quota(int64_t n, int k) {
  const int e = (int)(((uint32_t)CH * (uint32_t)k + (uint32_t)n - 1u) / (uint32_t)n);
  return e + 4 * ck_isqrt_ceil(e) + 16;
}
// Candidate slots per chunk for quota q: the quota plus room for the rest of
// the bin the q-th largest falls in (a chunk whose candidates would overflow
// them keeps only the bins above; the resolver then finds a floor above its
// threshold).
__host__ __device__ __forceinline__ constexpr int ck_slots_for(int q) { return (q + q / 8 + 32 + 31) / 32 * 32; }
template <int CH>
__host__ __device__ __forceinline__ constexpr int ck_slots(int64_t n, int k) {
  return ck_slots_for(ck_quota<CH>(n, k));
}
// An unused candidate slot: no real candidate has this pattern (its index
// would be 2^32 - 1).
constexpr uint64_t kNoCand = ~0ull;
static_assert(kCkChunk <= 65535, "a chunk's per-bin counts fit 16 bits");

// Workspace record per long row: counters ([0] arrivals), each chunk's
// packed (candidate count << 16 | bin floor), each chunk's histogram at and
// above its floor (16-bit counts, zeros below), each chunk's candidates (FP32
// bits << 32 | index, then unused markers) at chunk * ck_slots(n, k).
constexpr size_t kWsCtr = 0;
constexpr size_t kWsMeta = 64;
__host__ __device__ constexpr size_t ck_meta_bytes(int wmax) { return ((size_t)wmax * 4 + 255) / 256 * 256; }
__host__ __device__ constexpr size_t ck_hist_offset(int wmax) { return kWsMeta + ck_meta_bytes(wmax); }
__host__ __device__ constexpr size_t ck_cand_offset(int wmax) {
  return ck_hist_offset(wmax) + (size_t)wmax * kBins * 2;
}
// Records are whole blocks of kWsBlock bytes, so every row counter of every
// layout sits on the first word of such a block: a call that leaves those
// words zero leaves the workspace ready for any later shape.
constexpr size_t kWsBlock = (size_t)64 << 10;
// min_cut: the shortest row the launch may split (the per-chunk slots only
// shrink as rows grow).
static size_t ck_record_bytes(int32_t max_len, int32_t k, int32_t min_cut = kLongMin) {
  const int wmax = (max_len + kCkChunk - 1) / kCkChunk;
  const size_t b = ck_cand_offset(wmax) + (size_t)wmax * ck_slots<kCkChunk>(min_cut, k) * 8;
  return (b + kWsBlock - 1) / kWsBlock * kWsBlock;
}

template <int CAP, int RP = kRowPages>
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
  uint32_t bmax;
  uint32_t inbin;
  uint64_t red_and[16], red_or[16];
  uint32_t out_ctr;       // output positions handed out by the boundary refinement
  int32_t row_pages[RP];  // page ids 0 .. row_npages-1 of a whole row's request (fused translation)
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

// Entries 4*(lane_quad + uniform_quad) .. +3 of a row in one 16-byte load
// (the row starts 16-byte aligned; the resource's range check returns 0
// past its end).
__device__ __forceinline__ u32x4_t row_quad(const RowReader& rd, int lane_quad, int uniform_quad) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(rd.rsrc, lane_quad * 16, uniform_quad * 16, 0));
}

// Row index of a lane's register entry i, recomputed at each use: left to
// itself the compiler keeps all V of these (and their bounds tests) live
// across the kernel.  VEC = 1: entry i is base + i*NT + lane.  VEC = 4 (rows
// read 16 bytes per lane): entries 4q .. 4q+3 are the four consecutive
// entries at base + 4*(q*NT + lane).
template <int NT, int VEC = 1>
__device__ __forceinline__ int entry_index(int base, int i) {
  int idx = VEC == 1 ? base + i * NT + (int)threadIdx.x
                     : base + ((i / VEC) * NT + (int)threadIdx.x) * VEC + (i % VEC);
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

// Reserves cnt consecutive slots per lane (any cnt >= 0) from *counter with
// one LDS atomic per wave; returns this lane's first slot.  All 64 lanes must
// call.
__device__ __forceinline__ uint32_t wave_reserve_n(uint32_t* counter, uint32_t cnt) {
  const uint32_t incl = wave_incl_scan(cnt);
  uint32_t base = 0;
  if (lane_id() == 63) base = atomicAdd(counter, incl);
  base = readlane(base, 63);
  return base + incl - cnt;
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
template <int NT, int CAP, int RP>
__device__ __forceinline__ uint32_t block_excl_scan(TopkShared<CAP, RP>& s, uint32_t x, uint32_t& total) {
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

// The whole workgroup resolves the boundary bin from s.cand[0..nc) (nc > need
// >= 1, nc <= CAP): each lane holds up to PER candidates in registers
// (candidate i*NT + lane).  An exact MSB-first radix selection on the 64-bit
// keys, 8-bit digits after the bits all candidates share: per pass every lane
// adds its matching candidates to an LDS digit histogram, one barrier, then
// every wave finds the same digit from that histogram by itself.  Three digit
// buffers rotate (in s.hist, free once the threshold bin is known), so one
// barrier per pass suffices: the buffer pass p + 1 fills was last read in
// pass p - 2 and is cleared during pass p.  The `need` winners are written
// at out[base ...] (and chosen[base ...]) in an unspecified order, each wave
// taking its positions with one LDS atomic.
// AO: the caller has already published (before a barrier) s.red_and[0] and
// s.red_or[0], zeroed digit buffers 0 and 1 (s.hist[0 .. 512)) and
// s.out_ctr.  The two words are the AND and the OR of the nc keys, or any
// pair whose highest differing bit is at or above the keys' own and on whose
// bits above it every key agrees with them (the passes then start from a
// higher bit).  Without AO the exact AND and OR are found here, at the cost
// of one more barrier.
template <int NT, int CAP, int RP, int PER, bool AO = false>
__device__ __forceinline__ void block_refine_per(TopkShared<CAP, RP>& s, uint32_t nc, uint32_t need,
                                                 int32_t* __restrict__ out, int32_t* chosen, uint32_t base, int limit) {
  static_assert(3 * 256 <= kBins, "three digit buffers fit in the histogram's storage");
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t* const dig = s.hist;
  uint64_t key[PER];
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
  if (AO) {
    a = s.red_and[0];
    o = s.red_or[0];
  } else {
    a = wave_and64(a);
    o = wave_or64(o);
    if (lane_id() == 0) {
      s.red_and[wave] = a;
      s.red_or[wave] = o;
    }
    for (int i = tid; i < 512; i += NT) dig[i] = 0;  // buffers 0 and 1
    if (tid == 0) s.out_ctr = 0;
    __syncthreads();
    a = ~0ull;
    o = 0ull;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      a &= s.red_and[w];
      o |= s.red_or[w];
    }
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
  uint32_t pos = base + wave_reserve_n(&s.out_ctr, cnt);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if ((uint32_t)(i * NT + tid) < nc && (key[i] & mask) >= prefix) {
      if (pos < (uint32_t)limit) {
        const int idx = index_of(key[i]);
        if (out) out[pos] = idx;
        if (chosen) chosen[pos] = idx;
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

template <int NT, int CAP, int RP>
__device__ __forceinline__ void rank_refine(TopkShared<CAP, RP>& s, uint32_t nc, uint32_t need,
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

template <int NT, int CAP, int RP, bool AO = false>
__device__ __forceinline__ void block_refine(TopkShared<CAP, RP>& s, uint32_t nc, uint32_t need, int32_t* __restrict__ out,
                                             int32_t* chosen, uint32_t base, int limit) {
  constexpr int PMAX = (CAP + NT - 1) / NT;
  if (PMAX > 1 && nc <= (uint32_t)NT) block_refine_per<NT, CAP, RP, 1, AO>(s, nc, need, out, chosen, base, limit);
  else if (PMAX > 2 && nc <= 2u * NT) block_refine_per<NT, CAP, RP, 2, AO>(s, nc, need, out, chosen, base, limit);
  else if (PMAX > 4 && nc <= 4u * NT) block_refine_per<NT, CAP, RP, 4, AO>(s, nc, need, out, chosen, base, limit);
  else block_refine_per<NT, CAP, RP, PMAX, AO>(s, nc, need, out, chosen, base, limit);
}

// Block-wide fallback when the boundary bin overflows the LDS list: radix
// passes re-read the row (entries in bin T), the digit histogram is built by
// every lane, the decisions are taken by wave 0.  Rare (tie storms).
template <int NT, int CAP, int RP>
__device__ __forceinline__ void block_refine_from_row(TopkShared<CAP, RP>& s, const float* __restrict__ row, int n, uint32_t T,
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
template <int NT, int V, int CAP, int RP>
__device__ __forceinline__ void emit_tile(TopkShared<CAP, RP>& s, float (&x)[V], int base, int n, uint32_t T,
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

// Block-wide threshold over the 1,024 bins, held B = 1024/NT per lane from
// the top (lane i owns bins 1023 - B*i down to 1024 - B*(i+1); c[j] is the
// count of bin 1023 - B*i - j): the largest bin T whose suffix count reaches
// m, the count strictly above T and the count in T.  One DPP scan per wave,
// the wave totals through LDS: two barriers, no serial wave.  T = above =
// inbin = 0 if no bin qualifies (m above the total).  All lanes call.
template <int NT, int CAP, int RP>
__device__ __forceinline__ void block_threshold(TopkShared<CAP, RP>& s, const uint32_t (&c)[kBins / NT], uint32_t m,
                                                uint32_t& T, uint32_t& above, uint32_t& inbin) {
  constexpr int B = kBins / NT;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < B; ++i) t += c[i];
  const uint32_t incl = wave_incl_scan(t);
  if (lane == 63) s.wave_tot[wave] = incl;
  if (tid == 0) {
    s.T = 0;
    s.above = 0;
    s.inbin = 0;
  }
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) off += w < wave ? s.wave_tot[w] : 0u;
  uint32_t acc = off + incl - t;  // entries in the bins above this lane's
  if (acc < m && acc + t >= m) {
    bool found = false;
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if (!found && acc + c[i] >= m) {
        s.T = (uint32_t)(kBins - 1 - B * tid - i);
        s.above = acc;
        s.inbin = c[i];
        found = true;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  T = s.T;
  above = s.above;
  inbin = s.inbin;
}

// The threshold of the histogram in s.hist into s.T / s.above (all lanes
// call; the counts are published by the caller's barrier), block-wide: each
// lane reads its kBins/NT bins.  One wave scanning all 1,024 bins while the
// others waited measured slower in every shape (a lone 2,048-entry row
// 5.6 -> 5.1 us, the verify batch 18.4 -> 17.5 us, prefill 131.0 -> 130.2 us).
template <int NT, int CAP, int RP>
__device__ __forceinline__ void row_threshold(TopkShared<CAP, RP>& s, uint32_t m) {
  constexpr int B = kBins / NT;
  uint32_t c[B];
#pragma unroll
  for (int i = 0; i < B; ++i) c[i] = s.hist[kBins - 1 - B * (int)threadIdx.x - i];
  uint32_t T, above, inbin;
  block_threshold<NT>(s, c, m, T, above, inbin);
}

// One workgroup selects a whole row with n > m.  Rows of up to NT*V entries
// are read once and held in registers; longer rows are streamed: once for
// the histogram (skipped when it is ready), once in NT*V-entry tiles for
// emission.  HIST_READY: s.hist
// already holds the row's histogram (long-row finisher).  All lanes call.
// VEC = 4: the register path reads its entries 16 bytes per lane (the
// caller's row starts 16-byte aligned and holds at least n rounded up to 4
// entries).
template <int NT, int V, int CAP, int RP, bool HIST_READY, bool STREAM, class PF, int VEC = 1>
__device__ __forceinline__ void select_row(TopkShared<CAP, RP>& s, const float* __restrict__ row, int n, int m,
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
    // With a few entries per lane the values stay in registers, and the
    // boundary list gets its exact keys at once (no re-read round trip).
    constexpr bool KEEP_X = V <= 4;
    static_assert(VEC == 1 || (VEC == 4 && V % 4 == 0 && !STREAM), "16-byte reads: whole quads, registers only");
    uint32_t pb[P];
    float x[V];
    if constexpr (VEC == 4) {
      // V/4 loads per lane instead of V: a wave has at most 63 vector memory
      // operations outstanding, so V = 64 one-dword loads (plus the page
      // prefetch) made the last ones wait for the first to return.  The
      // quad holding entry n-1 is read whole (its entries past n are masked
      // by index below).
      const RowReader rq(row, (n + 3) & ~3);
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const u32x4_t v = row_quad(rq, tid, q * NT);
        x[4 * q] = __uint_as_float(v.x);
        x[4 * q + 1] = __uint_as_float(v.y);
        x[4 * q + 2] = __uint_as_float(v.z);
        x[4 * q + 3] = __uint_as_float(v.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) x[i] = rd.at(tid, i * NT);  // every load in flight at once
    }
    pf.issue();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (p % 4 == 0) __builtin_amdgcn_sched_barrier(0);  // a few bins live at a time
      const uint32_t B = bin_pair(x[2 * p], x[2 * p + 1]);
      uint32_t code;
      // Pair p is entries 2p, 2p+1 of every lane: with VEC = 4 half of quad
      // p/2.  Checked for the whole workgroup at once.
      if ((VEC == 4 ? (p / 2 + 1) * NT * 4 : (2 * p + 2) * NT) <= n) {  // inside the row for every lane
        if (!HIST_READY) {
          atomicAdd(&s.hist[B & 0xFFFFu], 1u);
          atomicAdd(&s.hist[B >> 16], 1u);
        }
        code = B + 0x00010001u;
      } else {
        const bool ok0 = entry_index<NT, VEC>(0, 2 * p) < n, ok1 = entry_index<NT, VEC>(0, 2 * p + 1) < n;
        if (!HIST_READY && ok0) atomicAdd(&s.hist[B & 0xFFFFu], 1u);
        if (!HIST_READY && ok1) atomicAdd(&s.hist[B >> 16], 1u);
        code = (ok0 ? (B & 0xFFFFu) + 1u : 0u) | (ok1 ? (B & 0xFFFF0000u) + 0x00010000u : 0u);
      }
      asm volatile("" : "+v"(code));  // packed here, not sunk past the loop
      pb[p] = code;
    }
    pf.commit(s);
    __syncthreads();
    row_threshold<NT>(s, (uint32_t)m);
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
        const int idx = entry_index<NT, VEC>(0, i);
        if (out) out[pu] = idx;
        if (keep) s.chosen[pu] = idx;
      }
      ++pu;
    }
    if (KEEP_X) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if ((eqm >> i) & 1ull) {
          if (pe < (uint32_t)CAP) s.cand[pe] = composite_key(x[i], entry_index<NT, VEC>(0, i));
          ++pe;
        }
      }
    } else {
      while (eqm) {
        const int i = __builtin_ctzll(eqm);
        eqm &= eqm - 1;
        if (pe < (uint32_t)CAP) s.cand[pe] = (uint64_t)(uint32_t)entry_index<NT, VEC>(0, i);  // index only, for now
        ++pe;
      }
    }
    up_pos = total >> 20;
    cand_pos = total & 0xFFFFFu;
    __syncthreads();
    // Exact keys of the listed boundary entries, when a refinement needs them
    // (already there when the values were kept).
    const uint32_t nc = cand_pos, need = (uint32_t)m - above;
    if (!KEEP_X && nc <= (uint32_t)CAP && need < nc) {
      for (uint32_t j = tid; j < nc; j += NT) {
        const int idx = (int)(uint32_t)s.cand[j];
        s.cand[j] = composite_key(rd[idx], idx);
      }
    } else if (!KEEP_X && nc <= (uint32_t)CAP) {
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
    row_threshold<NT>(s, (uint32_t)m);
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
    } else if (!(NT == kManyNT && V == kManyVpt) && nc <= (uint32_t)kRankMax && nc <= (uint32_t)NT) {
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

// Fused translation.  Selection position q of row r holding block j becomes
// output entries q*c .. q*c+c-1 (positions c*j .. c*j+c-1); after the m
// chosen blocks come the pending positions c*n_vis .. t, then -1.  slot =
// page_table[b][pos/64]*64 + pos mod 64 (-1 for an invalid block or page).
struct RowGeom {
  int b, t, nv, p;
};

// A row's request, position, visible blocks and pending count, split so
// that its reads can be issued long before the values are needed: start() reads the row's position and the first 64 request
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
  // Entries per lane per round.  4 against 8: the long-row selection 14.8 ->
  // 14.5 us, the prefill selection 133-138 -> 132-133 us (back-to-back
  // events, same box; 2 per lane measured between the two).  Less unrolled
  // code, which runs once per row and cold.
  constexpr int E = 4;
  const int c = tr.c, sh = c == 4 ? 2 : 0;
  const int nblk = c * m, total = nblk + g.p;
  const int32_t* pt = tr.page_table + (int64_t)g.b * tr.pt_stride;
  int32_t* orow = tr.out_slots + (int64_t)r * tr.ld_out;
  int32_t* prow = tr.out_pos ? tr.out_pos + (int64_t)r * tr.ld_out : nullptr;
  if (CACHED) {
    // Branch-free: a round's selection reads, then its page-id reads, are
    // issued together (indices clamped into range, results unused where they
    // do not apply), and the stores go through buffer resources whose range
    // check drops entries at or past ld_out (and every position store when
    // there is no position output).
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(orow, (short)0, tr.ld_out * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(prow ? prow : orow, (short)0, prow ? tr.ld_out * 4 : 0, 0x00020000);
    const int mlast = max(m - 1, 0);
    for (int i0 = 0; i0 < tr.ld_out; i0 += E * NT) {
      int j[E], ps[E], pg[E];
#pragma unroll
      for (int e = 0; e < E; ++e) j[e] = chosen[min((i0 + e * NT + (int)threadIdx.x) >> sh, mlast)];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = i0 + e * NT + (int)threadIdx.x;
        const int pb = j[e] >= 0 && j[e] < g.nv ? c * j[e] + (i & (c - 1)) : -1;
        ps[e] = i < nblk ? pb : i < total ? c * g.nv + (i - nblk) : -1;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) pg[e] = cached[max(ps[e], 0) >> 6];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t off = (uint32_t)(i0 + e * NT + (int)threadIdx.x) * 4u;
        const int slot = ps[e] >= 0 && pg[e] >= 0 ? pg[e] * kPage + (ps[e] & (kPage - 1)) : -1;
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)slot, ors, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)ps[e], prs, off, 0, 0);
      }
    }
  } else {
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
        if (ps >= 0 && (ps >> 6) < tr.pt_stride) pg = (ps >> 6) < ncached ? cached[ps >> 6] : pt[ps >> 6];
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

// Page ids of a row's first RP logical pages, for its fused
// translation: read right after the row's scores are issued (so their
// latency hides behind the binning) and put in LDS before the barrier that
// follows it.  Without them the translation waited for page-table reads that
// also waited for the selection's stores (vector memory operations retire in
// order).  ON = false: does nothing.
template <int NT, bool ON, int RP = kRowPages>
struct RowPagePrefetch {
  static constexpr int PER = (RP + NT - 1) / NT;
  const Translate& tr;
  int r;
  RowGeomReads gr;
  RowGeom g{};
  int np = 0;
  int32_t v[PER];
  __device__ __forceinline__ void issue() {
    if (!ON) return;
    g = row_geometry_finish(tr, r, gr);
    np = g.t >= 0 ? min((g.t >> 6) + 1, min(RP, tr.pt_stride)) : 0;
    const int32_t* pt = tr.page_table + (int64_t)g.b * tr.pt_stride;
    // Unconditional loads at clamped indices (a request's page-table row
    // holds pt_stride >= 1 entries), masked in commit(): a conditional load
    // would end in a wait at its branch join.
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = pt[min(i * NT + (int)threadIdx.x, max(np - 1, 0))];
  }
  template <int CAP>
  __device__ __forceinline__ void commit(TopkShared<CAP, RP>& s) {
    if (!ON) return;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = i * NT + (int)threadIdx.x;
      if (idx < RP) s.row_pages[idx] = idx < np ? v[i] : -1;
    }
    if (threadIdx.x == 0) s.row_npages = (uint32_t)np;
  }
};

// The whole selection of one row by one workgroup, any n.
template <int NT, int VPT, int CAP, bool TRANSLATE, bool STREAM = true, int RP, int VEC = 1>
__device__ __forceinline__ void select_whole_row(TopkShared<CAP, RP>& s, const float* __restrict__ row, int n, int m, int k,
                                 int32_t* __restrict__ out, int32_t* __restrict__ sel_count, int r,
                                 const Translate& tr) {
  const int tid = threadIdx.x;
  RowGeomReads gr{};
  if (TRANSLATE) gr = row_geometry_start(tr, r);  // in flight during the selection
  RowPagePrefetch<NT, TRANSLATE, RP> pf{tr, r, gr};
  // The selection is staged in LDS and written out once it is complete: a
  // global store issued early would hold up every later wait for a load
  // (vector memory operations retire in order).
  if (m == n) {
    pf.issue();
    for (int i = tid; i < n; i += NT) s.chosen[i] = i;
    pf.commit(s);
  } else {
    select_row<NT, VPT, CAP, RP, false, STREAM, decltype(pf), VEC>(s, row, n, m, nullptr, true, pf);
  }
  __syncthreads();
  for (int i = tid; i < k; i += NT) out[i] = i < m ? s.chosen[i] : -1;
  if (tid == 0) sel_count[r] = m;
  if (TRANSLATE) translate_row<NT>(tr, pf.g, r, m, s.chosen, s.row_pages, (int)s.row_npages);
}

// One workgroup of NT lanes per row.  Four shapes: 1,024 lanes holding 16
// entries each when the batch has few rows (each row gets a whole CU; longer
// rows are streamed), 512 lanes holding 64 entries each for rows of up to
// 32,768 entries (two rows per CU, one pass), 256 lanes holding 64 entries
// each when it has many rows (several rows per CU, so one row's latency chain
// overlaps the others'), and 512 lanes holding 4 entries each for rows of up
// to 2,048 entries in small batches.  A single 2,048-entry row measured
// 8.5 us (1,024 x 16), 7.4 us (128 x 16), 6.8 us (1,024 x 2), 6.4 us
// (256 x 8) and 5.8 us (512 x 4) in the kernel trace: this selection is one
// workgroup's latency chain, and both its barriers (more waves) and its
// unrolled per-entry code (more entries per lane, cold in the instruction
// cache on the compute unit that runs it) lengthen it.
template <bool TRANSLATE, int NT, int VPT, int CAP, int VEC = 1>
__global__ __launch_bounds__(NT, NT == kManyNT ? 4 : NT == kMidNT ? 2 : 1) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, Translate tr) {
  __shared__ TopkShared<CAP> s;
  const int r = blockIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  const int m = min(k, n);
  // The many-rows and mid shapes are launched only for rows of at most
  // NT*VPT entries.
  select_whole_row<NT, VPT, CAP, TRANSLATE, NT == kRowNT, kRowPages, VEC>(s, scores + (int64_t)r * ld, n, m, k,
                                                                         sel + (int64_t)r * k, sel_count, r, tr);
}

template <int V>
struct IntTag {
  static constexpr int value = V;
};

// Long rows, one launch.  Every workgroup holds the row kernels' shared
// memory (histogram, boundary list, selection, a page cache sized for long
// rows).
struct ChunkShared {
  TopkShared<kCkCand, kCkPages> t;
  int32_t trash32[kCkNT];   // per-lane targets of writes that do not apply
  uint64_t trash64[kCkNT];
};

// Data crossing workgroups inside the launch (a chunk's candidates,
// histogram and packed floor/count, the arrival counter) moves only through
// device-scope atomic loads and stores with relaxed order.  On gfx950 these
// are performed at the device coherence point rather than in a workgroup's
// XCD-local L2, and a store decrements the vector memory counter only once
// it has been performed there, so "s_waitcnt vmcnt(0)" after a chunk's
// stores and before its arrival means: every store is visible to any
// device-scope load issued after the arrival is counted.  The resolving
// workgroup issues its loads only after its own arrival returned the final
// count.  A release/acquire pair would also order these, but at device scope
// it compiles to a write-back (and, for acquire, an invalidation) of the
// whole per-XCD L2, which measured far costlier than the kernel; nothing here
// relies on plain (L2-cached) stores becoming visible inside the launch.
__device__ __forceinline__ void ws_store32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_store64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same store through a buffer resource (cache policy sc1, which is what
// the device-scope store above compiles to): low word lo, high word hi at
// byte offset off; offsets at or past the resource's range are dropped.
typedef uint32_t bs_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void ws_buffer_store64(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t lo, uint32_t hi) {
  constexpr int kSc1 = 16;
  __builtin_amdgcn_raw_buffer_store_b64(bs_u32x2{lo, hi}, rs, off, 0, kSc1);
}
// Loads through a buffer resource with the same cache policy (sc1): offsets
// at or past the range return 0 without a memory access, so the loads are
// unconditional (no branch, no wait at a join) and cost nothing where they
// do not apply.
__device__ __forceinline__ uint64_t ws_buffer_load64(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  constexpr int kSc1 = 16;
  const bs_u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kSc1);
  return ((uint64_t)v.y << 32) | v.x;
}
__device__ __forceinline__ uint32_t ws_buffer_load32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  constexpr int kSc1 = 16;
  return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kSc1);
}

// Rows of >= kLongMin entries: one workgroup per CH = NT*16-entry chunk
// (grid y); shorter rows are selected whole by their first workgroup.
//
// Chunk phase.  The chunk's 16 values per lane stay in registers (loaded
// before the row's length is known, within max_len); their bins go into an
// LDS histogram.  With q = min(ck_quota(n, k), chunk length), the chunk's
// floor is the bin of its q-th largest entry, and every entry at or above
// the floor is a candidate.  If those would not fit in the chunk's slots, the
// floor moves one bin up (fewer than q candidates); if the chunk keeps every
// entry, its floor is 0.  It publishes its histogram at and above the floor,
// its candidates (written straight to its slots, positions handed out by one
// LDS reservation per wave) and (count, floor), waits for those stores and
// arrives on the row's counter.
//
// Resolution, by the last chunk to arrive.  Let U be the union of the
// candidates and T the threshold bin of U for k (from the sum of the
// published histograms).  Each chunk's candidates are all of its entries at
// or above its floor, so when T is at or above every floor, U holds every
// entry of the row in bins >= T: the row's own threshold is T, its
// above-threshold entries and its boundary bin are U's, and selecting within
// U is exact.  Otherwise (a chunk holding more of the row's top than its
// quota) the workgroup selects the whole row itself, streaming it.  The
// candidates are read back in one round trip (every chunk's slot range;
// unused slots carry a marker), emitted above T (one packed LDS reservation
// per wave) and refined in bin T on the composite (FP32 key, inverted
// index); then the selection is written out and translated, and the first
// word of each 64 KiB block of the row's record (its arrival counter among
// them) is left zero for the next call.
// One work item of the long-row selection: chunk w of row r, for a row of at
// least `cut` entries.  Without KNOWN_N the length is read from row_len while
// the chunk's score loads are in flight, and a shorter row is selected whole
// by its w == 0 item (its other items do nothing); with KNOWN_N the caller
// gives the length and passes only chunks of rows split at `cut`.  All lanes
// call; every return is uniform.
template <bool TRANSLATE, int NT, bool KNOWN_N, int ALL = kCkAll>
__device__ __forceinline__ void chunk_item(ChunkShared& cs, int r, int w, int n_given, int cut,
                                           const float* __restrict__ scores, int64_t ld,
                                           const int32_t* __restrict__ row_len, int32_t max_len, int32_t k,
                                           int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
                                           uint8_t* __restrict__ ws, int64_t rec_bytes, int32_t wmax,
                                           const Translate& tr) {
  constexpr int VPT = kCkVpt, CH = NT * VPT, B = kBins / NT, P = VPT / 2;
  static_assert(B == 2, "the published histogram packs each lane's two bins into one 32-bit store");
  static_assert(CH <= 65535, "a chunk's per-bin counts fit 16 bits");
  TopkShared<kCkCand, kCkPages>& s = cs.t;
  const int tid = threadIdx.x;
  const int lo = w * CH;
  const float* row = scores + (int64_t)r * ld;
  // The chunk's loads go out with the row-length read (the row holds
  // max_len readable entries); entries at or past the length are masked.
  const RowReader rdx(row, KNOWN_N ? n_given : max_len);
  float x[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) x[i] = rdx.at(tid, lo + i * NT);
  const int n = KNOWN_N ? n_given : max(0, min(row_len[r], max_len));
  int32_t* out = sel + (int64_t)r * k;
  // The branches on the row length come after the binning below, which
  // consumes the loads above: left before it, they let the compiler sink
  // the loads into the branch, after the length's round trip.
  const int nchunk = (n + CH - 1) / CH;
  const int qn = ck_quota<CH>(max(n, cut), k);  // used only when n >= cut
  const int Q = ck_slots_for(qn);
  const int nck = min(CH, n - lo);
  const uint32_t q = (uint32_t)min(qn, nck);
  uint8_t* rec = ws + (size_t)r * (size_t)rec_bytes;
  uint32_t* ctr = reinterpret_cast<uint32_t*>(rec + kWsCtr);
  uint32_t* meta = reinterpret_cast<uint32_t*>(rec + kWsMeta);
  uint16_t* ghist = reinterpret_cast<uint16_t*>(rec + ck_hist_offset(wmax));
  uint64_t* gcand = reinterpret_cast<uint64_t*>(rec + ck_cand_offset(wmax));

  RowGeomReads gr{};
  if (TRANSLATE) gr = row_geometry_start(tr, r);  // for the resolving workgroup; in flight from the start
  for (int i = tid; i < kBins; i += NT) s.hist[i] = 0;
  if (tid == 0) {
    s.bmax = 0;
    s.emit = 0;
  }
  __syncthreads();
  // Bins in pairs, kept as codes (bin + 1, 0 past the row) two per register.
  uint32_t pb[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint32_t Bp = bin_pair(x[2 * p], x[2 * p + 1]);
    uint32_t code;
    if (lo + (2 * p + 2) * NT <= n) {  // the whole pair lies inside the row, for every lane
      atomicAdd(&s.hist[Bp & 0xFFFFu], 1u);
      atomicAdd(&s.hist[Bp >> 16], 1u);
      code = Bp + 0x00010001u;
    } else {
      const bool ok0 = lo + entry_index<NT>(0, 2 * p) < n, ok1 = lo + entry_index<NT>(0, 2 * p + 1) < n;
      if (ok0) atomicAdd(&s.hist[Bp & 0xFFFFu], 1u);
      if (ok1) atomicAdd(&s.hist[Bp >> 16], 1u);
      code = (ok0 ? (Bp & 0xFFFFu) + 1u : 0u) | (ok1 ? (Bp & 0xFFFF0000u) + 0x00010000u : 0u);
    }
    asm volatile("" : "+v"(code));
    pb[p] = code;
  }
  __syncthreads();
  if (!KNOWN_N && n < cut) {
    if (w == 0) select_whole_row<NT, VPT, kCkCand, TRANSLATE>(s, row, n, min(k, n), k, out, sel_count, r, tr);
    return;
  }
  if (lo >= n) return;
  uint32_t hc[B];
#pragma unroll
  for (int i = 0; i < B; ++i) hc[i] = s.hist[kBins - 1 - B * tid - i];
  uint32_t bq, aq, hq;
  block_threshold<NT>(s, hc, q, bq, aq, hq);
  uint32_t fl, cc;
  if (aq + hq == (uint32_t)nck && nck <= Q) {
    fl = 0;  // every entry kept
    cc = (uint32_t)nck;
  } else if (aq + hq <= (uint32_t)Q) {
    fl = bq;
    cc = aq + hq;
  } else {
    fl = bq + 1;
    cc = aq;
  }
  // Bit i: entry i is a candidate (code > fl, i.e. a bin >= fl inside the row).
  const uint32_t tge = fl * 0x00010001u;
  uint32_t gw = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const bs_ushort2 wt = {(uint16_t)(1u << (2 * p)), (uint16_t)(2u << (2 * p))};
    gw = __builtin_amdgcn_udot2(__builtin_bit_cast(bs_ushort2, pk_gt_flags(pb[p], tge)), wt, gw, false);
  }
  // Candidates go straight to this chunk's slots (one LDS atomic per wave
  // hands out the positions), unused slots get the marker, and the histogram
  // at and above the floor is published as 16-bit counts (this lane's two
  // bins, adjacent, in one store).
  // The stores are unconditional: a lane's non-candidate entries get an
  // offset outside the buffer's range, which the hardware drops (no branch).
  uint64_t* mine = gcand + (size_t)w * Q;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(mine, (short)0, Q * 8, 0x00020000);
  uint32_t pos = wave_reserve_n(&s.emit, (uint32_t)__builtin_popcount(gw));
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const uint32_t on = (gw >> i) & 1u;
    ws_buffer_store64(crs, on ? pos * 8u : 0x80000000u, (uint32_t)(lo + i * NT + tid), __float_as_uint(x[i]));
    pos += on;
  }
  for (uint32_t j = cc + tid; j < (uint32_t)Q; j += NT) ws_store64(&mine[j], kNoCand);
  {
    const uint32_t b0 = (uint32_t)(kBins - 1 - 2 * tid);  // hc[0]; hc[1] is bin b0 - 1
    const uint32_t pk = ((b0 >= fl ? hc[0] : 0u) << 16) | (b0 - 1 >= fl ? hc[1] : 0u);
    ws_store32(reinterpret_cast<uint32_t*>(ghist) + (size_t)w * (kBins / 2) + (b0 - 1) / 2, pk);
  }
  if (tid == 0) ws_store32(&meta[w], (cc << 16) | fl);
  __builtin_amdgcn_s_waitcnt(0);  // every store of this lane performed before the chunk arrives
  __syncthreads();
  if (tid == 0)
    s.last = __hip_atomic_fetch_add(&ctr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nchunk - 1);
  __syncthreads();
  if (!s.last) return;

  // ---- Resolution (the last chunk to arrive) ----
  const int nall = nchunk * Q;
  const bool fits = nall <= ALL && nchunk <= kCkMeta;
  // The candidates are held PA per lane: 8 when they fit (most rows), else
  // 16, else (ALL = 16,384: the one-launch grid, whose few workgroups per row
  // leave room for the registers) 32, which keeps rows of about a million
  // entries at k = 2,048 off the streaming fallback.  Separate copies of the
  // resolution, so that the common one carries the fewest registers and
  // instructions (its code is cold on the compute unit that resolves, so its
  // length costs time too).
  auto resolve = [&](auto pa_tag) __attribute__((always_inline)) {
    constexpr int PA = decltype(pa_tag)::value;
    RowPagePrefetch<NT, TRANSLATE, kCkPages> pf{tr, r, gr};
    uint64_t v[PA];
    uint32_t hs[B];
#pragma unroll
    for (int i = 0; i < B; ++i) hs[i] = 0;
    // Every load below is unconditional, through buffer resources covering
    // just the valid range (lanes past it read 0 without a memory access), and
    // masked once it has arrived: a load under a condition ends in a wait at
    // the branch join, which would serialise the round trips.
    const uint32_t vmeta = fits ? (uint32_t)nchunk * 4u : 0u, vcand = fits ? (uint32_t)nall * 8u : 0u;
    const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(meta, (short)0, vmeta, 0x00020000);
    const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(gcand, (short)0, vcand, 0x00020000);
    const __amdgpu_buffer_rsrc_t hrs =
        __builtin_amdgcn_make_buffer_rsrc(ghist, (short)0, fits ? (uint32_t)nchunk * kBins * 2u : 0u, 0x00020000);
    const uint32_t mt = ws_buffer_load32(mrs, (uint32_t)tid * 4u);
#pragma unroll
    for (int p = 0; p < PA; ++p) v[p] = ws_buffer_load64(grs, (uint32_t)(p * NT + tid) * 8u);
    // The union's histogram: the sum of the chunks' published histograms
    // (one packed load per chunk per lane), 32 chunks' loads in flight at a
    // time (one round trip up to 32 chunks).
    for (int c0 = 0; c0 < (fits ? nchunk : 0); c0 += 32) {
      uint32_t h[32];
#pragma unroll
      for (int u = 0; u < 32; ++u)
        h[u] = ws_buffer_load32(hrs, ((uint32_t)(c0 + u) * (kBins / 2) + (uint32_t)(kBins / 2 - 1 - tid)) * 4u);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        hs[0] += h[u] >> 16;
        hs[1] += h[u] & 0xFFFFu;
      }
    }
#pragma unroll
    for (int p = 0; p < PA; ++p) v[p] = p * NT + tid < nall ? v[p] : kNoCand;
    pf.issue();
    if (tid < nchunk) atomicMax(&s.bmax, mt & 0xFFFFu);
    // The boundary refinement's state, set up ahead of its barrier-free
    // start: digit buffers 0 and 1, the AND / OR of the boundary keys
    // (accumulated by the emission below) and the output counter.
    for (int i = tid; i < 512; i += NT) s.hist[i] = 0;
    if (tid == 0) {
      s.emit = 0;
      s.red_and[0] = ~0ull;
      s.red_or[0] = 0ull;
      s.out_ctr = 0;
    }
    pf.commit(s);
    __syncthreads();
    uint32_t T = 0, above = 0, inT = 0;
    block_threshold<NT>(s, hs, (uint32_t)k, T, above, inT);
    const bool fast = fits && T >= s.bmax;
    if (fast) {
      // Code per slot: bin + 1 for a candidate, 0 for an unused slot.
      uint32_t code[PA];
#pragma unroll
      for (int p = 0; p < PA; ++p) {
        const uint32_t b = bin_of(__uint_as_float((uint32_t)(v[p] >> 32))) + 1u;
        code[p] = v[p] != kNoCand ? b : 0u;
      }
      // Above T: the selection (LDS); in T: the boundary list as composite
      // keys.  Positions: one packed (above << 16 | in-bin) reservation per
      // wave.  Every slot writes both lists, the ones it does not belong to at
      // this lane's own scratch entries (no branch per slot).
      const uint32_t t1 = T + 1u;
      uint32_t upm = 0, eqm = 0;
#pragma unroll
      for (int p = 0; p < PA; ++p) {
        upm |= (code[p] > t1 ? 1u : 0u) << p;
        eqm |= (code[p] == t1 ? 1u : 0u) << p;
      }
      const uint32_t base =
          wave_reserve_n(&s.emit, ((uint32_t)__builtin_popcount(upm) << 16) | (uint32_t)__builtin_popcount(eqm));
      uint32_t pu = base >> 16, pe = base & 0xFFFFu;
      // AND / OR of the boundary keys' upper halves (the FP32 keys); when
      // those are all equal the index halves are taken as all-different,
      // which only adds radix passes over the index bits (exact either way).
      uint32_t ka = ~0u, ko = 0u;
#pragma unroll
      for (int p = 0; p < PA; ++p) {
        const uint32_t up = (upm >> p) & 1u, eq = (eqm >> p) & 1u;
        int32_t* du = up && pu < (uint32_t)k ? &s.chosen[pu] : &cs.trash32[tid];
        uint64_t* de = eq && pe < (uint32_t)kCkCand ? &s.cand[pe] : &cs.trash64[tid];
        const uint64_t ck = composite_key(__uint_as_float((uint32_t)(v[p] >> 32)), (int)(uint32_t)v[p]);
        *du = (int)(uint32_t)v[p];
        *de = ck;
        ka &= eq ? (uint32_t)(ck >> 32) : ~0u;
        ko |= eq ? (uint32_t)(ck >> 32) : 0u;
        pu += up;
        pe += eq;
      }
      ka = wave_bits32<true>(ka);
      ko = wave_bits32<false>(ko);
      if (lane_id() == 0) {
        atomicAnd(&s.red_and[0], (uint64_t)ka << 32);
        atomicOr(&s.red_or[0], ((uint64_t)ko << 32) | 0xFFFFFFFFull);
      }
      __syncthreads();
      const uint32_t nc = s.emit & 0xFFFFu, need = (uint32_t)k - above;
      if (need >= 1 && need <= (uint32_t)k) {
        if (nc <= (uint32_t)kCkCand) {
          if (need >= nc) {
            for (uint32_t i = tid; i < nc; i += NT) s.chosen[above + i] = index_of(s.cand[i]);
          } else if (nc <= (uint32_t)kRankMax) {
            rank_refine<NT>(s, nc, need, nullptr, s.chosen, above);
          } else {
            block_refine<NT, kCkCand, kCkPages, true>(s, nc, need, nullptr, s.chosen, above, k);
          }
          __syncthreads();
        } else {
          if (tid == 0) s.emit = above;
          __syncthreads();
          block_refine_from_row<NT>(s, row, n, T, need, nullptr, s.chosen, k);
        }
      }
      for (int i = tid; i < k; i += NT) out[i] = s.chosen[i];
      if (tid == 0) sel_count[r] = k;
      if (TRANSLATE) translate_row<NT>(tr, pf.g, r, k, s.chosen, s.row_pages, (int)s.row_npages);
    } else {
      // Some chunk held more of the row's top than its quota: select the whole
      // row here, streaming it (exact; rare on unclustered rows).
      select_whole_row<NT, VPT, kCkCand, TRANSLATE>(s, row, n, k, k, out, sel_count, r, tr);
    }
  };
  if (nall <= 8 * NT) {
    resolve(IntTag<8>{});
  } else if (ALL <= kCkAll || nall <= kCkAll) {
    resolve(IntTag<kCkAll / NT>{});
  } else {
    if constexpr (ALL > kCkAll) resolve(IntTag<ALL / NT>{});
  }
  // Leave the first word of every kWsBlock-byte block of the row's record
  // zero: every layout a later call may lay over the workspace (other row
  // counts, lengths, k) puts its row counters on such words, and everything
  // else a call reads it has written first.
  for (int i = tid; i < (int)(rec_bytes / kWsBlock); i += NT)
    ws_store32(reinterpret_cast<uint32_t*>(rec + (size_t)i * kWsBlock), 0u);
}

// One workgroup per (row, chunk) of the grid; rows shorter than kLongMin are
// selected whole by their first workgroup.
template <bool TRANSLATE, int NT, int ALL>
__global__ __launch_bounds__(NT, 1) void topk_chunked_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, uint8_t* __restrict__ ws,
    int64_t rec_bytes, int32_t wmax, Translate tr) {
  __shared__ ChunkShared cs;
  chunk_item<TRANSLATE, NT, false, ALL>(cs, blockIdx.x, blockIdx.y, 0, kLongMin, scores, ld, row_len, max_len, k, sel,
                                        sel_count, ws, rec_bytes, wmax, tr);
}

// Planning (TopK-V2: a planning kernel reads the batch's row lengths once,
// picks the length from which rows are split over several workgroups, and
// lays out the work list the selection's workgroups take their items from;
// the list serves every call on the same lengths, e.g. all layers of one
// step).
//
// The plan: a header of kPlanHeader int32 (item count, the split length,
// num_rows, max_len, chunk item count), then the items, one int4 {row,
// chunk, length, 0} each: first one item per kCkChunk-entry chunk of every
// row at least the split length long (in row order), then one item per
// shorter row, chunk kPlanWhole (selected whole: in registers up to
// kCkChunk entries, streamed past that).  Split rows come first so that
// their chains (chunks, then the resolution) start before the short rows.
//
// The split length: kPlanMinCut (rows of three or more chunks are split) when
// the resulting items all fit on the device at once (`pool` workgroups: the
// compute units times the selection's workgroups per unit), which shortens
// the longest item while units would otherwise idle; kLongMin (five or more
// chunks) otherwise, where the rows alone keep every unit busy and a split
// only adds the resolution's extra round trips.
constexpr int kPlanNT = 1024;
constexpr int kPlanRegs = 4;  // rows per lane kept in registers between the passes
constexpr int kPlanWhole = -1;
constexpr int kPlanMinCut = 2 * kCkChunk + 1;
constexpr int kPlanHeader = 8;  // int32 words before the items (16-byte aligned)
static_assert(kPlanMinCut <= kLongMin, "the split lengths the planner picks between");

__device__ __forceinline__ uint32_t plan_chunks_of(int n) { return (uint32_t)((n + kCkChunk - 1) / kCkChunk); }

// Block-wide exclusive scan of one value per lane (kPlanNT lanes); `tot`
// receives the block's total.  Two barriers; `sh` holds kPlanNT / 64 words.
__device__ __forceinline__ uint32_t plan_block_scan(uint32_t x, uint32_t* sh, uint32_t& tot) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(x);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < kPlanNT / 64; ++w) {
    off += w < wave ? sh[w] : 0u;
    tot += sh[w];
  }
  __syncthreads();
  return off + incl - x;
}

__global__ __launch_bounds__(kPlanNT) void topk_plan_kernel(const int32_t* __restrict__ row_len, int32_t num_rows,
                                                            int32_t max_len, int32_t pool,
                                                            int32_t* __restrict__ plan) {
  __shared__ uint32_t red[3][kPlanNT / 64];
  __shared__ uint32_t scan_c[kPlanNT / 64], scan_w[kPlanNT / 64];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // Pass 1: per lane, the rows tid, tid + kPlanNT, ... (the first kPlanRegs
  // kept): items at the low split length, and chunk items at either length.
  int nreg[kPlanRegs];
  uint32_t items_lo = 0, chunks_lo = 0, chunks_hi = 0;
  auto count = [&](int n) {
    const uint32_t ch = plan_chunks_of(n);
    items_lo += n >= kPlanMinCut ? ch : 1u;
    chunks_lo += n >= kPlanMinCut ? ch : 0u;
    chunks_hi += n >= kLongMin ? ch : 0u;
  };
#pragma unroll
  for (int i = 0; i < kPlanRegs; ++i) {
    const int r = i * kPlanNT + tid;
    nreg[i] = r < num_rows ? max(0, min(row_len[r], max_len)) : -1;
  }
#pragma unroll
  for (int i = 0; i < kPlanRegs; ++i)
    if (nreg[i] >= 0) count(nreg[i]);
  for (int r = kPlanRegs * kPlanNT + tid; r < num_rows; r += kPlanNT) count(max(0, min(row_len[r], max_len)));
  // The three totals: wave sums, then one barrier.
  items_lo = wave_incl_scan(items_lo);
  chunks_lo = wave_incl_scan(chunks_lo);
  chunks_hi = wave_incl_scan(chunks_hi);
  if (lane == 63) {
    red[0][wave] = items_lo;
    red[1][wave] = chunks_lo;
    red[2][wave] = chunks_hi;
  }
  __syncthreads();
  uint32_t t_items = 0, t_lo = 0, t_hi = 0;
#pragma unroll
  for (int w = 0; w < kPlanNT / 64; ++w) {
    t_items += red[0][w];
    t_lo += red[1][w];
    t_hi += red[2][w];
  }
  const bool low = t_items <= (uint32_t)pool;
  const int cut = low ? kPlanMinCut : kLongMin;
  const uint32_t total_chunks = low ? t_lo : t_hi;
  // Pass 2: chunk items at base_c + their rank, whole-row items after every
  // chunk item.
  int4* items = reinterpret_cast<int4*>(plan + kPlanHeader);
  uint32_t base_c = 0, base_w = total_chunks;
  // One block of kPlanNT rows (r0 uniform; n < 0 past the last row).
  auto place = [&](int r0, int n) {
    const int r = r0 + tid;
    const bool split = n >= cut, whole = n >= 0 && !split;
    const uint32_t cc = split ? plan_chunks_of(n) : 0u;
    uint32_t tc, tw;
    const uint32_t oc = base_c + plan_block_scan(cc, scan_c, tc);
    const uint32_t ow = base_w + plan_block_scan(whole ? 1u : 0u, scan_w, tw);
    for (uint32_t c = 0; c < cc; ++c) items[oc + c] = int4{r, (int)c, n, 0};
    if (whole) items[ow] = int4{r, kPlanWhole, n, 0};
    base_c += tc;
    base_w += tw;
  };
#pragma unroll
  for (int i = 0; i < kPlanRegs; ++i)
    if (i * kPlanNT < num_rows) place(i * kPlanNT, nreg[i]);
  for (int r0 = kPlanRegs * kPlanNT; r0 < num_rows; r0 += kPlanNT) {
    const int r = r0 + tid;
    place(r0, r < num_rows ? max(0, min(row_len[r], max_len)) : -1);
  }
  if (tid == 0) {
    plan[0] = (int32_t)base_w;
    plan[1] = cut;
    plan[2] = num_rows;
    plan[3] = max_len;
    plan[4] = (int32_t)total_chunks;
  }
}

// The planned selection: one workgroup per slot of the work list, the slots
// past the plan's item count exiting at once.  The hardware dispatcher acts
// as the persistent pool: it starts a workgroup on a compute unit as soon as
// one retires there, and items never wait on each other (a split row is
// resolved by whichever of its chunks arrives last).  A software loop over
// items in each workgroup was measured against it at compile time: the loop
// keeps its per-lane invariants live across iterations and needs 195 VGPRs
// (one workgroup per compute unit) where one item per workgroup needs 111
// (two).
template <bool TRANSLATE, int NT, int ALL = kCkAll>
__global__ __launch_bounds__(NT, 1) void topk_planned_kernel(
    const float* __restrict__ scores, int64_t ld, int32_t num_rows, int32_t max_len, int32_t k,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, uint8_t* __restrict__ ws, int64_t rec_bytes,
    int32_t wmax, const int32_t* __restrict__ plan, Translate tr) {
  __shared__ ChunkShared cs;
  // The item count, the split length and this slot's item in one round trip
  // (the grid has one workgroup per slot of the plan, so the read is in
  // bounds).
  const int total = plan[0];
  const int cut = max(plan[1], kPlanMinCut);
  const int4 cur = reinterpret_cast<const int4*>(plan + kPlanHeader)[blockIdx.x];
  if ((int)blockIdx.x >= total) return;
  const int r = cur.x, n = max(0, min(cur.z, max_len));
  if ((unsigned)r >= (unsigned)num_rows) return;  // never, for a plan made for this batch
  if (cur.y == kPlanWhole) {
    // The row in registers, in the shape that holds it with the fewest
    // entries per lane (the short-row shapes' latency grows with the entries
    // per lane); streamed only for lengths no plan of this batch gives a
    // whole-row item.
    const float* row = scores + (int64_t)r * ld;
    int32_t* out = sel + (int64_t)r * k;
    if (n <= NT * kSmallVpt)
      select_whole_row<NT, kSmallVpt, kCkCand, TRANSLATE, false>(cs.t, row, n, min(k, n), k, out, sel_count, r, tr);
    else if (n <= NT * kCkVpt)
      select_whole_row<NT, kCkVpt, kCkCand, TRANSLATE, false>(cs.t, row, n, min(k, n), k, out, sel_count, r, tr);
    else if (n <= NT * kMidVpt)
      select_whole_row<NT, kMidVpt, kCkCand, TRANSLATE, false>(cs.t, row, n, min(k, n), k, out, sel_count, r, tr);
    else
      select_whole_row<NT, kCkVpt, kCkCand, TRANSLATE, true>(cs.t, row, n, min(k, n), k, out, sel_count, r, tr);
  } else if (n >= cut && (unsigned)cur.y < (unsigned)min(wmax, (n + kCkChunk - 1) / kCkChunk)) {
    chunk_item<TRANSLATE, NT, true, ALL>(cs, r, cur.y, n, cut, scores, ld, nullptr, max_len, k, sel, sel_count, ws,
                                         rec_bytes, wmax, tr);
  }
}

static bool use_long_path(int32_t max_len) { return max_len >= kLongMin; }

constexpr int kMaxDevices = 64;

size_t topk_plan_items(int32_t num_rows, int32_t max_len) {
  const int64_t per_row = max_len >= kPlanMinCut ? (max_len + kCkChunk - 1) / kCkChunk : 1;
  return (size_t)num_rows * (size_t)per_row;
}

size_t topk_plan_bytes(int32_t num_rows, int32_t max_len) {
  return (size_t)kPlanHeader * 4 + topk_plan_items(num_rows, max_len) * sizeof(int4);
}
static_assert(kPlanHeader * 4 % sizeof(int4) == 0, "items stay 16-byte aligned");

size_t topk_planned_workspace_size(int32_t num_rows, int32_t max_len, int32_t k) {
  return max_len >= kPlanMinCut ? (size_t)num_rows * ck_record_bytes(max_len, k, kPlanMinCut) : 0;
}

// Workgroups of the planned selection the current device holds at once
// (compute units times resident workgroups per unit), found once per device;
// the planner splits more rows while the items fit in it.
static std::atomic<int> g_pool[kMaxDevices];

static int planned_pool() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int pool = g_pool[dev].load(std::memory_order_relaxed);
  if (pool == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(
                                                               &topk_planned_kernel<true, kCkNT>),
                                                     kCkNT, 0) != hipSuccess)
      return 0;
    pool = std::max(1, cus) * std::max(1, occ);
    g_pool[dev].store(pool, std::memory_order_relaxed);
  }
  return pool;
}

int launch_topk_plan(const int32_t* row_len, int32_t num_rows, int32_t max_len, int32_t* plan, hipStream_t stream) {
  const int pool = planned_pool();
  if (pool <= 0) return BS_ERR_LAUNCH;
  hipLaunchKernelGGL(topk_plan_kernel, dim3(1), dim3(kPlanNT), 0, stream, row_len, num_rows, max_len, pool, plan);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

int launch_select_translate_planned(const float* scores, int64_t ld, int32_t num_rows, int32_t max_len, int32_t k,
                                    const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos, int32_t c,
                                    const int32_t* page_table, int32_t pt_stride, int32_t* sel, int32_t* sel_count,
                                    int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out,
                                    const int32_t* plan, void* workspace, hipStream_t stream) {
  const Translate tr{req_row_ptr, num_req, row_pos, c, page_table, pt_stride, out_slots, out_pos, out_count, ld_out};
  const int grid = (int)topk_plan_items(num_rows, max_len);
  const int wmax = std::max(1, (max_len + kCkChunk - 1) / kCkChunk);
  const int64_t rec = max_len >= kPlanMinCut ? (int64_t)ck_record_bytes(max_len, k, kPlanMinCut) : 0;
  // As in the one-launch grid: the 32-per-lane resolver only when a max_len
  // row has more candidate slots than the 16-per-lane form holds.
  const int64_t slots = (int64_t)wmax * ck_slots<kCkChunk>(std::max(max_len, kPlanMinCut), k);
  if (slots > kCkAll)
    hipLaunchKernelGGL((topk_planned_kernel<true, kCkNT, 2 * kCkAll>), dim3(grid), dim3(kCkNT), 0, stream, scores, ld,
                       num_rows, max_len, k, sel, sel_count, static_cast<uint8_t*>(workspace), rec, wmax, plan, tr);
  else
    hipLaunchKernelGGL((topk_planned_kernel<true, kCkNT>), dim3(grid), dim3(kCkNT), 0, stream, scores, ld, num_rows,
                       max_len, k, sel, sel_count, static_cast<uint8_t*>(workspace), rec, wmax, plan, tr);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

size_t topk_workspace_size(int32_t num_rows, int32_t max_len, int32_t k) {
  return use_long_path(max_len) ? (size_t)num_rows * ck_record_bytes(max_len, k) : 0;
}

template <bool TRANSLATE>
static int launch_select(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows, int32_t max_len,
                         int32_t k, int32_t* sel, int32_t* sel_count, void* workspace, const Translate& tr,
                         hipStream_t stream) {
  // Rows that start 16-byte aligned (ld a multiple of 4, aligned base) are
  // read 16 bytes per lane by the 512-lane x 64-entry shape: 16 loads per
  // lane instead of 64 (a wave has at most 63 loads outstanding).  Verify
  // batch (384 rows): 18.5 -> 17.8 us back to back, bitwise the same output.
  const bool quads = ld % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  if (use_long_path(max_len)) {
    const int wmax = (max_len + kCkChunk - 1) / kCkChunk;
    // The resolver that holds 32 candidates per lane needs twice the
    // registers (one workgroup per CU instead of two): launched only when a
    // row of max_len entries has more candidate slots than the 16-per-lane
    // form holds (about a million entries at k = 2,048).  Either form is exact
    // for every row; a row beyond its capacity is streamed whole.
    const int64_t slots = (int64_t)wmax * ck_slots<kCkChunk>(std::max(max_len, kLongMin), k);
    if (slots > kCkAll)
      hipLaunchKernelGGL((topk_chunked_kernel<TRANSLATE, kCkNT, 2 * kCkAll>), dim3(num_rows, wmax), dim3(kCkNT), 0,
                         stream, scores, ld, row_len, max_len, k, sel, sel_count, static_cast<uint8_t*>(workspace),
                         (int64_t)ck_record_bytes(max_len, k), wmax, tr);
    else
      hipLaunchKernelGGL((topk_chunked_kernel<TRANSLATE, kCkNT, kCkAll>), dim3(num_rows, wmax), dim3(kCkNT), 0,
                         stream, scores, ld, row_len, max_len, k, sel, sel_count, static_cast<uint8_t*>(workspace),
                         (int64_t)ck_record_bytes(max_len, k), wmax, tr);
  } else if (num_rows >= kManyMinRows && max_len <= kManyNT * kManyVpt) {
    // One-dword reads here: the 16-byte form measured 134.0-135.5 against
    // 137.7-139.7 us on the 8,192-row prefill selection (same box, back to
    // back).  Six rows share a CU and their loads already fill its memory
    // pipeline (the loads' issue alone takes ~2 us of a row's 22 in either
    // form).
    hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kManyNT, kManyVpt, kManyCand>), dim3(num_rows), dim3(kManyNT), 0,
                       stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  } else if (max_len > kRowNT * kRowVpt) {
    if (quads)
      hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kMidNT, kMidVpt, kMidCand, 4>), dim3(num_rows), dim3(kMidNT), 0,
                         stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
    else
      hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kMidNT, kMidVpt, kMidCand>), dim3(num_rows), dim3(kMidNT), 0,
                         stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  } else if (max_len <= kSmallNT * kSmallVpt) {
    hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kSmallNT, kSmallVpt, kRowCand>), dim3(num_rows), dim3(kSmallNT), 0,
                       stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  } else {
    hipLaunchKernelGGL((topk_rows_kernel<TRANSLATE, kRowNT, kRowVpt, kRowCand>), dim3(num_rows), dim3(kRowNT), 0,
                       stream, scores, ld, row_len, max_len, k, sel, sel_count, tr);
  }
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

// Scratch for callers that cannot allocate (idx_select_translate_noalloc):
// the long-row records live in this array, one copy per GPU, zero at load.
// Every call leaves the first word of each 64 KiB block of the records it
// used zero, as it does for a caller's workspace, which is all the next call
// needs.  Host code never uses the array's name as an address: the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::atomic<void*> g_scratch_addr[kMaxDevices];

static void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_addr[dev].store(p, std::memory_order_release);  // every thread finds the same address
  }
  return p;
}

int launch_select_translate_noalloc(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows,
                                    int32_t max_len, int32_t k, const int32_t* req_row_ptr, int32_t num_req,
                                    const int32_t* row_pos, int32_t c, const int32_t* page_table, int32_t pt_stride,
                                    int32_t* sel, int32_t* sel_count, int32_t* out_slots, int32_t* out_pos,
                                    int32_t* out_count, int32_t ld_out, hipStream_t stream) {
  void* ws = nullptr;
  if (topk_workspace_size(num_rows, max_len, k) > 0) {
    ws = scratch_address();
    if (ws == nullptr) return BS_ERR_LAUNCH;
  }
  const Translate tr{req_row_ptr, num_req, row_pos, c, page_table, pt_stride, out_slots, out_pos, out_count, ld_out};
  return launch_select<true>(scores, ld, row_len, num_rows, max_len, k, sel, sel_count, ws, tr, stream);
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
