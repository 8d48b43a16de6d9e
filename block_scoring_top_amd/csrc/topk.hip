// topk.hip - exact top-k per FP32 score row, as a selection rather than a sort.
//
// Follows the TopK-V2 description (GLM-5.2 on SGLang blog, Kernel Optimization
// > TopK-V2, text and Figures 2-3): each FP32 score is rounded to FP16 and
// mapped to an order-preserving 16-bit key whose upper 10 bits index a
// 1,024-bin histogram; the bin holding the m-th largest score is located;
// scores in higher bins are emitted directly; the boundary bin is resolved
// exactly.  The page leaves the exact tie rule open; here equal scores go to
// the lower index, so the boundary is resolved by radix selection on the
// 64-bit pair (FP32 key, inverted index), which makes every key unique and the
// result exactly m entries.
//
// CDNA4 has no thread-block clusters or distributed shared memory, so the
// blog's 8-CTA cluster becomes:
//   * rows up to 16,384 entries: one 1,024-lane workgroup keeps the row in
//     registers (16 per lane) between the histogram and emission passes;
//   * rows up to 32,768 entries: one workgroup streams the row twice;
//   * longer rows: one workgroup per 4,096-entry chunk.  Each builds an LDS
//     histogram and merges it into the row's global histogram with
//     device-scope atomics (first launch).  In the second launch every
//     chunk's workgroup reads the merged histogram, finds the threshold bin,
//     emits its own above-threshold entries through a global atomic cursor and
//     appends its boundary candidates to a workspace list.  A third launch
//     (one workgroup per row) resolves the boundary bin and restores the
//     row's workspace to zero.  The hand-offs sit at kernel boundaries: an
//     in-kernel device-scope fence on gfx950 writes back and invalidates the
//     per-XCD L2, which costs far more than a launch; and no workgroup ever
//     waits on another, so co-residency is never assumed.
#include "device.h"
#include "kernels.h"

namespace bs {

constexpr int kTkBlock = 1024;
constexpr int kTkWaves = kTkBlock / 64;
constexpr int kTkVpt = 16;                         // register path: values per lane
constexpr int kTkShortMax = kTkBlock * kTkVpt;     // 16,384
constexpr int kTkLongMin = 32769;                  // rows this long use several workgroups
constexpr int kTkChunk = 4096;                     // entries per workgroup on long rows
static_assert(kTkChunk % kTkBlock == 0, "a long-row chunk is a whole number of passes");
constexpr int kTkCand = 4096;                      // boundary candidates kept in LDS / workspace

// Workspace record per row (long rows only): merged histogram, counters,
// candidate list.
constexpr size_t kWsHist = 0;
constexpr size_t kWsCtr = kBins * 4;  // [0] emit cursor, [1] candidates, [2] threshold bin, [3] count above it
constexpr size_t kWsCand = kWsCtr + 64;
constexpr size_t kWsRow = kWsCand + (size_t)kTkCand * 8;

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t hist_digit[256];
  uint64_t cand[kTkCand];
  uint32_t wave_sum[kTkWaves];
  uint64_t kmin, kmax;
  uint32_t emit;
  uint32_t ncand;
  uint32_t T;
  uint32_t above;
  uint32_t base_up, base_cand;
};

__device__ __forceinline__ uint64_t composite_key(float v, int idx) {
  return ((uint64_t)key32_of(v) << 32) | (uint32_t)(~(uint32_t)idx);
}

__device__ __forceinline__ int index_of(uint64_t key) { return (int)(~(uint32_t)key); }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m), hi = __shfl_xor((uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Reserves a slot per lane with `p` set, one atomic per wave.  All 64 lanes
// must call.  Returns the slot for lanes with `p` (undefined otherwise).
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, bool p) {
  const uint64_t mask = __ballot(p);
  const uint32_t n = (uint32_t)__popcll(mask);
  uint32_t base = 0;
  if (n != 0) {
    if (lane_id() == 0) base = atomicAdd(counter, n);
    base = __shfl(base, 0);
  }
  return base + lanes_below(mask);
}

// Largest bin T of h[0..nb) (nb <= kTkBlock) whose suffix count reaches m,
// and the count strictly above it; m must be in [1, sum h].  Results in
// s.T / s.above.  All lanes must call.
__device__ void find_threshold(const uint32_t* h, int nb, uint32_t m, TopkShared& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {  // only kept if no bin qualifies (m above the total: misuse)
    s.T = 0;
    s.above = 0;
  }
  const int bin = nb - 1 - tid;  // reversed: a prefix over lanes is a suffix over bins
  const uint32_t v = tid < nb ? h[bin] : 0u;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s.wave_sum[wave] = x;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += s.wave_sum[w];
  x += off;
  if (tid < nb && x >= m && x - v < m) {
    s.T = (uint32_t)bin;
    s.above = x - v;
  }
  __syncthreads();
}

// Resolves the boundary bin: among the candidates (FROM_ROW: entries of the
// row in bin T, re-read from memory; else s.cand[0..nc)), emits the `need`
// largest composite keys through s.emit into out[].  All lanes must call.
template <bool FROM_ROW>
__device__ void refine(TopkShared& s, const float* __restrict__ row, int n, uint32_t T, uint32_t nc,
                       uint32_t need, int32_t* __restrict__ out, int limit) {
  const int tid = threadIdx.x;
  auto for_each = [&](auto&& f) {
    if (FROM_ROW) {
      for (int i = tid; i < n; i += kTkBlock) {
        const float v = row[i];
        if (bin_of(v) == T) f(composite_key(v, i));
      }
    } else {
      for (int i = tid; i < (int)nc; i += kTkBlock) f(s.cand[i]);
    }
  };
  if (!FROM_ROW && need == nc) {
    const uint32_t base = s.emit;
    for (int i = tid; i < (int)nc; i += kTkBlock)
      if (base + i < (uint32_t)limit) out[base + i] = index_of(s.cand[i]);
    __syncthreads();
    return;
  }
  // The common leading bits of all candidates need no pass.
  uint64_t lo = ~0ull, hi = 0ull;
  for_each([&](uint64_t key) {
    lo = key < lo ? key : lo;
    hi = key > hi ? key : hi;
  });
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t a = shfl_xor64(lo, d), b = shfl_xor64(hi, d);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if (tid == 0) {
    s.kmin = ~0ull;
    s.kmax = 0ull;
  }
  __syncthreads();
  if ((tid & 63) == 0) {
    atomicMin(reinterpret_cast<unsigned long long*>(&s.kmin), (unsigned long long)lo);
    atomicMax(reinterpret_cast<unsigned long long*>(&s.kmax), (unsigned long long)hi);
  }
  __syncthreads();
  const uint64_t kmin = s.kmin, kmax = s.kmax;
  // highest differing bit (kmax != kmin whenever need < nc; 0 otherwise, a misuse)
  int hb = kmax != kmin ? 63 - __clzll((long long)(kmax ^ kmin)) : 0;
  uint64_t mask = ~((2ull << hb) - 1ull);
  uint64_t prefix = kmax & mask;
  uint32_t remaining = need;
  for (;;) {
    const int width = hb + 1 < 8 ? hb + 1 : 8;
    const int shift = hb + 1 - width;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += kTkBlock) s.hist_digit[i] = 0;
    __syncthreads();
    for_each([&](uint64_t key) {
      if ((key & mask) == prefix) atomicAdd(&s.hist_digit[(key >> shift) & (uint64_t)(nb - 1)], 1u);
    });
    __syncthreads();
    find_threshold(s.hist_digit, nb, remaining, s);
    const uint32_t d = s.T;
    remaining -= s.above;
    prefix |= (uint64_t)d << shift;
    mask |= (uint64_t)(nb - 1) << shift;
    const bool settled = s.hist_digit[d] == remaining;
    __syncthreads();
    if (settled || shift == 0) break;
    hb = shift - 1;
  }
  // Emit every candidate whose leading bits (under mask) are >= prefix:
  // exactly `need` of them.
  if (FROM_ROW) {
    for (int base = 0; base < n; base += kTkBlock) {
      const int i = base + tid;
      bool p = false;
      if (i < n) {
        const float v = row[i];
        p = bin_of(v) == T && (composite_key(v, i) & mask) >= prefix;
      }
      const uint32_t pos = wave_reserve(&s.emit, p);
      if (p && pos < (uint32_t)limit) out[pos] = i;
    }
  } else {
    for (int base = 0; base < (int)nc; base += kTkBlock) {
      const int i = base + tid;
      const bool p = i < (int)nc && (s.cand[i] & mask) >= prefix;
      const uint32_t pos = wave_reserve(&s.emit, p);
      if (p && pos < (uint32_t)limit) out[pos] = index_of(s.cand[i]);
    }
  }
  __syncthreads();
}

// Appends a boundary candidate for lanes with `p`.
__device__ __forceinline__ void push_candidate(TopkShared& s, bool p, float v, int idx) {
  const uint32_t pos = wave_reserve(&s.ncand, p);
  if (p && pos < (uint32_t)kTkCand) s.cand[pos] = composite_key(v, idx);
}

// One workgroup selects a whole row (n > m).  REG: the row is held in
// registers between passes (n <= kTkShortMax).
template <bool REG>
__device__ void select_row(TopkShared& s, const float* __restrict__ row, int n, int m, int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += kTkBlock) s.hist[i] = 0;
  if (tid == 0) {
    s.emit = 0;
    s.ncand = 0;
  }
  __syncthreads();
  float v[REG ? kTkVpt : 1];
  if (REG) {
#pragma unroll
    for (int i = 0; i < kTkVpt; ++i) {
      const int idx = tid + i * kTkBlock;
      v[i] = idx < n ? row[idx] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kTkVpt; ++i)
      if (tid + i * kTkBlock < n) atomicAdd(&s.hist[bin_of(v[i])], 1u);
  } else {
    for (int idx = tid; idx < n; idx += kTkBlock) atomicAdd(&s.hist[bin_of(row[idx])], 1u);
  }
  __syncthreads();
  find_threshold(s.hist, kBins, (uint32_t)m, s);
  const uint32_t T = s.T, above = s.above;
  if (REG) {
#pragma unroll
    for (int i = 0; i < kTkVpt; ++i) {
      const int idx = tid + i * kTkBlock;
      const bool valid = idx < n;
      const uint32_t b = bin_of(v[i]);
      const bool up = valid && b > T;
      const uint32_t pos = wave_reserve(&s.emit, up);
      if (up && pos < (uint32_t)m) out[pos] = idx;
      push_candidate(s, valid && b == T, v[i], idx);
    }
  } else {
    for (int base = 0; base < n; base += kTkBlock) {
      const int idx = base + tid;
      const bool valid = idx < n;
      const float x = valid ? row[idx] : 0.0f;
      const uint32_t b = bin_of(x);
      const bool up = valid && b > T;
      const uint32_t pos = wave_reserve(&s.emit, up);
      if (up && pos < (uint32_t)m) out[pos] = idx;
      push_candidate(s, valid && b == T, x, idx);
    }
  }
  __syncthreads();
  const uint32_t nc = s.ncand, need = (uint32_t)m - above;
  if (nc <= (uint32_t)kTkCand) refine<false>(s, row, n, T, nc, need, out, m);
  else refine<true>(s, row, n, T, nc, need, out, m);
}

__device__ __forceinline__ uint8_t* ws_row(uint8_t* ws, int r) { return ws + (size_t)r * kWsRow; }

__global__ __launch_bounds__(kTkBlock) void topk_main_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, uint8_t* __restrict__ ws) {
  __shared__ TopkShared s;
  const int r = blockIdx.x, w = blockIdx.y, tid = threadIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  const int m = min(k, n);
  const float* row = scores + (int64_t)r * ld;
  int32_t* out = sel + (int64_t)r * k;

  if (n >= kTkLongMin) {
    // Long row, first launch: this chunk's histogram merged into the row's.
    const int lo = w * kTkChunk;
    if (lo >= n) return;
    const int hi = min(n, lo + kTkChunk);
    s.hist[tid] = 0;
    __syncthreads();
    for (int idx = lo + tid; idx < hi; idx += kTkBlock) atomicAdd(&s.hist[bin_of(row[idx])], 1u);
    __syncthreads();
    const uint32_t cnt = s.hist[tid];
    if (cnt != 0) atomicAdd(reinterpret_cast<uint32_t*>(ws_row(ws, r) + kWsHist) + tid, cnt);
    return;
  }
  if (w != 0) return;
  for (int i = m + tid; i < k; i += kTkBlock) out[i] = -1;
  if (tid == 0) sel_count[r] = m;
  if (m == n) {
    for (int i = tid; i < n; i += kTkBlock) out[i] = i;
    return;
  }
  if (n <= kTkShortMax) select_row<true>(s, row, n, m, out);
  else select_row<false>(s, row, n, m, out);
}

// Long rows, second launch: every chunk's workgroup finds the threshold bin
// from the merged histogram, emits its above-threshold entries and appends
// its boundary candidates to the row's workspace list.
__global__ __launch_bounds__(kTkBlock) void topk_long_emit_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, uint8_t* __restrict__ ws) {
  __shared__ TopkShared s;
  const int r = blockIdx.x, w = blockIdx.y, tid = threadIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  if (n < kTkLongMin) return;
  if (w * kTkChunk >= n) return;
  const int m = k;  // n > 2048 >= k
  const float* row = scores + (int64_t)r * ld;
  int32_t* out = sel + (int64_t)r * k;
  uint8_t* rec = ws_row(ws, r);
  const uint32_t* gh = reinterpret_cast<const uint32_t*>(rec + kWsHist);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(rec + kWsCtr);
  uint64_t* gcand = reinterpret_cast<uint64_t*>(rec + kWsCand);

  s.hist[tid] = gh[tid];
  if (tid == 0) {
    s.emit = 0;
    s.ncand = 0;
  }
  __syncthreads();
  find_threshold(s.hist, kBins, (uint32_t)m, s);
  const uint32_t T = s.T;
  if (w == 0 && tid == 0) {
    ctr[2] = T;
    ctr[3] = s.above;
  }
  // Reserve output positions inside the workgroup first (LDS atomics), then
  // one device-scope atomic per list for the whole workgroup: same-address
  // device atomics serialise, so per-wave reservations would queue up.
  const int lo = w * kTkChunk, hi = min(n, lo + kTkChunk);
  constexpr int kPer = kTkChunk / kTkBlock;
  float x[kPer];
  bool up[kPer], eq[kPer];
  uint32_t lup[kPer], lcand[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = lo + i * kTkBlock + tid;
    const bool valid = idx < hi;
    x[i] = valid ? row[idx] : 0.0f;
    const uint32_t b = bin_of(x[i]);
    up[i] = valid && b > T;
    eq[i] = valid && b == T;
    lup[i] = wave_reserve(&s.emit, up[i]);
    lcand[i] = wave_reserve(&s.ncand, eq[i]);
  }
  __syncthreads();
  if (tid == 0) {
    s.base_up = s.emit ? atomicAdd(&ctr[0], s.emit) : 0u;
    s.base_cand = s.ncand ? atomicAdd(&ctr[1], s.ncand) : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = lo + i * kTkBlock + tid;
    const uint32_t pos = s.base_up + lup[i];
    if (up[i] && pos < (uint32_t)m) out[pos] = idx;
    const uint32_t cpos = s.base_cand + lcand[i];
    if (eq[i] && cpos < (uint32_t)kTkCand) gcand[cpos] = composite_key(x[i], idx);
  }
}

// Long rows, third launch: one workgroup per row resolves the boundary bin
// from the candidate list (or by re-reading the row if the list overflowed)
// and leaves the row's workspace zero-filled.  The kernel boundaries between
// the three launches make every workgroup's writes visible without fences.
__global__ __launch_bounds__(kTkBlock) void topk_long_finish_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ row_len, int32_t max_len,
    int32_t k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, uint8_t* __restrict__ ws) {
  __shared__ TopkShared s;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = max(0, min(row_len[r], max_len));
  if (n < kTkLongMin) return;
  const int m = k;
  const float* row = scores + (int64_t)r * ld;
  int32_t* out = sel + (int64_t)r * k;
  uint8_t* rec = ws_row(ws, r);
  uint32_t* gh = reinterpret_cast<uint32_t*>(rec + kWsHist);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(rec + kWsCtr);
  uint64_t* gcand = reinterpret_cast<uint64_t*>(rec + kWsCand);
  const uint32_t nc = ctr[1], T = ctr[2], above = ctr[3];
  const uint32_t need = (uint32_t)m - above;
  if (tid == 0) s.emit = above;
  if (nc <= (uint32_t)kTkCand)
    for (int i = tid; i < (int)nc; i += kTkBlock) s.cand[i] = gcand[i];
  __syncthreads();
  if (nc <= (uint32_t)kTkCand) refine<false>(s, row, n, T, nc, need, out, m);
  else refine<true>(s, row, n, T, nc, need, out, m);
  if (tid == 0) sel_count[r] = m;
  // Leave the row's workspace zero-filled for the next call.
  gh[tid] = 0;
  if (tid < 16) ctr[tid] = 0;
  const int used = (int)min(nc, (uint32_t)kTkCand);
  for (int i = tid; i < used; i += kTkBlock) gcand[i] = 0;
}

size_t topk_workspace_size(int32_t num_rows, int32_t max_len, int32_t /*k*/) {
  return max_len >= kTkLongMin ? (size_t)num_rows * kWsRow : 0;
}

int launch_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows, int32_t max_len,
                int32_t k, int32_t* sel, int32_t* sel_count, void* workspace, hipStream_t stream) {
  const bool any_long = max_len >= kTkLongMin;
  const int nchunk = any_long ? (max_len + kTkChunk - 1) / kTkChunk : 1;
  dim3 grid(num_rows, nchunk), block(kTkBlock);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipLaunchKernelGGL(topk_main_kernel, grid, block, 0, stream, scores, ld, row_len, max_len, k, sel,
                     sel_count, ws);
  if (hipGetLastError() != hipSuccess) return BS_ERR_LAUNCH;
  if (any_long) {
    hipLaunchKernelGGL(topk_long_emit_kernel, grid, block, 0, stream, scores, ld, row_len, max_len, k, sel, ws);
    if (hipGetLastError() != hipSuccess) return BS_ERR_LAUNCH;
    hipLaunchKernelGGL(topk_long_finish_kernel, dim3(num_rows), block, 0, stream, scores, ld, row_len, max_len,
                       k, sel, sel_count, ws);
    if (hipGetLastError() != hipSuccess) return BS_ERR_LAUNCH;
  }
  return BS_OK;
}

}  // namespace bs
