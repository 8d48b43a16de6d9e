// compress.hip - key compression and store, the step just upstream of the
// scorer.
//
// Page "Qwen3.8-Flash-Next Day-0 in SGLang", QSA section: the indexer has one
// shared key head; each run of 4 raw index keys becomes one compressed key by
// an FP32 average, a normalisation and a rotation with the MRoPE position of
// the run's first token, stored as bf16 at the page-aligned full_slot/4; the
// raw keys of a request's unfinished block are held in a 4-slot ring instead
// of a full-context raw-key cache.
//
// Readings: the average is ((k0 + k1) + k2) + k3 in FP32 times 0.25; the
// normalisation is division by the L2 norm (a zero mean stays zero); the
// rotation pairs dims (i, i + rot/2) over the first rot dims (rotate-half),
// pair i turning by P * theta^(-2i/rot) where P is the t, h or w component of
// the block's MRoPE position chosen by contiguous sections.  The ring's final
// state is that of writing every new token at slot p mod 4 in position order.
//
// One wavefront per compressed key (blockIdx.y = request, blockIdx.x = the
// request's n-th completed block).  The work is a short dependent chain, so
// every global load is issued up front.  Lanes load the 4 raw keys as
// 16-byte chunks into LDS, then own dims (lane, lane + 64): FP32 mean, a
// wave-wide max and sum of squares (scaled by the max so that neither
// overflows nor underflows), angles reduced in FP64 and turned into FP32
// sin/cos, FP32 rotation, one rounding to bf16, and a coalesced 256-byte
// store.  The first wave of each request also updates its ring, after it has
// consumed any ring entries.
#include <cmath>

#include "device.h"
#include "kernels.h"

namespace bs {

namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// FP32 -> bf16 bit pattern, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace

__global__ __launch_bounds__(64) void compress_kernel(
    const uint16_t* __restrict__ k_raw, int32_t num_tok, const int32_t* __restrict__ req_tok_ptr,
    const int32_t* __restrict__ tok_start, const int32_t* __restrict__ mrope_pos, int32_t max_tok,
    int32_t rot, int32_t sec0, int32_t sec01, double base,
    uint16_t* ring, int32_t* ring_pos,
    const int32_t* __restrict__ page_table, int32_t pt_stride,
    uint16_t* __restrict__ kcache, int64_t num_pages) {
  __shared__ __align__(16) uint16_t raw[4][kDim];
  __shared__ float ys[kDim];
  __shared__ __align__(16) uint16_t outs[kDim];

  const int b = blockIdx.y, item = blockIdx.x, lane = threadIdx.x;
  const int tp = req_tok_ptr[b];
  const int64_t s = tok_start[b];
  const int n = min(req_tok_ptr[b + 1] - tp, max_tok);
  if (s < 0 || n <= 0) return;
  const int64_t e = s + n - 1;                  // last new position
  const int64_t j0 = s >> 2;                    // block of the first new token
  const int64_t nb = ((e + 1) >> 2) - j0;       // blocks completed by this call
  if (item >= (nb > 1 ? nb : 1)) return;
  // k_raw row of new position p >= s, clamped into the buffer
  auto row_of = [&](int64_t p) -> int64_t {
    const int64_t t = tp + (p - s);
    return t < 0 ? 0 : (t >= num_tok ? num_tok - 1 : t);
  };
  const int u = lane >> 4, c16 = lane & 15;     // raw key u, 16-byte chunk c16

  // Ring update of the request's first wave: slot u ends up holding the
  // newest token p <= e with p mod 4 == u, when that token is new.  Its
  // loads read k_raw only and are issued first; its stores come last.
  const int64_t pu = e - ((e - u) & 3);
  const bool ring_slot = item == 0 && pu >= s;
  uint4 ring_val = make_uint4(0, 0, 0, 0);
  if (ring_slot) ring_val = reinterpret_cast<const uint4*>(k_raw + row_of(pu) * kDim)[c16];

  if (item < nb) {
    const int64_t j = j0 + item;
    const int64_t p = 4 * j + u;
    const uint16_t* src = p >= s ? k_raw + row_of(p) * kDim : ring + ((int64_t)b * 4 + u) * kDim;
    const uint4 v = reinterpret_cast<const uint4*>(src)[c16];
    const int64_t lp = (4 * j) >> 6;            // logical page of the block
    const int page = lp < pt_stride ? page_table[(int64_t)b * pt_stride + lp] : -1;
    int P[3];
    const int64_t pf = 4 * j;                   // the block's first token
    if (mrope_pos == nullptr) {
      P[0] = P[1] = P[2] = (int)pf;
    } else {
      const int32_t* mp = pf >= s ? mrope_pos + row_of(pf) * 3 : ring_pos + (int64_t)b * 3;
      P[0] = mp[0];
      P[1] = mp[1];
      P[2] = mp[2];
    }
    reinterpret_cast<uint4*>(&raw[u][0])[c16] = v;

    // Rotation of the pairs of this lane's dims (lane, lane + 64), in
    // revolutions: frequency base^i with base = theta^(-2/rot) (squarings in
    // FP64), angle P * base^i / (2 pi) reduced exactly to [-1/2, 1/2] in
    // FP64, then sin and cos of pi * 2f in FP32.
    const int half = rot >> 1;
    float cs[2], sn[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = lane + 64 * h;
      cs[h] = 1.f;
      sn[h] = 0.f;
      if (d < rot) {
        const int i = d < half ? d : d - half;
        const int comp = i < sec0 ? 0 : (i < sec01 ? 1 : 2);
        double f = 1.0, bb = base;
#pragma unroll
        for (int bit = 0; bit < 6; ++bit) {
          if ((i >> bit) & 1) f *= bb;
          bb *= bb;
        }
        const double rev = (double)P[comp] * f * 0.15915494309189535;  // 1 / (2 pi)
        const float fr = (float)(rev - rint(rev));
        sincospif(2.f * fr, &sn[h], &cs[h]);
      }
    }
    __syncthreads();

    float m[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = lane + 64 * h;
      float acc = bf16_bits_to_f32(raw[0][d]);
      acc += bf16_bits_to_f32(raw[1][d]);
      acc += bf16_bits_to_f32(raw[2][d]);
      acc += bf16_bits_to_f32(raw[3][d]);
      m[h] = acc * 0.25f;
    }
    const float amax = wave_max(fmaxf(fabsf(m[0]), fabsf(m[1])));
    float y0 = 0.f, y1 = 0.f;
    if (amax > 0.f) {
      const float a0 = m[0] / amax, a1 = m[1] / amax;
      const float r = 1.0f / sqrtf(wave_sum(a0 * a0 + a1 * a1));
      y0 = a0 * r;
      y1 = a1 * r;
    }
    ys[lane] = y0;
    ys[lane + 64] = y1;
    __syncthreads();

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int d = lane + 64 * h;
      float out = ys[d];
      if (d < rot) out = d < half ? ys[d] * cs[h] - ys[d + half] * sn[h] : ys[d] * cs[h] + ys[d - half] * sn[h];
      outs[d] = (uint16_t)f32_to_bf16_rne(out);
    }
    __syncthreads();

    if (page >= 0 && page < num_pages) {
      uint16_t* dst = kcache + ((int64_t)page * (kPage / 4) + (j & (kPage / 4 - 1))) * kDim;
      reinterpret_cast<uint32_t*>(dst)[lane] = reinterpret_cast<const uint32_t*>(outs)[lane];
    }
  }

  if (item == 0) {
    // The block above read its ring entries into LDS before its first
    // barrier, so these stores come after those reads.
    if (ring_slot) reinterpret_cast<uint4*>(ring + ((int64_t)b * 4 + u) * kDim)[c16] = ring_val;
    const int64_t p0 = e - (e & 3);             // newest block start <= e
    if (ring_pos != nullptr && lane < 3 && p0 >= s)
      ring_pos[(int64_t)b * 3 + lane] = mrope_pos != nullptr ? mrope_pos[row_of(p0) * 3 + lane] : (int32_t)p0;
  }
}

int launch_compress(const uint16_t* k_raw, int32_t num_tok, const int32_t* req_tok_ptr, const int32_t* tok_start,
                    const int32_t* mrope_pos, int32_t num_req, int32_t max_tok, int32_t rotary_dim,
                    int32_t sec_t, int32_t sec_h, double theta, uint16_t* ring, int32_t* ring_pos,
                    const int32_t* page_table, int32_t pt_stride, uint16_t* kcache, int64_t num_pages,
                    hipStream_t stream) {
  const int items = max(1, (max_tok + 3) / 4);
  // theta^(-2/rot), the ratio of successive pair frequencies
  const double base = rotary_dim > 0 ? std::pow(theta, -2.0 / (double)rotary_dim) : 1.0;
  hipLaunchKernelGGL(compress_kernel, dim3(items, num_req), dim3(64), 0, stream, k_raw, num_tok, req_tok_ptr,
                     tok_start, mrope_pos, max_tok, rotary_dim, sec_t, sec_t + sec_h, base, ring, ring_pos,
                     page_table, pt_stride, kcache, num_pages);
  return hipGetLastError() == hipSuccess ? BS_OK : BS_ERR_LAUNCH;
}

}  // namespace bs
