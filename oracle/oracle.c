/*
 * CPU oracle for the sparse-attention indexer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header, table or constant with the HIP path and
 * includes nothing from it.
 *
 * Each function writes out the plain definition of one step, slowly and in
 * double precision where arithmetic is involved:
 *
 *   oracle_score             QSA block score (page "Qwen3.8-Flash-Next Day-0 in
 *                            SGLang", theainews.cc, section on Qwen sparse
 *                            attention (QSA), the score equation s_{t,b}).
 *   oracle_topk              top-k as a full sort by (score desc, index asc)
 *                            (GLM-5.2 SGLang blog, aihot.virxact.com, Kernel
 *                            Optimization > TopK-V2: exactly k entries,
 *                            runtime k up to 2048; the lower-index tie-break
 *                            is the reading taken where the page only says
 *                            "exact radix tie-break").
 *   oracle_expand_translate  block -> token positions, append the unfinished
 *                            block's tokens, logical -> physical slot (QSA
 *                            section: 512 blocks -> 2048 positions + 0..3
 *                            pending; TopK-V2 Figure 2 caption: translation to
 *                            physical KV-cache slots; vllm-sparse-mla-blackwell,
 *                            shadowgraph.io, Design notes: index >= 0 sentinel).
 *   oracle_expand_translate_shared  the same with the tail extended to the
 *                            row's current position (QSA section, IndexShare
 *                            MTP: a captured selection reused across draft
 *                            steps, the positions drafted since appended).
 *   oracle_compress_store    key compression upstream of the scorer (QSA
 *                            section: 4 raw index keys averaged in FP32,
 *                            normalised, rotated with the MRoPE position of
 *                            the block's first token; a 4-slot raw-key ring
 *                            per request; full_slot/4 addressing).
 *   oracle_topk_hist         the TopK-V2 steps in the blog's order (FP16 key,
 *                            10-bit bins, threshold bin, direct emission,
 *                            exact refinement of the boundary bin), written
 *                            independently as a self-check of oracle_topk.
 *
 * Readings taken where the pages leave a step open:
 *   - a query row at 0-based position t sees blocks j with c*j+c-1 <= t, i.e.
 *     n_vis = floor((t+1)/c); its unfinished block's tokens c*n_vis .. t are
 *     the pending tail;
 *   - block j of a request lives at compressed slot
 *     page_table[(c*j)/64] * (64/c) + j mod (64/c)  (the page's "full_slot/4"
 *     addressing for c = 4, the full slot for c = 1);
 *   - -0.0 and +0.0 are equal scores;
 *   - FP32 -> FP16 is IEEE round-to-nearest-even with overflow to infinity.
 *
 * Floating point: scores are formed in double precision from the exact bf16
 * inputs and rounded once to FP32, the score type the TopK-V2 section fixes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#if defined(__F16C__)
#include <immintrin.h>
#endif

#define OR_HEADS 4
#define OR_DIM 128
#define OR_PAGE 64
#define OR_BINS 1024

enum { OR_OK = 0, OR_ERR_ARG = -2, OR_ERR_DATA = -5 };

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Number of compressed blocks a row at position t can see. */
int oracle_n_vis(int32_t t, int32_t c) { return (t + 1) / c; }

/* ------------------------------------------------------------------------ */
/* Score: s[t,b] = (1/sqrt(128)) * sum over the 4 heads of ReLU(<q[t,h], kbar[b]>),
 * over the visible blocks b of the row (QSA section, score equation).        */
/* ------------------------------------------------------------------------ */
int oracle_score(const uint16_t* q, const uint16_t* kcache, int64_t num_pages,
                 const int32_t* page_table, int32_t pt_stride,
                 const int32_t* req_row_ptr, int32_t num_req,
                 const int32_t* row_pos, int32_t num_rows, int32_t c,
                 float* scores, int64_t ld, int32_t* row_len) {
  if (c != 1 && c != 4) return OR_ERR_ARG;
  if (num_rows < 0 || num_req < 0) return OR_ERR_ARG;
  const int32_t per_page = OR_PAGE / c;
  const double scale = 1.0 / sqrt((double)OR_DIM);
  int status = OR_OK;
  for (int32_t b = 0; b < num_req; ++b) {
    for (int32_t r = req_row_ptr[b]; r < req_row_ptr[b + 1]; ++r) {
      const int32_t t = row_pos[r];
      const int32_t nv = oracle_n_vis(t, c);
      if (t < 0 || nv > ld || ((int64_t)t / OR_PAGE) >= pt_stride) { status = OR_ERR_DATA; continue; }
      row_len[r] = nv;
      int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
      for (int32_t j = 0; j < nv; ++j) {
        const int32_t page = page_table[(int64_t)b * pt_stride + (int64_t)c * j / OR_PAGE];
        if (page < 0 || page >= num_pages) { bad = 1; continue; }
        const uint16_t* key = kcache + ((int64_t)page * per_page + j % per_page) * OR_DIM;
        double head_sum = 0.0;
        for (int h = 0; h < OR_HEADS; ++h) {
          const uint16_t* qh = q + ((int64_t)r * OR_HEADS + h) * OR_DIM;
          double dot = 0.0;
          for (int d = 0; d < OR_DIM; ++d) dot += bf16_value(qh[d]) * bf16_value(key[d]);
          head_sum += dot > 0.0 ? dot : 0.0;
        }
        scores[(int64_t)r * ld + j] = (float)(head_sum * scale);
      }
      if (bad) status = OR_ERR_DATA;
    }
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Top-k by definition: a full sort by (score descending, index ascending),  */
/* then the first min(k, n).  The chosen indices are returned ascending.      */
/* ------------------------------------------------------------------------ */
typedef struct {
  float v;
  int32_t i;
} or_entry;

static int by_score_desc_index_asc(const void* a, const void* b) {
  const or_entry* x = (const or_entry*)a;
  const or_entry* y = (const or_entry*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->i > y->i) - (x->i < y->i);
}

static int int_asc(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int oracle_topk(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_rows,
                int32_t k, int32_t* sel, int32_t* count) {
  if (k < 1 || num_rows < 0) return OR_ERR_ARG;
  int status = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t r = 0; r < num_rows; ++r) {
    const int32_t n = row_len[r];
    int32_t* out = sel + (int64_t)r * k;
    for (int32_t i = 0; i < k; ++i) out[i] = -1;
    count[r] = 0;
    if (n < 0 || n > ld) {
#pragma omp atomic write
      status = OR_ERR_DATA;
      continue;
    }
    const float* row = scores + (int64_t)r * ld;
    or_entry* e = (or_entry*)malloc(sizeof(or_entry) * (size_t)(n > 0 ? n : 1));
    int has_nan = 0;
    for (int32_t i = 0; i < n; ++i) {
      e[i].v = row[i];
      e[i].i = i;
      if (isnan(row[i])) has_nan = 1;
    }
    if (has_nan) {
      free(e);
#pragma omp atomic write
      status = OR_ERR_DATA;
      continue;
    }
    qsort(e, (size_t)n, sizeof(or_entry), by_score_desc_index_asc);
    const int32_t m = n < k ? n : k;
    for (int32_t i = 0; i < m; ++i) out[i] = e[i].i;
    qsort(out, (size_t)m, sizeof(int32_t), int_asc);
    count[r] = m;
    free(e);
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Expand, append, translate.  Chosen block j covers tokens c*j .. c*j+c-1;  */
/* the unfinished block's tokens c*n_vis .. t follow; each position p maps to */
/* physical slot page_table[p / 64] * 64 + p mod 64.  Canonical order: block  */
/* positions ascending, then pending positions ascending; -1 pads the row.    */
/* ------------------------------------------------------------------------ */
/* Rows of one expansion; the pending tail of row r ends at tail_end[r]      */
/* (its own position when tail_end is NULL).                                 */
static int expand_rows(const int32_t* sel, const int32_t* sel_count, int32_t k,
                       const int32_t* req_row_ptr, int32_t num_req, const int32_t* row_pos,
                       const int32_t* tail_end, int32_t max_advance, int32_t c,
                       const int32_t* page_table, int32_t pt_stride,
                       int32_t* out_slots, int32_t* out_pos, int32_t* out_count, int32_t ld_out) {
  int status = OR_OK;
  for (int32_t b = 0; b < num_req; ++b) {
    for (int32_t r = req_row_ptr[b]; r < req_row_ptr[b + 1]; ++r) {
      int32_t* slots = out_slots + (int64_t)r * ld_out;
      int32_t* pos = out_pos + (int64_t)r * ld_out;
      for (int32_t i = 0; i < ld_out; ++i) slots[i] = pos[i] = -1;
      out_count[r] = 0;
      const int32_t t = row_pos[r];
      const int32_t te = tail_end ? tail_end[r] : t;
      const int32_t nv = oracle_n_vis(t, c);
      const int32_t m = sel_count[r];
      if (t < 0 || m < 0 || m > k || te < t || te - t > max_advance || ((int64_t)te / OR_PAGE) >= pt_stride) {
        status = OR_ERR_DATA;
        continue;
      }
      int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
      memcpy(blocks, sel + (int64_t)r * k, sizeof(int32_t) * (size_t)m);
      qsort(blocks, (size_t)m, sizeof(int32_t), int_asc);
      int bad = 0;
      for (int32_t i = 0; i < m; ++i)
        if (blocks[i] < 0 || blocks[i] >= nv || (i > 0 && blocks[i] == blocks[i - 1])) bad = 1;
      if (bad) { free(blocks); status = OR_ERR_DATA; continue; }
      int32_t n = 0;
      for (int32_t i = 0; i < m; ++i)
        for (int32_t u = 0; u < c; ++u) pos[n++] = c * blocks[i] + u;
      for (int32_t p = c * nv; p <= te; ++p) pos[n++] = p;
      for (int32_t i = 0; i < n; ++i) {
        const int32_t page = page_table[(int64_t)b * pt_stride + pos[i] / OR_PAGE];
        slots[i] = page < 0 ? -1 : page * OR_PAGE + pos[i] % OR_PAGE;
        if (page < 0) bad = 1;
      }
      if (bad) status = OR_ERR_DATA;
      out_count[r] = n;
      free(blocks);
    }
  }
  return status;
}

int oracle_expand_translate(const int32_t* sel, const int32_t* sel_count, int32_t k,
                            const int32_t* req_row_ptr, int32_t num_req,
                            const int32_t* row_pos, int32_t num_rows, int32_t c,
                            const int32_t* page_table, int32_t pt_stride,
                            int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                            int32_t ld_out) {
  if (c != 1 && c != 4) return OR_ERR_ARG;
  if (k < 1 || num_rows < 0 || num_req < 0 || ld_out < k * c + c - 1) return OR_ERR_ARG;
  return expand_rows(sel, sel_count, k, req_row_ptr, num_req, row_pos, NULL, 0, c, page_table, pt_stride,
                     out_slots, out_pos, out_count, ld_out);
}

/* ------------------------------------------------------------------------ */
/* IndexShare expansion (QSA page, section "IndexShare MTP"): a selection    */
/* captured for a row at position t0 is kept while the row advances; at      */
/* position t1 (t0 <= t1 <= t0 + max_advance) the chosen blocks expand as    */
/* before and the tail holds the captured pending tokens followed by every   */
/* position since, i.e. c*n_vis(t0) .. t1.  ld_out >= k*c + c - 1 +          */
/* max_advance.                                                              */
/* ------------------------------------------------------------------------ */
int oracle_expand_translate_shared(const int32_t* sel, const int32_t* sel_count, int32_t k,
                                   const int32_t* req_row_ptr, int32_t num_req,
                                   const int32_t* row_pos, const int32_t* row_pos_now, int32_t num_rows,
                                   int32_t c, int32_t max_advance,
                                   const int32_t* page_table, int32_t pt_stride,
                                   int32_t* out_slots, int32_t* out_pos, int32_t* out_count,
                                   int32_t ld_out) {
  if (c != 1 && c != 4) return OR_ERR_ARG;
  if (k < 1 || num_rows < 0 || num_req < 0 || max_advance < 0 || max_advance > 1024 ||
      ld_out < k * c + c - 1 + max_advance)
    return OR_ERR_ARG;
  return expand_rows(sel, sel_count, k, req_row_ptr, num_req, row_pos, row_pos_now, max_advance, c, page_table,
                     pt_stride, out_slots, out_pos, out_count, ld_out);
}

/* ------------------------------------------------------------------------ */
/* Double -> bf16 bit pattern, round to nearest, ties to even, in one step   */
/* (a pass through FP32 would round twice); overflow -> infinity.  A value   */
/* in [2^e, 2^(e+1)) has the quantum 2^(e-7); below 2^-126 the quantum is    */
/* 2^-133 (bf16 subnormals).                                                 */
/* ------------------------------------------------------------------------ */
uint16_t oracle_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0u;
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  const double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  int e = ilogb(a);
  if (e < -126) e = -126;
  const double quantum = ldexp(1.0, e - 7);
  const double r = nearbyint(a / quantum) * quantum; /* a / quantum is exact */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
  const float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------------ */
/* Key compression and store, the step just upstream of the scorer (QSA      */
/* section: the indexer's one shared key head; every 4 raw index keys are    */
/* averaged in FP32, normalised and rotated with the MRoPE position of their */
/* first token into one bf16 compressed key; the raw keys of a request's     */
/* unfinished block wait in a 4-slot ring; the compressed cache is addressed */
/* page-aligned at full_slot/4).                                             */
/*                                                                           */
/* Readings, where the page names the steps only:                            */
/*  - a request's new tokens are taken in position order.  The token at      */
/*    position p goes to ring slot p mod 4; when p mod 4 == 0 its MRoPE      */
/*    position (t, h, w) becomes the ring's block position; when             */
/*    p mod 4 == 3 the ring's 4 keys form block p/4, stored at               */
/*    page_table[b][(4j)/64] * 16 + j mod 16;                                */
/*  - average: ((k0 + k1) + k2) + k3 in FP32, times 0.25 (exact);            */
/*  - normalise: divide by the L2 norm; a zero mean stays zero;              */
/*  - rotate: rotate-half pairs (i, i + rot/2) over the first rot dims, the  */
/*    other dims pass through.  Pair i has the frequency theta^(-2i/rot) and */
/*    takes its position from component t when i < sec[0], h when            */
/*    i < sec[0] + sec[1], w otherwise (contiguous MRoPE sections; a text    */
/*    token has t = h = w = its position, which makes the layout moot).      */
/*    out_i = y_i cos a - y_{i+rot/2} sin a,                                 */
/*    out_{i+rot/2} = y_{i+rot/2} cos a + y_i sin a;                         */
/*  - the result is rounded once to bf16 (nearest, ties to even).           */
/* Normalisation and rotation run in double precision from the FP32 mean;    */
/* `exact` (optional, the shape of kcache) receives the unrounded values of  */
/* every key written.                                                        */
/*                                                                           */
/* k_raw [T][128] bf16: the new tokens; request b owns tokens                */
/* req_tok_ptr[b] .. req_tok_ptr[b+1]-1 at positions tok_start[b] + i.       */
/* mrope_pos [T][3] or NULL (text positions).  ring [num_req][4][128] bf16,  */
/* ring_pos [num_req][3] (required with mrope_pos; read only then).          */
/* ------------------------------------------------------------------------ */
static void compress_block(const uint16_t* ring4, const int32_t* P, int32_t rot, const int32_t* sec,
                           double theta, double* out) {
  float mean[OR_DIM];
  for (int d = 0; d < OR_DIM; ++d) {
    float s = (float)bf16_value(ring4[d]);
    s += (float)bf16_value(ring4[OR_DIM + d]);
    s += (float)bf16_value(ring4[2 * OR_DIM + d]);
    s += (float)bf16_value(ring4[3 * OR_DIM + d]);
    mean[d] = s * 0.25f;
  }
  double ss = 0.0;
  for (int d = 0; d < OR_DIM; ++d) ss += (double)mean[d] * (double)mean[d];
  const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
  double y[OR_DIM];
  for (int d = 0; d < OR_DIM; ++d) y[d] = (double)mean[d] * inv;
  const int32_t half = rot / 2;
  for (int d = 0; d < OR_DIM; ++d) out[d] = y[d];
  for (int32_t i = 0; i < half; ++i) {
    const int comp = i < sec[0] ? 0 : (i < sec[0] + sec[1] ? 1 : 2);
    const double angle = (double)P[comp] * pow(theta, -2.0 * (double)i / (double)rot);
    const double ca = cos(angle), sa = sin(angle);
    out[i] = y[i] * ca - y[i + half] * sa;
    out[i + half] = y[i + half] * ca + y[i] * sa;
  }
}

int oracle_compress_store(const uint16_t* k_raw, const int32_t* req_tok_ptr, const int32_t* tok_start,
                          const int32_t* mrope_pos, int32_t num_req,
                          int32_t rotary_dim, const int32_t* sections, double theta,
                          uint16_t* ring, int32_t* ring_pos,
                          const int32_t* page_table, int32_t pt_stride,
                          uint16_t* kcache, int64_t num_pages, double* exact) {
  if (num_req < 0 || rotary_dim < 0 || rotary_dim > OR_DIM || (rotary_dim & 1)) return OR_ERR_ARG;
  if (sections[0] < 0 || sections[1] < 0 || sections[2] < 0 ||
      sections[0] + sections[1] + sections[2] != rotary_dim / 2)
    return OR_ERR_ARG;
  if (!(theta > 0.0) || isinf(theta) || (mrope_pos && !ring_pos)) return OR_ERR_ARG;
  const int32_t per_page = OR_PAGE / 4;
  int status = OR_OK;
  for (int32_t b = 0; b < num_req; ++b) {
    const int32_t s = tok_start[b], n = req_tok_ptr[b + 1] - req_tok_ptr[b];
    if (s < 0 || n < 0) { status = OR_ERR_DATA; continue; }
    uint16_t* ring4 = ring + (int64_t)b * 4 * OR_DIM;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t p = s + i;
      const int64_t tok = (int64_t)req_tok_ptr[b] + i;
      memcpy(ring4 + (p % 4) * OR_DIM, k_raw + tok * OR_DIM, sizeof(uint16_t) * OR_DIM);
      if (p % 4 == 0 && ring_pos)
        for (int u = 0; u < 3; ++u) ring_pos[(int64_t)b * 3 + u] = mrope_pos ? mrope_pos[tok * 3 + u] : p;
      if (p % 4 != 3) continue;
      const int32_t j = p / 4;
      int32_t P[3];
      for (int u = 0; u < 3; ++u) P[u] = mrope_pos ? ring_pos[(int64_t)b * 3 + u] : 4 * j;
      if ((4 * (int64_t)j) / OR_PAGE >= pt_stride) { status = OR_ERR_DATA; continue; }
      const int32_t page = page_table[(int64_t)b * pt_stride + (4 * j) / OR_PAGE];
      if (page < 0 || page >= num_pages) { status = OR_ERR_DATA; continue; }
      double out[OR_DIM];
      compress_block(ring4, P, rotary_dim, sections, theta, out);
      const int64_t slot = (int64_t)page * per_page + j % per_page;
      for (int d = 0; d < OR_DIM; ++d) {
        kcache[slot * OR_DIM + d] = oracle_f64_to_bf16(out[d]);
        if (exact) exact[slot * OR_DIM + d] = out[d];
      }
    }
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* FP32 -> FP16, IEEE 754 round to nearest, ties to even; overflow -> inf;    */
/* FP16 subnormals kept; NaN -> quiet NaN.  Written from the binary16 and     */
/* binary32 formats with integer arithmetic only.                             */
/* ------------------------------------------------------------------------ */
uint16_t oracle_f32_to_f16(uint32_t x) {
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const int32_t exp = (int32_t)((x >> 23) & 0xFFu);
  const uint32_t man = x & 0x7FFFFFu;
  if (exp == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? (0x200u | (man >> 13)) : 0u));
  if (exp == 0) return sign; /* FP32 zero or subnormal: below 2^-126, rounds to +-0 */
  const int32_t e = exp - 127;          /* value = m24 * 2^(e-23) */
  const uint64_t m24 = (uint64_t)man | 0x800000u;
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  uint32_t shift;                        /* right shift to the FP16 quantum */
  if (e >= -14) shift = 13;              /* normal: quantum 2^(e-10) */
  else shift = (uint32_t)(-e - 1);       /* subnormal: quantum 2^-24 */
  uint64_t mant, rem, half;
  if (shift >= 40) { mant = 0; rem = m24; half = (uint64_t)1 << 39; }
  else {
    mant = m24 >> shift;
    rem = m24 & (((uint64_t)1 << shift) - 1);
    half = (uint64_t)1 << (shift - 1);
  }
  if (rem > half || (rem == half && (mant & 1))) mant += 1;
  uint32_t h;
  if (e >= -14) h = ((uint32_t)(e + 14) << 10) + (uint32_t)mant; /* mant in [0x400, 0x800] */
  else h = (uint32_t)mant;                                          /* may carry to 0x400 */
  return (uint16_t)(sign | h);
}

/* Order-preserving 16-bit key of an FP16 pattern: non-negative values get the
 * sign bit set, negative values are bit-inverted; -0 is first folded to +0 so
 * equal values get equal keys (TopK-V2, Figure 3 caption). */
uint16_t oracle_key16(uint16_t h) {
  if (h == 0x8000u) h = 0;
  return (h & 0x8000u) ? (uint16_t)(~h & 0xFFFFu) : (uint16_t)(h | 0x8000u);
}

uint32_t oracle_key32(uint32_t u) {
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* The coarse bin: the upper 10 bits of the 16-bit key (1,024 bins). */
int32_t oracle_bin(float v) { return (int32_t)(oracle_key16(oracle_f32_to_f16(f32_bits(v))) >> 6); }

typedef struct {
  uint32_t key;
  int32_t i;
} or_cand;

static int cand_desc(const void* a, const void* b) {
  const or_cand* x = (const or_cand*)a;
  const or_cand* y = (const or_cand*)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1;
  return (x->i > y->i) - (x->i < y->i);
}

/* TopK-V2's steps on one row, in the order the blog gives them:
 *  1. round each FP32 score to FP16, map to the order-preserving key, count
 *     the upper 10 key bits in a 1,024-bin histogram;
 *  2. find the bin holding the m-th largest score (m = min(k, n));
 *  3. emit every score in a higher bin directly;
 *  4. resolve the boundary bin exactly on the FP32 key, lower index first on
 *     equal keys, to return exactly m entries.
 * hist (1,024 counts) is returned for the check that it sums to n.  The
 * chosen indices come back ascending.  Returns the number chosen. */
int32_t oracle_topk_hist(const float* row, int32_t n, int32_t k, int32_t* sel, uint32_t* hist) {
  for (int i = 0; i < OR_BINS; ++i) hist[i] = 0;
  const int32_t m = n < k ? n : k;
  for (int32_t i = 0; i < n; ++i) hist[oracle_bin(row[i])] += 1;
  if (m == n) {
    for (int32_t i = 0; i < n; ++i) sel[i] = i;
    return m;
  }
  int32_t T = OR_BINS - 1;
  uint32_t above = 0; /* entries in bins > T */
  while (above + hist[T] < (uint32_t)m) above += hist[T--];
  int32_t out = 0;
  for (int32_t i = 0; i < n; ++i)
    if (oracle_bin(row[i]) > T) sel[out++] = i;
  or_cand* cand = (or_cand*)malloc(sizeof(or_cand) * (size_t)(hist[T] > 0 ? hist[T] : 1));
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i)
    if (oracle_bin(row[i]) == T) {
      cand[nc].key = oracle_key32(f32_bits(row[i]));
      cand[nc].i = i;
      ++nc;
    }
  qsort(cand, (size_t)nc, sizeof(or_cand), cand_desc);
  for (int32_t j = 0; j < m - (int32_t)above; ++j) sel[out++] = cand[j].i;
  free(cand);
  qsort(sel, (size_t)out, sizeof(int32_t), int_asc);
  return out;
}

/* ------------------------------------------------------------------------ */
/* Exhaustive self-checks over every FP32 bit pattern.                         */
/* ------------------------------------------------------------------------ */

/* oracle_f32_to_f16 against the host's F16C hardware conversion on all 2^32
 * inputs.  NaN inputs only need a NaN result.  Returns mismatches, or -1 when
 * F16C was not compiled in. */
int64_t oracle_check_f16_all(void) {
#if defined(__F16C__)
  int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t x = 0; x <= 0xFFFFFFFFll; ++x) {
    const uint32_t u = (uint32_t)x;
    const uint16_t mine = oracle_f32_to_f16(u);
    const float f = bits_f32(u);
    if (isnan(f)) {
      if ((mine & 0x7C00u) != 0x7C00u || (mine & 0x3FFu) == 0) ++bad;
      continue;
    }
    const uint16_t hw = (uint16_t)_cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT);
    if (mine != hw) ++bad;
  }
  return bad;
#else
  return -1;
#endif
}

/* Walks every non-NaN FP32 pattern in increasing value order (from -inf down
 * the negative patterns to -0, then +0 up to +inf), checks with the hardware's
 * float compare that each step does increase the value (or is -0 -> +0), and
 * that oracle_key32 increases strictly along the chain except for -0 -> +0,
 * where the keys are equal.  *visited gets the chain length (4,278,190,082
 * patterns).  Returns the number of violations. */
int64_t oracle_check_key32_chain(int64_t* visited) {
  int64_t bad = 0, n = 0;
  /* negative side: each step goes from pattern u+1 to the larger value u,
   * for u = 0xFF7FFFFF (from -inf) down to 0x80000000 (-0) */
#pragma omp parallel for schedule(static) reduction(+ : bad, n)
  for (int64_t x = 0x80000000ll; x <= 0xFF7FFFFFll; ++x) {
    const uint32_t u = (uint32_t)x, lo = u + 1u;
    if (!(bits_f32(lo) < bits_f32(u))) ++bad;
    if (!(oracle_key32(lo) < oracle_key32(u))) ++bad;
    ++n;
  }
  /* -0 -> +0: equal values, equal keys */
  if (!(bits_f32(0x80000000u) == bits_f32(0u))) ++bad;
  if (oracle_key32(0x80000000u) != oracle_key32(0u)) ++bad;
  /* positive side: from pattern u-1 to the larger value u, up to +inf */
#pragma omp parallel for schedule(static) reduction(+ : bad, n)
  for (int64_t x = 1; x <= 0x7F800000ll; ++x) {
    const uint32_t u = (uint32_t)x, lo = u - 1u;
    if (!(bits_f32(lo) < bits_f32(u))) ++bad;
    if (!(oracle_key32(lo) < oracle_key32(u))) ++bad;
    ++n;
  }
  *visited = n + 2; /* steps + 1 = patterns; plus the -0 -> +0 step */
  return bad;
}
