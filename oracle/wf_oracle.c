/*
 * wf_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, fp64 CPU statement of what block-causal chunk attention computes, plus an
 * independent e4m3 (OCP "E4M3FN") codec and block quantizer.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It shares no code, header,
 * table or constant with the GPU library: everything here is written from the definitions.
 *
 * Definitions followed (the pages give prose, no formula):
 *  - Wave Forcing project page, "01 - The design gap", column "C - Directed live frontier":
 *    attention is full inside a chunk and block-causal across chunks.
 *  - same page, "Key observation": the only edge removed is the reverse noisy -> clean one, so a
 *    chunk never reads a later, noisier chunk.
 *  - KipQuest paper page, "The deep dive": a chunk reads the anchor, the clean history, the live
 *    store and every earlier, cleaner chunk in flight, never a later one; producers write K/V
 *    into their final slots and the consumer reads them where they lie.
 *  - project page, "03 - End-to-end KV transport", panel "03 - Layout": each producer owns a fixed
 *    slot in the consumer's buffer and attention reads the prefix in place.
 *  Reading taken where the pages are silent: "earlier/cleaner" is the order given by chunk_order
 *  (smaller = cleaner); key chunk b is visible to query chunk a iff order[b] <= order[a]; b == a
 *  is always visible (full attention inside the chunk).  Equal orders (allowed only where the
 *  caller asks for them) make those chunks see each other both ways, the live bidirectional
 *  window of Rolling Forcing (project page, "01 - The design gap", column "A - Live frontier").
 *
 * The attention is the textbook two-pass softmax: s_j = scale * <q, k_j>, m = max_j s_j,
 * Z = sum_j exp(s_j - m), o = sum_j exp(s_j - m) / Z * v_j, lse = m + log Z.  No tiling, no
 * online rescaling, no reordering beyond the plain sums.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC wf_oracle.c -o libwf_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of this library (its own numbering). */
#define OR_OK 0
#define OR_BAD_ARG 1
#define OR_NO_MEM 2

/* ------------------------------------------------------------------------------------------ */
/* Generic masked attention for one head: the definition with an explicit 0/1 mask.            */
/* q [nq,d], k [nk,d], v [nk,d] row-major; allowed [nq,nk] (1 = key visible).                   */
/* out [nq,d], lse [nq].  A row with no visible key gets NaN output and lse = -inf.             */
/* ------------------------------------------------------------------------------------------ */
int oracle_attn_masked(int64_t nq, int64_t nk, int32_t d, double scale, const double* q,
                       const double* k, const double* v, const uint8_t* allowed, double* out,
                       double* lse, int32_t nthreads) {
  if (nq < 0 || nk < 0 || d < 1 || !q || !out || !lse || (nk > 0 && (!k || !v || !allowed)))
    return OR_BAD_ARG;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int fail = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    if (!s) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < nq; ++i) {
      if (!s) continue;
      const double* qi = q + i * d;
      double m = -INFINITY;
      for (int64_t j = 0; j < nk; ++j) {
        if (!allowed[i * nk + j]) continue;
        double acc = 0.0;
        for (int32_t c = 0; c < d; ++c) acc += qi[c] * k[j * d + c];
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
      }
      double* oi = out + i * d;
      if (m == -INFINITY) { /* no visible key: undefined, flagged */
        for (int32_t c = 0; c < d; ++c) oi[c] = NAN;
        lse[i] = -INFINITY;
        continue;
      }
      double z = 0.0;
      for (int64_t j = 0; j < nk; ++j)
        if (allowed[i * nk + j]) z += exp(s[j] - m);
      for (int32_t c = 0; c < d; ++c) oi[c] = 0.0;
      for (int64_t j = 0; j < nk; ++j) {
        if (!allowed[i * nk + j]) continue;
        double p = exp(s[j] - m) / z;
        for (int32_t c = 0; c < d; ++c) oi[c] += p * v[j * d + c];
      }
      lse[i] = m + log(z);
    }
    free(s);
  }
  return fail ? OR_NO_MEM : OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Chunk-table attention over a paged K/V pool.                                                 */
/*                                                                                              */
/* chunk c has chunk_tokens[c] tokens; its logical pages are page_offsets[c] .. [c+1]-1 and     */
/* token u of chunk c lives in physical page page_ids[page_offsets[c] + u / page_size], slot    */
/* u % page_size.  Pools are [num_pages, page_size, H, d]; q is [Lq, H, d] where the query rows */
/* are the tokens of query_chunks[0], query_chunks[1], ... concatenated.                        */
/* rows[n_rows] lists the query rows to evaluate; out is [n_rows, H, d], lse is [n_rows, H].    */
/* sumw2 (NULL: not computed) is [n_rows, H]: the sum over visible keys of the squared softmax  */
/* weights, sum_j (exp(s_j - m) / Z)^2.  It is no part of the attention; the tests use it to    */
/* size the spread that rounding each weight before the normaliser is summed leaves in an LSE.  */
/* ------------------------------------------------------------------------------------------ */
int oracle_attn_rows(int32_t num_chunks, const int32_t* chunk_tokens, const int32_t* chunk_order,
                     const int32_t* page_offsets, const int32_t* page_ids, int32_t num_pages,
                     int32_t page_size, int32_t num_query_chunks, const int32_t* query_chunks,
                     int32_t H, int32_t d, double scale, const double* q, const double* k_pool,
                     const double* v_pool, int64_t n_rows, const int64_t* rows, double* out,
                     double* lse, double* sumw2, int32_t nthreads) {
  if (num_chunks < 1 || !chunk_tokens || !chunk_order || !page_offsets || !page_ids ||
      num_pages < 1 || page_size < 1 || num_query_chunks < 1 || !query_chunks || H < 1 || d < 1 ||
      !q || !k_pool || !v_pool || n_rows < 0 || (n_rows > 0 && (!rows || !out || !lse)))
    return OR_BAD_ARG;
  /* row -> (query chunk, token) via the concatenation of the query chunks */
  int64_t* qstart = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_query_chunks + 1));
  if (!qstart) return OR_NO_MEM;
  qstart[0] = 0;
  for (int32_t i = 0; i < num_query_chunks; ++i) {
    int32_t a = query_chunks[i];
    if (a < 0 || a >= num_chunks) { free(qstart); return OR_BAD_ARG; }
    qstart[i + 1] = qstart[i] + chunk_tokens[a];
  }
  const int64_t lq = qstart[num_query_chunks];
  int64_t total_keys = 0;
  for (int32_t b = 0; b < num_chunks; ++b) {
    total_keys += chunk_tokens[b];
    for (int64_t p = page_offsets[b]; p < page_offsets[b + 1]; ++p)
      if (page_ids[p] < 0 || page_ids[p] >= num_pages) { free(qstart); return OR_BAD_ARG; }
  }
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= lq) { free(qstart); return OR_BAD_ARG; }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int fail = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)total_keys);
    const double** vrow = (const double**)malloc(sizeof(double*) * (size_t)total_keys);
    if (!s || !vrow) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < n_rows; ++r) {
      for (int32_t h = 0; h < H; ++h) {
        if (!s || !vrow) continue;
        const int64_t row = rows[r];
        int32_t qi = 0;
        while (row >= qstart[qi + 1]) ++qi;
        const int32_t a = query_chunks[qi];
        const double* qv = q + (row * H + h) * (int64_t)d;
        /* pass 1: scores over every visible key, and their max */
        int64_t n = 0;
        double m = -INFINITY;
        for (int32_t b = 0; b < num_chunks; ++b) {
          if (chunk_order[b] > chunk_order[a]) continue; /* later, noisier chunk: never read */
          for (int32_t u = 0; u < chunk_tokens[b]; ++u) {
            const int64_t page = page_ids[page_offsets[b] + u / page_size];
            const int64_t slot = page * page_size + u % page_size;
            const double* kv = k_pool + (slot * H + h) * (int64_t)d;
            double acc = 0.0;
            for (int32_t c = 0; c < d; ++c) acc += qv[c] * kv[c];
            s[n] = scale * acc;
            vrow[n] = v_pool + (slot * H + h) * (int64_t)d;
            if (s[n] > m) m = s[n];
            ++n;
          }
        }
        /* pass 2: normaliser and weighted sum of V */
        double z = 0.0;
        for (int64_t j = 0; j < n; ++j) z += exp(s[j] - m);
        double* o = out + (r * H + h) * (int64_t)d;
        for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
        double w2 = 0.0;
        for (int64_t j = 0; j < n; ++j) {
          const double p = exp(s[j] - m) / z;
          for (int32_t c = 0; c < d; ++c) o[c] += p * vrow[j][c];
          w2 += p * p;
        }
        lse[r * H + h] = m + log(z);
        if (sumw2) sumw2[r * H + h] = w2;
      }
    }
    free(s);
    free((void*)vrow);
  }
  free(qstart);
  return fail ? OR_NO_MEM : OR_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* e4m3 ("E4M3FN" in the OCP 8-bit floating point specification): 1 sign bit, 4 exponent bits */
/* with bias 7, 3 mantissa bits, no infinities; S.1111.111 is NaN, so the largest finite       */
/* magnitude is 1.110b * 2^8 = 448.  Exponent field 0 holds subnormals m * 2^-9.               */
/* ------------------------------------------------------------------------------------------ */
double oracle_e4m3_decode(uint8_t code) {
  const int sign = code >> 7;
  const int e = (code >> 3) & 0xF;
  const int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Round x to the nearest e4m3 value, ties to the even code (even mantissa), saturating to
 * +-448; NaN maps to 0x7F (sign kept).  The 127 non-negative finite magnitudes are increasing
 * in their code, so a bisection over codes finds the neighbours of |x|. */
uint8_t oracle_e4m3_encode(float x) {
  if (isnan(x)) return signbit(x) ? 0xFF : 0x7F;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 0x7E; /* decode(lo) <= a < decode(hi) */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
  }
  const double dlo = a - oracle_e4m3_decode((uint8_t)lo);
  const double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
  int code;
  if (dlo < dhi) code = lo;
  else if (dhi < dlo) code = hi;
  else code = (lo % 2 == 0) ? lo : hi;
  return sign | (uint8_t)code;
}

/* Block quantizer for [rows, H, d] fp32 data (bf16 values widened exactly): for each block of
 * 64 consecutive rows (the last one may be short) and each head, amax = max |x| over the block's
 * rows and all d channels (NaN entries ignored), scale = amax / 448, x8 = e4m3(x * (448/amax))
 * with the product clamped to [-448, 448]; amax == 0 gives scale 1 and multiplier 1.  All of
 * this is in fp32, so the code chosen for each element is an fp32 decision.
 * scales is [ceil(rows/64), H]. */
int oracle_quantize_e4m3(const float* x, int64_t rows, int32_t H, int32_t d, uint8_t* x8,
                         float* scales) {
  if (!x || !x8 || !scales || rows < 0 || H < 1 || d < 1) return OR_BAD_ARG;
  const int64_t nblk = (rows + 63) / 64;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < nblk; ++b) {
    for (int32_t h = 0; h < H; ++h) {
      const int64_t r0 = b * 64, r1 = (r0 + 64 < rows) ? r0 + 64 : rows;
      float amax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int32_t c = 0; c < d; ++c) {
          const float v = fabsf(x[(r * H + h) * (int64_t)d + c]);
          if (v > amax) amax = v; /* comparison with NaN is false: NaN ignored */
        }
      float scale = 1.0f, mult = 1.0f;
      if (amax > 0.0f) {
        scale = amax / 448.0f;
        mult = 448.0f / amax;
      }
      scales[b * H + h] = scale;
      for (int64_t r = r0; r < r1; ++r)
        for (int32_t c = 0; c < d; ++c) {
          const int64_t i = (r * H + h) * (int64_t)d + c;
          float y = x[i] * mult;
          if (y > 448.0f) y = 448.0f;
          if (y < -448.0f) y = -448.0f;
          x8[i] = oracle_e4m3_encode(y);
        }
    }
  }
  return OR_OK;
}

/* Dequantize: y = decode(x8) * scale of its (64-row block, head), in fp64. */
int oracle_dequantize_e4m3(const uint8_t* x8, const float* scales, int64_t rows, int32_t H,
                           int32_t d, double* y) {
  if (!x8 || !scales || !y || rows < 0 || H < 1 || d < 1) return OR_BAD_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t h = 0; h < H; ++h)
      for (int32_t c = 0; c < d; ++c) {
        const int64_t i = (r * H + h) * (int64_t)d + c;
        y[i] = oracle_e4m3_decode(x8[i]) * (double)scales[(r / 64) * H + h];
      }
  return OR_OK;
}

/* Merge attention results computed over disjoint key sets of the same query row:
 * lse = log(sum_i exp(lse_i)), o = sum_i exp(lse_i - lse) * o_i.  o_parts is [n_parts, n, d],
 * lse_parts is [n_parts, n]; out [n, d], lse [n].  Parts with lse = -inf (no keys) weigh 0. */
int oracle_merge_lse(int32_t n_parts, int64_t n, int32_t d, const double* o_parts,
                     const double* lse_parts, double* out, double* lse) {
  if (n_parts < 1 || n < 0 || d < 1 || !o_parts || !lse_parts || !out || !lse) return OR_BAD_ARG;
  for (int64_t i = 0; i < n; ++i) {
    double m = -INFINITY;
    for (int32_t p = 0; p < n_parts; ++p)
      if (lse_parts[p * n + i] > m) m = lse_parts[p * n + i];
    double z = 0.0;
    for (int32_t p = 0; p < n_parts; ++p) z += exp(lse_parts[p * n + i] - m);
    const double l = m + log(z);
    lse[i] = l;
    for (int32_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int32_t p = 0; p < n_parts; ++p) {
        const double w = exp(lse_parts[p * n + i] - l);
        if (w != 0.0) acc += w * o_parts[(p * n + i) * d + c];
      }
      out[i * d + c] = acc;
    }
  }
  return OR_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
