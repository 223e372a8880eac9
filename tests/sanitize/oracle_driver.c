/* Drives the C oracle (oracle/wf_oracle.c) over seeded random small chunk tables, the explicit-
 * mask form, the e4m3 codec and quantizer and the LSE merge.  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py (host code only), so an out-of-bounds
 * access or undefined operation in the oracle ends the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn_rows(int32_t num_chunks, const int32_t* chunk_tokens, const int32_t* chunk_order,
                     const int32_t* page_offsets, const int32_t* page_ids, int32_t num_pages,
                     int32_t page_size, int32_t num_query_chunks, const int32_t* query_chunks,
                     int32_t H, int32_t d, double scale, const double* q, const double* k_pool,
                     const double* v_pool, int64_t n_rows, const int64_t* rows, double* out,
                     double* lse, double* sumw2, int32_t nthreads);
int oracle_attn_masked(int64_t nq, int64_t nk, int32_t d, double scale, const double* q,
                       const double* k, const double* v, const uint8_t* allowed, double* out,
                       double* lse, int32_t nthreads);
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float x);
int oracle_quantize_e4m3(const float* x, int64_t rows, int32_t H, int32_t d, uint8_t* x8, float* scales);
int oracle_dequantize_e4m3(const uint8_t* x8, const float* scales, int64_t rows, int32_t H, int32_t d,
                           double* y);
int oracle_merge_lse(int32_t n_parts, int64_t n, int32_t d, const double* o_parts, const double* lse_parts,
                     double* out, double* lse);

static uint64_t state = 88172645463325252ull;
static uint32_t next_u32(void) {  /* xorshift64 */
  state ^= state << 13; state ^= state >> 7; state ^= state << 17;
  return (uint32_t)(state >> 32);
}
static int uni(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }
static double gauss(void) { return ((double)next_u32() / 4294967296.0 - 0.5) * 3.4; }

int main(void) {
  for (int it = 0; it < 40; ++it) {
    const int n = uni(1, 5), page = 64 * uni(1, 2), H = uni(1, 2), d = uni(0, 1) ? 64 : 32;
    int32_t tokens[5], order[5], offs[6] = {0}, q[5];
    for (int c = 0; c < n; ++c) { tokens[c] = uni(1, 150); order[c] = uni(0, n - 1); q[c] = c; }
    for (int c = 0; c < n; ++c) offs[c + 1] = offs[c] + (tokens[c] + page - 1) / page;
    const int npages = offs[n] + 1;
    int32_t* ids = malloc(sizeof(int32_t) * (size_t)offs[n]);
    for (int p = 0; p < offs[n]; ++p) ids[p] = npages - 1 - p;
    const int nq = uni(1, n);
    int64_t lq = 0;
    for (int i = 0; i < nq; ++i) lq += tokens[q[i]];
    const size_t pool = (size_t)npages * page * H * d;
    double* kp = malloc(sizeof(double) * pool);
    double* vp = malloc(sizeof(double) * pool);
    double* qq = malloc(sizeof(double) * (size_t)lq * H * d);
    for (size_t i = 0; i < pool; ++i) { kp[i] = gauss(); vp[i] = gauss(); }
    for (size_t i = 0; i < (size_t)lq * H * d; ++i) qq[i] = gauss();
    int64_t* rows = malloc(sizeof(int64_t) * (size_t)lq);
    for (int64_t r = 0; r < lq; ++r) rows[r] = r;
    double* out = malloc(sizeof(double) * (size_t)lq * H * d);
    double* lse = malloc(sizeof(double) * (size_t)lq * H);
    double* w2 = malloc(sizeof(double) * (size_t)lq * H);
    if (oracle_attn_rows(n, tokens, order, offs, ids, npages, page, nq, q, H, d, 0.0, qq, kp, vp, lq, rows,
                         out, lse, w2, 2) != 0) { printf("attn_rows\n"); return 1; }
    for (size_t i = 0; i < (size_t)lq * H; ++i) if (!(w2[i] > 0.0 && w2[i] <= 1.0)) { printf("sumw2\n"); return 1; }
    for (size_t i = 0; i < (size_t)lq * H * d; ++i) if (!isfinite(out[i])) { printf("nonfinite\n"); return 1; }
    free(ids); free(kp); free(vp); free(qq); free(rows); free(out); free(lse); free(w2);
  }
  {  /* explicit mask, one head */
    enum { NQ = 37, NK = 53, D = 16 };
    static double q[NQ * D], k[NK * D], v[NK * D], out[NQ * D], lse[NQ];
    static uint8_t allowed[NQ * NK];
    for (int i = 0; i < NQ * D; ++i) q[i] = gauss();
    for (int i = 0; i < NK * D; ++i) { k[i] = gauss(); v[i] = gauss(); }
    for (int i = 0; i < NQ * NK; ++i) allowed[i] = (uint8_t)(i % 3 != 0 || i % NK == 0);
    if (oracle_attn_masked(NQ, NK, D, 0.25, q, k, v, allowed, out, lse, 2) != 0) return 1;
  }
  for (int c = 0; c < 256; ++c) {  /* codec round trip on every finite code */
    const double x = oracle_e4m3_decode((uint8_t)c);
    if (!isnan(x) && oracle_e4m3_encode((float)x) != (uint8_t)c && !(x == 0.0)) { printf("codec %d\n", c); return 1; }
  }
  {  /* block quantizer, a short last block, and the LSE merge */
    enum { R = 130, HH = 3, DD = 64 };
    static float x[R * HH * DD], sc[3 * HH];
    static uint8_t x8[R * HH * DD];
    static double y[R * HH * DD];
    for (int i = 0; i < R * HH * DD; ++i) x[i] = (float)gauss();
    x[5] = NAN;
    if (oracle_quantize_e4m3(x, R, HH, DD, x8, sc) != 0) return 1;
    if (oracle_dequantize_e4m3(x8, sc, R, HH, DD, y) != 0) return 1;
    static double op[3 * 50 * 8], lp[3 * 50], mo[50 * 8], ml[50];
    for (int i = 0; i < 3 * 50 * 8; ++i) op[i] = gauss();
    for (int i = 0; i < 3 * 50; ++i) lp[i] = gauss() * 10;
    if (oracle_merge_lse(3, 50, 8, op, lp, mo, ml) != 0) return 1;
  }
  printf("OK\n");
  return 0;
}
