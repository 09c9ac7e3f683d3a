/*
 * CPU oracle for causal GQA prefill attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header or constant with the GPU
 * path.
 *
 * What it computes is the plain definition of the operation, in fp64:
 *
 *   for every request r, query token i of that request and q head h
 *     kv head   c = h / (Hq / Hkv)                      (consecutive q heads share a kv head)
 *     position  p = kv_len - qo_len + i                 (query block right-aligned to the KV)
 *     s_j       = sm_scale * <q[i,h,:], K_r[j,c,:]>      for 0 <= j <= p
 *     o         = sum_j exp(s_j - m) V_r[j,c,:] / sum_j exp(s_j - m),  m = max_j s_j
 *     lse       = m + log(sum_j exp(s_j - m))          (natural log)
 *
 * with K_r[j] read through the page table: page kv_indices[kv_indptr[r] + j / page_size],
 * slot j % page_size. Sources: causal scaled-dot-product attention over a paged KV cache, the
 * prefill operation of the sglang PR #46351 page (Motivation);
 * the query-to-position alignment is the one the sglang PR #46351 page states in its Fix
 * section and in the author's reply on tail alignment (row i sits at i + kv_len - qo_len,
 * key j is masked when j exceeds that position).
 *
 * fp8 keys/values use the OCP 8-bit E4M3 encoding (bias 7, no infinities, S.1111.111 is NaN),
 * decoded exactly and multiplied by the caller's scale.
 *
 * Every (token, head) row is computed on its own, so any subset of rows is exact and the
 * result of a row cannot depend on which other rows are in the batch.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit floating point, E4M3 variant: 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN; there is
 * no infinity, so exponent 15 with mantissa 0..6 are ordinary normals (max 448). */
double oracle_e4m3_to_double(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* E4M3 values of all 256 codes, filled once from oracle_e4m3_to_double (the same decode,
 * looked up instead of recomputed per element). */
static double g_e4m3[256];
static void fill_e4m3_table(void) {
  for (int c = 0; c < 256; ++c) g_e4m3[c] = oracle_e4m3_to_double((uint8_t)c);
}

static double load_kv(const void* pool, int kv_dtype, int64_t idx, double scale) {
  if (kv_dtype == 0) return oracle_bf16_to_double(((const uint16_t*)pool)[idx]);
  return g_e4m3[((const uint8_t*)pool)[idx]] * scale;
}

/* Index of the request owning global query token t (qo_indptr is non-decreasing). */
static int find_request(const int32_t* qo_indptr, int batch, int64_t t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (qo_indptr[mid] <= t) lo = mid; else hi = mid - 1;
  }
  /* skip empty requests that share the same start */
  while (lo + 1 < batch && qo_indptr[lo + 1] <= t) lo++;
  return lo;
}

static int64_t kv_len_of(const int32_t* kv_indptr, const int32_t* last_len, int page_size, int r) {
  int64_t np = kv_indptr[r + 1] - kv_indptr[r];
  return np > 0 ? (np - 1) * page_size + last_len[r] : 0;
}

/*
 * Attention rows over the paged KV cache.
 *
 * q        [Nq, hq, d] bf16 bits, Nq = qo_indptr[batch]
 * k_pool   [num_pages, page_size, hkv, d], bf16 bits (kv_dtype 0) or E4M3 codes (kv_dtype 1)
 * v_pool   same layout as k_pool
 * sel      optional list of n_sel global query tokens to compute (NULL: all Nq tokens, in order)
 * key_lo, key_hi
 *          keys outside [key_lo, key_hi) are left out (key_hi < 0 means no upper bound).
 *          The full operation is key_lo = 0, key_hi = -1. A row with no key in range
 *          gets o = 0 and lse = -inf (the empty softmax partial).
 * o        [n_rows, hq, d] fp64 out;  lse [n_rows, hq] fp64 out (natural log)
 *
 * Returns ORACLE_EINVAL if some request has qo_len > kv_len or a malformed table.
 */
int oracle_paged_prefill(int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t page_size,
                         int32_t kv_dtype, double sm_scale, double k_scale, double v_scale,
                         const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, const int32_t* kv_last_page_len,
                         const uint16_t* q, const void* k_pool, const void* v_pool,
                         int64_t n_sel, const int64_t* sel, int64_t key_lo, int64_t key_hi,
                         double* o, double* lse) {
  if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d <= 0 || page_size <= 0)
    return ORACLE_EINVAL;
  if (kv_dtype != 0 && kv_dtype != 1) return ORACLE_EINVAL;
  int64_t max_kv = 0;
  for (int r = 0; r < batch; ++r) {
    int64_t qo_len = qo_indptr[r + 1] - qo_indptr[r];
    int64_t np = kv_indptr[r + 1] - kv_indptr[r];
    if (qo_len < 0 || np < 0) return ORACLE_EINVAL;
    if (np > 0 && (kv_last_page_len[r] < 1 || kv_last_page_len[r] > page_size)) return ORACLE_EINVAL;
    int64_t kv_len = kv_len_of(kv_indptr, kv_last_page_len, page_size, r);
    if (qo_len > kv_len) return ORACLE_EINVAL;
    if (kv_len > max_kv) max_kv = kv_len;
  }
  fill_e4m3_table();
  const int64_t nq = qo_indptr[batch];
  const int64_t n_rows = sel ? n_sel : nq;
  const int group = hq / hkv;
  int bad = 0;

#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_kv > 0 ? max_kv : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t work = 0; work < n_rows * hq; ++work) {
      const int64_t row = work / hq;
      const int h = (int)(work % hq);
      const int64_t t = sel ? sel[row] : row;
      double* orow = o + (row * hq + h) * d;
      if (t < 0 || t >= nq) {
        bad = 1;
        continue;
      }
      const int r = find_request(qo_indptr, batch, t);
      const int64_t qo_len = qo_indptr[r + 1] - qo_indptr[r];
      const int64_t kv_len = kv_len_of(kv_indptr, kv_last_page_len, page_size, r);
      const int64_t i = t - qo_indptr[r];
      const int64_t pos = kv_len - qo_len + i;
      const int c = h / group;
      const uint16_t* qrow = q + (t * hq + h) * (int64_t)d;
      int64_t lo = key_lo > 0 ? key_lo : 0;
      int64_t hi = pos + 1;
      if (key_hi >= 0 && key_hi < hi) hi = key_hi;

      double m = -INFINITY;
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t page = kv_indices[kv_indptr[r] + j / page_size];
        const int64_t base = ((page * page_size + j % page_size) * hkv + c) * (int64_t)d;
        double dot = 0.0;
        for (int k = 0; k < d; ++k)
          dot += oracle_bf16_to_double(qrow[k]) * load_kv(k_pool, kv_dtype, base + k, k_scale);
        s[j] = sm_scale * dot;
        if (s[j] > m) m = s[j];
      }
      for (int k = 0; k < d; ++k) acc[k] = 0.0;
      double l = 0.0;
      for (int64_t j = lo; j < hi; ++j) {
        const int64_t page = kv_indices[kv_indptr[r] + j / page_size];
        const int64_t base = ((page * page_size + j % page_size) * hkv + c) * (int64_t)d;
        const double e = exp(s[j] - m);
        l += e;
        for (int k = 0; k < d; ++k) acc[k] += e * load_kv(v_pool, kv_dtype, base + k, v_scale);
      }
      if (hi <= lo) {
        for (int k = 0; k < d; ++k) orow[k] = 0.0;
        lse[row * hq + h] = -INFINITY;
      } else {
        for (int k = 0; k < d; ++k) orow[k] = acc[k] / l;
        lse[row * hq + h] = m + log(l);
      }
    }
    free(s);
    free(acc);
  }
  return bad ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * Combination of softmax partials over disjoint key sets (the states that fixed KV splits
 * produce). Partial s of a row is (o_s, lse_s) with lse_s the natural-log normaliser over its
 * keys; the combined row is the softmax over the union of the keys:
 *
 *   lse = log sum_s exp(lse_s),    o = sum_s exp(lse_s - lse) * o_s
 *
 * o_part [R, S, H, d], lse_part [R, S, H]; o [R, H, d], lse [R, H]. An empty partial
 * (lse_s = -inf) has weight zero. A row whose partials are all empty gets o = 0, lse = -inf.
 */
void oracle_merge_states(int64_t R, int32_t S, int32_t H, int32_t d, const double* o_part,
                         const double* lse_part, double* o, double* lse) {
#pragma omp parallel for schedule(static)
  for (int64_t rh = 0; rh < R * H; ++rh) {
    const int64_t r = rh / H;
    const int h = (int)(rh % H);
    double m = -INFINITY;
    for (int s = 0; s < S; ++s) {
      const double v = lse_part[(r * S + s) * H + h];
      if (v > m) m = v;
    }
    double* orow = o + rh * d;
    for (int k = 0; k < d; ++k) orow[k] = 0.0;
    if (m == -INFINITY) {
      lse[rh] = -INFINITY;
      continue;
    }
    double w_sum = 0.0;
    for (int s = 0; s < S; ++s) {
      const double w = exp(lse_part[(r * S + s) * H + h] - m);
      w_sum += w;
      const double* os = o_part + ((r * S + s) * H + h) * (int64_t)d;
      for (int k = 0; k < d; ++k) orow[k] += w * os[k];
    }
    for (int k = 0; k < d; ++k) orow[k] /= w_sum;
    lse[rh] = m + log(w_sum);
  }
}
