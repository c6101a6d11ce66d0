/*
 * pagedkv_oracle.c -- fp64 CPU reference for one paged-attention decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header or table with the HIP kernels.
 *
 * What it computes (plain definitions, no blocking or fusion):
 *
 *  - oracle_attn: for every sequence b and query head h, gather K and V rows through the
 *    block table and return softmax(scale * q K^T) V in fp64.  The block table maps a
 *    (sequence, logical block) pair to a physical block of a shared pool, and the blocks of
 *    one sequence need not be contiguous ("vllm-project-vllm -- L2", section 3 Q2 and
 *    section 6 "KV Cache Block Tables").  Decode attends one new query token per sequence
 *    over its whole cache (same page, section 7).  Query head h reads KV head h / (Hq/Hkv).
 *  - oracle_attn_partials: the same attention restricted to consecutive token partitions,
 *    returning per-partition (max score, sum of exp, normalised output).
 *  - oracle_lse_merge: combines such partials by log-sum-exp weighting.
 *  - oracle_kv_write: scatters new K/V rows into pool slots (slot = block*BS + offset);
 *    negative slots are skipped.  For an fp8 cache each element is quantised by
 *    oracle_fp8_encode.
 *  - fp8 codec: OCP E4M3FN (bias 7, max 448, NaN = S.1111.111, no infinities).  Decode
 *    follows the format definition; encode divides in fp32 and picks the nearest finite
 *    code, ties to the even code, saturating at +-448.
 *
 * Element types: 0 = fp16, 1 = bf16, 2 = fp8 e4m3fn (pools only).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F16 = 0, ODT_BF16 = 1, ODT_FP8 = 2 };

/* ---------------------------------------------------------------- element decoding */

static double f16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);     /* (1 + m/1024) * 2^(e-15) */
  return s ? -v : v;
}

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;              /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double oracle_fp8_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);                  /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp((double)(8 + m), e - 10);        /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

static double elem_value(const void* base, size_t idx, int dt) {
  switch (dt) {
    case ODT_F16: return f16_value(((const uint16_t*)base)[idx]);
    case ODT_BF16: return bf16_value(((const uint16_t*)base)[idx]);
    default: return oracle_fp8_decode(((const uint8_t*)base)[idx]);
  }
}

static size_t elem_size(int dt) { return dt == ODT_FP8 ? 1 : 2; }

/* ---------------------------------------------------------------- fp8 encode */

/* Values of the 127 non-negative finite codes, filled from oracle_fp8_decode. */
static double g_mag[127];
static int g_mag_ready = 0;

static void fp8_table_init(void) {
  if (g_mag_ready) return;
  for (int c = 0; c < 127; ++c) g_mag[c] = oracle_fp8_decode((uint8_t)c);
  g_mag_ready = 1;
}

/* Nearest finite E4M3FN magnitude code for a >= 0 (codes 0..126 are increasing in value);
   ties go to the even code; anything at or above 448 maps to 448 (code 126). */
static uint8_t fp8_nearest_magnitude(double a) {
  int lo = 0, hi = 126;                        /* invariant: value(lo) <= a < value(hi) */
  if (a >= 448.0) return 126;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g_mag[mid] <= a) lo = mid; else hi = mid;
  }
  double below = g_mag[lo], above = g_mag[lo + 1];
  double dlo = a - below, dhi = above - a;
  if (dlo < dhi) return (uint8_t)lo;
  if (dhi < dlo) return (uint8_t)(lo + 1);
  return (uint8_t)((lo % 2 == 0) ? lo : lo + 1);
}

uint8_t oracle_fp8_encode(float x, float scale) {
  fp8_table_init();
  float y = x / scale;                         /* IEEE fp32 division, round to nearest even */
  if (isnan(y)) return (uint8_t)(signbit(y) ? 0xFF : 0x7F);
  uint8_t mag = fp8_nearest_magnitude(fabs((double)y));
  return (uint8_t)(signbit(y) ? (0x80 | mag) : mag);
}

void oracle_fp8_encode_array(const float* x, int64_t n, float scale, uint8_t* out) {
  fp8_table_init();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(x[i], scale);
}

void oracle_fp8_decode_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_decode(c[i]);
}

/* ---------------------------------------------------------------- KV write */

/* key/value: [T, Hkv, D] in src_dt (fp16|bf16).  Caches: [NB, BS, Hkv, D] in cache_dt.
   Returns 0, or -1 if a slot is outside the pool (nothing is written for that row). */
int oracle_kv_write(const void* key, const void* value, void* key_cache, void* value_cache,
                    const int64_t* slot_mapping, int64_t T, int64_t num_blocks, int block_size,
                    int Hkv, int D, int src_dt, int cache_dt, float k_scale, float v_scale) {
  const size_t row = (size_t)Hkv * D;
  const size_t es = elem_size(src_dt), ec = elem_size(cache_dt);
  int bad = 0;
  fp8_table_init();
#pragma omp parallel for schedule(static) reduction(|| : bad)
  for (int64_t i = 0; i < T; ++i) {
    int64_t s = slot_mapping[i];
    if (s < 0) continue;                       /* padding token */
    if (s >= num_blocks * (int64_t)block_size) { bad = 1; continue; }
    int64_t blk = s / block_size, off = s % block_size;
    size_t dst = ((size_t)blk * block_size + (size_t)off) * row;
    size_t src = (size_t)i * row;
    for (int pass = 0; pass < 2; ++pass) {
      const void* in = pass ? value : key;
      void* cache = pass ? value_cache : key_cache;
      float sc = pass ? v_scale : k_scale;
      if (cache_dt == src_dt) {
        memcpy((char*)cache + dst * ec, (const char*)in + src * es, row * es);
      } else {
        for (size_t j = 0; j < row; ++j) {
          float x = (float)elem_value(in, src + j, src_dt);   /* fp16/bf16 -> fp32 is exact */
          ((uint8_t*)cache)[dst + j] = oracle_fp8_encode(x, sc);
        }
      }
    }
  }
  return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- attention */

typedef struct {
  const void* q; int q_dt;
  const void* kc; const void* vc; int kv_dt;
  const int32_t* bt; int max_blocks;
  const int32_t* lens;
  int B, Hq, Hkv, D, BS;
  double scale, k_scale, v_scale;
} attn_args;

/* Scores s_t = scale * sum_d q[d] * K_t[d] for t in [t0, t1) of sequence b, query head h. */
static void scores(const attn_args* a, int b, int h, int64_t t0, int64_t t1, double* s) {
  const int G = a->Hq / a->Hkv, g = h / G, D = a->D;
  const size_t qoff = ((size_t)b * a->Hq + h) * D;
  for (int64_t t = t0; t < t1; ++t) {
    int64_t blk = a->bt[(size_t)b * a->max_blocks + t / a->BS];
    int64_t off = t % a->BS;
    size_t krow = (((size_t)blk * a->BS + off) * a->Hkv + g) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += elem_value(a->q, qoff + d, a->q_dt) * (elem_value(a->kc, krow + d, a->kv_dt) * a->k_scale);
    s[t - t0] = a->scale * dot;
  }
}

/* softmax-weighted V over tokens [t0, t1): returns max score m, sum of exp l, and
   o = sum_t exp(s_t - m) V_t / l. */
static void attend_range(const attn_args* a, int b, int h, int64_t t0, int64_t t1, double* s,
                         double* m_out, double* l_out, double* o) {
  const int G = a->Hq / a->Hkv, g = h / G, D = a->D;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (t1 <= t0) { *m_out = -INFINITY; *l_out = 0.0; return; }
  scores(a, b, h, t0, t1, s);
  double m = -INFINITY;
  for (int64_t t = t0; t < t1; ++t) if (s[t - t0] > m) m = s[t - t0];
  double l = 0.0;
  for (int64_t t = t0; t < t1; ++t) {
    int64_t blk = a->bt[(size_t)b * a->max_blocks + t / a->BS];
    int64_t off = t % a->BS;
    size_t vrow = (((size_t)blk * a->BS + off) * a->Hkv + g) * D;
    double w = exp(s[t - t0] - m);
    l += w;
    for (int d = 0; d < D; ++d) o[d] += w * (elem_value(a->vc, vrow + d, a->kv_dt) * a->v_scale);
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  *m_out = m;
  *l_out = l;
}

static int check_args(const attn_args* a) {
  if (a->Hkv <= 0 || a->Hq % a->Hkv != 0 || a->D <= 0 || a->BS <= 0 || a->B < 0) return -2;
  for (int b = 0; b < a->B; ++b)
    if (a->lens[b] < 0 || a->lens[b] > (int64_t)a->max_blocks * a->BS) return -2;
  return 0;
}

/* out: [B, Hq, D] fp64.  A sequence with n = 0 gets zeros. */
int oracle_attn(const void* q, int q_dt, const void* key_cache, const void* value_cache, int kv_dt,
                const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                int B, int Hq, int Hkv, int D, int block_size,
                double scale, double k_scale, double v_scale, double* out, int nthreads) {
  attn_args a = {q, q_dt, key_cache, value_cache, kv_dt, block_tables, max_blocks, context_lens,
                 B, Hq, Hkv, D, block_size, scale, k_scale, v_scale};
  int rc = check_args(&a);
  if (rc) return rc;
  int64_t nmax = 0;
  for (int b = 0; b < B; ++b) if (context_lens[b] > nmax) nmax = context_lens[b];
  const int64_t units = (int64_t)B * Hq;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(nmax > 0 ? nmax : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      int b = (int)(u / Hq), h = (int)(u % Hq);
      double m, l;
      attend_range(&a, b, h, 0, context_lens[b], s, &m, &l, out + (size_t)u * D);
    }
    free(s);
  }
  return 0;
}

/* Partition p of sequence b covers tokens [p*PS, min((p+1)*PS, n)).  For p < ceil(n/PS):
   m[b,h,p] = max score, l[b,h,p] = sum exp(s - m), o[b,h,p,:] = normalised partial output.
   Entries for p >= ceil(n/PS) are left untouched.  Shapes [B,Hq,Pmax] and [B,Hq,Pmax,D]. */
int oracle_attn_partials(const void* q, int q_dt, const void* key_cache, const void* value_cache,
                         int kv_dt, const int32_t* block_tables, int max_blocks,
                         const int32_t* context_lens, int B, int Hq, int Hkv, int D, int block_size,
                         double scale, double k_scale, double v_scale, int partition_size, int Pmax,
                         double* m, double* l, double* o, int nthreads) {
  attn_args a = {q, q_dt, key_cache, value_cache, kv_dt, block_tables, max_blocks, context_lens,
                 B, Hq, Hkv, D, block_size, scale, k_scale, v_scale};
  int rc = check_args(&a);
  if (rc) return rc;
  if (partition_size <= 0) return -2;
  for (int b = 0; b < B; ++b)
    if ((context_lens[b] + partition_size - 1) / partition_size > Pmax) return -2;
  const int64_t units = (int64_t)B * Hq;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)partition_size);
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      int b = (int)(u / Hq);
      int64_t n = context_lens[b];
      int64_t P = (n + partition_size - 1) / partition_size;
      for (int64_t p = 0; p < P; ++p) {
        int64_t t0 = p * partition_size, t1 = t0 + partition_size < n ? t0 + partition_size : n;
        size_t idx = (size_t)u * Pmax + (size_t)p;
        attend_range(&a, b, (int)(u % Hq), t0, t1, s, m + idx, l + idx, o + idx * D);
      }
    }
    free(s);
  }
  return 0;
}

/* Log-sum-exp merge of R rows of partials: M = max_p m_p, w_p = l_p exp(m_p - M),
   out = sum_p w_p o_p / sum_p w_p over p < nparts[r].  A row with nparts = 0 gets zeros. */
void oracle_lse_merge(const double* m, const double* l, const double* o, const int32_t* nparts,
                      int64_t R, int Pmax, int D, double* out) {
  for (int64_t r = 0; r < R; ++r) {
    double* dst = out + (size_t)r * D;
    for (int d = 0; d < D; ++d) dst[d] = 0.0;
    int P = nparts[r];
    if (P <= 0) continue;
    double M = -INFINITY;
    for (int p = 0; p < P; ++p) if (m[(size_t)r * Pmax + p] > M) M = m[(size_t)r * Pmax + p];
    double wsum = 0.0;
    for (int p = 0; p < P; ++p) {
      size_t idx = (size_t)r * Pmax + p;
      double w = l[idx] * exp(m[idx] - M);
      wsum += w;
      for (int d = 0; d < D; ++d) dst[d] += w * o[idx * D + d];
    }
    for (int d = 0; d < D; ++d) dst[d] /= wsum;
  }
}
