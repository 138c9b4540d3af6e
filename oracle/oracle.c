/*
 * oracle.c - plain, slow, fp64 CPU oracle of the DSA / CSA hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this library. It shares no code, header, table or helper with the GPU
 * library; both read the same stored input bytes written by the seeded generator.
 *
 * Every step is the plain definition, in fp64, with no blocking, fusion or reordering:
 *   compress  : kv_c[j] = mean_{i<m} kv_raw[m*j + i]          ([P1] V4 CSA summary: every 4
 *               tokens' KV become one entry; [P4] CSA snippets: "e.g. average pooling")
 *   visibility: n_vis = min(N, floor((p + 1) / m))            (a query sees itself; only
 *               complete blocks; reading of [P5] s3 step 3 keep-all rule at context <= k)
 *   scores    : I[s] = sum_j w[j] * max(0, sum_d q_I[j,d] * k_I[s,d]),  s < n_vis
 *               ([P5] s1.3 lightning indexer, ReLU for throughput; formula as stated for
 *               the path: the page's own formula image is lost)
 *   top-k     : if n_vis <= k keep all; else the first k of a sort by (score desc, index asc)
 *               ([P5] s1.3 fine-grained sparse attention step 2; s3 step 3)
 *   attention : E = selected entries u raw window rows (p-W+1 .. p), one joint softmax,
 *               z = scale * q . K_e, out = sum softmax(z)_e * K_e[:D_V], lse = log sum exp z
 *               ([P5] s1.3 step 3, s1.4 MQA mode: one latent row shared by all heads;
 *               [P4] window KV concatenated with the compressed KV)
 *   sink      : optional per-head logit s_h joining that softmax with a zero value vector:
 *               out = sum_e exp(z_e) K_e[:D_V] / (sum_e exp(z_e) + exp(s_h)),
 *               lse = log(sum_e exp(z_e) + exp(s_h))   ([P4] CSA snippet 4.3: sliding window
 *               plus an attention sink; read as one learned logit per head, unscaled)
 *   ragged    : optional per-sequence entry count len_b: entries s >= len_b are not visible,
 *               n_vis = min(N, floor((p + 1) / m), len_b)
 * Sources: [P5] "DeepSeek-V3.2 sparse-attention principle and TPU adaptation" (trdm.cn);
 *          [P1] xhh.club "sparse" tag feed, DeepSeek-V4 CSA summary;
 *          [P4] Tencent Cloud developer search "compressed sparse attention (CSA)".
 * MXFP4 / MXFP8 decoding follows the OCP Microscaling Formats spec v1.0 (e2m1 and e4m3
 * elements, one E8M0 scale per 32 elements).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MXFP4 = 2, ORC_F64 = 3, ORC_MXFP8 = 4 };

/* ---- stored-value decoding (exact) ------------------------------------------------------ */

double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16; /* bf16 is the upper half of an IEEE binary32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP MX e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa. */
double orc_e2m1_to_double(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, mbit = code & 1;
  double mag = (e == 0) ? 0.5 * mbit                      /* subnormal: 0 or 0.5 */
                        : ldexp(1.0 + 0.5 * mbit, e - 1); /* 1, 1.5, 2, 3, 4, 6 */
  return s ? -mag : mag;
}

/* OCP e4m3 (FP8 "E4M3FN"): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN (no infinities). */
double orc_e4m3_to_double(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, mant = code & 7;
  if (e == 15 && mant == 7) return NAN;
  double mag = (e == 0) ? ldexp(mant / 8.0, -6) : ldexp(1.0 + mant / 8.0, e - 7);
  return s ? -mag : mag;
}

/* OCP MX E8M0 scale: 2^(byte - 127); 0xFF is NaN. */
double orc_e8m0_to_double(int byte) {
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, byte - 127);
}

static double ld(int dt, const void* p, int64_t i) {
  switch (dt) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)p)[i]);
    case ORC_F64: return ((const double*)p)[i];
    default: abort();
  }
}

void orc_decode(int dt, const void* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = ld(dt, src, i);
}

/* One MXFP4 row of D values: codes [D/2] (low nibble = even element), scales [D/32]. */
void orc_decode_mxfp4_row(const uint8_t* codes, const uint8_t* scales, int D, double* out) {
  for (int i = 0; i < D; ++i) {
    int byte = codes[i / 2];
    int code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    out[i] = orc_e2m1_to_double(code) * orc_e8m0_to_double(scales[i / 32]);
  }
}

/* One MXFP8 row of D values: e4m3 codes [D], scales [D/32]. */
void orc_decode_mxfp8_row(const uint8_t* codes, const uint8_t* scales, int D, double* out) {
  for (int i = 0; i < D; ++i) out[i] = orc_e4m3_to_double(codes[i]) * orc_e8m0_to_double(scales[i / 32]);
}

/* ---- step 0: CSA compression ------------------------------------------------------------ */

/* One sequence: raw [n_raw, D] of dtype dt -> out [floor(n_raw/m), D] fp64 means. */
void orc_compress_mean(int64_t n_raw, int D, int m, int dt, const void* raw, double* out) {
  int64_t nc = n_raw / m;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < nc; ++j) {
    for (int d = 0; d < D; ++d) {
      double s = 0.0;
      for (int i = 0; i < m; ++i) s += ld(dt, raw, (m * j + i) * (int64_t)D + d);
      out[j * D + d] = s / m;
    }
  }
}

/* ---- visibility ----------------------------------------------------------------------- */

int64_t orc_n_vis(int64_t p, int m, int64_t N) {
  if (p < 0) return 0;
  int64_t v = (p + 1) / m;
  return v < N ? v : N;
}

/* n_vis of a sequence holding len entries (ragged batches): min(n_vis, len), len >= 0 */
int64_t orc_n_vis_len(int64_t p, int m, int64_t N, int64_t len) {
  int64_t v = orc_n_vis(p, m, N);
  return v < len ? v : (len > 0 ? len : 0);
}

/* ---- step 1: lightning-indexer scores of one query -------------------------------------- */

/* qI [H_I, D_I] (dtype qdt; MXFP8: codes [H_I, D_I] and qscale [H_I, D_I/32]), w [H_I],
 * kI [N, D_I] (dtype kdt; MXFP4: codes [N, D_I/2] and kscale [N, D_I/32]; MXFP8: codes
 * [N, D_I] and kscale [N, D_I/32]) -> out[s] = score for s < n_vis, -inf for n_vis <= s < N. */
void orc_scores_row(int H_I, int D_I, int64_t N, int64_t n_vis, int qdt, const void* qI,
                    const uint8_t* qscale, const float* w, int kdt, const void* kI,
                    const uint8_t* kscale, double* out) {
  double* q = (double*)malloc(sizeof(double) * (size_t)H_I * D_I);
  if (qdt == ORC_MXFP8)
    for (int j = 0; j < H_I; ++j)
      orc_decode_mxfp8_row((const uint8_t*)qI + (int64_t)j * D_I, qscale + (int64_t)j * (D_I / 32),
                           D_I, q + (int64_t)j * D_I);
  else
    orc_decode(qdt, qI, (int64_t)H_I * D_I, q);
#pragma omp parallel
  {
    double* k = (double*)malloc(sizeof(double) * (size_t)D_I);
#pragma omp for schedule(static)
    for (int64_t s = 0; s < N; ++s) {
      if (s >= n_vis) {
        out[s] = -INFINITY;
        continue;
      }
      if (kdt == ORC_MXFP4)
        orc_decode_mxfp4_row((const uint8_t*)kI + s * (D_I / 2), kscale + s * (D_I / 32), D_I, k);
      else if (kdt == ORC_MXFP8)
        orc_decode_mxfp8_row((const uint8_t*)kI + s * D_I, kscale + s * (D_I / 32), D_I, k);
      else
        for (int d = 0; d < D_I; ++d) k[d] = ld(kdt, kI, s * (int64_t)D_I + d);
      double I = 0.0;
      for (int j = 0; j < H_I; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D_I; ++d) dot += q[(int64_t)j * D_I + d] * k[d];
        I += (double)w[j] * (dot > 0.0 ? dot : 0.0);
      }
      out[s] = I;
    }
    free(k);
  }
  free(q);
}

/* ---- step 2: top-k of one query --------------------------------------------------------- */

typedef struct { double v; int64_t s; } orc_pair;

static int by_score_desc_then_index(const void* a, const void* b) {
  const orc_pair* x = (const orc_pair*)a;
  const orc_pair* y = (const orc_pair*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int by_index(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* idx[0..k): the selected entries ascending, then -1. Returns the number selected. */
int orc_topk_row(const double* scores, int64_t n_vis, int k, int32_t* idx) {
  int cnt;
  if (n_vis <= k) {
    for (int64_t s = 0; s < n_vis; ++s) idx[s] = (int32_t)s;
    cnt = (int)n_vis;
  } else {
    orc_pair* a = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)n_vis);
    for (int64_t s = 0; s < n_vis; ++s) { a[s].v = scores[s]; a[s].s = s; }
    qsort(a, (size_t)n_vis, sizeof(orc_pair), by_score_desc_then_index);
    for (int i = 0; i < k; ++i) idx[i] = (int32_t)a[i].s;
    free(a);
    qsort(idx, (size_t)k, sizeof(int32_t), by_index);
    cnt = k;
  }
  for (int i = cnt; i < k; ++i) idx[i] = -1;
  return cnt;
}

/* ---- step 3: sparse MQA attention of one query ------------------------------------------ */

/* q [H, D_K] (qdt); kv [N, D_K] (kvdt) rows addressed by idx[0..k) (-1 = skip); kv_raw rows at
 * raw positions raw_base .. raw_base+n_raw-1 (rawdt), of which the window p-W+1 .. p (clipped
 * at 0 and to what kv_raw holds) joins the entry set. out [H, D_V], lse [H]. */
void orc_attend_row(int H, int D_K, int D_V, int qdt, const void* q, int kvdt, const void* kv,
                    const int32_t* idx, int k, int rawdt, const void* kv_raw, int64_t raw_base,
                    int64_t n_raw, int64_t p, int W, double scale, const double* sink,
                    double* out, double* lse) {
  /* entry list: (source, row) */
  int cap = k + (W > 0 ? W : 0);
  const void** src = (const void**)malloc(sizeof(void*) * (size_t)(cap > 0 ? cap : 1));
  int* sdt = (int*)malloc(sizeof(int) * (size_t)(cap > 0 ? cap : 1));
  int64_t* row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
  int E = 0;
  for (int i = 0; i < k; ++i)
    if (idx[i] >= 0) { src[E] = kv; sdt[E] = kvdt; row[E] = idx[i]; ++E; }
  if (W > 0 && kv_raw) {
    int64_t lo = p - W + 1;
    if (lo < 0) lo = 0;
    for (int64_t r = lo; r <= p; ++r)
      if (r >= raw_base && r < raw_base + n_raw) {
        src[E] = kv_raw; sdt[E] = rawdt; row[E] = r - raw_base; ++E;
      }
  }
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
    double* qh = (double*)malloc(sizeof(double) * (size_t)D_K);
#pragma omp for schedule(static)
    for (int h = 0; h < H; ++h) {
      double* o = out + (int64_t)h * D_V;
      for (int d = 0; d < D_V; ++d) o[d] = 0.0;
      const double s_h = sink ? sink[h] : -INFINITY; /* sink logit (value vector 0) */
      if (E == 0) {
        lse[h] = s_h;
        continue;
      }
      for (int d = 0; d < D_K; ++d) qh[d] = ld(qdt, q, (int64_t)h * D_K + d);
      double zmax = s_h;
      for (int e = 0; e < E; ++e) {
        double dot = 0.0;
        for (int d = 0; d < D_K; ++d) dot += qh[d] * ld(sdt[e], src[e], row[e] * D_K + d);
        z[e] = scale * dot;
        if (z[e] > zmax) zmax = z[e];
      }
      double sum = sink ? exp(s_h - zmax) : 0.0;
      for (int e = 0; e < E; ++e) {
        z[e] = exp(z[e] - zmax);
        sum += z[e];
      }
      for (int e = 0; e < E; ++e) {
        double pe = z[e] / sum;
        for (int d = 0; d < D_V; ++d) o[d] += pe * ld(sdt[e], src[e], row[e] * D_K + d);
      }
      lse[h] = zmax + log(sum);
    }
    free(qh);
    free(z);
  }
  free(src);
  free(sdt);
  free(row);
}

int orc_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
