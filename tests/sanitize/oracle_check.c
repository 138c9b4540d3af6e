/* oracle_check.c - drives every function of the CPU oracle (oracle/oracle.c) over small
 * inputs and their edge cases (empty and partial visibility, k above and below the visible
 * count, ties, -1 padding, a clipped raw window, attention sinks, every dtype), for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer. Test infrastructure: it checks memory
 * safety and defined behaviour plus a few invariants, not values (the pin tests do that).
 * Exit status 0 = clean; the sanitizers abort with a report otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_to_double(uint16_t bits);
double orc_e2m1_to_double(int code);
double orc_e4m3_to_double(int code);
double orc_e8m0_to_double(int byte);
void orc_decode(int dt, const void* src, int64_t n, double* dst);
void orc_decode_mxfp4_row(const uint8_t* codes, const uint8_t* scales, int D, double* out);
void orc_decode_mxfp8_row(const uint8_t* codes, const uint8_t* scales, int D, double* out);
void orc_compress_mean(int64_t n_raw, int D, int m, int dt, const void* raw, double* out);
int64_t orc_n_vis(int64_t p, int m, int64_t N);
int64_t orc_n_vis_len(int64_t p, int m, int64_t N, int64_t len);
void orc_scores_row(int H_I, int D_I, int64_t N, int64_t n_vis, int qdt, const void* qI,
                    const uint8_t* qscale, const float* w, int kdt, const void* kI,
                    const uint8_t* kscale, double* out);
int orc_topk_row(const double* scores, int64_t n_vis, int k, int32_t* idx);
void orc_attend_row(int H, int D_K, int D_V, int qdt, const void* q, int kvdt, const void* kv,
                    const int32_t* idx, int k, int rawdt, const void* kv_raw, int64_t raw_base,
                    int64_t n_raw, int64_t p, int W, double scale, const double* sink,
                    double* out, double* lse);

enum { F32 = 0, BF16 = 1, MXFP4 = 2, F64 = 3, MXFP8 = 4 };

static uint64_t st = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(void) { /* xorshift64* */
  st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
  return (uint32_t)((st * 0x2545f4914f6cdd1dull) >> 32);
}
static float frnd(void) { return (float)(rnd() % 2001) / 1000.0f - 1.0f; }
static uint16_t to_bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

/* exact-size heap buffers, so that any overrun hits a redzone */
static void* buf(size_t n) { void* p = malloc(n ? n : 1); memset(p, 0, n ? n : 1); return p; }

static void decoders(void) {
  double acc = 0.0;
  for (int c = 0; c < 16; ++c) acc += fabs(orc_e2m1_to_double(c));
  CHECK(acc == 2.0 * (0.5 + 1 + 1.5 + 2 + 3 + 4 + 6));
  for (int c = 0; c < 256; ++c) { double v = orc_e4m3_to_double(c); (void)v; }
  for (int c = 0; c < 255; ++c) CHECK(orc_e8m0_to_double(c) > 0.0);
  CHECK(isnan(orc_e8m0_to_double(255)));
  for (int b = 0; b < 65536; b += 97) { double v = orc_bf16_to_double((uint16_t)b); (void)v; }
  const int D = 128;
  uint8_t* c4 = buf(D / 2); uint8_t* c8 = buf(D); uint8_t* sc = buf(D / 32);
  for (int i = 0; i < D / 2; ++i) c4[i] = (uint8_t)rnd();
  for (int i = 0; i < D; ++i) c8[i] = (uint8_t)(rnd() % 0x7e);
  for (int i = 0; i < D / 32; ++i) sc[i] = (uint8_t)(120 + rnd() % 10);
  double* o = buf(sizeof(double) * D);
  orc_decode_mxfp4_row(c4, sc, D, o);
  orc_decode_mxfp8_row(c8, sc, D, o);
  float* f = buf(sizeof(float) * 7); uint16_t* h = buf(2 * 7); double* g = buf(8 * 7);
  for (int i = 0; i < 7; ++i) { f[i] = frnd(); h[i] = to_bf16(f[i]); g[i] = f[i]; }
  orc_decode(F32, f, 7, o); CHECK(o[6] == (double)f[6]);
  orc_decode(BF16, h, 7, o);
  orc_decode(F64, g, 7, o); CHECK(o[3] == g[3]);
  free(c4); free(c8); free(sc); free(o); free(f); free(h); free(g);
}

static void compress(void) {
  const int D = 8;
  for (int m = 1; m <= 5; ++m)
    for (int64_t n_raw = 0; n_raw <= 11; ++n_raw) {
      float* rf = buf(sizeof(float) * (size_t)(n_raw * D));
      uint16_t* rb = buf(2 * (size_t)(n_raw * D));
      for (int64_t i = 0; i < n_raw * D; ++i) { rf[i] = 1.5f; rb[i] = to_bf16(1.5f); }
      double* out = buf(sizeof(double) * (size_t)((n_raw / m) * D));
      orc_compress_mean(n_raw, D, m, F32, rf, out);
      for (int64_t i = 0; i < (n_raw / m) * D; ++i) CHECK(out[i] == 1.5);
      orc_compress_mean(n_raw, D, m, BF16, rb, out);
      free(rf); free(rb); free(out);
    }
}

static void visibility(void) {
  CHECK(orc_n_vis(-1, 1, 10) == 0);
  CHECK(orc_n_vis(2, 4, 10) == 0);
  CHECK(orc_n_vis(3, 4, 10) == 1);
  CHECK(orc_n_vis(1000, 1, 10) == 10);
  CHECK(orc_n_vis_len(1000, 1, 10, 4) == 4);
  CHECK(orc_n_vis_len(1000, 1, 10, 0) == 0);
  CHECK(orc_n_vis_len(5, 1, 10, -3) == 0);
}

static void scores_and_topk(void) {
  const int H_I = 4, D_I = 32;
  const int64_t N = 23;
  float* qf = buf(sizeof(float) * H_I * D_I); uint16_t* qb = buf(2 * H_I * D_I);
  uint8_t* q8 = buf(H_I * D_I); uint8_t* qs = buf(H_I * (D_I / 32));
  float* w = buf(sizeof(float) * H_I);
  float* kf = buf(sizeof(float) * (size_t)(N * D_I)); uint16_t* kb = buf(2 * (size_t)(N * D_I));
  uint8_t* k4 = buf((size_t)(N * D_I / 2)); uint8_t* k8 = buf((size_t)(N * D_I));
  uint8_t* ks = buf((size_t)(N * (D_I / 32)));
  for (int i = 0; i < H_I * D_I; ++i) { qf[i] = frnd(); qb[i] = to_bf16(qf[i]); q8[i] = (uint8_t)(rnd() % 0x7e); }
  for (int i = 0; i < H_I * (D_I / 32); ++i) qs[i] = 127;
  for (int j = 0; j < H_I; ++j) w[j] = (j & 1) ? -frnd() : frnd(); /* mixed signs */
  for (int64_t i = 0; i < N * D_I; ++i) { kf[i] = frnd(); kb[i] = to_bf16(kf[i]); k8[i] = (uint8_t)(rnd() % 0x7e); }
  for (int64_t i = 0; i < N * D_I / 2; ++i) k4[i] = (uint8_t)rnd();
  for (int64_t i = 0; i < N * (D_I / 32); ++i) ks[i] = (uint8_t)(125 + rnd() % 4);
  double* sc = buf(sizeof(double) * (size_t)N);
  int32_t* idx = buf(sizeof(int32_t) * 64);
  const int64_t nvs[] = {0, 1, 7, 22, 23};
  for (int a = 0; a < 5; ++a) {
    const int64_t nv = nvs[a];
    orc_scores_row(H_I, D_I, N, nv, F32, qf, NULL, w, F32, kf, NULL, sc);
    for (int64_t s = nv; s < N; ++s) CHECK(isinf(sc[s]) && sc[s] < 0);
    orc_scores_row(H_I, D_I, N, nv, BF16, qb, NULL, w, BF16, kb, NULL, sc);
    orc_scores_row(H_I, D_I, N, nv, BF16, qb, NULL, w, MXFP4, k4, ks, sc);
    orc_scores_row(H_I, D_I, N, nv, MXFP8, q8, qs, w, MXFP4, k4, ks, sc);
    orc_scores_row(H_I, D_I, N, nv, MXFP8, q8, qs, w, MXFP8, k8, ks, sc);
    const int ks_[] = {1, 5, 7, 22, 23, 64};
    for (int b = 0; b < 6; ++b) {
      const int k = ks_[b];
      int32_t* ix = buf(sizeof(int32_t) * (size_t)k);
      int cnt = orc_topk_row(sc, nv, k, ix);
      CHECK(cnt == (nv < k ? (int)nv : k));
      for (int i = 0; i < cnt; ++i) CHECK(ix[i] >= 0 && ix[i] < nv && (i == 0 || ix[i] > ix[i - 1]));
      for (int i = cnt; i < k; ++i) CHECK(ix[i] == -1);
      free(ix);
    }
  }
  /* ties: all equal scores keep the lowest indices */
  for (int64_t s = 0; s < N; ++s) sc[s] = 0.25;
  int32_t* ix = buf(sizeof(int32_t) * 5);
  orc_topk_row(sc, N, 5, ix);
  for (int i = 0; i < 5; ++i) CHECK(ix[i] == i);
  free(ix);
  free(qf); free(qb); free(q8); free(qs); free(w); free(kf); free(kb); free(k4); free(k8); free(ks);
  free(sc); free(idx);
}

static void attend(void) {
  const int H = 3, D_K = 16, D_V = 12, N = 9, n_raw = 6, W = 4;
  const int64_t raw_base = 10;
  float* qf = buf(sizeof(float) * H * D_K); uint16_t* qb = buf(2 * H * D_K);
  float* kvf = buf(sizeof(float) * N * D_K); uint16_t* kvb = buf(2 * N * D_K);
  float* rf = buf(sizeof(float) * n_raw * D_K); uint16_t* rb = buf(2 * n_raw * D_K);
  for (int i = 0; i < H * D_K; ++i) { qf[i] = frnd(); qb[i] = to_bf16(qf[i]); }
  for (int i = 0; i < N * D_K; ++i) { kvf[i] = frnd(); kvb[i] = to_bf16(kvf[i]); }
  for (int i = 0; i < n_raw * D_K; ++i) { rf[i] = frnd(); rb[i] = to_bf16(rf[i]); }
  double sink[3] = {0.0, -1.0, 2.0};
  double* out = buf(sizeof(double) * H * D_V); double* lse = buf(sizeof(double) * H);
  const int k = 5;
  int32_t* idx = buf(sizeof(int32_t) * k);
  const int32_t sets[3][5] = {{0, 3, 8, -1, -1}, {-1, -1, -1, -1, -1}, {1, 2, 4, 5, 7}};
  const int64_t ps[] = {0, 9, 12, 15, 40};
  for (int s = 0; s < 3; ++s)
    for (int a = 0; a < 5; ++a)
      for (int wv = 0; wv <= W; wv += W)
        for (int sk = 0; sk < 2; ++sk) {
          memcpy(idx, sets[s], sizeof(int32_t) * k);
          orc_attend_row(H, D_K, D_V, F32, qf, F32, kvf, idx, k, F32, wv ? rf : NULL, raw_base,
                         n_raw, ps[a], wv, 0.25, sk ? sink : NULL, out, lse);
          for (int i = 0; i < H * D_V; ++i) CHECK(isfinite(out[i]));
          orc_attend_row(H, D_K, D_V, BF16, qb, BF16, kvb, idx, k, BF16, wv ? rb : NULL,
                         raw_base, n_raw, ps[a], wv, 0.25, sk ? sink : NULL, out, lse);
        }
  /* no selected entry and no window: out = 0, lse = sink (or -inf) */
  orc_attend_row(H, D_K, D_V, F32, qf, F32, kvf, sets[1], k, F32, NULL, 0, 0, 3, 0, 0.25, NULL, out, lse);
  for (int h = 0; h < H; ++h) CHECK(isinf(lse[h]) && lse[h] < 0);
  orc_attend_row(H, D_K, D_V, F32, qf, F32, kvf, sets[1], k, F32, NULL, 0, 0, 3, 0, 0.25, sink, out, lse);
  for (int h = 0; h < H; ++h) CHECK(lse[h] == sink[h]);
  for (int i = 0; i < H * D_V; ++i) CHECK(out[i] == 0.0);
  /* k = 0 */
  orc_attend_row(H, D_K, D_V, F32, qf, F32, kvf, idx, 0, F32, rf, raw_base, n_raw, 12, W, 0.25, NULL, out, lse);
  free(qf); free(qb); free(kvf); free(kvb); free(rf); free(rb); free(out); free(lse); free(idx);
}

int main(void) {
  decoders();
  compress();
  visibility();
  scores_and_topk();
  attend();
  if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
  printf("oracle_check: ok\n");
  return 0;
}
