/* abi_check.c - the argument validation of libdsa's C ABI (include/dsa.h), driven from C for a
 * build whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer. Every call
 * here fails validation (or, with no usable gfx950 device, the device check) before anything
 * is launched, so it runs without a GPU and never dereferences the dummy device pointers.
 * It also compiles include/dsa.h as C. Exit status 0 = every status matched and the
 * sanitizers saw nothing. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsa.h"

#define P ((void*)(uintptr_t)0x10000) /* 16-byte aligned dummy device address */
#define PO(o) ((void*)((uintptr_t)0x10000 + (o)))

static int fails = 0;
#define EXPECT(call, want)                                                                  \
  do {                                                                                      \
    int got_ = (int)(call);                                                                 \
    if (got_ != (want)) {                                                                   \
      fprintf(stderr, "line %d: %s -> %d (%s), want %d\n", __LINE__, #call, got_,          \
              dsa_status_str(got_), (want));                                                \
      ++fails;                                                                              \
    }                                                                                       \
  } while (0)

static dsa_dims dims(int B, int T, int N, int H_I, int D_I, int H, int D_K, int D_V, int top_k,
                     int m, int W) {
  dsa_dims d = {B, T, N, H_I, D_I, H, D_K, D_V, top_k, m, W};
  return d;
}
static dsa_dims base(void) { return dims(2, 3, 100, 64, 128, 128, 576, 512, 32, 1, 0); }

static dsa_forward_args fargs(void) {
  dsa_forward_args a;
  memset(&a, 0, sizeof a);
  a.dt = DSA_BF16;
  a.k_dt = DSA_BF16;
  a.q_I = P; a.w = P; a.k_I = P; a.q = P; a.kv = P; a.q_pos = P; a.out = P;
  a.softmax_scale = 0.1f;
  return a;
}

static void status_and_version(void) {
  for (int c = 0; c <= 8; ++c) {
    const char* s = dsa_status_str(c);
    if (!s || strncmp(s, "DSA_", 4) != 0) { fprintf(stderr, "status %d: %s\n", c, s); ++fails; }
  }
  if (strcmp(dsa_status_str(-1), "unknown dsa_status") != 0) ++fails;
  if (strcmp(dsa_status_str(99), "unknown dsa_status") != 0) ++fails;
  if (dsa_version() != 220) ++fails;
  if (dsa_noalloc_scratch_bytes() != DSA_NOALLOC_SCRATCH_BYTES) ++fails;
}

static void indexer(void) {
  dsa_dims d = base(), e;
  EXPECT(indexer_scores(NULL, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 1);
  EXPECT(indexer_scores(&d, NULL, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 1);
  EXPECT(indexer_scores(&d, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, NULL, NULL, P, NULL), 1);
  EXPECT(indexer_scores(&d, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, PO(2), P, NULL), 4);
  e = base(); e.N = 0;
  EXPECT(indexer_scores(&e, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 2);
  e = base(); e.top_k = 5000;
  EXPECT(indexer_scores(&e, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 2);
  e = base(); e.B = -1;
  EXPECT(indexer_scores(&e, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 2);
  e = base(); e.T = 0x7fffffff; e.N = 0x7fffffff; /* products must not overflow int32 */
  int r = indexer_scores(&e, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL);
  if (r != 2 && r != 6) { fprintf(stderr, "huge dims -> %d\n", r); ++fails; }
  EXPECT(indexer_scores(&d, P, DSA_MXFP4, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 3);
  EXPECT(indexer_scores(&d, P, DSA_F32, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 3);
  EXPECT(indexer_scores(&d, P, DSA_BF16, NULL, P, P, NULL, DSA_MXFP4, P, NULL, P, NULL), 1);
  e = base(); e.D_I = 48;
  EXPECT(indexer_scores(&e, P, DSA_BF16, NULL, P, P, P, DSA_MXFP4, P, NULL, P, NULL), 2);
  EXPECT(indexer_scores(&d, P, DSA_BF16, NULL, P, P, P, DSA_BF16, P, NULL, P, NULL), 3);
  EXPECT(indexer_scores(&d, PO(8), DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 4);
  EXPECT(indexer_scores(&d, P, DSA_BF16, NULL, P, P, NULL, DSA_BF16, P, NULL, PO(4), NULL), 4);
  EXPECT(indexer_scores(&d, P, DSA_MXFP8, NULL, P, P, P, DSA_MXFP8, P, NULL, P, NULL), 1);
  EXPECT(indexer_scores(&d, P, DSA_MXFP8, P, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 3);
  EXPECT(indexer_scores(&d, P, DSA_MXFP8, PO(2), P, P, P, DSA_MXFP8, P, NULL, P, NULL), 4);
  EXPECT(indexer_scores(&d, P, (dsa_dtype)7, NULL, P, P, NULL, (dsa_dtype)7, P, NULL, P, NULL), 3);
  EXPECT(indexer_scores(&d, P, (dsa_dtype)-3, NULL, P, P, NULL, DSA_BF16, P, NULL, P, NULL), 3);
  EXPECT(kv_compress_mean(&d, (dsa_dtype)-1, P, 400, P, NULL), 3);
}

static void topk(void) {
  dsa_dims d = base(), e;
  EXPECT(topk_select(&d, NULL, P, NULL, P, NULL, 0, NULL), 1);
  EXPECT(topk_select(&d, PO(4), P, NULL, P, NULL, 0, NULL), 4);
  EXPECT(topk_select(&d, P, P, PO(1), P, NULL, 0, NULL), 4);
  e = base(); e.top_k = 0;
  EXPECT(topk_select(&e, P, P, NULL, P, NULL, 0, NULL), 2);
  e = base(); e.m = 0;
  EXPECT(topk_select(&e, P, P, NULL, P, NULL, 0, NULL), 2);
  e = base(); e.N = 1 << 24; /* long rows need a workspace */
  if (dsa_workspace_bytes(&e, DSA_OP_TOPK) > 0)
    EXPECT(topk_select(&e, P, P, NULL, P, NULL, 0, NULL), 5);
}

static int att(const dsa_dims* d, dsa_dtype dt, const void* q, const void* raw, int64_t base_,
               void* ws, size_t wsb, void* out, const float* sink) {
  return sparse_mla_attend(d, dt, q, P, P, raw, base_, 0, P, 0.1f, sink, out, NULL, ws, wsb,
                           NULL);
}

static void attend(void) {
  dsa_dims d = base(), e;
  EXPECT(att(&d, DSA_BF16, NULL, NULL, 0, NULL, 0, P, NULL), 1);
  e = base(); e.W = 16;
  EXPECT(att(&e, DSA_BF16, P, NULL, 0, NULL, 0, P, NULL), 1);
  EXPECT(att(&e, DSA_BF16, P, P, -1, NULL, 0, P, NULL), 2);
  e = base(); e.D_V = 600;
  EXPECT(att(&e, DSA_BF16, P, NULL, 0, NULL, 0, P, NULL), 2);
  e = base(); e.D_K = 1028;
  EXPECT(att(&e, DSA_BF16, P, NULL, 0, NULL, 0, P, NULL), 2);
  EXPECT(att(&d, DSA_MXFP4, P, NULL, 0, NULL, 0, P, NULL), 3);
  EXPECT(att(&d, DSA_BF16, P, NULL, 0, NULL, 0, PO(2), NULL), 4);
  EXPECT(att(&d, DSA_BF16, P, NULL, 0, NULL, 0, P, PO(2)), 4);
  e = dims(1, 1, 100, 64, 128, 128, 576, 512, 2048, 1, 0);
  size_t need = dsa_workspace_bytes(&e, DSA_OP_ATTEND);
  if (need == 0) ++fails;
  EXPECT(att(&e, DSA_BF16, P, NULL, 0, NULL, 0, P, NULL), 5);
  EXPECT(att(&e, DSA_BF16, P, NULL, 0, P, need - 1, P, NULL), 5);
}

static void attend_mxkv(void) {
  dsa_dims d = base(), e;
  EXPECT(sparse_mla_attend_mxkv(&d, P, P, NULL, DSA_MXFP8, P, NULL, 0, 0, P, 0.1f, NULL, P, NULL, NULL, 0, NULL), 1);
  EXPECT(sparse_mla_attend_mxkv(&d, P, NULL, P, DSA_MXFP8, P, NULL, 0, 0, P, 0.1f, NULL, P, NULL, NULL, 0, NULL), 1);
  e = dims(2, 3, 100, 64, 128, 128, 80, 64, 32, 1, 0);
  EXPECT(sparse_mla_attend_mxkv(&e, P, P, P, DSA_MXFP8, P, NULL, 0, 0, P, 0.1f, NULL, P, NULL, NULL, 0, NULL), 2);
  EXPECT(sparse_mla_attend_mxkv(&d, P, PO(8), P, DSA_MXFP8, P, NULL, 0, 0, P, 0.1f, NULL, P, NULL, NULL, 0, NULL), 4);
  e = base(); e.W = 16;
  EXPECT(sparse_mla_attend_mxkv(&e, P, P, P, DSA_MXFP8, P, NULL, 0, 0, P, 0.1f, NULL, P, NULL, NULL, 0, NULL), 1);
  EXPECT(sparse_mla_attend_mxkv(&e, P, P, P, DSA_MXFP8, P, P, -1, 0, P, 0.1f, NULL, P, NULL, NULL, 0, NULL), 2);
  /* unsplit calls expand the cache into the workspace: a call without one is refused */
  size_t need = dsa_workspace_bytes(&d, DSA_OP_ATTEND_MXKV);
  if (need < (size_t)2 * 100 * 576 * 2) ++fails;
  EXPECT(sparse_mla_attend_mxkv(&d, P, P, P, DSA_MXFP8, P, NULL, 0, 0, P, 0.1f, NULL, P, NULL, P, need - 1, NULL), 5);
}

static void forward(void) {
  dsa_dims d = base(), e;
  dsa_forward_args a = fargs();
  size_t need = dsa_workspace_bytes(&d, DSA_OP_FORWARD);
  if (need < 2 * 3 * 100 * 4 + 2 * 3 * 32 * 4) ++fails;
  EXPECT(dsa_forward(&d, NULL, P, need, NULL), 1);
  EXPECT(dsa_forward(NULL, &a, P, need, NULL), 1);
  EXPECT(dsa_forward(&d, &a, NULL, 0, NULL), 5);
  EXPECT(dsa_forward(&d, &a, P, need - 1, NULL), 5);
  a.compress = 1;
  EXPECT(dsa_forward(&d, &a, P, need, NULL), 1);
  a.kv_raw = P; a.n_raw = 399;
  e = base(); e.m = 4;
  EXPECT(dsa_forward(&e, &a, P, need, NULL), 2);
  a = fargs(); a.q_I = PO(8);
  EXPECT(dsa_forward(&d, &a, P, need, NULL), 4);
  a = fargs(); a.kv_scale = P; a.kv_dt = DSA_MXFP8; a.dt = DSA_F32;
  EXPECT(dsa_forward(&d, &a, P, need, NULL), 3);
  a = fargs(); a.kv_scale = P; a.kv_dt = DSA_BF16;   /* not an MX format */
  EXPECT(dsa_forward(&d, &a, P, need, NULL), 3);
  a = fargs(); a.events = (void* const*)P; a.n_events = -1;
  int r = dsa_forward(&d, &a, P, need, NULL);
  if (r == 0) { fprintf(stderr, "negative n_events accepted\n"); ++fails; }
  /* the no-alloc variant: same rules, plus its scratch limit */
  a = fargs();
  e = dims(1, 32768, 32768, 64, 128, 128, 576, 512, 2048, 1, 0);
  if (dsa_workspace_bytes(&e, DSA_OP_FORWARD) <= DSA_NOALLOC_SCRATCH_BYTES) ++fails;
  EXPECT(dsa_forward_noalloc(&e, &a, NULL), 8);
  e = dims(16, 1, 8192, 64, 128, 128, 576, 512, 2048, 1, 0);
  EXPECT(dsa_forward_noalloc(&e, NULL, NULL), 1);
  a.q = PO(4);
  EXPECT(dsa_forward_noalloc(&e, &a, NULL), 4);
}

static void hca(void) {
  dsa_forward_args a = fargs();
  a.q_I = NULL; a.w = NULL; a.k_I = NULL;
  dsa_dims dec = dims(2, 1, 8192, 64, 128, 128, 576, 512, 1, 128, 128);
  size_t need = dsa_workspace_bytes(&dec, DSA_OP_HCA);
  if (need == 0) ++fails;
  EXPECT(hca_forward(&dec, NULL, P, need, NULL), 1);
  EXPECT(hca_forward(&dec, &a, P, need, NULL), 1);
  a.kv_raw = P; a.n_raw = 128;
  EXPECT(hca_forward(&dec, &a, NULL, 0, NULL), 5);
  EXPECT(hca_forward(&dec, &a, P, need - 1, NULL), 5);
  dsa_dims big = dims(2, 1, 10240, 64, 128, 128, 576, 512, 1, 128, 1);
  EXPECT(hca_forward(&big, &a, P, (size_t)1 << 30, NULL), 2);
  a.compress = 1;
  EXPECT(hca_forward(&dec, &a, P, need, NULL), 2);
  a.compress = 0; a.q = PO(4);
  EXPECT(hca_forward(&dec, &a, P, need, NULL), 4);
}

static void compress(void) {
  dsa_dims d = base();
  d.m = 4;
  EXPECT(kv_compress_blocks(NULL, DSA_BF16, P, 400, P, 100, 0, 1, NULL), 1);
  EXPECT(kv_compress_blocks(&d, DSA_MXFP4, P, 400, P, 100, 0, 1, NULL), 3);
  EXPECT(kv_compress_blocks(&d, DSA_BF16, P, 400, P, 100, 5, 4, NULL), 2);
  EXPECT(kv_compress_blocks(&d, DSA_BF16, P, 400, P, 100, 0, 101, NULL), 2);
  EXPECT(kv_compress_blocks(&d, DSA_BF16, P, 399, P, 100, 99, 100, NULL), 2);
  EXPECT(kv_compress_blocks(&d, DSA_BF16, PO(8), 400, P, 100, 0, 1, NULL), 4);
  EXPECT(kv_compress_blocks(&d, DSA_BF16, P, -5, P, 100, 0, 1, NULL), 2);
  EXPECT(kv_compress_mean(&d, DSA_BF16, NULL, 400, P, NULL), 1);
  EXPECT(kv_compress_mean(&d, DSA_MXFP4, P, 400, P, NULL), 3);
  EXPECT(kv_compress_mean(&d, DSA_BF16, P, -1, P, NULL), 2);
  dsa_dims z = base(); z.m = 0;
  EXPECT(kv_compress_mean(&z, DSA_BF16, P, 400, P, NULL), 2);
}

static void workspace(void) {
  dsa_dims z = base(); z.N = 0;
  if (dsa_workspace_bytes(&z, DSA_OP_FORWARD) != 0) ++fails;
  if (dsa_workspace_bytes(NULL, DSA_OP_FORWARD) != 0) ++fails;
  dsa_dims d = base();
  if (dsa_workspace_bytes(&d, 99) != 0) ++fails;
  dsa_dims big = dims(1, 32768, 32768, 64, 128, 128, 576, 512, 2048, 1, 0);
  if (dsa_workspace_bytes(&big, DSA_OP_FORWARD) >= ((size_t)600 << 20)) ++fails;
  dsa_dims huge = dims(4, 1, 262144, 64, 128, 128, 576, 512, 1024, 4, 128);
  if (dsa_workspace_bytes(&huge, DSA_OP_FORWARD) == 0) ++fails;
}

int main(int argc, char** argv) {
  status_and_version();
  indexer();
  topk();
  attend();
  attend_mxkv();
  forward();
  hca();
  compress();
  workspace();
  if (argc > 1 && strcmp(argv[1], "--no-gpu") == 0) {
    dsa_dims d = dims(1, 1, 64, 64, 128, 128, 576, 512, 8, 1, 0);
    EXPECT(topk_select(&d, P, P, NULL, P, NULL, 0, NULL), 6);
  }
  if (fails) {
    fprintf(stderr, "abi_check: %d mismatches\n", fails);
    return 1;
  }
  printf("abi_check: ok\n");
  return 0;
}
