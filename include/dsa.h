/*
 * dsa.h - C ABI of the DeepSeek sparse-attention (DSA / CSA) hot path on MI355X (gfx950).
 *
 * The path has three steps, each a call below, plus a fused driver:
 *   1. indexer_scores    lightning-indexer score of every query against every visible key
 *   2. topk_select       per-query top-k of those scores
 *   3. sparse_mla_attend MQA-mode latent attention over the selected entries (+ raw window)
 *   0. kv_compress_mean  optional CSA step: mean-pool every m raw KV rows into one entry
 *   *  dsa_forward       0 -> 1 -> 2 -> 3 on one stream, with scores/idx kept in a workspace
 *   *  hca_forward       heavily compressed attention: 0 -> dense attention over every visible
 *                        compressed entry (+ raw window); no indexer, no selection
 *
 * Sources (web pages on the method; no code exists on them):
 *   [P5] "DeepSeek-V3.2 sparse-attention principle and TPU adaptation" (trdm.cn news 392380):
 *        s1.3 (lightning indexer; fine-grained sparse attention), s1.4 (MQA mode of MLA),
 *        s3 steps 2-4 (mqa logits -> top-k with the keep-all rule -> sparse MLA with index_mask).
 *   [P1] xhh.club "sparse" tag feed, DeepSeek-V4 CSA summary (4:1 compression, top-1024 blocks,
 *        64-head x 128-dim ReLU-weighted FP4 indexer).
 *   [P4] Tencent Cloud developer search "compressed sparse attention (CSA)": compress -> index
 *        select -> core attention; window KV concatenated with compressed KV; average pooling.
 *   [P3] wiki.gxlh.xyz "sparse attention" tag page, GLM-5.3 summary (IndexShare: one index
 *        selection reused by several layers) and DeepSeek-V4.1-Flash summary (the main latent
 *        KV cache stored in low precision).
 * The page's own index-score formula image is lost; the score used here is
 *   I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:]).
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller, contiguous row-major, 16-byte
 *     aligned. The library never allocates, frees or synchronises and keeps no state between
 *     calls except a per-device "is this gfx950" cache. Scratch memory comes from the caller
 *     (`ws`, sized by dsa_workspace_bytes).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is asynchronous.
 *   - Arguments are validated on the host before anything is launched; on any error nothing is
 *     launched and the status says why. Device faults surface at the caller's next sync.
 *   - Causality is expressed only through q_pos[B,T] (int32, raw 0-indexed position of each
 *     query token): entry s (token, or block of m tokens) is visible iff s < n_vis with
 *         n_vis = min(N, floor((q_pos + 1) / m)),
 *     i.e. a query sees itself (m == 1) and only complete blocks (m > 1).
 *   - Ragged batches: where a call takes seq_len[B] (int32, nullable), sequence b holds only
 *     seq_len[b] entries of its N-entry storage, and n_vis = min(N, floor((q_pos+1)/m),
 *     seq_len[b]) (a negative seq_len counts as 0). NULL = every sequence holds N.
 *   - Shapes use dsa_dims below. Value vectors are the first D_V columns of the key row
 *     (MQA-mode MLA: one latent row per entry shared by all H query heads, [P5] s1.4).
 *   - Thread safety: calls may run concurrently on different streams.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,      /* a required pointer is NULL                                   */
  DSA_ERR_SHAPE = 2,     /* a dimension is out of range or inconsistent                  */
  DSA_ERR_DTYPE = 3,     /* unsupported dtype or dtype combination                       */
  DSA_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                             */
  DSA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than dsa_workspace_bytes           */
  DSA_ERR_DEVICE = 6,    /* current HIP device is not gfx950, or the device query failed */
  DSA_ERR_LAUNCH = 7,    /* a kernel launch reported an error                            */
  DSA_ERR_SCRATCH = 8    /* dsa_forward_noalloc: the call needs more workspace than the
                            static scratch array holds (DSA_NOALLOC_SCRATCH_BYTES)        */
} dsa_status;

typedef enum dsa_dtype {
  DSA_F32 = 0,   /* IEEE binary32                                                         */
  DSA_BF16 = 1,  /* bfloat16 (upper half of binary32)                                     */
  DSA_MXFP4 = 2, /* OCP MX FP4: e2m1 codes, two per byte, LOW nibble = even element;
                    one E8M0 scale byte (2^(e-127)) per 32 consecutive elements.
                    Only for k_I.                                                        */
  DSA_MXFP8 = 3, /* OCP MX FP8: e4m3 (E4M3FN) codes, one per byte; one E8M0 scale byte
                    per 32 consecutive elements. For k_I and q_I (the indexer only).     */
  /* Not dtypes: these two widen the enumeration's range to every int32 value, so that any
     integer a caller passes is a defined dsa_dtype value, rejected with DSA_ERR_DTYPE. */
  DSA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  DSA_DTYPE_RANGE_MAX_ = 2147483647
} dsa_dtype;

typedef struct dsa_dims {
  int32_t B;     /* sequences                                                          */
  int32_t T;     /* query tokens per sequence                                          */
  int32_t N;     /* key entries per sequence: tokens (m == 1) or compressed blocks     */
  int32_t H_I;   /* indexer heads (64)                                                 */
  int32_t D_I;   /* indexer head dim (128)                                             */
  int32_t H;     /* attention query heads (128)                                        */
  int32_t D_K;   /* shared key dim: latent + rope (576)                                */
  int32_t D_V;   /* value dim = first D_V columns of the key row (512)                 */
  int32_t top_k; /* entries kept per query (2048 tokens / 1024 blocks)                 */
  int32_t m;     /* compression ratio: 1 = DSA over tokens, >1 = CSA over blocks       */
  int32_t W;     /* raw sliding window length for CSA (0 = none)                       */
} dsa_dims;

/* Limits checked by every call. */
#define DSA_MAX_TOPK 4096
#define DSA_MAX_DK 1024

/* Workspace query ops. */
#define DSA_OP_TOPK 1
#define DSA_OP_ATTEND 2
#define DSA_OP_FORWARD 3
#define DSA_OP_HCA 4
/* The same calls over an MX latent cache (sparse_mla_attend_mxkv, dsa_forward / hca_forward
 * with kv_scale != NULL): attention launches with many query rows (run unsplit) read a bf16
 * copy of the whole cache the call first writes into the workspace (B*N*D_K*2 bytes more). */
#define DSA_OP_ATTEND_MXKV 5
#define DSA_OP_FORWARD_MXKV 6
#define DSA_OP_HCA_MXKV 7
/* hca_forward: compressed entries plus window rows one query attends over (N + W) */
#define DSA_MAX_HCA_ENTRIES 10240

/* Human-readable name of a status code; never NULL. */
const char* dsa_status_str(int status);

/* ABI version (major * 100 + minor). */
int dsa_version(void);

/* Bytes of device workspace `op` needs for these dims (0 = none; a NULL ws is then fine).
 * Returns 0 for invalid dims as well; the call itself then reports the error. */
size_t dsa_workspace_bytes(const dsa_dims* d, int op);

/* Incremental compression for decoding ([P1] V4 CSA summary: one compressed entry per m
 * tokens; a decoder appends one as each block of m raw tokens completes). For every sequence b
 * and block j0 <= j < j1:
 *   kv_c[b, j, :] = (1/m) * sum_{i<m} kv_raw[b, m*j + i, :]
 * kv_raw: [B, raw_stride, D_K] of dtype dt (F32 or BF16); kv_c: [B, c_stride, D_K], same dtype;
 * needs j1 <= c_stride and m*j1 <= raw_stride (DSA_ERR_SHAPE otherwise). Arithmetic as
 * kv_compress_mean (fp32 sum, one RNE rounding); entries outside [j0, j1) are not touched.
 * Uses d->B, d->D_K, d->m. */
dsa_status kv_compress_blocks(const dsa_dims* d, dsa_dtype dt, const void* kv_raw,
                              int64_t raw_stride, void* kv_c, int64_t c_stride, int64_t j0,
                              int64_t j1, void* stream);

/* Step 0 - CSA token-dimension compression ([P1] V4 CSA summary; [P4] CSA snippets: m
 * consecutive tokens' KV pooled into one entry, average pooling named as one choice).
 *   kv_c[b, j, :] = (1/m) * sum_{i<m} kv_raw[b, m*j + i, :],   j < floor(n_raw / m)
 * kv_raw: [B, n_raw, D_K] of dtype dt (F32 or BF16); kv_c: [B, floor(n_raw/m), D_K], same dtype.
 * Summation in fp32, one final rounding (RNE) to dt. Uses d->B, d->D_K, d->m (>= 1). */
dsa_status kv_compress_mean(const dsa_dims* d, dsa_dtype dt, const void* kv_raw, int64_t n_raw,
                            void* kv_c, void* stream);

/* Step 1 - lightning-indexer scores ([P5] s1.3 lightning indexer; s3 step 2, the indexer's
 * multi-query logits with one key shared by all indexer heads).
 *   scores[b,t,s] = sum_{j<H_I} w[b,t,j] * max(0, sum_{d<D_I} q_I[b,t,j,d] * k_I[b,s,d])
 *                   for s < n_vis(b,t);   -inf for n_vis <= s < N.
 * q_I:    [B,T,H_I,D_I], dtype q_dt (F32 or BF16), or for q_dt == MXFP8 e4m3 codes
 *         [B,T,H_I,D_I] bytes
 * q_scale:[B,T,H_I,D_I/32] E8M0 bytes when q_dt == MXFP8, else must be NULL
 * w:      [B,T,H_I] fp32 (any sign)
 * k_I:    [B,N,D_I] of dtype k_dt (== q_dt), or for k_dt == MXFP4 codes [B,N,D_I/2] bytes,
 *         for k_dt == MXFP8 codes [B,N,D_I] bytes
 * k_scale:[B,N,D_I/32] E8M0 bytes when k_dt is MXFP4 or MXFP8, else must be NULL
 * q_pos:  [B,T] int32
 * seq_len:[B] int32 or NULL (ragged batch, see the conventions)
 * scores: [B,T,N] fp32 (written in full)
 * (q_dt, k_dt) pairs: (F32, F32), (BF16, BF16), (BF16, MXFP4), (BF16, MXFP8), (MXFP8, MXFP4),
 * (MXFP8, MXFP8); others give DSA_ERR_DTYPE. MX formats need D_I % 32 == 0.
 * Products are exact (every element is an exactly decoded stored value), accumulation fp32;
 * a bf16 q_I against MX keys enters the block-scaled MFMA as two fp8 parts (hi + lo, exact
 * except for values more than 2^13 below their 32-value block's largest, error < 2^-21 of it).
 */
dsa_status indexer_scores(const dsa_dims* d, const void* q_I, dsa_dtype q_dt,
                          const uint8_t* q_scale, const float* w, const void* k_I,
                          const uint8_t* k_scale, dsa_dtype k_dt, const int32_t* q_pos,
                          const int32_t* seq_len, float* scores, void* stream);

/* Step 2 - per-query top-k ([P5] s1.3: only the KV entries with the k highest index scores
 * take part; s3 step 3: every token is kept when the context is no longer than k; step 4's
 * index mask).
 *   n = n_vis(b,t). If n <= top_k: idx[b,t,0..n) = 0..n-1 (ascending).
 *   Else: idx[b,t,:] = the top_k entries s < n with the largest scores, ties broken toward the
 *   LOWER index (the result is the first top_k of a stable sort by descending score); the
 *   order inside the row is unspecified.
 *   Slots past the selected count are -1. -0.0 ranks equal to +0.0. Scores must not be NaN.
 * scores: [B,T,N] fp32 (entries s >= n_vis are ignored); idx: [B,T,top_k] int32; seq_len:
 * [B] int32 or NULL (ragged batch).
 * ws: dsa_workspace_bytes(d, DSA_OP_TOPK) bytes (may be 0). */
dsa_status topk_select(const dsa_dims* d, const float* scores, const int32_t* q_pos,
                       const int32_t* seq_len, int32_t* idx, void* ws, size_t ws_bytes,
                       void* stream);

/* Step 3 - sparse MQA-mode MLA attention ([P5] s1.3 "fine-grained sparse attention", s1.4,
 * s3 step 4; [P4] window KV concatenated with the compressed KV into one core attention).
 * For each (b,t,h) the entry set is
 *   E = { kv[b, idx[b,t,i], :] : idx[b,t,i] >= 0 }                       (i < top_k)
 *     u { kv_raw[b, r - raw_base, :] : max(0, p-W+1) <= r <= p,
 *                                      raw_base <= r < raw_base + n_raw } (p = q_pos[b,t])
 * one joint softmax over E (no de-duplication):
 *   z_e = softmax_scale * q[b,t,h,:D_K] . K_e[:D_K];  out[b,t,h,:] = sum_e softmax(z)_e K_e[:D_V]
 *   lse[b,t,h] = log sum_e exp(z_e).  Empty E: out = 0, lse = -inf.
 * Attention sink ([P4] CSA snippet 4.3: sliding window plus an attention sink): sink [H] fp32 or
 * NULL, one logit per head (not multiplied by softmax_scale) that joins the softmax with a zero
 * value vector: out = sum_e exp(z_e) K_e[:D_V] / (sum_e exp(z_e) + exp(sink[h])),
 * lse = log(sum_e exp(z_e) + exp(sink[h])); empty E then gives out = 0, lse = sink[h].
 * IndexShare ([P3] GLM-5.3 summary: layers reuse one index selection): a later layer passes the
 * idx a dsa_forward call returned (a->idx) with its own q / kv.
 * q: [B,T,H,D_K], kv: [B,N,D_K], kv_raw: [B,n_raw,D_K] (NULL iff W == 0), out: [B,T,H,D_V],
 * all of dtype dt (F32 or BF16); lse: [B,T,H] fp32 or NULL. idx values must be < N.
 * bf16: MFMA products, fp32 accumulation, online softmax, out rounded RNE.
 * ws: dsa_workspace_bytes(d, DSA_OP_ATTEND) bytes (split partials for few-query calls). */
dsa_status sparse_mla_attend(const dsa_dims* d, dsa_dtype dt, const void* q, const void* kv,
                             const int32_t* idx, const void* kv_raw, int64_t raw_base,
                             int64_t n_raw, const int32_t* q_pos, float softmax_scale,
                             const float* sink, void* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* Step 3 over a low-precision latent KV cache ([P3] V4.1-Flash summary: the main KV is kept
 * in FP4): the same attention as sparse_mla_attend with kv stored in an OCP MX format, kv_dt:
 * DSA_MXFP8 (e4m3 codes kv_codes [B,N,D_K] uint8) or DSA_MXFP4 (e2m1 codes, two per byte, low
 * nibble = even element: kv_codes [B,N,D_K/2]), with one E8M0 scale byte 2^(e-127) per 32
 * consecutive elements along D_K in kv_scale [B,N,D_K/32]. Entry e's row is K_e[d] =
 * code_value(d) * 2^(scale[d/32] - 127), exact in bf16; q, kv_raw (window rows) and out are
 * bf16, lse fp32. Needs D_K % 32 == 0 and the code bytes of one sequence below 2^32 (else
 * DSA_ERR_SHAPE), kv_dt MXFP8 or MXFP4 (else DSA_ERR_DTYPE); other rules and the sink as for
 * sparse_mla_attend with dt = BF16; ws: dsa_workspace_bytes(d, DSA_OP_ATTEND_MXKV) bytes. MFMA
 * shapes (D_K = 576, D_V = 512, H % 64 == 0): calls with few query rows (split attention,
 * decode) convert the rows they gather to bf16 inside the kernel; calls with many rows first
 * expand the whole cache to bf16 in ws, then attend at bf16 speed. Other shapes take the
 * scalar kernel. */
dsa_status sparse_mla_attend_mxkv(const dsa_dims* d, const void* q, const uint8_t* kv_codes,
                                  const uint8_t* kv_scale, dsa_dtype kv_dt, const int32_t* idx,
                                  const void* kv_raw,
                                  int64_t raw_base, int64_t n_raw, const int32_t* q_pos,
                                  float softmax_scale, const float* sink, void* out, float* lse,
                                  void* ws, size_t ws_bytes, void* stream);

/* Arguments of dsa_forward (pointers as in the calls above). */
typedef struct dsa_forward_args {
  dsa_dtype dt;          /* dtype of q_I, q, kv, kv_raw, out: F32 or BF16                 */
  dsa_dtype k_dt;        /* dtype of k_I: == dt, or MXFP4 / MXFP8 (with dt == BF16)       */
  const void* q_I;       /* [B,T,H_I,D_I]                                                 */
  const float* w;        /* [B,T,H_I]                                                     */
  const void* k_I;       /* [B,N,D_I] or MXFP4 codes [B,N,D_I/2]                          */
  const uint8_t* k_scale;/* [B,N,D_I/32] for MXFP4, else NULL                             */
  const void* q;         /* [B,T,H,D_K]                                                   */
  void* kv;              /* [B,N,D_K]; written first when compress != 0                   */
  const void* kv_raw;    /* [B,n_raw,D_K] raw rows at positions raw_base..; NULL if unused */
  int64_t raw_base;
  int64_t n_raw;
  int32_t compress;      /* != 0: kv = kv_compress_mean(kv_raw) (needs raw_base == 0 and
                            floor(n_raw / m) == N)                                       */
  const int32_t* q_pos;  /* [B,T]                                                         */
  float softmax_scale;
  void* out;             /* [B,T,H,D_V]                                                   */
  float* lse;            /* [B,T,H] or NULL                                               */
  float* scores;         /* [B,T,N] or NULL (then scores live in ws, masked tail unwritten)*/
  int32_t* idx;          /* [B,T,top_k] or NULL (then idx lives in ws)                    */
  void* const* events;   /* profiling aid, or NULL: timing-enabled hipEvent_t handles;
                            events[2i] and events[2i+1] receive the start and the end of the
                            i-th kernel this call launches (hipExtLaunchKernel stamps them with
                            that dispatch's own times, so nothing is inserted between the
                            kernels), as far as n_events reaches. The kernel order is:
                            [compress], then per query chunk indexer (one launch per sequence
                            segment of the chunk in prefill), [top-k,] attention[, split
                            combine]; the top-k is a kernel of its own unless the attention
                            selects the entries itself (MFMA shapes, N <= 32768, at most 128
                            query rows per chunk: the decode case); for rows longer than 32768
                            entries it is one kernel when the decode indexer with MX keys
                            already wrote the candidate segments, else two. */
  int32_t n_events;
  const uint8_t* q_scale;/* NULL, or the E8M0 scales [B,T,H_I,D_I/32] of an MXFP8 q_I (then q_I
                            holds e4m3 codes [B,T,H_I,D_I]); indexer only                 */
  const int32_t* seq_len;/* [B] or NULL: entries held per sequence (ragged batch)           */
  const float* sink;     /* [H] or NULL: attention-sink logit per head (sparse_mla_attend)  */
  const uint8_t* kv_scale;/* NULL, or the E8M0 scales [B,N,D_K/32] of an MX kv (then kv holds
                            its codes; dt == BF16, compress == 0), as in
                            sparse_mla_attend_mxkv                                        */
  dsa_dtype kv_dt;       /* with kv_scale: DSA_MXFP8 or DSA_MXFP4 (the codes' format)     */
} dsa_forward_args;

/* Fused path: [compress] -> indexer_scores -> topk_select -> sparse_mla_attend on `stream`
 * ([P5] key takeaways: light pre-scoring -> top-k sparse selection -> sparse MLA). For bf16
 * MFMA shapes with N <= 32768 and at most 128 query rows per chunk (decode) the attention
 * kernel performs the top-k selection itself (same selection as topk_select: ties to the
 * lowest indices, idx in ascending order); longer chunks run the top-k kernel, since every
 * workgroup of a row would repeat the selection.
 * When a->scores is NULL, queries are processed in chunks whose scores fit the workspace.
 * ws: dsa_workspace_bytes(d, DSA_OP_FORWARD) bytes. Graph-capturable (no sync, no alloc). */
dsa_status dsa_forward(const dsa_dims* d, const dsa_forward_args* a, void* ws, size_t ws_bytes,
                       void* stream);

/* Heavily compressed attention, HCA ([P4] Tencent Cloud CSA/HCA snippets: the second,
 * heavier compression of DeepSeek-V4 -- ratio m' = 128 against CSA's m = 4 -- runs dense
 * attention on the compressed sequence, with no sparse selection; the CSA snippets concatenate
 * the sliding-window KV with the compressed KV, and the same window is offered here, W >= 0).
 * For each (b,t,h), with p = q_pos[b,t] and n = n_vis = min(N, floor((p+1)/m)):
 *   E = { kv[b, j, :] : 0 <= j < n } u { the raw window rows of sparse_mla_attend },
 * one joint softmax over E as in sparse_mla_attend. a->compress != 0 first writes
 * kv = kv_compress_mean(kv_raw) (needs raw_base == 0, floor(n_raw / m) == N).
 * Uses from `a`: dt (F32 or BF16), q, kv, kv_raw, raw_base, n_raw, compress, q_pos, seq_len
 * (ragged batch), sink, softmax_scale, out, lse, events / n_events (kernel order: [compress,] attention[, split
 * combine]); the indexer fields (q_I, w, k_I, k_scale, k_dt, scores, idx) are ignored, and so
 * are d->top_k, d->H_I and d->D_I. Needs N + W <= DSA_MAX_HCA_ENTRIES (DSA_ERR_SHAPE otherwise).
 * ws: dsa_workspace_bytes(d, DSA_OP_HCA) bytes (split partials for few-query calls; may be 0).
 * Graph-capturable (no sync, no alloc). */
dsa_status hca_forward(const dsa_dims* d, const dsa_forward_args* a, void* ws, size_t ws_bytes,
                       void* stream);

/* Bytes of the static per-GPU scratch array behind dsa_forward_noalloc. */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* dsa_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The same launches and results as
 * dsa_forward, with the workspace taken from a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES bytes (one per GPU the library runs on, held until the process
 * ends) instead of a caller's buffer. The caller still passes inputs and outputs in `a`.
 * No hipMalloc / hipFree and no allocating library call, on any path. The array's address on
 * the current device is looked up once per device, on the first call there.
 *   - Returns DSA_ERR_SCRATCH, launching nothing, when dsa_workspace_bytes(d, DSA_OP_FORWARD)
 *     exceeds DSA_NOALLOC_SCRATCH_BYTES (the decode-sized workloads fit; a 32768-query
 *     prefill, whose scores alone take 256 MB, does not).
 *   - Every call on one GPU shares that GPU's array and finds the previous call's contents in
 *     it (nothing in it needs to start at zero). Calls that overlap in time on one GPU (two
 *     streams, two host threads) race on the array: serialise them.
 * Other errors as dsa_forward. */
dsa_status dsa_forward_noalloc(const dsa_dims* d, const dsa_forward_args* a, void* stream);

/* DSA_NOALLOC_SCRATCH_BYTES, for bindings that cannot read the macro. */
size_t dsa_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
