// api.cpp - the C ABI (include/dsa.h): argument validation, workspace sizing and dispatch.
//
// Every argument is checked on the host before anything touches HIP, so error paths launch
// nothing (and run without a GPU). Then the current device is checked to be gfx950 (cached per
// device), then kernels are launched on the caller's stream. No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "dsa.h"
#include "launch.h"

using namespace dsa;

thread_local KernelTimer* dsa::g_kernel_timer = nullptr;

namespace {

constexpr int kMaxW = 4096;
constexpr size_t kScoreChunkBytes = size_t(256) << 20;  // fused path: scores per chunk
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }  // NULL passes

dsa_status check_dims(const dsa_dims* d) {
  if (!d) return DSA_ERR_NULL;
  if (d->B < 1 || d->T < 1 || d->N < 1 || d->H_I < 1 || d->D_I < 1 || d->H < 1 || d->D_K < 8 ||
      d->D_V < 1 || d->top_k < 1 || d->m < 1 || d->W < 0)
    return DSA_ERR_SHAPE;
  if (d->top_k > DSA_MAX_TOPK || d->D_K > DSA_MAX_DK || d->W > kMaxW) return DSA_ERR_SHAPE;
  if (d->D_K % 8 || d->D_V % 8 || d->D_I % 8 || d->D_V > d->D_K) return DSA_ERR_SHAPE;
  // flattened element counts must fit the kernels' 64-bit indexing and 32-bit row counts
  const int64_t rows = (int64_t)d->B * d->T;
  if (rows > INT32_MAX || (int64_t)d->B * d->N > ((int64_t)1 << 40)) return DSA_ERR_SHAPE;
  return DSA_OK;
}

Shape to_shape(const dsa_dims* d) {
  return Shape{d->B, d->T, d->N, d->H_I, d->D_I, d->H, d->D_K, d->D_V, d->top_k, d->m, d->W};
}

bool fmt_ok(dsa_dtype t) { return t == DSA_F32 || t == DSA_BF16; }

// indexer argument rules shared by indexer_scores and dsa_forward
dsa_status check_indexer(const dsa_dims* d, dsa_dtype q_dt, const uint8_t* q_scale,
                         dsa_dtype k_dt, const uint8_t* k_scale) {
  const bool qmx = q_dt == DSA_MXFP8, kmx = k_dt == DSA_MXFP4 || k_dt == DSA_MXFP8;
  if (!fmt_ok(q_dt) && !qmx) return DSA_ERR_DTYPE;
  if (qmx != (q_scale != nullptr)) return qmx ? DSA_ERR_NULL : DSA_ERR_DTYPE;
  if (kmx != (k_scale != nullptr)) return kmx ? DSA_ERR_NULL : DSA_ERR_DTYPE;
  if (kmx) {
    if (q_dt != DSA_BF16 && !qmx) return DSA_ERR_DTYPE;  // MX keys pair with bf16 or MXFP8 q_I
  } else if (k_dt != q_dt) {
    return DSA_ERR_DTYPE;  // includes MXFP8 q_I against plain keys
  }
  if ((qmx || kmx) && d->D_I % 32) return DSA_ERR_SHAPE;
  const bool fast = (q_dt == DSA_BF16 || qmx) && d->H_I == 64 && d->D_I == 128;
  if (!fast && (int64_t)d->H_I * d->D_I > 8192) return DSA_ERR_SHAPE;  // generic kernel LDS
  return DSA_OK;
}

dsa_status check_attend_shape(const dsa_dims* d) {
  // generic kernel keeps q, the logits and the row pointers of one query in LDS
  const size_t e = (size_t)d->top_k + d->W;
  const size_t shm = sizeof(float) * (d->D_K + e + 1) + sizeof(void*) * e + 16;
  if (shm > 60 * 1024) return DSA_ERR_SHAPE;
  return DSA_OK;
}

std::atomic<int> g_dev_ok[64];  // 0 unknown, 1 gfx950, 2 other

// Workspace of dsa_forward_noalloc: one array per GPU, held until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device (looked up once per device).
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[64];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (nullptr when the lookup fails).
void* scratch_ptr(int dev) {
  if (void* p = g_scratch_ptr[dev].load(std::memory_order_acquire)) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (void* p = g_scratch_ptr[dev].load(std::memory_order_relaxed)) return p;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

dsa_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return DSA_ERR_DEVICE;
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSA_ERR_DEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? DSA_OK : DSA_ERR_DEVICE;
}

inline dsa_status launched(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

// Installs the caller's profiling events for the kernels of one dsa_forward call (launch()
// stamps pair i with the i-th kernel's start and end).
struct TimerScope {
  KernelTimer t;
  TimerScope(void* const* ev, int n) : t{ev, n, 0} {
    if (ev != nullptr && n > 0) g_kernel_timer = &t;
  }
  ~TimerScope() { g_kernel_timer = nullptr; }
};

int64_t forward_chunk_rows(const dsa_dims* d) {
  const int64_t rows = (int64_t)d->B * d->T;
  const int64_t per = std::max<int64_t>(1, (int64_t)(kScoreChunkBytes / ((size_t)d->N * 4)));
  return std::min(rows, per);
}

struct FwdLayout {
  size_t scores, idx, attend, total;
};

FwdLayout forward_layout(const dsa_dims* d, dsa_dtype dt) {
  const int64_t R = forward_chunk_rows(d);
  const Shape s = to_shape(d);
  FwdLayout L;
  L.scores = align_up((size_t)R * d->N * sizeof(float));
  L.idx = align_up((size_t)R * d->top_k * sizeof(int32_t));
  // chunks have R rows except possibly the last one; the split plan depends on the row count
  const int fmt = dt == DSA_BF16 ? FMT_BF16 : FMT_F32;
  const int64_t rows = (int64_t)d->B * d->T;
  const int64_t last = rows - (rows - 1) / R * R;
  L.attend = align_up(std::max(attend_ws_bytes(s, R, fmt), attend_ws_bytes(s, last, fmt)));
  L.total = L.scores + L.idx + L.attend + align_up(topk_ws_bytes(s, R));
  return L;
}

// HCA: the dims rules of the other calls except top_k (unused: every visible entry takes part),
// and a bound on the entries one query attends over.
dsa_status check_hca_dims(const dsa_dims* d) {
  if (!d) return DSA_ERR_NULL;
  dsa_dims c = *d;
  c.top_k = 1;
  if (dsa_status st = check_dims(&c)) return st;
  if ((int64_t)d->N + d->W > DSA_MAX_HCA_ENTRIES) return DSA_ERR_SHAPE;
  return DSA_OK;
}

// The attention kernels see HCA as "top_k = N entries with no index list" (idx == nullptr):
// entry j < N is compressed entry j itself, masked from n_vis on.
Shape hca_shape(const dsa_dims* d) {
  Shape s = to_shape(d);
  s.top_k = d->N;
  return s;
}

// An MX latent cache: whole scale blocks per row, and a sequence's code bytes addressable with
// 32-bit offsets (the MXFP4 codes take half the bytes of MXFP8 ones).
bool mxkv_shape_ok(const dsa_dims* d) {
  return d->D_K % 32 == 0 && (uint64_t)d->N * (uint64_t)d->D_K < (1ull << 32);
}
bool mxkv_dt_ok(dsa_dtype dt) { return dt == DSA_MXFP8 || dt == DSA_MXFP4; }
// the kernels' format code of an MX cache
int mxkv_fmt(dsa_dtype dt) { return dt == DSA_MXFP4 ? FMT_MXFP4 : FMT_MXFP8; }

// An MX cache read by attention launches that each hold many query rows (rows query rows per
// launch, the attention unsplit) is first expanded to bf16 in the workspace, once per call: the
// bf16 kernel then gathers it at full speed, and the expansion costs one pass over the cache.
// Few-row launches (decode) convert only the rows they gather, inside the attention kernel.
// Returns the bytes of that bf16 copy (0 = none).
size_t mxkv_expand_bytes(const Shape& s, const dsa_dims* d, int64_t rows_per_launch) {
  if (!(s.D_K == 576 && s.D_V == 512 && s.H % 64 == 0)) return 0;  // scalar kernel: decodes itself
  if (attend_splits(s, rows_per_launch, FMT_BF16) > 1) return 0;
  return align_up((size_t)d->B * d->N * d->D_K * 2);
}

// Argument rules of dsa_forward (everything but the workspace).
dsa_status check_forward(const dsa_dims* d, const dsa_forward_args* a) {
  if (dsa_status st = check_dims(d)) return st;
  if (!a) return DSA_ERR_NULL;
  if (dsa_status st = check_attend_shape(d)) return st;
  if (!fmt_ok(a->dt)) return DSA_ERR_DTYPE;
  const dsa_dtype qi_dt = a->q_scale != nullptr ? DSA_MXFP8 : a->dt;
  if (a->q_scale && a->dt != DSA_BF16) return DSA_ERR_DTYPE;
  if (dsa_status st = check_indexer(d, qi_dt, a->q_scale, a->k_dt, a->k_scale)) return st;
  if (a->q_scale && ((uintptr_t)a->q_scale & 3u)) return DSA_ERR_ALIGN;
  if (!a->q_I || !a->w || !a->k_I || !a->q || !a->kv || !a->q_pos || !a->out) return DSA_ERR_NULL;
  if ((d->W > 0 || a->compress) && !a->kv_raw) return DSA_ERR_NULL;
  if (a->raw_base < 0 || a->n_raw < 0) return DSA_ERR_SHAPE;
  if (a->compress && (a->raw_base != 0 || a->n_raw / d->m != d->N)) return DSA_ERR_SHAPE;
  // MXFP8 entries: bf16 q / kv_raw / out, stored (not compressed) entries, D_K % 32 == 0
  if (a->kv_scale && (a->dt != DSA_BF16 || a->compress || !mxkv_dt_ok(a->kv_dt)))
    return DSA_ERR_DTYPE;
  if (a->kv_scale && !mxkv_shape_ok(d)) return DSA_ERR_SHAPE;
  const void* ptrs16[] = {a->q_I, a->w, a->k_I, a->q, a->kv, a->out, a->kv_raw, a->scores,
                          a->idx};
  for (const void* p : ptrs16)
    if (p && !aligned16(p)) return DSA_ERR_ALIGN;
  if (!aligned4(a->seq_len) || !aligned4(a->sink)) return DSA_ERR_ALIGN;
  if (a->n_events < 0) return DSA_ERR_SHAPE;
  return DSA_OK;
}

// Workspace bytes of a validated dsa_forward call: the layout, plus the bf16 copy of an MXFP8
// cache when its attention launches are unsplit.
size_t forward_ws_need(const dsa_dims* d, const dsa_forward_args* a) {
  const FwdLayout L = forward_layout(d, a->dt);
  return L.total + (a->kv_scale ? mxkv_expand_bytes(to_shape(d), d, forward_chunk_rows(d)) : 0);
}

// The launches of dsa_forward on a validated call, with workspace ws (forward_ws_need bytes).
dsa_status run_forward(const dsa_dims* d, const dsa_forward_args* a, void* ws, hipStream_t st) {
  const FwdLayout L = forward_layout(d, a->dt);
  const dsa_dtype qi_dt = a->q_scale != nullptr ? DSA_MXFP8 : a->dt;
  const Shape s = to_shape(d);
  const int fmt = a->dt == DSA_BF16 ? FMT_BF16 : FMT_F32;
  TimerScope timer(a->events, a->n_events);
  if (a->compress) {
    if (hipError_t e = launch_compress(d->B, a->n_raw, d->D_K, d->m, fmt, a->kv_raw, a->kv, st))
      return launched(e);
  }
  char* wsb = static_cast<char*>(ws);
  float* ws_scores = reinterpret_cast<float*>(wsb);
  int32_t* ws_idx = reinterpret_cast<int32_t*>(wsb + L.scores);
  void* ws_att = wsb + L.scores + L.idx;
  void* ws_topk = wsb + L.scores + L.idx + L.attend;
  const int64_t rows = (int64_t)d->B * d->T;
  const int64_t R = forward_chunk_rows(d);  // the attention workspace is sized for R rows
  const bool keep_scores = a->scores != nullptr;
  // an MXFP8 cache read by unsplit attention launches: expanded to bf16 once, after the layout
  const void* kv_att = a->kv;
  const uint8_t* kv_sc = a->kv_scale;
  if (kv_sc != nullptr && mxkv_expand_bytes(s, d, R) > 0) {
    void* kv16 = wsb + L.total;
    if (hipError_t e = launch_mx_to_bf16(mxkv_fmt(a->kv_dt), static_cast<const uint8_t*>(a->kv),
                                         kv_sc, (int64_t)d->B * d->N, d->D_K, kv16, st))
      return launched(e);
    kv_att = kv16;
    kv_sc = nullptr;
  }
  const int kv_fmt = mxkv_fmt(a->kv_dt);
  for (int64_t q0 = 0; q0 < rows; q0 += R) {
    const int64_t nr = std::min(R, rows - q0);
    float* sc = keep_scores ? a->scores + (size_t)q0 * d->N : ws_scores;
    int32_t* ix = a->idx ? a->idx + (size_t)q0 * d->top_k : ws_idx;
    const bool fused = attend_fused_ok(s, fmt, nr);
    // long rows with MX keys: the indexer's epilogue also writes the top-k's candidate segments
    const int seg_stride = fused ? 0 : indexer_segment_stride(s, nr, (int)qi_dt, (int)a->k_dt);
    if (seg_stride > 0) {
      if (hipError_t e = launch_indexer_segments(s, q0, nr, a->q_I, (int)qi_dt, a->q_scale, a->w,
                                                 a->k_I, a->k_scale, (int)a->k_dt, a->q_pos,
                                                 a->seq_len, sc, keep_scores,
                                                 static_cast<uint8_t*>(ws_topk), st))
        return launched(e);
      if (hipError_t e = launch_topk_segments(s, q0, nr, sc, a->q_pos, a->seq_len, seg_stride, ix,
                                              ws_topk, st))
        return launched(e);
    } else if (hipError_t e = launch_indexer(s, q0, nr, a->q_I, (int)qi_dt, a->q_scale, a->w,
                                             a->k_I, a->k_scale, (int)a->k_dt, a->q_pos,
                                             a->seq_len, sc, keep_scores, st)) {
      return launched(e);
    }
    if (fused) {
      // top-k inside the attention kernel: idx is written only when the caller wants it
      if (hipError_t e = launch_attend_fused(s, q0, nr, a->q, kv_att, kv_sc, kv_fmt, sc,
                                             a->idx ? a->idx + (size_t)q0 * d->top_k : nullptr,
                                             d->W > 0 ? a->kv_raw : nullptr, a->raw_base,
                                             a->n_raw, a->q_pos, a->seq_len, a->sink,
                                             a->softmax_scale, a->out, a->lse, ws_att, st))
        return launched(e);
    } else {
      if (seg_stride == 0)
        if (hipError_t e = launch_topk(s, q0, nr, sc, a->q_pos, a->seq_len, ix, ws_topk, st))
          return launched(e);
      if (hipError_t e = launch_attend(s, q0, nr, fmt, a->q, kv_att, kv_sc, kv_fmt, ix,
                                       d->W > 0 ? a->kv_raw : nullptr, a->raw_base, a->n_raw,
                                       a->q_pos, nullptr, a->sink, a->softmax_scale, a->out,
                                       a->lse, ws_att, st))
        return launched(e);
    }
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_str(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a dimension is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: unsupported dtype or dtype combination";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_DEVICE: return "DSA_ERR_DEVICE: current HIP device is not gfx950";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH: a kernel launch failed";
    case DSA_ERR_SCRATCH:
      return "DSA_ERR_SCRATCH: the call needs more workspace than the static scratch array holds";
    default: return "unknown dsa_status";
  }
}

int dsa_version(void) { return 220; }

size_t dsa_workspace_bytes(const dsa_dims* d, int op) {
  if (op == DSA_OP_HCA || op == DSA_OP_HCA_MXKV) {
    if (check_hca_dims(d) != DSA_OK) return 0;
    const Shape s = hca_shape(d);
    const int64_t rows = (int64_t)d->B * d->T;
    if (op == DSA_OP_HCA_MXKV)
      return align_up(attend_ws_bytes(s, rows, FMT_BF16)) + mxkv_expand_bytes(s, d, rows);
    return std::max(attend_ws_bytes(s, rows, FMT_BF16), attend_ws_bytes(s, rows, FMT_F32));
  }
  if (check_dims(d) != DSA_OK) return 0;
  const Shape s = to_shape(d);
  const int64_t rows = (int64_t)d->B * d->T;
  switch (op) {
    case DSA_OP_TOPK: return topk_ws_bytes(s, rows);
    case DSA_OP_ATTEND:
      // the bf16 plan needs at least as much as the fp32 one
      return std::max(attend_ws_bytes(s, rows, FMT_BF16), attend_ws_bytes(s, rows, FMT_F32));
    case DSA_OP_FORWARD: return forward_layout(d, DSA_BF16).total;
    case DSA_OP_ATTEND_MXKV:
      return align_up(attend_ws_bytes(s, rows, FMT_BF16)) + mxkv_expand_bytes(s, d, rows);
    case DSA_OP_FORWARD_MXKV:
      return forward_layout(d, DSA_BF16).total + mxkv_expand_bytes(s, d, forward_chunk_rows(d));
    default: return 0;
  }
}

dsa_status kv_compress_mean(const dsa_dims* d, dsa_dtype dt, const void* kv_raw, int64_t n_raw,
                            void* kv_c, void* stream) {
  if (!d) return DSA_ERR_NULL;
  if (d->B < 1 || d->D_K < 8 || d->D_K % 8 || d->D_K > DSA_MAX_DK || d->m < 1 || n_raw < 0)
    return DSA_ERR_SHAPE;
  if (!fmt_ok(dt)) return DSA_ERR_DTYPE;
  if (!kv_raw || !kv_c) return DSA_ERR_NULL;
  if (!aligned16(kv_raw) || !aligned16(kv_c)) return DSA_ERR_ALIGN;
  if (dsa_status st = check_device()) return st;
  return launched(launch_compress(d->B, n_raw, d->D_K, d->m, dt == DSA_BF16 ? FMT_BF16 : FMT_F32,
                                  kv_raw, kv_c, (hipStream_t)stream));
}

dsa_status kv_compress_blocks(const dsa_dims* d, dsa_dtype dt, const void* kv_raw,
                              int64_t raw_stride, void* kv_c, int64_t c_stride, int64_t j0,
                              int64_t j1, void* stream) {
  if (!d) return DSA_ERR_NULL;
  if (d->B < 1 || d->D_K < 8 || d->D_K % 8 || d->D_K > DSA_MAX_DK || d->m < 1 || j0 < 0 ||
      j1 < j0 || raw_stride < 0 || c_stride < 0 || j1 > c_stride || j1 * d->m > raw_stride)
    return DSA_ERR_SHAPE;
  if (!fmt_ok(dt)) return DSA_ERR_DTYPE;
  if (!kv_raw || !kv_c) return DSA_ERR_NULL;
  if (!aligned16(kv_raw) || !aligned16(kv_c)) return DSA_ERR_ALIGN;
  if (dsa_status st = check_device()) return st;
  return launched(launch_compress_blocks(d->B, d->D_K, d->m, dt == DSA_BF16 ? FMT_BF16 : FMT_F32,
                                         kv_raw, raw_stride, kv_c, c_stride, j0, j1,
                                         (hipStream_t)stream));
}

dsa_status indexer_scores(const dsa_dims* d, const void* q_I, dsa_dtype q_dt,
                          const uint8_t* q_scale, const float* w, const void* k_I,
                          const uint8_t* k_scale, dsa_dtype k_dt, const int32_t* q_pos,
                          const int32_t* seq_len, float* scores, void* stream) {
  if (dsa_status st = check_dims(d)) return st;
  if (dsa_status st = check_indexer(d, q_dt, q_scale, k_dt, k_scale)) return st;
  if (!q_I || !w || !k_I || !q_pos || !scores) return DSA_ERR_NULL;
  if (!aligned16(q_I) || !aligned16(w) || !aligned16(k_I) || !aligned16(scores) ||
      (k_scale && ((uintptr_t)k_scale & 3u)) || (q_scale && ((uintptr_t)q_scale & 3u)) ||
      !aligned4(seq_len))
    return DSA_ERR_ALIGN;
  if (dsa_status st = check_device()) return st;
  const Shape s = to_shape(d);
  return launched(launch_indexer(s, 0, (int64_t)d->B * d->T, q_I, (int)q_dt, q_scale, w, k_I,
                                 k_scale, (int)k_dt, q_pos, seq_len, scores, true,
                                 (hipStream_t)stream));
}

dsa_status topk_select(const dsa_dims* d, const float* scores, const int32_t* q_pos,
                       const int32_t* seq_len, int32_t* idx, void* ws, size_t ws_bytes,
                       void* stream) {
  if (dsa_status st = check_dims(d)) return st;
  if (!scores || !q_pos || !idx) return DSA_ERR_NULL;
  if (!aligned16(scores) || !aligned16(idx) || !aligned4(seq_len)) return DSA_ERR_ALIGN;
  const size_t need = dsa_workspace_bytes(d, DSA_OP_TOPK);
  if (need && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (dsa_status st = check_device()) return st;
  return launched(launch_topk(to_shape(d), 0, (int64_t)d->B * d->T, scores, q_pos, seq_len, idx,
                              ws, (hipStream_t)stream));
}

dsa_status sparse_mla_attend(const dsa_dims* d, dsa_dtype dt, const void* q, const void* kv,
                             const int32_t* idx, const void* kv_raw, int64_t raw_base,
                             int64_t n_raw, const int32_t* q_pos, float softmax_scale,
                             const float* sink, void* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  if (dsa_status st = check_dims(d)) return st;
  if (dsa_status st = check_attend_shape(d)) return st;
  if (!fmt_ok(dt)) return DSA_ERR_DTYPE;
  if (!q || !kv || !idx || !q_pos || !out) return DSA_ERR_NULL;
  if (d->W > 0 && !kv_raw) return DSA_ERR_NULL;
  if (raw_base < 0 || n_raw < 0) return DSA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (kv_raw && !aligned16(kv_raw)) ||
      !aligned4(sink))
    return DSA_ERR_ALIGN;
  const Shape s = to_shape(d);
  const int fmt = dt == DSA_BF16 ? FMT_BF16 : FMT_F32;
  const size_t need = attend_ws_bytes(s, (int64_t)d->B * d->T, fmt);
  if (need && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return DSA_ERR_ALIGN;
  if (dsa_status st = check_device()) return st;
  return launched(launch_attend(s, 0, (int64_t)d->B * d->T, fmt, q, kv, nullptr, 0, idx,
                                d->W > 0 ? kv_raw : nullptr, raw_base, n_raw, q_pos, nullptr,
                                sink, softmax_scale, out, lse, ws, (hipStream_t)stream));
}

dsa_status sparse_mla_attend_mxkv(const dsa_dims* d, const void* q, const uint8_t* kv_codes,
                                  const uint8_t* kv_scale, dsa_dtype kv_dt, const int32_t* idx,
                                  const void* kv_raw, int64_t raw_base, int64_t n_raw,
                                  const int32_t* q_pos, float softmax_scale, const float* sink,
                                  void* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (dsa_status st = check_dims(d)) return st;
  if (dsa_status st = check_attend_shape(d)) return st;
  if (!mxkv_dt_ok(kv_dt)) return DSA_ERR_DTYPE;
  if (!mxkv_shape_ok(d)) return DSA_ERR_SHAPE;
  if (!q || !kv_codes || !kv_scale || !idx || !q_pos || !out) return DSA_ERR_NULL;
  if (d->W > 0 && !kv_raw) return DSA_ERR_NULL;
  if (raw_base < 0 || n_raw < 0) return DSA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(kv_codes) || !aligned16(out) ||
      (kv_raw && !aligned16(kv_raw)) || !aligned4(sink))
    return DSA_ERR_ALIGN;
  const Shape s = to_shape(d);
  const int64_t rows = (int64_t)d->B * d->T;
  const size_t part = attend_ws_bytes(s, rows, FMT_BF16);
  const size_t expand = mxkv_expand_bytes(s, d, rows);
  const size_t need = (expand ? align_up(part) : part) + expand;
  if (need && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return DSA_ERR_ALIGN;
  if (dsa_status st = check_device()) return st;
  hipStream_t st = (hipStream_t)stream;
  const void* kv_att = kv_codes;
  const uint8_t* kv_sc = kv_scale;
  if (expand) {
    void* kv16 = static_cast<char*>(ws) + align_up(part);
    if (hipError_t e = launch_mx_to_bf16(mxkv_fmt(kv_dt), kv_codes, kv_scale,
                                         (int64_t)d->B * d->N, d->D_K, kv16, st))
      return launched(e);
    kv_att = kv16;
    kv_sc = nullptr;
  }
  return launched(launch_attend(s, 0, rows, FMT_BF16, q, kv_att, kv_sc, mxkv_fmt(kv_dt), idx,
                                d->W > 0 ? kv_raw : nullptr, raw_base, n_raw, q_pos, nullptr,
                                sink, softmax_scale, out, lse, ws, st));
}

dsa_status dsa_forward(const dsa_dims* d, const dsa_forward_args* a, void* ws, size_t ws_bytes,
                       void* stream) {
  if (dsa_status st = check_forward(d, a)) return st;
  if (ws && !aligned16(ws)) return DSA_ERR_ALIGN;
  if (!ws || ws_bytes < forward_ws_need(d, a)) return DSA_ERR_WORKSPACE;
  if (dsa_status st = check_device()) return st;
  return run_forward(d, a, ws, (hipStream_t)stream);
}

size_t dsa_noalloc_scratch_bytes(void) { return DSA_NOALLOC_SCRATCH_BYTES; }

dsa_status dsa_forward_noalloc(const dsa_dims* d, const dsa_forward_args* a, void* stream) {
  if (dsa_status st = check_forward(d, a)) return st;
  if (forward_ws_need(d, a) > (size_t)DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_SCRATCH;
  if (dsa_status st = check_device()) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_DEVICE;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return DSA_ERR_DEVICE;
  return run_forward(d, a, ws, (hipStream_t)stream);
}

dsa_status hca_forward(const dsa_dims* d, const dsa_forward_args* a, void* ws, size_t ws_bytes,
                       void* stream) {
  if (dsa_status st = check_hca_dims(d)) return st;
  if (!a) return DSA_ERR_NULL;
  if (!fmt_ok(a->dt)) return DSA_ERR_DTYPE;
  if (!a->q || !a->kv || !a->q_pos || !a->out) return DSA_ERR_NULL;
  if ((d->W > 0 || a->compress) && !a->kv_raw) return DSA_ERR_NULL;
  if (a->raw_base < 0 || a->n_raw < 0) return DSA_ERR_SHAPE;
  if (a->compress && (a->raw_base != 0 || a->n_raw / d->m != d->N)) return DSA_ERR_SHAPE;
  if (a->kv_scale && (a->dt != DSA_BF16 || a->compress || !mxkv_dt_ok(a->kv_dt)))
    return DSA_ERR_DTYPE;
  if (a->kv_scale && !mxkv_shape_ok(d)) return DSA_ERR_SHAPE;
  const Shape s = hca_shape(d);
  const int fmt = a->dt == DSA_BF16 ? FMT_BF16 : FMT_F32;
  if (fmt == FMT_F32 || !(s.D_K == 576 && s.D_V == 512 && s.H % 64 == 0)) {
    // the scalar kernel keeps a query's logits and row pointers in LDS
    dsa_dims c = *d;
    c.top_k = d->N;
    if (dsa_status st = check_attend_shape(&c)) return st;
  }
  const void* ptrs16[] = {a->q, a->kv, a->out, a->kv_raw, ws};
  for (const void* p : ptrs16)
    if (p && !aligned16(p)) return DSA_ERR_ALIGN;
  if (!aligned4(a->seq_len) || !aligned4(a->sink)) return DSA_ERR_ALIGN;
  const int64_t rows = (int64_t)d->B * d->T;
  const size_t part = attend_ws_bytes(s, rows, fmt);
  const size_t expand = a->kv_scale ? mxkv_expand_bytes(s, d, rows) : 0;
  const size_t need = (expand ? align_up(part) : part) + expand;
  if (need && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  if (a->n_events < 0) return DSA_ERR_SHAPE;
  if (dsa_status st = check_device()) return st;
  hipStream_t st = (hipStream_t)stream;
  TimerScope timer(a->events, a->n_events);
  if (a->compress) {
    if (hipError_t e = launch_compress(d->B, a->n_raw, d->D_K, d->m, fmt, a->kv_raw, a->kv, st))
      return launched(e);
  }
  const void* kv_att = a->kv;
  const uint8_t* kv_sc = a->kv_scale;
  if (expand) {
    void* kv16 = static_cast<char*>(ws) + align_up(part);
    if (hipError_t e = launch_mx_to_bf16(mxkv_fmt(a->kv_dt), static_cast<const uint8_t*>(a->kv),
                                         kv_sc, (int64_t)d->B * d->N, d->D_K, kv16, st))
      return launched(e);
    kv_att = kv16;
    kv_sc = nullptr;
  }
  return launched(launch_attend(s, 0, rows, fmt, a->q, kv_att, kv_sc, mxkv_fmt(a->kv_dt), nullptr,
                                d->W > 0 ? a->kv_raw : nullptr, a->raw_base, a->n_raw, a->q_pos,
                                a->seq_len, a->sink, a->softmax_scale, a->out, a->lse, ws, st));
}

}  // extern "C"
