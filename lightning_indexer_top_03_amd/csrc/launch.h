// launch.h - host-side launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace dsa {

// Per-kernel timing for a caller's profiling events. While a KernelTimer is installed on the
// calling thread, every launch() takes the next two events of its list and passes them to
// hipExtLaunchKernel, which stamps them with that dispatch's own start and end times: no
// marker packet sits between the kernels, so they run as in an untimed call.
struct KernelTimer {
  void* const* ev;
  int n, next;
};
extern thread_local KernelTimer* g_kernel_timer;

// k<<<grid, block, shm, st>>>(a...), timed when a KernelTimer is installed.
template <typename... P, typename... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t shm, hipStream_t st,
                         A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  if (KernelTimer* t = g_kernel_timer) {
    const int i = t->next;
    t->next += 2;
    hipEvent_t e0 = i < t->n ? static_cast<hipEvent_t>(t->ev[i]) : nullptr;
    hipEvent_t e1 = i + 1 < t->n ? static_cast<hipEvent_t>(t->ev[i + 1]) : nullptr;
    if (e0 != nullptr || e1 != nullptr) {
      std::tuple<P...> v{static_cast<P>(a)...};
      void* args[sizeof...(P) + 1];
      std::apply([&args](auto&... x) {
        int j = 0;
        ((args[j++] = static_cast<void*>(&x)), ...);
      }, v);
      return hipExtLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, shm, st, e0,
                                e1, 0);
    }
  }
  k<<<grid, block, shm, st>>>(static_cast<P>(a)...);
  return hipGetLastError();
}

enum Fmt { FMT_F32 = 0, FMT_BF16 = 1, FMT_MXFP4 = 2, FMT_MXFP8 = 3 };

struct Shape {
  int B, T, N, H_I, D_I, H, D_K, D_V, top_k, m, W;
};

// Query-side tensors are indexed by the flattened row qi = b*T + t; a call covers the rows
// qi0 .. qi0+nrows-1, and its row-relative buffers (scores, idx) start at row qi0.

// ---- step 0 ----
hipError_t launch_compress(int B, int64_t n_raw, int D, int m, int fmt, const void* kv_raw,
                           void* kv_c, hipStream_t st);
// Incremental compression: for every sequence b, kv_c[b, j, :] = mean of kv_raw[b, m*j + i, :]
// (i < m) for the blocks j0 <= j < j1; kv_raw holds raw_stride rows per sequence, kv_c
// c_stride entries.
hipError_t launch_compress_blocks(int B, int D, int m, int fmt, const void* kv_raw,
                                  int64_t raw_stride, void* kv_c, int64_t c_stride, int64_t j0,
                                  int64_t j1, hipStream_t st);

// An MX latent cache (fmt FMT_MXFP8: e4m3 codes [rows, D]; FMT_MXFP4: e2m1 code pairs
// [rows, D/2], low nibble first; E8M0 scales [rows, D/32]) expanded to bf16 [rows, D] (exact).
hipError_t launch_mx_to_bf16(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int D, void* out, hipStream_t st);

// ---- step 1 ----
// scores: [nrows, N] row-relative. fill_masked: write -inf for s >= n_vis. seq_len (nullable):
// entries held per sequence (ragged batch), clamping n_vis.
hipError_t launch_indexer(const Shape& s, int64_t qi0, int64_t nrows, const void* q_I, int q_fmt,
                          const uint8_t* q_scale, const float* w, const void* k_I,
                          const uint8_t* k_scale, int k_fmt, const int32_t* q_pos,
                          const int32_t* seq_len, float* scores, bool fill_masked,
                          hipStream_t st);

// The decode indexer over long rows (N > 8 * 4096) with MX keys, fused with the first stage of
// the long-row top-k: besides the scores it writes the rows' candidate segments (select.h
// chunk_filter layout, one per workgroup of 4096 keys) into seg_ws (topk_ws_bytes). The
// stride is the argument launch_topk_segments needs; 0 = launch_indexer_segments does not
// apply to this call (it then returns hipErrorInvalidValue).
int indexer_segment_stride(const Shape& s, int64_t nrows, int q_fmt, int k_fmt);
hipError_t launch_indexer_segments(const Shape& s, int64_t qi0, int64_t nrows, const void* q_I,
                                   int q_fmt, const uint8_t* q_scale, const float* w,
                                   const void* k_I, const uint8_t* k_scale, int k_fmt,
                                   const int32_t* q_pos, const int32_t* seq_len, float* scores,
                                   bool fill_masked, uint8_t* seg_ws, hipStream_t st);

// ---- step 2 ----
// scores: [nrows, N] row-relative, idx: [nrows, top_k] row-relative, rows qi0 .. qi0+nrows-1.
size_t topk_ws_bytes(const Shape& s, int64_t nrows);
hipError_t launch_topk(const Shape& s, int64_t qi0, int64_t nrows, const float* scores,
                       const int32_t* q_pos, const int32_t* seq_len, int32_t* idx, void* ws,
                       hipStream_t st);
// The select of long rows (N > 32768) over candidate segments the decode indexer already wrote
// (launch_indexer with a segment workspace): chunk g's first keys start at g * stride.
hipError_t launch_topk_segments(const Shape& s, int64_t qi0, int64_t nrows, const float* scores,
                                const int32_t* q_pos, const int32_t* seq_len, int stride,
                                int32_t* idx, const void* ws, hipStream_t st);

// ---- step 3 ----
// idx: [nrows, top_k] row-relative; q/out/lse indexed by the flattened row qi.
int attend_splits(const Shape& s, int64_t nrows, int fmt);
size_t attend_ws_bytes(const Shape& s, int64_t nrows, int fmt);
// seq_len (nullable): entries per sequence (limits the dense idx == nullptr case and the fused
// selection); sink (nullable): one logit per head joining the softmax with a zero value vector.
// kv_scale (nullable): kv holds MX entries of kv_fmt (FMT_MXFP8: e4m3 code bytes [B, N, D_K];
// FMT_MXFP4: e2m1 code pairs [B, N, D_K / 2]), E8M0 scales [B, N, D_K / 32]; q, kv_raw and out
// stay in fmt.
hipError_t launch_attend(const Shape& s, int64_t qi0, int64_t nrows, int fmt, const void* q,
                         const void* kv, const uint8_t* kv_scale, int kv_fmt,
                         const int32_t* idx, const void* kv_raw, int64_t raw_base, int64_t n_raw,
                         const int32_t* q_pos, const int32_t* seq_len, const float* sink,
                         float scale, void* out, float* lse, void* ws, hipStream_t st);

// Fused top-k + attention (dsa_forward): every workgroup of a row selects the row's top-k from
// the indexer scores itself and attends over its split of it; idx_out (nullable) receives the
// selection in ascending index order. attend_fused_ok: bf16 MFMA shapes with N <= 32768 and at
// most 128 query rows per launch.
bool attend_fused_ok(const Shape& s, int fmt, int64_t nrows);
hipError_t launch_attend_fused(const Shape& s, int64_t qi0, int64_t nrows, const void* q,
                               const void* kv, const uint8_t* kv_scale, int kv_fmt,
                               const float* scores, int32_t* idx_out, const void* kv_raw,
                               int64_t raw_base,
                               int64_t n_raw, const int32_t* q_pos, const int32_t* seq_len,
                               const float* sink, float scale, void* out, float* lse, void* ws,
                               hipStream_t st);

}  // namespace dsa
