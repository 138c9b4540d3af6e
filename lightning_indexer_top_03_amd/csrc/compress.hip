// compress.hip - CSA token-dimension compression on gfx950 (HBM-bound streaming kernel).
//
//   kv_c[b, j, :] = (1/m) * sum_{i<m} kv_raw[b, m*j + i, :]
//
// (xhh.club DeepSeek-V4 CSA summary: every 4 tokens' KV cache becomes one entry; Tencent Cloud
// CSA snippets: a light compression function over m consecutive tokens, e.g. average pooling.)
// Each thread owns one 16-byte column chunk of one output entry: m coalesced 16-byte loads,
// fp32 sum, one division by m, one RNE rounding, one 16-byte store.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

__global__ __launch_bounds__(256) void compress_mean_bf16(const uint16_t* __restrict__ raw,
                                                          int64_t n_raw, int D, int m,
                                                          int64_t nc, int64_t total,
                                                          uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int cpr = D / 8;
  const int64_t c = t % cpr;
  const int64_t bj = t / cpr;  // b * nc + j
  const int64_t b = bj / nc, j = bj % nc;
  const uint16_t* src = raw + ((size_t)b * n_raw + (size_t)j * m) * D + 8 * c;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < m; ++i) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + (size_t)i * D));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += __uint_as_float(v[k] << 16);
      acc[2 * k + 1] += __uint_as_float(v[k] & 0xffff0000u);
    }
  }
  const float fm = (float)m;
  u32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[2 * k] / fm, acc[2 * k + 1] / fm);
  *reinterpret_cast<u32x4_t*>(out + (size_t)bj * D + 8 * c) = o;
}

__global__ __launch_bounds__(256) void compress_mean_f32(const float* __restrict__ raw,
                                                         int64_t n_raw, int D, int m, int64_t nc,
                                                         int64_t total, float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int cpr = D / 4;
  const int64_t c = t % cpr;
  const int64_t bj = t / cpr;
  const int64_t b = bj / nc, j = bj % nc;
  const float* src = raw + ((size_t)b * n_raw + (size_t)j * m) * D + 4 * c;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < m; ++i) acc += *reinterpret_cast<const f32x4_t*>(src + (size_t)i * D);
  const float fm = (float)m;
  *reinterpret_cast<f32x4_t*>(out + (size_t)bj * D + 4 * c) =
      f32x4_t{acc[0] / fm, acc[1] / fm, acc[2] / fm, acc[3] / fm};
}

}  // namespace

hipError_t launch_compress(int B, int64_t n_raw, int D, int m, int fmt, const void* kv_raw,
                           void* kv_c, hipStream_t st) {
  const int64_t nc = n_raw / m;
  if (nc <= 0) return hipSuccess;
  const int64_t total = (int64_t)B * nc * (fmt == FMT_BF16 ? D / 8 : D / 4);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (fmt == FMT_BF16)
    return launch(compress_mean_bf16, blocks, 256, 0, st, static_cast<const uint16_t*>(kv_raw),
                  n_raw, D, m, nc, total, static_cast<uint16_t*>(kv_c));
  return launch(compress_mean_f32, blocks, 256, 0, st, static_cast<const float*>(kv_raw), n_raw, D,
                m, nc, total, static_cast<float*>(kv_c));
}

}  // namespace dsa
