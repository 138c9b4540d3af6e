// compress.hip - CSA token-dimension compression on gfx950 (HBM-bound streaming kernel).
//
//   kv_c[b, j, :] = (1/m) * sum_{i<m} kv_raw[b, m*j + i, :]
//
// (xhh.club DeepSeek-V4 CSA summary: every 4 tokens' KV cache becomes one entry; Tencent Cloud
// CSA snippets: a light compression function over m consecutive tokens, e.g. average pooling.)
// Each thread owns one 16-byte column chunk of one output entry: m coalesced 16-byte loads,
// fp32 sum, one division by m, one RNE rounding, one 16-byte store. The kernels cover the blocks
// j0 .. j0 + nc - 1 of every sequence (all of them for a whole cache; the newest one when a
// decoder appends a block every m tokens); kv_raw holds raw_stride rows per sequence and kv_c
// c_stride entries.
//
// mxfp8_to_bf16 expands an MXFP8 latent cache (the V4.1-Flash summary on the "sparse attention"
// tag page: the main KV kept in low precision) to bf16 for attention calls with many query rows,
// which then read the cache at bf16 speed; it is HBM-bound the same way.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

__global__ __launch_bounds__(256) void compress_mean_bf16(const uint16_t* __restrict__ raw,
                                                          int64_t raw_stride, int D, int m,
                                                          int64_t j0, int64_t nc,
                                                          int64_t c_stride, int64_t total,
                                                          uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int cpr = D / 8;
  const int64_t c = t % cpr;
  const int64_t bj = t / cpr;  // b * nc + j
  const int64_t b = bj / nc, j = j0 + bj % nc;
  const uint16_t* src = raw + ((size_t)b * raw_stride + (size_t)j * m) * D + 8 * c;
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
  *reinterpret_cast<u32x4_t*>(out + ((size_t)b * c_stride + j) * D + 8 * c) = o;
}

__global__ __launch_bounds__(256) void compress_mean_f32(const float* __restrict__ raw,
                                                         int64_t raw_stride, int D, int m,
                                                         int64_t j0, int64_t nc, int64_t c_stride,
                                                         int64_t total, float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int cpr = D / 4;
  const int64_t c = t % cpr;
  const int64_t bj = t / cpr;
  const int64_t b = bj / nc, j = j0 + bj % nc;
  const float* src = raw + ((size_t)b * raw_stride + (size_t)j * m) * D + 4 * c;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < m; ++i) acc += *reinterpret_cast<const f32x4_t*>(src + (size_t)i * D);
  const float fm = (float)m;
  *reinterpret_cast<f32x4_t*>(out + ((size_t)b * c_stride + j) * D + 4 * c) =
      f32x4_t{acc[0] / fm, acc[1] / fm, acc[2] / fm, acc[3] / fm};
}

// An MXFP8 latent cache expanded to bf16 (exact: e4m3 x 2^(e-127) fits bf16): thread i takes
// codes 8i .. 8i+7 of the flattened [rows, D] codes and their E8M0 scale (one per 32 codes).
__global__ __launch_bounds__(256) void mxfp8_to_bf16(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int D,
                                                     int64_t units, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= units) return;
  const int64_t per_row = D / 8;
  const int64_t row = i / per_row, u = i - row * per_row;
  const u32x2_t w = *reinterpret_cast<const u32x2_t*>(codes + 8 * i);
  const uint32_t e = scales[row * (D / 32) + u / 4];
  const float sc = __uint_as_float(e != 0u ? e << 23 : 0x00400000u);  // 2^(e-127)
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, true);
  *reinterpret_cast<u32x4_t*>(out + 8 * i) =
      u32x4_t{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
              __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// The same for an MXFP4 cache (e2m1 x 2^(e-127) fits bf16): thread i takes code bytes
// 4i .. 4i+3 (codes 8i .. 8i+7, low nibble first) of the flattened [rows, D / 2] codes.
__global__ __launch_bounds__(256) void mxfp4_to_bf16(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int D,
                                                     int64_t units, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= units) return;
  const int64_t per_row = D / 8;
  const int64_t row = i / per_row, u = i - row * per_row;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + 4 * i);
  const uint32_t e = scales[row * (D / 32) + u / 4];
  const float sc = __uint_as_float(e != 0u ? e << 23 : 0x00400000u);  // 2^(e-127)
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
  *reinterpret_cast<u32x4_t*>(out + 8 * i) =
      u32x4_t{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
              __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

}  // namespace

hipError_t launch_mx_to_bf16(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int D, void* out, hipStream_t st) {
  const int64_t units = rows * (D / 8);
  if (units <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((units + 255) / 256);
  if (fmt == FMT_MXFP4)
    return launch(mxfp4_to_bf16, blocks, 256, 0, st, codes, scales, D, units,
                  static_cast<uint16_t*>(out));
  return launch(mxfp8_to_bf16, blocks, 256, 0, st, codes, scales, D, units,
                static_cast<uint16_t*>(out));
}

hipError_t launch_compress_blocks(int B, int D, int m, int fmt, const void* kv_raw,
                                  int64_t raw_stride, void* kv_c, int64_t c_stride, int64_t j0,
                                  int64_t j1, hipStream_t st) {
  const int64_t nc = j1 - j0;
  if (nc <= 0) return hipSuccess;
  const int64_t total = (int64_t)B * nc * (fmt == FMT_BF16 ? D / 8 : D / 4);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (fmt == FMT_BF16)
    return launch(compress_mean_bf16, blocks, 256, 0, st, static_cast<const uint16_t*>(kv_raw),
                  raw_stride, D, m, j0, nc, c_stride, total, static_cast<uint16_t*>(kv_c));
  return launch(compress_mean_f32, blocks, 256, 0, st, static_cast<const float*>(kv_raw),
                raw_stride, D, m, j0, nc, c_stride, total, static_cast<float*>(kv_c));
}

hipError_t launch_compress(int B, int64_t n_raw, int D, int m, int fmt, const void* kv_raw,
                           void* kv_c, hipStream_t st) {
  return launch_compress_blocks(B, D, m, fmt, kv_raw, n_raw, kv_c, n_raw / m, 0, n_raw / m, st);
}

}  // namespace dsa
