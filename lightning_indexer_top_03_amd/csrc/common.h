// common.h - device-side helpers shared by the gfx950 kernels of the DSA / CSA path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even, one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Visible entries of a query at raw position p with compression m over N entries.
__device__ __forceinline__ int n_visible(int p, int m, int N) {
  if (p < 0) return 0;
  int v = (p + 1) / m;
  return v < N ? v : N;
}

// The same in a ragged batch: sequence b holds seq_len[b] entries (seq_len may be null).
__device__ __forceinline__ int n_visible(int p, int m, int N, const int32_t* seq_len, int b) {
  const int v = n_visible(p, m, N);
  if (seq_len == nullptr) return v;
  const int L = seq_len[b];
  return v < L ? v : (L > 0 ? L : 0);
}

// Order-preserving map fp32 -> uint32 (larger float <=> larger key); -0 ranks as +0.
// Workgroup id -> work item, XCD-major: workgroups are dealt to the 8 XCDs round-robin
// (id % 8), so with T % 8 == 0 XCD x runs items x*T/8 .. (x+1)*T/8 - 1 in order and work items
// that share data stay in one XCD's L2.
__device__ __forceinline__ int xcd_item(int lin, int T) {
  const int remapped = (lin & 7) * (T >> 3) + (lin >> 3);
  return (T & 7) ? lin : remapped;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace dsa
