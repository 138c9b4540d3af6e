// indexer.hip - lightning-indexer scores on gfx950.
//
//   I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:])     for s < n_vis(t), else -inf
//
// ("DeepSeek-V3.2 sparse-attention principle and TPU adaptation", s1.3 lightning indexer:
// a low-dimensional per-token key, a ReLU instead of a softmax for throughput; s3 step 2:
// "mqa logits", the key is shared by all indexer heads.)
//
// Three kernels:
//  * indexer_decode_mfma  - few query rows, long key ranges: the query's 64x128 q_I stays in
//    registers as MFMA A operands; every wave streams its own 32-key tiles of k_I straight
//    from HBM into B operands (16-byte loads, two tiles in flight). bf16 or MXFP4 keys (FP4
//    codes dequantised by v_cvt_scalef32_pk_bf16_fp4 into exact bf16).
//  * indexer_prefill_mfma - many query rows of one sequence: each wave keeps 64 keys of k_I
//    in registers, the workgroup walks 32 queries whose q_I is staged in LDS.
//  * indexer_generic      - any H_I / D_I, fp32 or bf16 (and MXFP4) inputs; scalar fp32.
// All three fuse ReLU, the head weights and the 64-head reduction into the epilogue, so the
// [H_I x N] per-head products never leave registers.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace dsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// E8M0 byte -> fp32 scale 2^(e-127).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// ------------------------------------------------------------------------------------------
// Decode-shaped kernel. H_I = 64, D_I = 128.
//
// MFMA v_mfma_f32_32x32x16_bf16, C[32 heads x 32 keys] += A[heads x 16] * B[16 x keys].
// Lane l = (n = l % 32, h = l / 32). The contraction index of MFMA kk, slot i is dim
// 64*h + 8*kk + i for both operands, so a lane reads 128 contiguous bytes of its q_I row
// (A) and of its key row (B). Output: acc[hb][4*j + i] = head hb*32 + 8*j + 4*h + i, key n.
// ------------------------------------------------------------------------------------------
template <int KFMT>
struct KeyTile {
  u32x4_t v[8];
};

template <int KFMT>
__device__ __forceinline__ void load_key_tile(KeyTile<KFMT>& kt, const uint8_t* __restrict__ kI,
                                              const uint8_t* __restrict__ ksc, size_t row, int h,
                                              float& s_lo, float& s_hi) {
  if constexpr (KFMT == FMT_BF16) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(kI + row * 256 + 128 * h);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kt.v[kk] = __builtin_nontemporal_load(p + kk);
  } else {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(kI + row * 64 + 32 * h);
    kt.v[0] = __builtin_nontemporal_load(p);
    kt.v[1] = __builtin_nontemporal_load(p + 1);
    uint32_t sc = *reinterpret_cast<const uint16_t*>(ksc + row * 4 + 2 * h);
    s_lo = e8m0_scale(sc & 0xffu);
    s_hi = e8m0_scale(sc >> 8);
  }
}

template <int KFMT>
__device__ __forceinline__ bf16x8_t key_operand(const KeyTile<KFMT>& kt, int kk, float s_lo,
                                                float s_hi) {
  if constexpr (KFMT == FMT_BF16) {
    return as_bf16x8(kt.v[kk]);
  } else {
    // dims 64h + 8kk .. +7 are code bytes 4kk .. 4kk+3 of the lane's 32-byte chunk
    uint32_t cw = kt.v[kk >> 2][kk & 3];
    float sc = kk < 4 ? s_lo : s_hi;
    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0);
    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1);
    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2);
    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3);
    bf16x8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
  }
}

constexpr int kDecodeMaxIters = 16;  // 32-key tiles per wave

template <int KFMT, int ITERS>
__global__ __launch_bounds__(256) void indexer_decode_mfma(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const uint8_t* __restrict__ ksc, const int32_t* __restrict__ q_pos, int T, int N, int m,
    int64_t qi0, float* __restrict__ scores, int fill_masked) {
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int nv = n_visible(q_pos[qi], m, N);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  constexpr int keys_per_wave = 32 * ITERS;
  const int key0 = (blockIdx.x * 4 + wv) * keys_per_wave;
  float* __restrict__ srow = scores + (size_t)row * N;
  __shared__ float sres[4][32 * ITERS];

  if (key0 >= nv) {
    if (fill_masked)
      for (int s = key0 + lane; s < min(key0 + keys_per_wave, N); s += 64) srow[s] = kNegInf;
    return;
  }

  // q_I fragments (A operands) and the weights of the heads this lane's outputs belong to.
  const uint16_t* qrow = qI + (size_t)qi * (64 * 128);
  u32x4_t qa[2][8];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qa[hb][kk] = *reinterpret_cast<const u32x4_t*>(qrow + (hb * 32 + n) * 128 + 64 * h + 8 * kk);
  float wr[2][16];
  const float* wrow = w + (size_t)qi * 64;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(wrow + hb * 32 + 8 * j + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[hb][4 * j + i] = w4[i];
    }
  // complete the q_I / w loads before the key pipeline and make the values opaque, so that the
  // compiler neither waits for them inside the pipeline (draining the prefetched tile) nor
  // re-loads them next to each use
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) asm volatile("" : "+v"(qa[hb][kk]));
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wr[hb][r]));
  }

  const size_t base_row = (size_t)b * N;
  const int last = min(key0 + keys_per_wave, nv);  // exclusive end of computed keys
  const int ntiles = (last - key0 + 31) / 32;      // wave-uniform
  // Two register buffers, ping-pong: the next tile is always requested (rows clamped to the
  // sequence) before the current one is consumed, with no branch around the loads, so the
  // wait for the current tile leaves the next one in flight.
  KeyTile<KFMT> ta, tb;
  float lo_a = 0.f, hi_a = 0.f, lo_b = 0.f, hi_b = 0.f;
  auto tile_row = [&](int t) { return base_row + min(key0 + 32 * t + n, N - 1); };
  auto consume = [&](const KeyTile<KFMT>& kt, float slo, float shi, int t) {
    f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8_t kb = key_operand<KFMT>(kt, kk, slo, shi);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[0][kk]), kb, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[1][kk]), kb, acc1, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part += wr[0][r] * fmaxf(acc0[r], 0.f);
      part += wr[1][r] * fmaxf(acc1[r], 0.f);
    }
    part += __shfl_xor(part, 32, 64);
    // scores go to LDS (no vector-memory counter traffic inside the pipeline), flushed below
    if (h == 0) sres[wv][32 * t + n] = part;
  };
  // Straight-line, branch-free (ITERS is a compile-time count): the loads of tile t+1 are issued
  // before tile t is consumed. Rows past the wave's visible range are clamped and their results
  // never flushed; computing them keeps the code free of branches the loads could sink into.
  load_key_tile<KFMT>(ta, kI, ksc, tile_row(0), h, lo_a, hi_a);
#pragma unroll
  for (int t = 0; t < ITERS; ++t) {
    if (t % 2 == 0) {
      if (t + 1 < ITERS) load_key_tile<KFMT>(tb, kI, ksc, tile_row(t + 1), h, lo_b, hi_b);
      __builtin_amdgcn_sched_barrier(0);  // keep the next tile's loads ahead of this tile's use
      consume(ta, lo_a, hi_a, t);
    } else {
      if (t + 1 < ITERS) load_key_tile<KFMT>(ta, kI, ksc, tile_row(t + 1), h, lo_a, hi_a);
      __builtin_amdgcn_sched_barrier(0);
      consume(tb, lo_b, hi_b, t);
    }
  }
  // flush this wave's scores: computed keys (masked past n_vis), then -inf past the visible end
  const int kend = min(key0 + keys_per_wave, N);
  for (int s = key0 + lane; s < kend; s += 64) {
    const int o = s - key0;
    if (o < 32 * ntiles)
      srow[s] = s < nv ? sres[wv][o] : kNegInf;
    else if (fill_masked)
      srow[s] = kNegInf;
  }
}

// ------------------------------------------------------------------------------------------
// Decode-shaped kernel, bf16 keys, streamed through LDS. Reading rows straight into the MFMA
// operand layout (each lane 16 B of its own 256-byte row per load) makes every load instruction
// touch 64 rows and runs at a fraction of HBM speed, so all global traffic here is fully
// coalesced DMA (global_load_lds_dwordx4: lane l of instruction j moves 16 bytes at 1024*j+16*l):
//  * the query's q_I (64 rows x 256 B) is staged once per workgroup and read back as A operands;
//  * each of the 8 waves streams its own 32-key tiles (8 KB) through a 2-stage LDS ring.
// Row r of a staged block keeps its 16-byte chunk c in slot c ^ (r % 16), so the 8 lanes a
// ds_read_b128 phase serves hit distinct banks. Key-ring stages are only read by the wave that
// filled them, after an explicit s_waitcnt vmcnt; q_I is shared behind one barrier.
// ------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kDecWaves = 8;

__device__ __forceinline__ float relu_bits(float x) {
  // max(x, 0) on the IEEE bit pattern: negative values (sign bit set) are negative as int32
  return __int_as_float(max(__float_as_int(x), 0));
}

template <int ITERS>
__global__ __launch_bounds__(kDecWaves * 64, 1) void indexer_decode_dma(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ kI,
    const int32_t* __restrict__ q_pos, int T, int N, int m, int64_t qi0,
    float* __restrict__ scores, int fill_masked) {
  __shared__ __attribute__((aligned(16))) char sq[64 * 256];
  __shared__ __attribute__((aligned(16))) char sk[kDecWaves][2][32 * 256];
  __shared__ float sres[kDecWaves][32 * ITERS];
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int nv = n_visible(q_pos[qi], m, N);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  constexpr int keys_per_wave = 32 * ITERS;
  const int key0_wg = blockIdx.x * kDecWaves * keys_per_wave;
  const int key0 = key0_wg + wv * keys_per_wave;
  float* __restrict__ srow = scores + (size_t)row * N;

  if (key0_wg >= nv) {  // the whole workgroup is past the visible range
    if (fill_masked)
      for (int s = key0_wg + (int)threadIdx.x; s < min(key0_wg + kDecWaves * keys_per_wave, N);
           s += kDecWaves * 64)
        srow[s] = kNegInf;
    return;
  }
  const size_t base_row = (size_t)b * N;
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sk[wv][0][0]);
  const uint32_t qlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sq[0]);
  const int r4 = lane >> 4, c16 = lane & 15;
  auto issue = [&](int t) {  // tile t of this wave into stage t % 2
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + r4;
      const size_t krow = base_row + min(key0 + 32 * t + r, N - 1);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(kI + krow * 256 + 16 * (c16 ^ (r & 15))),
          (lds_void_t*)(uintptr_t)(ring + (t & 1) * (32 * 256) + 1024 * j), 16, 0, 0);
    }
  };
  issue(0);
  if (ITERS > 1) issue(1);
  {  // q_I: 16 KB, two 1 KB DMAs per wave (rows 8*wv .. 8*wv+7)
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(qI + (size_t)qi * (64 * 128));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 8 * wv + 4 * j + r4;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(qsrc + r * 256 + 16 * (c16 ^ (r & 15))),
          (lds_void_t*)(uintptr_t)(qlds + (8 * wv + 4 * j) * 256), 16, 0, 0);
    }
  }
  float wr[2][16];
  const float* wrow = w + (size_t)qi * 64;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(wrow + hb * 32 + 8 * j + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[hb][4 * j + i] = w4[i];
    }
  // Everything issued so far has landed once this returns (the counter drains in order).
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wr[hb][r]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();  // every wave's share of q_I is in LDS
  u32x4_t qa[2][8];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int r = hb * 32 + n;
      qa[hb][kk] = *reinterpret_cast<const u32x4_t*>(&sq[r * 256 + 16 * ((8 * h + kk) ^ (r & 15))]);
    }

  const int last = min(key0 + keys_per_wave, nv);
  const int ntiles = last > key0 ? (last - key0 + 31) / 32 : 0;
#pragma unroll
  for (int t = 0; t < ITERS; ++t) {
    if (t >= 2) {
      if (t + 1 < ITERS)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // tile t landed, tile t+1 in flight
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const char* st = &sk[wv][t & 1][0];
    u32x4_t kb[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      kb[kk] = *reinterpret_cast<const u32x4_t*>(st + n * 256 + 16 * ((8 * h + kk) ^ (n & 15)));
    __builtin_amdgcn_sched_barrier(0);  // all eight LDS reads in flight before the MFMAs
    f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[0][kk]), as_bf16x8(kb[kk]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[1][kk]), as_bf16x8(kb[kk]), acc1, 0, 0, 0);
    }
    if (t + 2 < ITERS) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this stage's reads are done
      issue(t + 2);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part += wr[0][r] * relu_bits(acc0[r]);
      part += wr[1][r] * relu_bits(acc1[r]);
    }
    part += __shfl_xor(part, 32, 64);
    if (h == 0) sres[wv][32 * t + n] = part;
  }
  const int kend = min(key0 + keys_per_wave, N);
  for (int s = key0 + lane; s < kend; s += 64) {
    const int o = s - key0;
    if (o < 32 * ntiles)
      srow[s] = s < nv ? sres[wv][o] : kNegInf;
    else if (fill_masked)
      srow[s] = kNegInf;
  }
}

// ------------------------------------------------------------------------------------------
// Prefill-shaped kernel (bf16). H_I = 64, D_I = 128. Workgroup = kPfQ queries of one sequence x
// the key blocks (256 keys) g, g + gridDim.x, ... (g: its key group) below the queries' visible
// range: a grid of every (key block, query block) pair would be mostly blocks past the causal
// edge, and dispatching those alone costs more than a tenth of the kernel. Per key block, wave
// wv holds keys kbase + 64*wv + 32*kb + n (kb = 0, 1) as B operands in registers; the queries'
// q_I (64 x 128, 16 KB) and w (64) stream through a 3-stage LDS ring by DMA, two queries ahead
// of the MFMAs (row hr keeps its 16-byte chunk c in slot c ^ (hr % 16): the A-operand reads are
// conflict-free). One barrier per query; the DMA waits are explicit, so the barrier never
// drains the queries in flight.
// ------------------------------------------------------------------------------------------
constexpr int kPfKeys = 256;
constexpr int kPfQ = 32;
constexpr int kPfKeyGroups = 16;  // workgroups per query block

__global__ __launch_bounds__(256) void indexer_prefill_mfma(
    const uint16_t* __restrict__ qI, const float* __restrict__ w, const uint16_t* __restrict__ kI,
    const int32_t* __restrict__ q_pos, int T, int N, int m, int b, int t0, int nt,
    float* __restrict__ scores, int fill_masked) {
  __shared__ __attribute__((aligned(16))) char sq[3][64 * 256];
  __shared__ __attribute__((aligned(16))) float sw[3][64];
  __shared__ int snv[kPfQ];
  __shared__ int smax;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // the gridDim.x workgroups of a query block are consecutive work items, one XCD's: they
  // stream the same q_I rows, which then stay in that XCD's L2
  const int item = xcd_item(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int kgrp = item % gridDim.x;
  const int r0 = (item / gridDim.x) * kPfQ;  // first row (relative to t0) of this tile
  const int nrows = min(kPfQ, nt - r0);
  const int64_t qi0 = (int64_t)b * T + t0 + r0;

  if (tid == 0) smax = 0;
  __syncthreads();
  if (tid < nrows) {
    int v = n_visible(q_pos[qi0 + tid], m, N);
    snv[tid] = v;
    atomicMax(&smax, v);
  }
  __syncthreads();
  const int maxnv = smax;
  const size_t base_row = (size_t)b * N;
  const uint32_t qlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sq[0][0]);
  const uint32_t wlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sw[0][0]);
  for (int kblk = kgrp; kblk * kPfKeys < N; kblk += gridDim.x) {
    const int kbase = kblk * kPfKeys;
    if (kbase >= maxnv) {
      if (fill_masked)
        for (int r = 0; r < nrows; ++r)
          for (int s = kbase + tid; s < min(kbase + kPfKeys, N); s += 256)
            scores[(size_t)(r0 + r) * N + s] = kNegInf;
      continue;
    }

    // this wave's keys as B operands: kf[0..1][kk]
    u32x4_t kf[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int s = min(kbase + 64 * wv + 32 * kb + n, N - 1);
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(kI + (base_row + s) * 128 + 64 * h);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) kf[kb][kk] = p[kk];
    }

    // DMA of query r into stage buf: wave wv moves q_I rows 16*wv .. 16*wv+15 (four 1 KB
    // instructions); wave 0 also moves w (16 lanes x 16 B). Wave 0 issues 5 instructions per
    // query, the others 4.
    auto stage = [&](int r, int buf) {
      const char* src = reinterpret_cast<const char*>(qI + (size_t)(qi0 + r) * (64 * 128));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hr = 16 * wv + 4 * j + (lane >> 4), c = lane & 15;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(src + hr * 256 + 16 * (c ^ (hr & 15))),
            (lds_void_t*)(uintptr_t)(qlds + buf * (64 * 256) + (16 * wv + 4 * j) * 256), 16, 0, 0);
      }
      if (wv == 0 && lane < 16)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(w + (size_t)(qi0 + r) * 64 + 4 * lane),
            (lds_void_t*)(uintptr_t)(wlds + buf * 256), 16, 0, 0);
    };
    stage(0, 0);
    if (nrows > 1) stage(1, 1);

    for (int r = 0; r < nrows; ++r) {
      const int buf = r % 3;
      // query r landed (query r+1's DMAs may still be in flight), then every wave's share is
      // visible after the barrier; stage (r+2)%3 was last read in iteration r-1
      if (r + 1 < nrows) {
        if (wv == 0) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      if (r + 2 < nrows) stage(r + 2, (r + 2) % 3);
      const int nv = snv[r];
      float* srow = scores + (size_t)(r0 + r) * N;
      if (kbase < nv) {
        const char* qb = &sq[buf][0];
        u32x4_t a[2][8];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const int hr = hb * 32 + n;
            a[hb][kk] = *reinterpret_cast<const u32x4_t*>(qb + hr * 256 + 16 * ((8 * h + kk) ^ (hr & 15)));
          }
        f32x16_t acc[2][2] = {};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            acc[hb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[hb][kk]), as_bf16x8(kf[0][kk]), acc[hb][0], 0, 0, 0);
            acc[hb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[hb][kk]), as_bf16x8(kf[1][kk]), acc[hb][1], 0, 0, 0);
          }
        // lane (n, h) holds rows 8*(i/4) + 4*h + i%4 of each 32-head block: w of those heads
        float part[2] = {0.f, 0.f};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(&sw[buf][hb * 32 + 8 * q4 + 4 * h]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              part[0] += w4[i] * relu_bits(acc[hb][0][4 * q4 + i]);
              part[1] += w4[i] * relu_bits(acc[hb][1][4 * q4 + i]);
            }
          }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float v = part[kb] + __shfl_xor(part[kb], 32, 64);
          int s = kbase + 64 * wv + 32 * kb + n;
          if (h == 0 && s < N && (fill_masked || s < nv)) srow[s] = (s < nv) ? v : kNegInf;
        }
      } else if (fill_masked) {
        for (int s = kbase + tid; s < min(kbase + kPfKeys, N); s += 256) srow[s] = kNegInf;
      }
    }
    // every wave is done with the ring before the next key block restages it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }
}

// ------------------------------------------------------------------------------------------
// Generic scalar kernel: any H_I * D_I <= 16384, fp32 / bf16 queries, fp32 / bf16 / MXFP4 keys.
// One thread per key; q_I and w of the query row in LDS (as fp32).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float load_val(const void* p, size_t i, int fmt) {
  return fmt == FMT_F32 ? reinterpret_cast<const float*>(p)[i]
                        : bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ float fp4_val(uint32_t code) {
  // e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0
  uint32_t e = (code >> 1) & 3u, mb = code & 1u;
  float mag = e == 0 ? 0.5f * (float)mb : ldexpf(1.0f + 0.5f * (float)mb, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

__global__ __launch_bounds__(256) void indexer_generic(
    const void* __restrict__ qI, int q_fmt, const float* __restrict__ w,
    const void* __restrict__ kI, const uint8_t* __restrict__ ksc, int k_fmt,
    const int32_t* __restrict__ q_pos, int T, int N, int m, int H_I, int D_I, int64_t qi0,
    float* __restrict__ scores, int fill_masked) {
  extern __shared__ float sm[];  // [H_I*D_I] q, [H_I] w
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int nv = n_visible(q_pos[qi], m, N);
  float* sqf = sm;
  float* swf = sm + H_I * D_I;
  for (int i = threadIdx.x; i < H_I * D_I; i += blockDim.x)
    sqf[i] = load_val(qI, (size_t)qi * H_I * D_I + i, q_fmt);
  for (int i = threadIdx.x; i < H_I; i += blockDim.x) swf[i] = w[(size_t)qi * H_I + i];
  __syncthreads();
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= N) return;
  float* srow = scores + (size_t)row * N;
  if (s >= nv) {
    if (fill_masked) srow[s] = kNegInf;
    return;
  }
  const size_t krow = (size_t)b * N + s;
  float acc = 0.f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.f;
    for (int d = 0; d < D_I; ++d) {
      float kv;
      if (k_fmt == FMT_MXFP4) {
        uint32_t byte = reinterpret_cast<const uint8_t*>(kI)[krow * (D_I / 2) + d / 2];
        uint32_t code = (d & 1) ? (byte >> 4) : (byte & 15u);
        kv = fp4_val(code) * e8m0_scale(ksc[krow * (D_I / 32) + d / 32]);
      } else {
        kv = load_val(kI, krow * D_I + d, k_fmt);
      }
      dot += sqf[j * D_I + d] * kv;
    }
    acc += swf[j] * fmaxf(dot, 0.f);
  }
  srow[s] = acc;
}

}  // namespace

hipError_t launch_indexer(const Shape& s, int64_t qi0, int64_t nrows, const void* q_I, int q_fmt,
                          const float* w, const void* k_I, const uint8_t* k_scale, int k_fmt,
                          const int32_t* q_pos, float* scores, bool fill_masked,
                          hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const bool fast = q_fmt == FMT_BF16 && (k_fmt == FMT_BF16 || k_fmt == FMT_MXFP4) &&
                    s.H_I == 64 && s.D_I == 128;
  const int fm = fill_masked ? 1 : 0;
  if (fast && k_fmt == FMT_BF16 && nrows >= 64) {
    // prefill: one launch per sequence segment (a workgroup's queries share one sequence)
    for (int64_t q = qi0; q < qi0 + nrows;) {
      const int b = (int)(q / s.T);
      const int64_t seg_end = std::min<int64_t>(qi0 + nrows, (int64_t)(b + 1) * s.T);
      const int t0 = (int)(q - (int64_t)b * s.T);
      const int nt = (int)(seg_end - q);
      dim3 grid(std::min((s.N + kPfKeys - 1) / kPfKeys, kPfKeyGroups), (nt + kPfQ - 1) / kPfQ);
      hipError_t e = launch(indexer_prefill_mfma, grid, 256, 0, st,
                            static_cast<const uint16_t*>(q_I), w,
                            static_cast<const uint16_t*>(k_I), q_pos, s.T, s.N, s.m, b, t0, nt,
                            scores + (size_t)(q - qi0) * s.N, fm);
      if (e != hipSuccess) return e;
      q = seg_end;
    }
    return hipSuccess;
  }
  if (fast) {
    // keys per wave: enough work per wave to amortise the q_I fragments, while the grid still
    // fills the chip (~1024 workgroups)
    const int64_t total = nrows * (int64_t)s.N;
    int64_t it = total / (32LL * 2048);  // ~2048 waves: two per SIMD
    int iters = 1;
    while (iters < kDecodeMaxIters && 2 * iters <= it) iters *= 2;
    const int keys_per_wg = 4 * 32 * iters;
    dim3 grid((s.N + keys_per_wg - 1) / keys_per_wg, (unsigned)nrows);
    const uint16_t* qp = static_cast<const uint16_t*>(q_I);
    const uint8_t* kp = static_cast<const uint8_t*>(k_I);
#define DSA_DEC(F, I)                                                                     \
  return launch(indexer_decode_mfma<F, I>, grid, 256, 0, st, qp, w, kp, k_scale, q_pos, s.T, \
                s.N, s.m, qi0, scores, fm)
#define DSA_DEC_ITERS(F)        \
  switch (iters) {              \
    case 1: DSA_DEC(F, 1);      \
    case 2: DSA_DEC(F, 2);      \
    case 4: DSA_DEC(F, 4);      \
    case 8: DSA_DEC(F, 8);      \
    default: DSA_DEC(F, 16);    \
  }
    if (k_fmt == FMT_BF16) {
      // 8 waves per workgroup, ~2 tiles per wave: 256 workgroups at 16 x 8192 keys
      int it2 = 1;
      while (it2 < 16 && (int64_t)2 * it2 * 32 * kDecWaves * 256 <= total) it2 *= 2;
      const int kpw = kDecWaves * 32 * it2;
      dim3 g2((s.N + kpw - 1) / kpw, (unsigned)nrows);
      const uint8_t* kb = static_cast<const uint8_t*>(k_I);
#define DSA_DMA(I)                                                                          \
  return launch(indexer_decode_dma<I>, g2, kDecWaves * 64, 0, st, qp, w, kb, q_pos, s.T, s.N, \
                s.m, qi0, scores, fm)
      switch (it2) {
        case 1: DSA_DMA(1);
        case 2: DSA_DMA(2);
        case 4: DSA_DMA(4);
        case 8: DSA_DMA(8);
        default: DSA_DMA(16);
      }
#undef DSA_DMA
    }
    DSA_DEC_ITERS(FMT_MXFP4)
#undef DSA_DEC_ITERS
#undef DSA_DEC
  }
  dim3 grid((s.N + 255) / 256, (unsigned)nrows);
  size_t shm = sizeof(float) * ((size_t)s.H_I * s.D_I + s.H_I);
  return launch(indexer_generic, grid, 256, shm, st, q_I, q_fmt, w, k_I, k_scale, k_fmt, q_pos, s.T,
                s.N, s.m, s.H_I, s.D_I, qi0, scores, fm);
}

}  // namespace dsa
