// indexer.hip - lightning-indexer scores on gfx950.
//
//   I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j,:] . k_I[s,:])     for s < n_vis(t), else -inf
//
// ("DeepSeek-V3.2 sparse-attention principle and TPU adaptation", s1.3 lightning indexer:
// a low-dimensional per-token key, a ReLU instead of a softmax for throughput; s3 step 2:
// "mqa logits", the key is shared by all indexer heads.)
//
// Kernels:
//  * indexer_decode_dma     - few query rows, bf16 keys: the query's 64x128 q_I is staged once
//    per workgroup and held as MFMA A operands; every wave streams its own 32-key tiles of k_I
//    from HBM into a private LDS ring by DMA (v_mfma_f32_32x32x16_bf16).
//  * indexer_decode_fp4_dma - few query rows, MXFP4 keys: the same ring of 64-key tiles, fed
//    to the block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with the FP4 codes and E8M0
//    scales as stored and q_I split into two scaled fp8 operands.
//  * indexer_prefill_mfma   - many query rows of one sequence: each wave keeps 64 keys of k_I
//    in registers, the workgroup walks 32 queries whose q_I is staged in LDS.
//  * indexer_generic        - any H_I / D_I, fp32 or bf16 (and MXFP4) inputs; scalar fp32.
// All of them fuse ReLU, the head weights and the 64-head reduction into the epilogue, so the
// [H_I x N] per-head products never leave registers.
#include "common.h"
#include "launch.h"
#include "select.h"

#include <algorithm>

namespace dsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// E8M0 byte -> fp32 scale 2^(e-127).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
  return e == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
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
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ seq_len, int T, int N, int m,
    int64_t qi0, float* __restrict__ scores, int fill_masked) {
  __shared__ __attribute__((aligned(16))) char sq[64 * 256];
  __shared__ __attribute__((aligned(16))) char sk[kDecWaves][2][32 * 256];
  __shared__ float sres[kDecWaves][32 * ITERS];
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int nv = n_visible(q_pos[qi], m, N, seq_len, b);
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
  // Every wave's q_I DMAs and w loads enter the CU's address queue ahead of all key DMAs (behind
  // them, they would wait out every wave's two tiles); only tile 0 is issued before the full
  // wait the first use of w needs (the compiler cannot count LDS DMAs out of a partial wait),
  // tile 1 right after it.
  __builtin_amdgcn_s_barrier();
  issue(0);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wr[hb][r]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (ITERS > 1) issue(1);
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
    if (t >= 1) {  // (tile 0 landed in the prologue's wait)
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
// Decode-shaped kernel, MX keys (MXFP4: 64 code bytes per key; MXFP8: 128 code bytes per key;
// both with 4 E8M0 scale bytes per key), on the block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4, which takes the codes and their E8M0 scales as they are
// stored (no per-element conversion).
//  * q_I either is MXFP8 itself (QMX: codes and scales go straight into the A operands) or is
//    bf16 and enters as two fp8 (e4m3) operands, q = hi + lo, each with its own E8M0 scale per
//    32 dims: with e the exponent of the block's largest |q|, hi = RNE(q / 2^(e-7)) and
//    lo = RNE((q - hi 2^(e-7)) / 2^(e-11)). A bf16 value has 8 significant bits and hi keeps 4,
//    so the remainder has at most 4 and lo holds it exactly, except for values more than 2^13
//    below the block maximum, where the error stays below 2^(e-21). Products of fp8 and fp4 /
//    fp8 values are exact and accumulate in fp32.
//  * Operand layouts of the instruction (checked on gfx950): an fp4 operand (16 bytes per lane)
//    has lane (c, h) = row or key c, contraction indices 32h .. 32h+31 in nibble order; an fp8
//    operand (32 bytes per lane) has indices 16h .. 16h+15 in bytes 0..15 and 32+16h .. 47+16h
//    in bytes 16..31; the scale of (row or key c, index block b) comes from lane c + 32b.
//    Contraction step s covers dims 64s .. 64s+63, so each index block is one MX block.
//  * Keys stream through LDS: each of the 8 waves runs its own 4-stage ring of tiles (64 FP4
//    keys or 32 FP8 keys: 4 KB of codes in four fully coalesced 1 KB DMAs, scales in one
//    4-byte-per-lane DMA), dealt round-robin over the row's waves so that at any moment the
//    whole grid streams one contiguous window of the key cache (a cold read of this size runs
//    ~25% faster that way than when every wave streams a contiguous range of its own). The
//    16-byte chunks of a code row are XOR-swizzled so that the 16 lanes of a ds_read_b128 phase
//    cover all 64 banks once.
//  * The MFMAs of a 32-key group are issued before the epilogue of the previous group, one
//    MFMA per eight epilogue instructions, so the VALU work overlaps this wave's own MFMAs.
// ------------------------------------------------------------------------------------------
constexpr int kMxStages = 4;          // ring stages per wave
constexpr int kMxStage = 4096 + 256;  // codes + scales per stage

typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int KFMT>
struct MxKeys {
  static constexpr int kTile = KFMT == FMT_MXFP4 ? 64 : 32;  // keys per tile
  static constexpr int kRow = KFMT == FMT_MXFP4 ? 64 : 128;  // code bytes per key
  static constexpr int kChunks = kRow / 16;
  static constexpr int kGroups = kTile / 32;                 // 32-key groups per tile
  static constexpr int kFmt = KFMT == FMT_MXFP4 ? 4 : 0;     // MFMA operand format
  // swizzled slot of 16-byte chunk c of tile row r
  __device__ static int slot(int r, int c) {
    return KFMT == FMT_MXFP4 ? (c ^ ((r >> 2) & 3)) : (c ^ ((r >> 1) & 7));
  }
};

template <int KFMT, bool QMX, int ITERS, bool FILT>
__global__ __launch_bounds__(kDecWaves * 64, 1) void indexer_decode_mx_dma(
    const void* __restrict__ qI, const uint8_t* __restrict__ qsc, const float* __restrict__ w,
    const uint8_t* __restrict__ kI, const uint8_t* __restrict__ ksc,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ seq_len, int T, int N, int m,
    int64_t qi0, float* __restrict__ scores, int fill_masked, int top_k,
    uint8_t* __restrict__ seg_ws) {
  using K = MxKeys<KFMT>;
  constexpr int TK = K::kTile;
  constexpr int NP = QMX ? 1 : 2;  // q parts: the MXFP8 q_I itself, or hi + lo
  static_assert(ITERS * TK <= 512, "the scores of a wave are staged in the q_I operand buffer");
  // sq: fp8 codes of a bf16 q_I's two parts, [part][head][8 chunks of 16 B] (chunk c of head r
  // in slot c ^ (r & 7)); then reused for the scores
  __shared__ __attribute__((aligned(16))) char sq[2 * 64 * 128];
  __shared__ uint32_t sqs[2][64];  // their E8M0 scale bytes: [part][head] x 4 blocks
  __shared__ __attribute__((aligned(16))) char sk[kDecWaves][kMxStages][kMxStage];
  float (*sres)[ITERS * TK] = reinterpret_cast<float (*)[ITERS * TK]>(&sq[0]);
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int nv = n_visible(q_pos[qi], m, N, seq_len, b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  // tile t of wave gw: keys (t GW + gw) * TK ..
  const int gw = blockIdx.x * kDecWaves + wv, GW = gridDim.x * kDecWaves;
  auto tile_key = [&](int t) { return (t * GW + gw) * TK; };
  float* __restrict__ srow = scores + (size_t)row * N;

  if (blockIdx.x * kDecWaves * TK >= nv) {  // every tile of the workgroup is masked
    if (fill_masked)
      for (int t = 0; t < ITERS; ++t)
        if (lane < TK && tile_key(t) + lane < N) srow[tile_key(t) + lane] = kNegInf;
    return;
  }
  const size_t base_row = (size_t)b * N;
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sk[wv][0][0]);
  // head weights of the rows this lane's accumulators hold
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
  // q_I loads: an MXFP8 q_I straight into the A operands (row 32hb + n, dims 64s + 16h .. +15
  // and 64s + 32 + 16h .. +15, scale of block 2s + h); a bf16 q_I per thread for the split
  i32x8_t qa[NP][2][2];
  int qs[NP][2][2];
  u32x4_t q0 = {}, q1 = {};
  uint32_t qsw[2] = {0u, 0u};
  const int qh = tid >> 3, qc = tid & 7;
  if constexpr (QMX) {
    const uint8_t* qrow = static_cast<const uint8_t*>(qI) + (size_t)qi * (64 * 128);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const uint8_t* qr = qrow + (32 * hb + n) * 128;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(qr + 64 * s2 + 16 * h);
        const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(qr + 64 * s2 + 32 + 16 * h);
        qa[0][hb][s2] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                                (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
      }
      qsw[hb] = *reinterpret_cast<const uint32_t*>(qsc + ((size_t)qi * 64 + 32 * hb + n) * 4);
    }
  } else {
    const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(qI) +
                                                           (size_t)qi * (64 * 128) + qh * 128 + 16 * qc);
    q0 = qsrc[0];
    q1 = qsrc[1];
  }
  // tile t of this wave into stage t % kMxStages: 5 DMA instructions
  auto issue = [&](int t) {
    const uint32_t sb = ring + (t % kMxStages) * kMxStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (1024 / K::kRow) * j + lane / K::kChunks, c = lane % K::kChunks;
      // keys past the visible range re-read the last visible row (served by L2)
      const size_t krow = base_row + min(tile_key(t) + r, nv - 1);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(kI + krow * K::kRow + 16 * K::slot(r, c)),
          (lds_void_t*)(uintptr_t)(sb + 1024 * j), 16, 0, 0);
    }
    const size_t srow_k = base_row + min(tile_key(t) + lane, nv - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ksc + srow_k * 4),
                                     (lds_void_t*)(uintptr_t)(sb + 4096), 4, 0, 0);
  };
  constexpr int kPre = ITERS < kMxStages ? ITERS : kMxStages;
  constexpr int kHead = kPre < 2 ? kPre : 2;
  // Every wave's q_I and w loads enter the CU's address queue ahead of all the key DMAs
  // (queued behind the other waves' DMAs they would wait out tens of them). Their first use
  // makes the compiler wait for every memory instruction in flight (it cannot count LDS DMAs
  // out of a partial wait), so only the first kHead tiles are issued before it, the rest once
  // q_I is in its operand registers.
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int t = 0; t < kHead; ++t) issue(t);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(wr[hb][r]));
  asm volatile("" : "+v"(q0), "+v"(q1), "+v"(qsw[0]), "+v"(qsw[1]));
  if constexpr (QMX) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) asm volatile("" : "+v"(qa[0][hb][s2]));
  }
  if constexpr (QMX) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) qs[0][hb][s2] = (int)((qsw[hb] >> (8 * (2 * s2 + h))) & 0xffu);
  } else {
    // thread t converts head t / 8, dims 16 (t % 8) .. +15 into the two fp8 parts
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(q0[i] & 0xffffu));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(q0[i] >> 16));
      v[8 + 2 * i] = bf16_to_f32((uint16_t)(q1[i] & 0xffffu));
      v[8 + 2 * i + 1] = bf16_to_f32((uint16_t)(q1[i] >> 16));
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // the other 16 dims of the 32-dim block
    // exponent of the block maximum (clamped so both scale bytes stay in range)
    const int e = amax > 0.f ? max(((int)(__float_as_uint(amax) >> 23) & 0xff) - 127, -100) : 0;
    const float inv_hi = __uint_as_float((uint32_t)(127 - (e - 7)) << 23);  // 2^-(e-7)
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hp = 0, lp = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float a = v[4 * i + 2 * j] * inv_hi, c = v[4 * i + 2 * j + 1] * inv_hi;
        const uint32_t hc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, c, 0, false) & 0xffffu;
        const float ra = (a - __builtin_amdgcn_cvt_f32_fp8(hc, 0)) * 16.f;
        const float rc = (c - __builtin_amdgcn_cvt_f32_fp8(hc, 1)) * 16.f;
        const uint32_t lc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ra, rc, 0, false) & 0xffffu;
        hp |= hc << (16 * j);
        lp |= lc << (16 * j);
      }
      hw[i] = hp;
      lw[i] = lp;
    }
    const int slot = qc ^ (qh & 7);
    *reinterpret_cast<u32x4_t*>(&sq[qh * 128 + 16 * slot]) = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
    *reinterpret_cast<u32x4_t*>(&sq[64 * 128 + qh * 128 + 16 * slot]) = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
    if ((qc & 1) == 0) {  // one scale byte per 32-dim block: hi 2^(e-7), lo 2^(e-11)
      reinterpret_cast<uint8_t*>(&sqs[0][qh])[qc >> 1] = (uint8_t)(e + 120);
      reinterpret_cast<uint8_t*>(&sqs[1][qh])[qc >> 1] = (uint8_t)(e + 116);
    }
    __syncthreads();
#pragma unroll
    for (int pt = 0; pt < NP; ++pt)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int r = 32 * hb + n;
        const uint32_t sc4 = sqs[pt][r];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int c0 = 4 * s2 + h, c1 = 4 * s2 + 2 + h;  // 16-byte chunks
          const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(&sq[pt * 64 * 128 + r * 128 + 16 * (c0 ^ (r & 7))]);
          const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(&sq[pt * 64 * 128 + r * 128 + 16 * (c1 ^ (r & 7))]);
          qa[pt][hb][s2] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                                   (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
          qs[pt][hb][s2] = (int)((sc4 >> (8 * (2 * s2 + h))) & 0xffu);  // block 2s + h
        }
      }
  }
  // the other prefetched tiles, after the last LDS read the compiler would hold behind them
#pragma unroll
  for (int t = kHead; t < kPre; ++t) issue(t);
  // every wave holds its A operands before the buffer is reused for the scores
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();

  // Software pipeline over the K::kGroups * ITERS groups of 32 keys (group g: tile
  // g / kGroups, keys 32 (g % kGroups) ..): the MFMAs of group g + 1 are issued before the
  // epilogue of group g, one MFMA per eight epilogue instructions. Two accumulator pairs
  // alternate.
  constexpr int G = K::kGroups * ITERS;
  auto tile_ready = [&](int t) {
    if (t > 0 && t + kMxStages - 1 < ITERS) {
      // stage (t-1) % kMxStages: its B-operand reads completed before their MFMAs issued
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(t + kMxStages - 1);
    }
    // tile t landed; the tiles after it (up to three) may still be in flight
    const int after = min(ITERS - 1 - t, kMxStages - 1);
    switch (after) {
      case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
  };
  auto mfma_group = [&](int g, f32x16_t& acc0, f32x16_t& acc1) {
    const char* st = &sk[wv][(g / K::kGroups) % kMxStages][0];
    const int r = 32 * (g % K::kGroups) + n;
    const uint32_t ks = *reinterpret_cast<const uint32_t*>(st + 4096 + 4 * r);
    i32x8_t kb[2];
    int kss[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      kss[s2] = (int)((ks >> (8 * (2 * s2 + h))) & 0xffu);  // scale of block 2s + h
      if constexpr (KFMT == FMT_MXFP4) {
        // key r, step s: 16-byte chunk 2s + h of its codes
        const u32x4_t c4 = *reinterpret_cast<const u32x4_t*>(st + r * 64 + 16 * K::slot(r, 2 * s2 + h));
        kb[s2] = i32x8_t{(int)c4[0], (int)c4[1], (int)c4[2], (int)c4[3], 0, 0, 0, 0};
      } else {
        // key r, step s: chunks 4s + h and 4s + 2 + h (the fp8 operand layout)
        const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(st + r * 128 + 16 * K::slot(r, 4 * s2 + h));
        const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(st + r * 128 + 16 * K::slot(r, 4 * s2 + 2 + h));
        kb[s2] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                         (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
      }
    }
    acc0 = f32x16_t{};
    acc1 = f32x16_t{};
#pragma unroll
    for (int pt = 0; pt < NP; ++pt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[pt][0][s2], kb[s2], acc0, 0, K::kFmt, 0, qs[pt][0][s2], 0, kss[s2]);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[pt][1][s2], kb[s2], acc1, 0, K::kFmt, 0, qs[pt][1][s2], 0, kss[s2]);
      }
  };
  auto epilogue = [&](int g, const f32x16_t& acc0, const f32x16_t& acc1) {
    float p4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p4[i & 3] += wr[0][i] * relu_bits(acc0[i]);
      p4[(i + 2) & 3] += wr[1][i] * relu_bits(acc1[i]);
    }
    float part = (p4[0] + p4[1]) + (p4[2] + p4[3]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    part = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // both halves: heads 4h.. of every 8
    if (h == 0) sres[wv][32 * g + n] = part;
  };
  f32x16_t accA0, accA1, accB0, accB1;
  tile_ready(0);
  mfma_group(0, accA0, accA1);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g + 1 < G) {
      if ((g + 1) % K::kGroups == 0) tile_ready((g + 1) / K::kGroups);
      if (g & 1) mfma_group(g + 1, accA0, accA1);
      else mfma_group(g + 1, accB0, accB1);
    }
    if (g & 1) epilogue(g, accB0, accB1);
    else epilogue(g, accA0, accA1);
    if (g + 1 < G) {
#pragma unroll
      for (int k = 0; k < 4 * NP; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 16 / NP, 0);  // epilogue instructions
      }
    }
  }
#pragma unroll
  for (int t = 0; t < ITERS; ++t) {
    const int s = tile_key(t) + lane;
    if (lane < TK) {
      if (s < nv) srow[s] = sres[wv][TK * t + lane];
      else if (fill_masked && s < N) srow[s] = kNegInf;
    }
  }
  if constexpr (FILT) {
    // The long-row top-k's first stage on the scores still in LDS (select.h chunk_filter):
    // this workgroup's keys are one chunk; thread (wv, lane) takes its wave's staged scores
    // 8 lane .. 8 lane + 7 (one tile, ascending keys, so the visible ones come first).
    static_assert(ITERS * TK == 8 * 64, "one chunk = 8 staged scores per thread");
    if (nv <= top_k) return;  // the select keeps every visible entry
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with its ring, which now holds the select state
    SelShared<kDecWaves>& sh = *reinterpret_cast<SelShared<kDecWaves>*>(&sk[0][0][0]);
    const int t = (8 * lane) / TK, off = (8 * lane) % TK;
    const int e0 = tile_key(t) + off;
    uint32_t key[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) key[j] = order_key(sres[wv][8 * lane + j]);
    const int nvt = max(0, min(8, nv - e0));
    chunk_filter<kDecWaves, 8>(key, nvt, nv, top_k, sh, seg_ws + (size_t)row * long_row_bytes(gridDim.x),
                               gridDim.x, blockIdx.x, [&](int j) { return e0 + j; });
  }
}

// ------------------------------------------------------------------------------------------
// Prefill-shaped kernel (bf16). H_I = 64, D_I = 128. Workgroup = kPfQ queries of one sequence x
// the key blocks (256 keys) g, g + gridDim.x, ... (g: its key group) below the queries' visible
// range: a grid of every (key block, query block) pair would be mostly blocks past the causal
// edge, and dispatching those alone costs more than a tenth of the kernel. When a query block
// sees fewer key blocks than there are key groups (early causal chunks), the spare groups split
// its queries instead of idling: group g takes key block g % nkb and the (g / nkb)-th part of the
// rows. Per key block, wave wv holds keys kbase + 64*wv + 32*kb + n (kb = 0, 1) as B operands in
// registers; the queries' q_I (64 x 128, 16 KB) and w (64) stream through a 3-stage LDS ring by
// buffer-to-LDS DMA (one 32-bit offset register per DMA), two queries ahead of the MFMAs (row hr
// keeps its 16-byte chunk c in slot c ^ (hr % 16): the A-operand reads are conflict-free). One
// barrier per query; the DMA waits are explicit, so the barrier never drains the queries in
// flight. The MFMAs run one 32-head x 32-key block at a time (8 chained MFMAs, then that block's
// ReLU and head weights), so A operands and accumulators take 48 registers instead of 128: the
// kernel fits 168 VGPRs and three waves per SIMD (three workgroups per CU), which hides more of
// the epilogue and the DMA issue behind other waves' MFMAs than two did. The per-key sums run in
// the same order as with all four blocks in flight (head block, then 4-row group, then row).
// ------------------------------------------------------------------------------------------
constexpr int kPfKeys = 256;
constexpr int kPfQ = 32;
constexpr int kPfKeyGroups = 96;     // workgroups per query block (at most)
constexpr int kPfMinQ = 8;           // fewest queries per workgroup when queries are split

template <bool FILL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void
indexer_prefill_mfma(const uint16_t* __restrict__ qI, const float* __restrict__ w,
                     const uint16_t* __restrict__ kI, const int32_t* __restrict__ q_pos,
                     const int32_t* __restrict__ seq_len, int T, int N, int m, int b, int t0,
                     int nt, float* __restrict__ scores) {
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
    int v = n_visible(q_pos[qi0 + tid], m, N, seq_len, b);
    snv[tid] = v;
    atomicMax(&smax, v);
  }
  __syncthreads();
  const int maxnv = smax;
  const size_t base_row = (size_t)b * N;
  const uint32_t qlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sq[0][0]);
  const uint32_t wlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sw[0][0]);
  // byte offset of this lane's q_I DMA j within a query's 16 KB: (d0 ^ 64 j) + 1024 j
  const uint32_t d0 = (16 * wv + (lane >> 4)) * 256 + 16 * ((lane & 15) ^ (lane >> 4));

  // key blocks and rows of this workgroup (FILL: every key block, masked ones set to -inf)
  int kfirst = kgrp, kstep = gridDim.x, rbeg = 0, rend = nrows;
  const int nkbv = (maxnv + kPfKeys - 1) / kPfKeys;  // visible key blocks of the query block
  if (!FILL && nkbv > 0 && nkbv < (int)gridDim.x) {
    const int parts = min((int)gridDim.x / nkbv, max(1, nrows / kPfMinQ));
    if (kgrp >= parts * nkbv) return;  // uniform over the workgroup, after its last barrier
    const int part = kgrp / nkbv;
    kfirst = kgrp % nkbv;
    kstep = nkbv;
    rbeg = part * nrows / parts;
    rend = (part + 1) * nrows / parts;
  }
  for (int kblk = kfirst; kblk * kPfKeys < N; kblk += kstep) {
    const int kbase = kblk * kPfKeys;
    if (kbase >= maxnv) {
      if (FILL)
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
    // query, the others 4. The buffer descriptors cover exactly the query's q_I row and w row.
    auto stage = [&](int r, int buf) {
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(qI + (size_t)(qi0 + r) * (64 * 128)), (short)0, 64 * 256,
          0x00020000);
      uint32_t dd = d0;
      asm volatile("" : "+v"(dd));  // rebuilt per query: no loop-invariant offsets held
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (lds_void_t*)(uintptr_t)(qlds + buf * (64 * 256) + (16 * wv + 4 * j) * 256), 16,
            (dd ^ (64 * j)) + 1024 * j, 0, 0, 0);
      if (wv == 0 && lane < 16) {
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(w + (size_t)(qi0 + r) * 64), (short)0, 256, 0x00020000);
        uint32_t wo;  // 16 x lane id, computed here (a loop-invariant copy would be spilled)
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\t"
                     "v_lshlrev_b32 %0, 4, %0"
                     : "=v"(wo));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t*)(uintptr_t)(wlds + buf * 256),
                                                 16, wo, 0, 0, 0);
      }
    };
    stage(rbeg, 0);
    if (rbeg + 1 < rend) stage(rbeg + 1, 1);

    for (int r = rbeg; r < rend; ++r) {
      const int buf = (r - rbeg) % 3;
      // query r landed (query r+1's DMAs may still be in flight), then every wave's share is
      // visible after the barrier; stage (r+2)%3 was last read in iteration r-1
      if (r + 1 < rend) {
        if (wv == 0) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      if (r + 2 < rend) stage(r + 2, (r - rbeg + 2) % 3);
      const int nv = snv[r];
      float* srow = scores + (size_t)(r0 + r) * N;
      if (kbase < nv) {
        const char* qb = &sq[buf][0];
        // row n's chunk 8h + kk sits at slot (8h + kk) ^ (n & 15): byte offset abase ^ 16 kk
        uint32_t abase = n * 256 + 128 * (h ^ ((n >> 3) & 1)) + 16 * (n & 7);
        asm volatile("" : "+v"(abase));  // rebuilt per query: no loop-invariant offsets held
        float part[2] = {0.f, 0.f};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          __builtin_amdgcn_sched_barrier(0);
          u32x4_t a[8];
#pragma unroll
          for (int kk = 0; kk < 8; ++kk)
            a[kk] = *reinterpret_cast<const u32x4_t*>(qb + hb * 8192 + (abase ^ (16 * kk)));
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            __builtin_amdgcn_sched_barrier(0);
            f32x16_t acc = {};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kk]), as_bf16x8(kf[kb][kk]),
                                                            acc, 0, 0, 0);
            // lane (n, h) holds rows 8*(i/4) + 4*h + i%4 of the 32-head block: w of those heads
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(&sw[buf][hb * 32 + 8 * q4 + 4 * h]);
#pragma unroll
              for (int i = 0; i < 4; ++i) part[kb] += w4[i] * relu_bits(acc[4 * q4 + i]);
            }
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          float v = part[kb] + __shfl_xor(part[kb], 32, 64);
          int s = kbase + 64 * wv + 32 * kb + n;
          if (h == 0 && s < N && (FILL || s < nv)) srow[s] = (s < nv) ? v : kNegInf;
        }
      } else if (FILL) {
        for (int s = kbase + tid; s < min(kbase + kPfKeys, N); s += 256) srow[s] = kNegInf;
      }
    }
    // every wave is done with the ring before the next key block restages it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }
}

// ------------------------------------------------------------------------------------------
// Prefill-shaped kernel, MXFP8 q_I with MX keys (MXFP8 or MXFP4), on the block-scaled MFMA:
// the structure of indexer_prefill_mfma (a workgroup = kPfQ queries of one sequence x the key
// blocks g, g + gridDim.x, ..., spare key groups splitting the queries, each wave holding 64
// keys as B operands in registers, q_I and w streamed through a 3-stage LDS ring by DMA two
// queries ahead, one 32-head block at a time so that three waves fit per SIMD), with the
// operands in their stored codes: per query and wave, 8 v_mfma_scale_f32_32x32x64_f8f6f4 (2 head
// blocks x 2 key blocks x 2 steps of 64 dims) in place of 32 v_mfma_f32_32x32x16_bf16. Operand
// layouts as in
// indexer_decode_mx_dma. A query's ring stage: 8 KB of e4m3 codes (row hr keeps its 16-byte
// chunk c in slot c ^ ((hr >> 1) & 7)), its 256 scale bytes and its 64 weights.
// ------------------------------------------------------------------------------------------
constexpr int kPfMxStage = 64 * 128 + 256 + 256;

template <int KFMT, bool FILL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void
indexer_prefill_mx(const uint8_t* __restrict__ qI, const uint8_t* __restrict__ qsc,
                   const float* __restrict__ w, const uint8_t* __restrict__ kI,
                   const uint8_t* __restrict__ ksc, const int32_t* __restrict__ q_pos,
                   const int32_t* __restrict__ seq_len, int T, int N, int m, int b, int t0, int nt,
                   float* __restrict__ scores) {
  using K = MxKeys<KFMT>;
  __shared__ __attribute__((aligned(16))) char sq[3][kPfMxStage];
  __shared__ int snv[kPfQ];
  __shared__ int smax;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int item = xcd_item(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int kgrp = item % gridDim.x;
  const int r0 = (item / gridDim.x) * kPfQ;  // first row (relative to t0) of this tile
  const int nrows = min(kPfQ, nt - r0);
  const int64_t qi0 = (int64_t)b * T + t0 + r0;

  if (tid == 0) smax = 0;
  __syncthreads();
  if (tid < nrows) {
    int v = n_visible(q_pos[qi0 + tid], m, N, seq_len, b);
    snv[tid] = v;
    atomicMax(&smax, v);
  }
  __syncthreads();
  const int maxnv = smax;
  const size_t base_row = (size_t)b * N;
  const uint32_t qlds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)&sq[0][0]);
  // key blocks and rows of this workgroup, as in indexer_prefill_mfma
  int kfirst = kgrp, kstep = gridDim.x, rbeg = 0, rend = nrows;
  const int nkbv = (maxnv + kPfKeys - 1) / kPfKeys;
  if (!FILL && nkbv > 0 && nkbv < (int)gridDim.x) {
    const int parts = min((int)gridDim.x / nkbv, max(1, nrows / kPfMinQ));
    if (kgrp >= parts * nkbv) return;  // uniform over the workgroup, after its last barrier
    const int part = kgrp / nkbv;
    kfirst = kgrp % nkbv;
    kstep = nkbv;
    rbeg = part * nrows / parts;
    rend = (part + 1) * nrows / parts;
  }
  for (int kblk = kfirst; kblk * kPfKeys < N; kblk += kstep) {
    const int kbase = kblk * kPfKeys;
    if (kbase >= maxnv) {
      if (FILL)
        for (int r = 0; r < nrows; ++r)
          for (int s = kbase + tid; s < min(kbase + kPfKeys, N); s += 256)
            scores[(size_t)(r0 + r) * N + s] = kNegInf;
      continue;
    }

    // this wave's keys as B operands: key kbase + 64 wv + 32 kb + n, step s2
    i32x8_t kf[2][2];
    uint32_t ksw[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const size_t krow = base_row + min(kbase + 64 * wv + 32 * kb + n, N - 1);
      const uint8_t* p = kI + krow * K::kRow;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if constexpr (KFMT == FMT_MXFP4) {
          const u32x4_t c4 = *reinterpret_cast<const u32x4_t*>(p + 16 * (2 * s2 + h));
          kf[kb][s2] = i32x8_t{(int)c4[0], (int)c4[1], (int)c4[2], (int)c4[3], 0, 0, 0, 0};
        } else {
          const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(p + 16 * (4 * s2 + h));
          const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(p + 16 * (4 * s2 + 2 + h));
          kf[kb][s2] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                               (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        }
      }
      ksw[kb] = *reinterpret_cast<const uint32_t*>(ksc + krow * 4);
    }

    // DMA of query r into stage buf: wave wv moves code rows 16 wv .. 16 wv + 15 (two 1 KB
    // instructions); wave 0 also moves w (16 lanes x 16 B), wave 1 the scales (64 lanes x 4 B).
    // Waves 0 and 1 issue 3 instructions per query, waves 2 and 3 two.
    auto stage = [&](int r, int buf) {
      const uint8_t* src = qI + (size_t)(qi0 + r) * (64 * 128);
      const uint32_t sb = qlds + buf * kPfMxStage;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int u = 2 * wv + j, hr = 8 * u + (lane >> 3), c = lane & 7;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(src + hr * 128 + 16 * (c ^ ((hr >> 1) & 7))),
            (lds_void_t*)(uintptr_t)(sb + 1024 * u), 16, 0, 0);
      }
      if (wv == 0 && lane < 16)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(w + (size_t)(qi0 + r) * 64 + 4 * lane),
            (lds_void_t*)(uintptr_t)(sb + 8192 + 256), 16, 0, 0);
      if (wv == 1)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(qsc + ((size_t)(qi0 + r) * 64 + lane) * 4),
            (lds_void_t*)(uintptr_t)(sb + 8192), 4, 0, 0);
    };
    stage(rbeg, 0);
    if (rbeg + 1 < rend) stage(rbeg + 1, 1);

    for (int r = rbeg; r < rend; ++r) {
      const int buf = (r - rbeg) % 3;
      // query r landed (query r+1's DMAs may still be in flight), then every wave's share is
      // visible after the barrier; stage (r+2)%3 was last read in iteration r-1
      if (r + 1 < rend) {
        if (wv < 2) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      if (r + 2 < rend) stage(r + 2, (r - rbeg + 2) % 3);
      const int nv = snv[r];
      float* srow = scores + (size_t)(r0 + r) * N;
      if (kbase < nv) {
        const char* qb = &sq[buf][0];
        // lane (n, h) holds rows 8*(i/4) + 4*h + i%4 of each 32-head block: w of those heads
        const float* wb = reinterpret_cast<const float*>(qb + 8192 + 256);
        float part[2] = {0.f, 0.f};
        // one 32-head block at a time (fewer live registers: three waves per SIMD)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          __builtin_amdgcn_sched_barrier(0);
          const int hr = 32 * hb + n;
          i32x8_t a[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int c0 = 4 * s2 + h, c1 = 4 * s2 + 2 + h;
            const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(qb + hr * 128 + 16 * (c0 ^ ((hr >> 1) & 7)));
            const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(qb + hr * 128 + 16 * (c1 ^ ((hr >> 1) & 7)));
            a[s2] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                            (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
          }
          const uint32_t qsw = *reinterpret_cast<const uint32_t*>(qb + 8192 + 4 * hr);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            f32x16_t acc = {};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int qs = (int)((qsw >> (8 * (2 * s2 + h))) & 0xffu);
              const int ks = (int)((ksw[kb] >> (8 * (2 * s2 + h))) & 0xffu);
              acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s2], kf[kb][s2], acc, 0,
                                                                    K::kFmt, 0, qs, 0, ks);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(wb + hb * 32 + 8 * q4 + 4 * h);
#pragma unroll
              for (int i = 0; i < 4; ++i) part[kb] += w4[i] * relu_bits(acc[4 * q4 + i]);
            }
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[kb]), __float_as_uint(part[kb]), false, false);
          const float v = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
          int s = kbase + 64 * wv + 32 * kb + n;
          if (h == 0 && s < N && (FILL || s < nv)) srow[s] = (s < nv) ? v : kNegInf;
        }
      } else if (FILL) {
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

// e4m3 (OCP E4M3FN) code -> value: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0
__device__ __forceinline__ float fp8_val(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, mb = code & 7u;
  const float mag = e == 0 ? ldexpf((float)mb, -9) : ldexpf(1.0f + 0.125f * (float)mb, (int)e - 7);
  return (code & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ float fp4_val(uint32_t code) {
  // e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0
  uint32_t e = (code >> 1) & 3u, mb = code & 1u;
  float mag = e == 0 ? 0.5f * (float)mb : ldexpf(1.0f + 0.5f * (float)mb, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

__global__ __launch_bounds__(256) void indexer_generic(
    const void* __restrict__ qI, int q_fmt, const uint8_t* __restrict__ qsc,
    const float* __restrict__ w, const void* __restrict__ kI, const uint8_t* __restrict__ ksc,
    int k_fmt,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ seq_len, int T, int N, int m,
    int H_I, int D_I, int64_t qi0, float* __restrict__ scores, int fill_masked) {
  extern __shared__ float sm[];  // [H_I*D_I] q, [H_I] w
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int nv = n_visible(q_pos[qi], m, N, seq_len, b);
  float* sqf = sm;
  float* swf = sm + H_I * D_I;
  for (int i = threadIdx.x; i < H_I * D_I; i += blockDim.x) {
    const size_t e = (size_t)qi * H_I * D_I + i;
    sqf[i] = q_fmt == FMT_MXFP8
                 ? fp8_val(static_cast<const uint8_t*>(qI)[e]) * e8m0_scale(qsc[e / 32])
                 : load_val(qI, e, q_fmt);
  }
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
  auto kval = [&](int d) -> float {
    if (k_fmt == FMT_MXFP4) {
      uint32_t byte = reinterpret_cast<const uint8_t*>(kI)[krow * (D_I / 2) + d / 2];
      uint32_t code = (d & 1) ? (byte >> 4) : (byte & 15u);
      return fp4_val(code) * e8m0_scale(ksc[krow * (D_I / 32) + d / 32]);
    }
    if (k_fmt == FMT_MXFP8)
      return fp8_val(reinterpret_cast<const uint8_t*>(kI)[krow * D_I + d]) *
             e8m0_scale(ksc[krow * (D_I / 32) + d / 32]);
    return load_val(kI, krow * D_I + d, k_fmt);
  };
  float acc = 0.f;
  if (H_I <= 8) {
    // few heads: each key value is loaded once and feeds every head's dot product; the loads
    // of a block of dims are in flight together (one at a time, every product waited out a
    // cache round trip)
    float dot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int d = 0; d < D_I; ++d) {
      const float kv = kval(d);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < H_I) dot[j] += sqf[j * D_I + d] * kv;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < H_I) acc += swf[j] * fmaxf(dot[j], 0.f);
  } else {
    for (int j = 0; j < H_I; ++j) {
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D_I; ++d) dot += sqf[j * D_I + d] * kval(d);
      acc += swf[j] * fmaxf(dot, 0.f);
    }
  }
  srow[s] = acc;
}

}  // namespace

hipError_t launch_indexer(const Shape& s, int64_t qi0, int64_t nrows, const void* q_I, int q_fmt,
                          const uint8_t* q_scale, const float* w, const void* k_I,
                          const uint8_t* k_scale, int k_fmt, const int32_t* q_pos,
                          const int32_t* seq_len, float* scores, bool fill_masked,
                          hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const bool shape_ok = s.H_I == 64 && s.D_I == 128;
  const bool kmx = k_fmt == FMT_MXFP4 || k_fmt == FMT_MXFP8;
  const int fm = fill_masked ? 1 : 0;
  if (shape_ok && q_fmt == FMT_BF16 && k_fmt == FMT_BF16 && nrows >= 64) {
    // prefill: one launch per sequence segment (a workgroup's queries share one sequence)
    for (int64_t q = qi0; q < qi0 + nrows;) {
      const int b = (int)(q / s.T);
      const int64_t seg_end = std::min<int64_t>(qi0 + nrows, (int64_t)(b + 1) * s.T);
      const int t0 = (int)(q - (int64_t)b * s.T);
      const int nt = (int)(seg_end - q);
      dim3 grid(std::min((s.N + kPfKeys - 1) / kPfKeys, kPfKeyGroups), (nt + kPfQ - 1) / kPfQ);
      const uint16_t* qp = static_cast<const uint16_t*>(q_I);
      const uint16_t* kp = static_cast<const uint16_t*>(k_I);
      float* sc = scores + (size_t)(q - qi0) * s.N;
      hipError_t e = fm ? launch(indexer_prefill_mfma<true>, grid, 256, 0, st, qp, w, kp, q_pos,
                                 seq_len, s.T, s.N, s.m, b, t0, nt, sc)
                        : launch(indexer_prefill_mfma<false>, grid, 256, 0, st, qp, w, kp, q_pos,
                                 seq_len, s.T, s.N, s.m, b, t0, nt, sc);
      if (e != hipSuccess) return e;
      q = seg_end;
    }
    return hipSuccess;
  }
  if (shape_ok && q_fmt == FMT_MXFP8 && kmx && nrows >= 64) {
    // prefill with an MXFP8 q_I: one launch per sequence segment, as above
    for (int64_t q = qi0; q < qi0 + nrows;) {
      const int b = (int)(q / s.T);
      const int64_t seg_end = std::min<int64_t>(qi0 + nrows, (int64_t)(b + 1) * s.T);
      const int t0 = (int)(q - (int64_t)b * s.T);
      const int nt = (int)(seg_end - q);
      dim3 grid(std::min((s.N + kPfKeys - 1) / kPfKeys, kPfKeyGroups), (nt + kPfQ - 1) / kPfQ);
      const uint8_t* qp = static_cast<const uint8_t*>(q_I);
      const uint8_t* kp = static_cast<const uint8_t*>(k_I);
      float* sc = scores + (size_t)(q - qi0) * s.N;
      hipError_t e;
      if (k_fmt == FMT_MXFP4)
        e = fm ? launch(indexer_prefill_mx<FMT_MXFP4, true>, grid, 256, 0, st, qp, q_scale, w, kp,
                        k_scale, q_pos, seq_len, s.T, s.N, s.m, b, t0, nt, sc)
               : launch(indexer_prefill_mx<FMT_MXFP4, false>, grid, 256, 0, st, qp, q_scale, w, kp,
                        k_scale, q_pos, seq_len, s.T, s.N, s.m, b, t0, nt, sc);
      else
        e = fm ? launch(indexer_prefill_mx<FMT_MXFP8, true>, grid, 256, 0, st, qp, q_scale, w, kp,
                        k_scale, q_pos, seq_len, s.T, s.N, s.m, b, t0, nt, sc)
               : launch(indexer_prefill_mx<FMT_MXFP8, false>, grid, 256, 0, st, qp, q_scale, w, kp,
                        k_scale, q_pos, seq_len, s.T, s.N, s.m, b, t0, nt, sc);
      if (e != hipSuccess) return e;
      q = seg_end;
    }
    return hipSuccess;
  }
  const int64_t total = nrows * (int64_t)s.N;
  const uint8_t* kp = static_cast<const uint8_t*>(k_I);
  if (shape_ok && q_fmt == FMT_BF16 && k_fmt == FMT_BF16) {
    // 8 waves per workgroup, ~2 tiles per wave: 256 workgroups at 16 x 8192 keys
    const uint16_t* qp = static_cast<const uint16_t*>(q_I);
    int it2 = 1;
    while (it2 < 16 && (int64_t)2 * it2 * 32 * kDecWaves * 256 <= total) it2 *= 2;
    const int kpw = kDecWaves * 32 * it2;
    dim3 g2((s.N + kpw - 1) / kpw, (unsigned)nrows);
#define DSA_DMA(I)                                                                          \
  return launch(indexer_decode_dma<I>, g2, kDecWaves * 64, 0, st, qp, w, kp, q_pos, seq_len, \
                s.T, s.N, s.m, qi0, scores, fm)
    switch (it2) {
      case 1: DSA_DMA(1);
      case 2: DSA_DMA(2);
      case 4: DSA_DMA(4);
      case 8: DSA_DMA(8);
      default: DSA_DMA(16);
    }
#undef DSA_DMA
  }
  if (shape_ok && kmx && (q_fmt == FMT_BF16 || q_fmt == FMT_MXFP8)) {
    // MX keys: 8 waves per workgroup, tiles of 64 (FP4) or 32 (FP8) keys, ~256 workgroups
    const int tk = k_fmt == FMT_MXFP4 ? 64 : 32, max_it = 512 / tk;
    int it = 1;
    while (it < max_it && (int64_t)2 * it * tk * kDecWaves * 256 <= total) it *= 2;
    const int kpw = kDecWaves * tk * it;
    dim3 g((s.N + kpw - 1) / kpw, (unsigned)nrows);
#define DSA_MX(KF, QM, I)                                                                        \
  return launch(indexer_decode_mx_dma<KF, QM, I, false>, g, kDecWaves * 64, 0, st, q_I, q_scale, w, \
                kp, k_scale, q_pos, seq_len, s.T, s.N, s.m, qi0, scores, fm, s.top_k, nullptr)
#define DSA_MX_IT(KF, QM)        \
  switch (it) {                  \
    case 1: DSA_MX(KF, QM, 1);   \
    case 2: DSA_MX(KF, QM, 2);   \
    case 4: DSA_MX(KF, QM, 4);   \
    case 8: DSA_MX(KF, QM, 8);   \
    default:                     \
      if constexpr (KF == FMT_MXFP8) { DSA_MX(KF, QM, 16); }  \
      else { DSA_MX(KF, QM, 8); } \
  }
    if (k_fmt == FMT_MXFP4) {
      if (q_fmt == FMT_MXFP8) DSA_MX_IT(FMT_MXFP4, true)
      DSA_MX_IT(FMT_MXFP4, false)
    }
    if (q_fmt == FMT_MXFP8) DSA_MX_IT(FMT_MXFP8, true)
    DSA_MX_IT(FMT_MXFP8, false)
#undef DSA_MX_IT
#undef DSA_MX
  }
  dim3 grid((s.N + 255) / 256, (unsigned)nrows);
  size_t shm = sizeof(float) * ((size_t)s.H_I * s.D_I + s.H_I);
  return launch(indexer_generic, grid, 256, shm, st, q_I, q_fmt, q_scale, w, k_I, k_scale, k_fmt,
                q_pos, seq_len, s.T, s.N, s.m, s.H_I, s.D_I, qi0, scores, fm);
}

int indexer_segment_stride(const Shape& s, int64_t nrows, int q_fmt, int k_fmt) {
  const bool shape_ok = s.H_I == 64 && s.D_I == 128;
  const bool kmx = k_fmt == FMT_MXFP4 || k_fmt == FMT_MXFP8;
  if (!shape_ok || !kmx || s.N <= kLongChunk * 8 || nrows <= 0) return 0;
  if (q_fmt == FMT_MXFP8 && nrows >= 64) return 0;  // the prefill-shaped kernel
  if (q_fmt != FMT_BF16 && q_fmt != FMT_MXFP8) return 0;
  // the decode kernel's plan (launch_indexer) must be the one with 4096 keys per workgroup,
  // the chunk size of the segment workspace
  const int tk = k_fmt == FMT_MXFP4 ? 64 : 32, max_it = 512 / tk;
  const int64_t total = nrows * (int64_t)s.N;
  int it = 1;
  while (it < max_it && (int64_t)2 * it * tk * kDecWaves * 256 <= total) it *= 2;
  return it == max_it ? kDecWaves * tk : 0;
}

hipError_t launch_indexer_segments(const Shape& s, int64_t qi0, int64_t nrows, const void* q_I,
                                   int q_fmt, const uint8_t* q_scale, const float* w,
                                   const void* k_I, const uint8_t* k_scale, int k_fmt,
                                   const int32_t* q_pos, const int32_t* seq_len, float* scores,
                                   bool fill_masked, uint8_t* seg_ws, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  if (indexer_segment_stride(s, nrows, q_fmt, k_fmt) == 0) return hipErrorInvalidValue;
  const int fm = fill_masked ? 1 : 0;
  const uint8_t* kp = static_cast<const uint8_t*>(k_I);
  const dim3 g((s.N + kLongChunk - 1) / kLongChunk, (unsigned)nrows);
#define DSA_MXF(KF, QM, I)                                                                      \
  return launch(indexer_decode_mx_dma<KF, QM, I, true>, g, kDecWaves * 64, 0, st, q_I, q_scale, w, \
                kp, k_scale, q_pos, seq_len, s.T, s.N, s.m, qi0, scores, fm, s.top_k, seg_ws)
  if (k_fmt == FMT_MXFP4) {
    if (q_fmt == FMT_MXFP8) DSA_MXF(FMT_MXFP4, true, 8);
    DSA_MXF(FMT_MXFP4, false, 8);
  }
  if (q_fmt == FMT_MXFP8) DSA_MXF(FMT_MXFP8, true, 16);
  DSA_MXF(FMT_MXFP8, false, 16);
#undef DSA_MXF
}

}  // namespace dsa
