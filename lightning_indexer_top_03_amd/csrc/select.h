// select.h - block-wide top-k selection primitives shared by the top-k kernel and the fused
// top-k + attention path (gfx950, wave64).
//
// ("DeepSeek-V3.2 sparse-attention principle and TPU adaptation", s1.3 fine-grained sparse
// attention step 2: keep the entries of the top-k index scores; s3 step 3: keep every entry
// when the visible context is no longer than k.)
//
// A block of NW waves selects, from n visible entries of one row, the k with the largest
// scores; ties at the k-th value go to the lowest indices, so the set is the first k of a
// stable descending sort. Thread t owns the contiguous entries PER*t .. PER*t+PER-1 and keeps
// their order keys (common.h order_key) in registers.
//  * block_threshold: the bits every visible key shares (block AND / OR) are skipped; the rest
//    are resolved 8 bits at a time. Each wave counts into its own 256-bin LDS histogram (no
//    atomics shared between waves, no clearing barrier), then wave 0 sums the NW histograms and
//    finds the bin holding the need-th largest key with one DPP prefix scan over the bins in
//    descending order. Result: tau (the k-th largest key), need (how many tau-valued keys to
//    take) and the count of tau-valued keys.
//  * block_ranks: two block prefix scans give each thread the rank, in ascending index order,
//    of its first selected entry and how many of its tau-valued entries it takes.
#pragma once

#include "common.h"

namespace dsa {

// inclusive prefix sum over the 64 lanes of a wave with DPP (row shifts, then row broadcasts)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

template <int NW>
struct __attribute__((aligned(16))) SelShared {
  uint32_t hist[NW][256];
  uint32_t wtot[NW < 4 ? 4 : NW];
  uint32_t red_and[NW], red_or[NW];
  uint32_t bin, above, cnt;
};

// exclusive prefix sum over the block of v; also returns the block total. Ends with a barrier,
// so wtot can be reused at once.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SelShared<NW>& sh,
                                                    uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) sh.wtot[wv] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = sh.wtot[w];
    before += w < wv ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Threshold of the k largest among the valid keys (key[j], j < nv, of every thread), n > k.
template <int NW, int PER>
__device__ __forceinline__ void block_threshold(const uint32_t (&key)[PER], int nv, uint32_t k,
                                                SelShared<NW>& sh, uint32_t& tau,
                                                uint32_t& need, uint32_t& cnt_eq,
                                                uint32_t n) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < nv) {
      kand &= key[j];
      kor |= key[j];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kand &= __shfl_xor(kand, o, 64);
    kor |= __shfl_xor(kor, o, 64);
  }
  if (lane == 0) {
    sh.red_and[wv] = kand;
    sh.red_or[wv] = kor;
  }
  __syncthreads();
  kand = 0xffffffffu;
  kor = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kand &= sh.red_and[w];
    kor |= sh.red_or[w];
  }
  const uint32_t diff = kand ^ kor;  // bits that vary across the visible row
  uint32_t prefix = kand, pmask = 0xffffffffu;
  need = k;
  cnt_eq = n;
  if (diff != 0) {
    const int top = 31 - __clz(diff);  // highest varying bit
    pmask = top == 31 ? 0u : (~0u << (top + 1));
    prefix = kand & pmask;
    for (int hi = top; hi >= 0; hi -= 8) {
      const int width = hi + 1 < 8 ? hi + 1 : 8;
      const int shift = hi + 1 - width;
      const uint32_t bmask = (1u << width) - 1u;
      uint32_t* h = sh.hist[wv];
      // this wave's histogram: cleared and filled by the wave alone (LDS ops of a wave are
      // performed in order)
      *reinterpret_cast<u32x4_t*>(&h[4 * lane]) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (j < nv && (key[j] & pmask) == prefix) atomicAdd(&h[(key[j] >> shift) & bmask], 1u);
      __syncthreads();
      if (wv == 0) {
        // lane l: bins 255-4l .. 252-4l, highest first, summed over the NW wave histograms
        uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const u32x4_t t4 = *reinterpret_cast<const u32x4_t*>(&sh.hist[w][252 - 4 * lane]);
          c[0] += t4[3];  // bin 255 - 4l
          c[1] += t4[2];
          c[2] += t4[1];
          c[3] += t4[0];  // bin 252 - 4l
        }
        const uint32_t local = c[0] + c[1] + c[2] + c[3];
        const uint32_t inc = wave_incl_scan(local);  // keys in bins >= 252 - 4l
        const uint32_t excl = inc - local;
        if (inc >= need && excl < need) {
          uint32_t a = excl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (a + c[j] >= need) {
              sh.bin = (uint32_t)(255 - 4 * lane - j);
              sh.above = a;
              sh.cnt = c[j];
              break;
            }
            a += c[j];
          }
        }
      }
      __syncthreads();
      const uint32_t bin = sh.bin;
      prefix |= bin << shift;
      need -= sh.above;
      pmask |= bmask << shift;
      cnt_eq = sh.cnt;
      __syncthreads();  // before the next pass clears the histograms
    }
  }
  tau = prefix;
}

// Rank (in ascending index order) of this thread's first selected entry, and how many of its
// tau-valued entries it takes; selected = key > tau, or key == tau among the first `need`
// tau-valued entries of the row.
template <int NW, int PER>
__device__ __forceinline__ void block_ranks(const uint32_t (&key)[PER], int nv, uint32_t tau,
                                            uint32_t need, uint32_t cnt_eq, SelShared<NW>& sh,
                                            uint32_t& base, uint32_t& take_eq) {
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < nv) {
      n_gt += key[j] > tau ? 1u : 0u;
      n_eq += key[j] == tau ? 1u : 0u;
    }
  }
  uint32_t tot;
  take_eq = n_eq;
  if (cnt_eq != need) {  // tau tied beyond what is needed: the lowest-index ones
    const uint32_t eq_before = block_excl_scan<NW>(n_eq, sh, tot);
    take_eq = eq_before >= need ? 0u : min(n_eq, need - eq_before);
  }
  base = block_excl_scan<NW>(n_gt + take_eq, sh, tot);
}

// Load the order keys of entries PER*t .. PER*t+PER-1 of a row of n visible scores (clamped,
// branch-free addresses; 16-byte loads when the row allows), returns the valid count.
template <int PER>
__device__ __forceinline__ int load_keys(const float* __restrict__ s, int N, int n,
                                         uint32_t (&key)[PER]) {
  const int e0 = PER * (int)threadIdx.x;
  if ((N & 3) == 0 && (reinterpret_cast<uintptr_t>(s) & 15) == 0) {
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(s + min(e0 + j, ((n - 1) & ~3)));
#pragma unroll
      for (int i = 0; i < 4; ++i) key[j + i] = order_key(v[i]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) key[j] = order_key(s[min(e0 + j, n - 1)]);
  }
  return max(0, min(PER, n - e0));
}

}  // namespace dsa
