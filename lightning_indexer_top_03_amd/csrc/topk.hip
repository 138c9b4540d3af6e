// topk.hip - per-query top-k selection on gfx950.
//
// ("DeepSeek-V3.2 sparse-attention principle and TPU adaptation", s1.3 fine-grained sparse
// attention: keep only the entries of the top-k index scores; s3 step 3: when the visible
// context is no longer than k every token is kept.)
//
// Radix select on an order-preserving uint32 image of the fp32 scores, one workgroup per query
// row: histogram passes over 12-bit digits of the bits that vary within the row narrow the k-th
// largest key down to one exact value tau and the count `need` of tau-valued entries to take;
// a final pass emits every entry above tau and the `need` LOWEST-index entries equal to tau (a
// block-wide ordered scan, only when tau is tied), so the set equals the first k of a stable
// descending sort.
// Rows whose n_vis <= k take every visible entry. Unused slots are -1.
#include "common.h"
#include "launch.h"
#include "select.h"

#include <mutex>

namespace dsa {

namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kDigit = 12;               // bits per radix digit
constexpr int kBins = 1 << kDigit;       // 4096 bins, 4 per thread
constexpr int kLdsMaxN = 32768;          // rows up to this many entries are staged in LDS

struct __attribute__((aligned(16))) TkShared {
  uint32_t hist[kBins];
  uint32_t wave_tot[kTkWaves];
  uint32_t red_and[kTkWaves], red_or[kTkWaves];
  uint32_t bin, above, pos, taken_eq;
};

// Block-wide search of the bin holding the need-th largest element counting from the top:
// thread t owns bins 4t .. 4t+3; a suffix scan over threads (shuffles within a wave, wave totals
// through LDS) finds the owning thread, which writes the bin and the count strictly above it.
// The bins hold at least `need` elements, so exactly one thread hits. Ends with a barrier.
__device__ __forceinline__ void find_bin(TkShared& sh, uint32_t need) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const u32x4_t c = *reinterpret_cast<const u32x4_t*>(&sh.hist[4 * tid]);
  const uint32_t local = c[0] + c[1] + c[2] + c[3];
  uint32_t suf = local;  // inclusive suffix over lanes lane..63
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  if (lane == 0) sh.wave_tot[wv] = suf;
  __syncthreads();
  for (int w = wv + 1; w < kTkWaves; ++w) suf += sh.wave_tot[w];
  const uint32_t excl = suf - local;
  if (suf >= need && excl < need) {
    uint32_t a = excl;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (a + c[j] >= need) {
        sh.bin = (uint32_t)(4 * tid + j);
        sh.above = a;
        break;
      }
      a += c[j];
    }
  }
  __syncthreads();
}

// Append index i to out for every lane with take set: one LDS atomic per wave (the ballot's
// popcount), each lane then writes at base + its rank among the taking lanes.
__device__ __forceinline__ void append(bool take, int i, uint32_t* pos, int32_t* __restrict__ out) {
  const unsigned long long bal = __ballot(take);
  if (bal == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)bal) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(pos, (uint32_t)__popcll(bal));
  base = __shfl(base, leader, 64);
  if (take) out[base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull))] = i;
}

// One workgroup per query row. LDS_KEYS: the row's order keys are staged in LDS (rows of at
// most kLdsMaxN entries); otherwise every pass re-reads the scores from global memory (L2).
// The bits every visible key shares (block-wide AND / OR) are skipped, so the first digit
// already splits the row: scores of one row typically share sign and exponent, and digits over
// those bits would put the whole row into a handful of bins and serialise the LDS atomics.
template <bool LDS_KEYS>
__global__ __launch_bounds__(kTkThreads) void topk_radix_row(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int64_t qi0, int N,
    int m, int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t skey[];  // [n] when LDS_KEYS
  __shared__ TkShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = blockIdx.x;
  const int n = n_visible(q_pos[qi0 + row], m, N);
  int32_t* __restrict__ out = idx + row * (int64_t)k;
  const float* __restrict__ s = scores + row * (int64_t)N;
  auto key = [&](int i) -> uint32_t {
    if constexpr (LDS_KEYS)
      return skey[i];
    else
      return order_key(s[i]);
  };

  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t kand = 0xffffffffu, kor = 0u;
  if constexpr (LDS_KEYS) {
    // every load in flight before the first use (clamped addresses, no branches): a loop over
    // the runtime n would wait for each load in turn
    constexpr int kPer = kLdsMaxN / kTkThreads;
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (j * kTkThreads < n) v[j] = s[min(tid + j * kTkThreads, n - 1)];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * kTkThreads;
      if (i < n) {
        const uint32_t u = order_key(v[j]);
        skey[i] = u;
        kand &= u;
        kor |= u;
      }
    }
  } else {
    for (int base = 0; base < n; base += 8 * kTkThreads) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = s[min(base + tid + j * kTkThreads, n - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (base + tid + j * kTkThreads < n) {
          const uint32_t u = order_key(v[j]);
          kand &= u;
          kor |= u;
        }
      }
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
  if (tid == 0) {
    sh.pos = 0;
    sh.taken_eq = 0;
  }
  __syncthreads();
  kand = 0xffffffffu;
  kor = 0u;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    kand &= sh.red_and[w];
    kor |= sh.red_or[w];
  }
  const uint32_t diff = kand ^ kor;  // bits that vary across the visible row
  uint32_t prefix = kand;            // every bit is shared when diff == 0
  uint32_t need = (uint32_t)k, cnt_eq = (uint32_t)n;
  if (diff != 0) {
    const int top = 31 - __clz(diff);  // highest varying bit
    uint32_t pmask = top == 31 ? 0u : (~0u << (top + 1));
    prefix = kand & pmask;
    for (int hi = top; hi >= 0; hi -= kDigit) {
      const int width = hi + 1 < kDigit ? hi + 1 : kDigit;
      const int shift = hi + 1 - width;
      const uint32_t bmask = (1u << width) - 1u;
      *reinterpret_cast<u32x4_t*>(&sh.hist[4 * tid]) = u32x4_t{0u, 0u, 0u, 0u};
      __syncthreads();
      for (int i = tid; i < n; i += kTkThreads) {
        const uint32_t u = key(i);
        if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & bmask], 1u);
      }
      __syncthreads();
      find_bin(sh, need);
      const uint32_t bin = sh.bin;
      prefix |= bin << shift;
      need -= sh.above;
      pmask |= bmask << shift;
      cnt_eq = sh.hist[bin];
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;
  if (cnt_eq == need) {
    for (int base = 0; base < n; base += kTkThreads) {  // block-uniform trip count
      const int i = base + tid;
      append(i < n && key(i) >= tau, i, &sh.pos, out);
    }
    return;
  }
  // tau tied beyond what is needed: keys above tau in any order, tau-valued ones by index
  for (int base = 0; base < n; base += kTkThreads) {
    const int i = base + tid;
    const uint32_t u = i < n ? key(i) : 0u;
    append(i < n && u > tau, i, &sh.pos, out);
    const bool eq = i < n && u == tau;
    const unsigned long long bal = __ballot(eq);
    if (lane == 0) sh.wave_tot[wv] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = sh.taken_eq;
    for (int w = 0; w < wv; ++w) before += sh.wave_tot[w];
    before += (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    append(eq && before < need, i, &sh.pos, out);
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kTkWaves; ++w) tot += sh.wave_tot[w];
      sh.taken_eq += tot;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// topk_radix_reg<PER>: rows of at most 1024*PER visible entries, one 1024-thread workgroup per
// row. Thread t owns the contiguous entries PER*t .. PER*t+PER-1 and keeps their order keys in
// registers for the whole kernel; the threshold and the ranks come from select.h
// (block_threshold: 8-bit digits into a shared LDS histogram, one barrier per pass, small
// boundary bins ranked directly; block_ranks: one block prefix scan). The selection is written
// in ascending index order, so the output order is deterministic.
// ------------------------------------------------------------------------------------------
template <int PER>
__global__ __launch_bounds__(kTkThreads) void topk_radix_reg(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int64_t qi0, int N,
    int m, int k, int32_t* __restrict__ idx) {
  __shared__ SelShared<kTkWaves> sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = n_visible(q_pos[qi0 + row], m, N);
  int32_t* __restrict__ out = idx + row * (int64_t)k;
  const float* __restrict__ s = scores + row * (int64_t)N;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t key[PER];
  const int nv = load_keys<PER>(s, N, n, key);
  uint32_t tau, need, cnt_eq;
  block_threshold<kTkWaves, PER>(key, nv, (uint32_t)k, sh, tau, need, cnt_eq, (uint32_t)n);
  uint32_t base, take_eq, nsel;
  block_ranks<kTkWaves, PER>(key, nv, tau, need, sh, base, take_eq, nsel);
  const int e0 = PER * tid;
  const auto sel = select_mask<PER>(key, nv, tau, take_eq);
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if ((sel >> j) & 1) out[base + sel_rank(sel, j)] = e0 + j;
}

}  // namespace

size_t topk_ws_bytes(const Shape&, int64_t) { return 0; }

hipError_t launch_topk(const Shape& s, int64_t qi0, int64_t nrows, const float* scores,
                       const int32_t* q_pos, int32_t* idx, void*, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  // rows hold at most N visible entries
  const dim3 grid((unsigned)nrows);
  if (s.N <= 8 * kTkThreads)
    return launch(topk_radix_reg<8>, grid, kTkThreads, 0, st, scores, q_pos, qi0, s.N, s.m,
                  s.top_k, idx);
  if (s.N <= 16 * kTkThreads)
    return launch(topk_radix_reg<16>, grid, kTkThreads, 0, st, scores, q_pos, qi0, s.N, s.m,
                  s.top_k, idx);
  if (s.N <= kLdsMaxN)
    return launch(topk_radix_reg<32>, grid, kTkThreads, 0, st, scores, q_pos, qi0, s.N, s.m,
                  s.top_k, idx);
  return launch(topk_radix_row<false>, grid, kTkThreads, 0, st, scores, q_pos, qi0, s.N, s.m,
                s.top_k, idx);
}

}  // namespace dsa
