// topk.hip - per-query top-k selection on gfx950.
//
// ("DeepSeek-V3.2 sparse-attention principle and TPU adaptation", s1.3 fine-grained sparse
// attention: keep only the entries of the top-k index scores; s3 step 3: when the visible
// context is no longer than k every token is kept.)
//
// Radix select on an order-preserving uint32 image of the fp32 scores, one workgroup per query
// row: three histogram passes (bits 31..21, 20..10, 9..0) narrow the k-th largest key down to
// one exact value tau and the count `need` of tau-valued entries to take; a final pass emits
// every entry above tau and the `need` LOWEST-index entries equal to tau (a block-wide ordered
// scan, only when tau is tied), so the set equals the first k of a stable descending sort.
// Rows whose n_vis <= k take every visible entry. Unused slots are -1.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kBins = 2048;

struct TkShared {
  uint32_t hist[kBins];
  uint32_t wave_cnt[kTkWaves];
  uint32_t bin, above, pos, taken_eq;
};

// Find, among the bins of hist, the one holding the need-th largest element counting from the
// top; the lane that finds it writes the bin and the count strictly above it to LDS. Run by
// wave 0 only. The bins hold at least `need` elements in total, so exactly one lane hits.
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nbins, uint32_t need,
                                         uint32_t* bin_out, uint32_t* above_out) {
  const int lane = threadIdx.x & 63;
  const int per = nbins / 64;  // bins per lane; lane 63 owns the highest bins
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[lane * per + i];
  // inclusive suffix sum over lanes: lane L holds the count of lanes L..63
  uint32_t suf = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  if (suf >= need && suf - local < need) {
    uint32_t above = suf - local;
    for (int i = per - 1; i >= 0; --i) {
      uint32_t c = hist[lane * per + i];
      if (above + c >= need) {
        *bin_out = (uint32_t)(lane * per + i);
        *above_out = above;
        break;
      }
      above += c;
    }
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_radix_row(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int64_t qi0, int N,
    int m, int k, int32_t* __restrict__ idx) {
  __shared__ TkShared sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = n_visible(q_pos[qi0 + row], m, N);
  int32_t* __restrict__ out = idx + row * (int64_t)k;
  const float* __restrict__ s = scores + row * (int64_t)N;

  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }

  // ---- radix passes: (shift, bits) = (21, 11), (10, 11), (0, 10) ----
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k, cnt_eq = 0;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t bmask = (1u << widths[pass]) - 1u;
    for (int i = tid; i < kBins; i += kTkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTkThreads) {
      uint32_t u = order_key(s[i]);
      if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & bmask], 1u);
    }
    __syncthreads();
    if (tid < 64) find_bin(sh.hist, kBins, need, &sh.bin, &sh.above);
    __syncthreads();
    const uint32_t bin = sh.bin;
    prefix |= bin << shift;
    need -= sh.above;
    pmask |= bmask << shift;
    cnt_eq = sh.hist[bin];
    __syncthreads();
  }
  const uint32_t tau = prefix;

  // ---- emission ----
  if (tid == 0) {
    sh.pos = 0;
    sh.taken_eq = 0;
  }
  __syncthreads();
  if (cnt_eq == need) {
    for (int i = tid; i < n; i += kTkThreads) {
      uint32_t u = order_key(s[i]);
      if (u >= tau) out[atomicAdd(&sh.pos, 1u)] = i;
    }
    return;
  }
  // tau is tied beyond what is needed: entries above tau in any order, the tau-valued ones in
  // ascending index order until `need` are taken.
  const int lane = tid & 63, wv = tid >> 6;
  for (int base = 0; base < n; base += kTkThreads) {
    const int i = base + tid;
    uint32_t u = i < n ? order_key(s[i]) : 0u;
    if (i < n && u > tau) out[atomicAdd(&sh.pos, 1u)] = i;
    const bool eq = i < n && u == tau;
    const unsigned long long bal = __ballot(eq);
    if (lane == 0) sh.wave_cnt[wv] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = sh.taken_eq;
    for (int j = 0; j < wv; ++j) before += sh.wave_cnt[j];
    before += (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (eq && before < need) out[atomicAdd(&sh.pos, 1u)] = i;
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int j = 0; j < kTkWaves; ++j) tot += sh.wave_cnt[j];
      sh.taken_eq += tot;
    }
    __syncthreads();
  }
}

// LDS-resident variant for rows of at most kLdsMaxN entries: the row's keys are staged in LDS
// once and every pass reads them from there. The bits every visible key shares (a block-wide
// AND / OR) are skipped, so the first 11-bit digit already splits the row (scores of one row
// typically share sign and exponent; digits over those bits would put the whole row into a
// handful of bins and serialise the LDS atomics).
constexpr int kLdsMaxN = 32768;

__global__ __launch_bounds__(kTkThreads) void topk_radix_row_lds(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos, int64_t qi0, int N,
    int m, int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t skey[];  // [n]
  __shared__ TkShared sh;
  __shared__ uint32_t red_and[kTkWaves], red_or[kTkWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = blockIdx.x;
  const int n = n_visible(q_pos[qi0 + row], m, N);
  int32_t* __restrict__ out = idx + row * (int64_t)k;
  const float* __restrict__ s = scores + row * (int64_t)N;

  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t kand = 0xffffffffu, kor = 0u;
  for (int i = tid; i < n; i += kTkThreads) {
    const uint32_t u = order_key(s[i]);
    skey[i] = u;
    kand &= u;
    kor |= u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kand &= __shfl_xor(kand, o, 64);
    kor |= __shfl_xor(kor, o, 64);
  }
  if (lane == 0) {
    red_and[wv] = kand;
    red_or[wv] = kor;
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
    kand &= red_and[w];
    kor |= red_or[w];
  }
  const uint32_t diff = kand ^ kor;  // bits that vary across the visible row
  uint32_t prefix = kand;            // all bits equal when diff == 0
  uint32_t need = (uint32_t)k, cnt_eq = (uint32_t)n;
  if (diff != 0) {
    const int top = 31 - __clz(diff);  // highest varying bit
    uint32_t pmask = top == 31 ? 0u : (~0u << (top + 1));
    prefix = kand & pmask;
    for (int hi = top; hi >= 0; hi -= 11) {
      const int width = hi + 1 < 11 ? hi + 1 : 11;
      const int shift = hi + 1 - width;
      const uint32_t bmask = (1u << width) - 1u;
      for (int i = tid; i < kBins; i += kTkThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kTkThreads) {
        const uint32_t u = skey[i];
        if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & bmask], 1u);
      }
      __syncthreads();
      if (tid < 64) find_bin(sh.hist, kBins, need, &sh.bin, &sh.above);
      __syncthreads();
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
    for (int i = tid; i < n; i += kTkThreads)
      if (skey[i] >= tau) out[atomicAdd(&sh.pos, 1u)] = i;
    return;
  }
  // tau tied beyond what is needed: keys above tau in any order, tau-valued ones by index
  for (int base = 0; base < n; base += kTkThreads) {
    const int i = base + tid;
    const uint32_t u = i < n ? skey[i] : 0u;
    if (i < n && u > tau) out[atomicAdd(&sh.pos, 1u)] = i;
    const bool eq = i < n && u == tau;
    const unsigned long long bal = __ballot(eq);
    if (lane == 0) sh.wave_cnt[wv] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = sh.taken_eq;
    for (int w = 0; w < wv; ++w) before += sh.wave_cnt[w];
    before += (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
    if (eq && before < need) out[atomicAdd(&sh.pos, 1u)] = i;
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kTkWaves; ++w) tot += sh.wave_cnt[w];
      sh.taken_eq += tot;
    }
    __syncthreads();
  }
}

}  // namespace

size_t topk_ws_bytes(const Shape&, int64_t) { return 0; }

hipError_t launch_topk(const Shape& s, int64_t qi0, int64_t nrows, const float* scores,
                       const int32_t* q_pos, int32_t* idx, void*, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  // rows hold at most N visible entries
  if (s.N <= kLdsMaxN) {
    const size_t shm = sizeof(uint32_t) * (size_t)s.N;
    static bool attr_set = false;  // raise the dynamic LDS limit once (128 KB at N = 32768)
    if (!attr_set) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_radix_row_lds),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMaxN * 4);
      attr_set = true;
    }
    topk_radix_row_lds<<<dim3((unsigned)nrows), kTkThreads, shm, st>>>(scores, q_pos, qi0, s.N,
                                                                       s.m, s.top_k, idx);
  } else {
    topk_radix_row<<<dim3((unsigned)nrows), kTkThreads, 0, st>>>(scores, q_pos, qi0, s.N, s.m,
                                                                 s.top_k, idx);
  }
  return hipGetLastError();
}

}  // namespace dsa
