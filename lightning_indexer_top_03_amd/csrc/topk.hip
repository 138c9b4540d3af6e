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

// Exact radix select over one whole row of n > k visible scores, re-read from global memory
// (L2) on every pass; one 1024-thread workgroup. The bits every visible key shares (block-wide
// AND / OR) are skipped, so the first digit already splits the row: scores of one row typically
// share sign and exponent, and digits over those bits would put the whole row into a handful of
// bins and serialise the LDS atomics. Used for long rows only when the filtered path below
// cannot prove its candidate set complete.
__device__ void radix_row_exact(const float* __restrict__ s, int n, int k,
                                int32_t* __restrict__ out, TkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto key = [&](int i) -> uint32_t { return order_key(s[i]); };
  uint32_t kand = 0xffffffffu, kor = 0u;
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
// Rows longer than kLdsMaxN (CSA decode: 262144 blocks per row) in two launches, so that the
// whole GPU works on a handful of rows instead of one workgroup per row:
//  * topk_long_filter, one 512-thread workgroup per kLongChunk entries of a row: the chunk's
//    local threshold tau_g = its r-th largest key with r = ceil(2k * chunk / n) + 16 (about
//    twice the chunk's fair share of the top k), then every key >= tau_g of the chunk goes, in
//    index order, to the chunk's candidate segment (indices and keys), with its count and tau_g.
//  * topk_long_select, one 1024-thread workgroup per row: the segments are concatenated in
//    chunk order (so candidate order is index order) into LDS and the top k of the candidates
//    are selected with the same ties-to-lowest-index rule. The result is exact whenever the
//    selected threshold tau >= tau_g for every chunk: an entry that is not a candidate lies
//    below its chunk's tau_g <= tau, so every entry >= tau is a candidate. When that check
//    fails, or a segment overflowed, or there are more candidates than the registers hold, the
//    workgroup falls back to the exact whole-row radix select above.
// ------------------------------------------------------------------------------------------
constexpr int kLongChunk = 4096;                // entries per filter workgroup
constexpr int kFiltThreads = 512;               // 8 entries per thread
constexpr int kLongSeg = 1024;                  // candidate slots per chunk
constexpr int kLongCap = 8 * kTkThreads;        // candidates ranked in registers by the select
constexpr int kLongMaxChunks = 4 * kTkThreads;  // chunks per row the select kernel can scan

// Per-row workspace of the long-row path: counts[G], taus[G], cand_idx[G][kLongSeg],
// cand_key[G][kLongSeg].
__host__ __device__ inline size_t long_row_bytes(int G) {
  return (size_t)G * (8 + 8 * (size_t)kLongSeg);
}

__global__ __launch_bounds__(kFiltThreads) void topk_long_filter(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ seq_len, int T, int64_t qi0, int N, int m, int k, int G,
    uint8_t* __restrict__ ws) {
  constexpr int NW = kFiltThreads / 64, PER = kLongChunk / kFiltThreads;
  __shared__ SelShared<NW> sh;
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int c0 = g * kLongChunk;
  // the chunk's loads depend on N only (clamped to the row), so they are in flight while
  // q_pos is read; entries at or past n_vis are masked below
  uint32_t key[PER];
  load_keys<PER>(scores + row * (int64_t)N + c0, N, min(kLongChunk, N - c0), key);
  const int n = n_visible(q_pos[qi0 + row], m, N, seq_len, (int)((qi0 + row) / T));
  if (n <= k) return;  // the select kernel keeps every visible entry
  uint8_t* rws = ws + row * long_row_bytes(G);
  uint32_t* counts = reinterpret_cast<uint32_t*>(rws);
  uint32_t* taus = counts + G;
  int32_t* cidx = reinterpret_cast<int32_t*>(taus + G) + (size_t)g * kLongSeg;
  uint32_t* ckey = reinterpret_cast<uint32_t*>(taus + G) + (size_t)G * kLongSeg + (size_t)g * kLongSeg;
  if (c0 >= n) {
    if (tid == 0) {
      counts[g] = 0u;
      taus[g] = 0u;
    }
    return;
  }
  const int cn = min(kLongChunk, n - c0);
  const int nv = max(0, min(PER, cn - PER * tid));
  const int64_t r64 = (2 * (int64_t)k * cn + n - 1) / n + 16;
  uint32_t tau = 0u;  // every key >= 0: the whole chunk is a candidate
  if (r64 < cn) {
    uint32_t need, cnt_eq;
    block_threshold<NW, PER>(key, nv, (uint32_t)r64, sh, tau, need, cnt_eq, (uint32_t)cn);
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) cnt += (j < nv && key[j] >= tau) ? 1u : 0u;
  uint32_t total;
  const uint32_t pos = block_excl_scan<NW>(cnt, sh, total);
  if (total <= (uint32_t)kLongSeg) {
    uint32_t o = pos;
    const int e0 = c0 + PER * tid;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (j < nv && key[j] >= tau) {
        cidx[o] = e0 + j;
        ckey[o] = key[j];
        ++o;
      }
    }
  }
  if (tid == 0) {
    counts[g] = total <= (uint32_t)kLongSeg ? total : 0xffffffffu;  // overflow marker
    taus[g] = tau;
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_long_select(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ seq_len, int T, int64_t qi0, int N, int m, int k, int G,
    const uint8_t* __restrict__ ws, int32_t* __restrict__ idx) {
  constexpr int PER = kLongCap / kTkThreads;
  struct Fast {
    SelShared<kTkWaves> sel;
    uint32_t off[kLongMaxChunks], cnt[kLongMaxChunks];
    int32_t cidx[kLongCap];
    uint32_t ckey[kLongCap];
    uint32_t tau_max, bad;
  };
  __shared__ __attribute__((aligned(16))) char smem[sizeof(Fast) > sizeof(TkShared) ? sizeof(Fast) : sizeof(TkShared)];
  Fast& f = *reinterpret_cast<Fast*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = blockIdx.x;
  const uint8_t* rws = ws + row * long_row_bytes(G);
  const uint32_t* counts = reinterpret_cast<const uint32_t*>(rws);
  const uint32_t* taus = counts + G;
  const int32_t* sidx = reinterpret_cast<const int32_t*>(taus + G);
  const uint32_t* skey = reinterpret_cast<const uint32_t*>(taus + G) + (size_t)G * kLongSeg;
  // Everything the fast path reads is requested up front, at addresses that depend on G only
  // (in flight together with q_pos): this thread's four counts and tau_g, and for wave w the
  // first 64 slots of segments w, w + 16, w + 32, w + 48 (slots past a segment's count hold
  // stale values and are dropped).
  constexpr int U = 4;
  uint32_t c[4], t4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int gj = min(4 * tid + j, G - 1);
    c[j] = counts[gj];
    t4[j] = taus[gj];
  }
  int32_t pi[U];
  uint32_t pk[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t gj = (size_t)min(wv + kTkWaves * u, G - 1);
    pi[u] = sidx[gj * kLongSeg + lane];
    pk[u] = skey[gj * kLongSeg + lane];
  }
  const int n = n_visible(q_pos[qi0 + row], m, N, seq_len, (int)((qi0 + row) / T));
  int32_t* __restrict__ out = idx + row * (int64_t)k;
  const float* __restrict__ s = scores + row * (int64_t)N;
  if (n <= k) {
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int Gn = (n + kLongChunk - 1) / kLongChunk;  // chunks holding visible entries
  bool fast = Gn <= kLongMaxChunks;
  uint32_t total = 0;
  if (fast) {
    // thread t owns chunks 4t .. 4t+3: their counts, running offsets and the largest tau_g
    uint32_t local = 0, tmax = 0, bad = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = 4 * tid + j < Gn;
      c[j] = in ? c[j] : 0u;
      bad |= c[j] > (uint32_t)kLongSeg ? 1u : 0u;
      c[j] = c[j] > (uint32_t)kLongSeg ? 0u : c[j];
      tmax = max(tmax, in ? t4[j] : 0u);
      local += c[j];
    }
    if (tid == 0) {
      f.tau_max = 0u;
      f.bad = 0u;
    }
    const uint32_t before = block_excl_scan<kTkWaves>(local, f.sel, total);
    uint32_t o = before;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gj = 4 * tid + j;
      if (gj < Gn) {
        f.off[gj] = o;
        f.cnt[gj] = c[j];
      }
      o += c[j];
    }
    tmax = wave_max(tmax);
    bad = wave_max(bad);
    if (lane == 0) {
      atomicMax(&f.tau_max, tmax);
      atomicOr(&f.bad, bad);
    }
    __syncthreads();
    fast = f.bad == 0u && total >= (uint32_t)k && total <= (uint32_t)kLongCap;
    if (fast) {
      // concatenate the segments in chunk order: the prefetched slots first, then whatever
      // lies beyond them (segments past 64, slots past 64)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int gj = wv + kTkWaves * u;
        if (gj < Gn && (uint32_t)lane < f.cnt[gj]) {
          f.cidx[f.off[gj] + lane] = pi[u];
          f.ckey[f.off[gj] + lane] = pk[u];
        }
      }
      for (int gj = wv; gj < Gn; gj += kTkWaves) {
        const uint32_t cg = f.cnt[gj], og = f.off[gj];
        for (uint32_t i = (gj < U * kTkWaves ? 64u : 0u) + lane; i < cg; i += 64) {
          f.cidx[og + i] = sidx[(size_t)gj * kLongSeg + i];
          f.ckey[og + i] = skey[(size_t)gj * kLongSeg + i];
        }
      }
      __syncthreads();
      uint32_t key[PER];
      const int e0 = PER * tid;
      const int nv = max(0, min(PER, (int)total - e0));
#pragma unroll
      for (int j = 0; j < PER; ++j) key[j] = f.ckey[min(e0 + j, (int)total - 1)];
      uint32_t tau, need, cnt_eq;
      block_threshold<kTkWaves, PER>(key, nv, (uint32_t)k, f.sel, tau, need, cnt_eq, total);
      if (tau >= f.tau_max) {  // block-uniform: the candidate set holds the row's top k
        uint32_t base, take_eq, nsel;
        block_ranks<kTkWaves, PER>(key, nv, tau, need, f.sel, base, take_eq, nsel);
        const auto sel = select_mask<PER>(key, nv, tau, take_eq);
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if ((sel >> j) & 1) out[base + sel_rank(sel, j)] = f.cidx[e0 + j];
        return;
      }
    }
    __syncthreads();  // the fallback reuses the shared memory
  }
  radix_row_exact(s, n, k, out, *reinterpret_cast<TkShared*>(smem));
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
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ seq_len, int T, int64_t qi0, int N, int m, int k,
    int32_t* __restrict__ idx) {
  __shared__ SelShared<kTkWaves> sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int n = n_visible(q_pos[qi0 + row], m, N, seq_len, (int)((qi0 + row) / T));
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

size_t topk_ws_bytes(const Shape& s, int64_t nrows) {
  if (s.N <= kLdsMaxN) return 0;
  const int G = (s.N + kLongChunk - 1) / kLongChunk;
  return (size_t)nrows * long_row_bytes(G);
}

hipError_t launch_topk(const Shape& s, int64_t qi0, int64_t nrows, const float* scores,
                       const int32_t* q_pos, const int32_t* seq_len, int32_t* idx, void* ws,
                       hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  // rows hold at most N visible entries
  const dim3 grid((unsigned)nrows);
  if (s.N <= 8 * kTkThreads)
    return launch(topk_radix_reg<8>, grid, kTkThreads, 0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m,
                  s.top_k, idx);
  if (s.N <= 16 * kTkThreads)
    return launch(topk_radix_reg<16>, grid, kTkThreads, 0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m,
                  s.top_k, idx);
  if (s.N <= kLdsMaxN)
    return launch(topk_radix_reg<32>, grid, kTkThreads, 0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m,
                  s.top_k, idx);
  const int G = (s.N + kLongChunk - 1) / kLongChunk;
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (hipError_t e = launch(topk_long_filter, dim3((unsigned)G, (unsigned)nrows), kFiltThreads,
                            0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m, s.top_k, G, w))
    return e;
  return launch(topk_long_select, grid, kTkThreads, 0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m,
                s.top_k, G, static_cast<const uint8_t*>(w), idx);
}

}  // namespace dsa
