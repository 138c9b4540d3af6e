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
  uint32_t bin, above;
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

// Exact radix select over one whole row of n > k visible scores, re-read from global memory
// (L2) on every pass; one 1024-thread workgroup. The bits every visible key shares (block-wide
// AND / OR) are skipped, so the first digit already splits the row: scores of one row typically
// share sign and exponent, and digits over those bits would put the whole row into a handful of
// bins and serialise the LDS atomics. Used for long rows only when the filtered path below
// cannot prove its candidate set complete. The selection is written in ascending index order,
// as on every other path, so a row's result does not depend on the timing of the waves.
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
  uint32_t need = (uint32_t)k;
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
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;
  // the selection in ascending index order, one block of kTkThreads entries at a time: one
  // block scan of the packed (greater, equal) flags gives each entry its output slot; entries
  // equal to tau are taken while fewer than need of them precede (lowest indices first)
  uint32_t pos = 0, eq_run = 0;
  for (int base = 0; base < n; base += kTkThreads) {  // block-uniform trip count
    const int i = base + tid;
    const uint32_t u = i < n ? key(i) : 0u;
    const uint32_t gt = (i < n && u > tau) ? 1u : 0u, eq = (i < n && u == tau) ? 1u : 0u;
    const uint32_t v = (gt << 16) | eq;  // at most kTkThreads of each: 16 bits hold the counts
    const uint32_t inc = wave_incl_scan(v);
    if (lane == 63) sh.wave_tot[wv] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t t = sh.wave_tot[w];
      before += w < wv ? t : 0u;
      tot += t;
    }
    __syncthreads();  // sh.wave_tot is rewritten by the next block
    const uint32_t ex = before + inc - v;
    const uint32_t gt_before = ex >> 16, eq_before = eq_run + (ex & 0xffffu);
    const uint32_t taken_before = min(eq_before, need) - min(eq_run, need);
    if (gt || (eq && eq_before < need)) out[pos + gt_before + taken_before] = i;
    const uint32_t eq_tot = tot & 0xffffu;
    pos += (tot >> 16) + (min(eq_run + eq_tot, need) - min(eq_run, need));
    eq_run += eq_tot;
  }
}

// ------------------------------------------------------------------------------------------
// Rows longer than kLdsMaxN (CSA decode: 262144 blocks per row): the whole GPU works on a
// handful of rows through per-chunk candidate segments (select.h chunk_filter):
//  * the segments come from topk_long_filter, one 512-thread workgroup per kLongChunk
//    contiguous entries of a row, or straight from the decode indexer's epilogue, which runs the
//    same filter on the scores it just computed (then a "chunk" is the set of keys one indexer
//    workgroup scored, and segment order is not index order);
//  * topk_long_select, one 1024-thread workgroup per row: the segments are concatenated in
//    chunk order into LDS and the top k of the candidates are selected. With contiguous chunks
//    candidate order is index order, so ties at tau go to the lowest indices as everywhere
//    else; with the indexer's segments the fast path is taken only when no tau-valued entry
//    has to be left out. The result is exact whenever tau >= tau_g for every chunk. When that
//    check fails, or a segment overflowed, or there are more candidates than the registers hold,
//    the workgroup falls back to the exact whole-row radix select above, over the row's scores.
// ------------------------------------------------------------------------------------------
constexpr int kFiltThreads = 512;               // 8 entries per thread
constexpr int kLongCap = 8 * kTkThreads;        // candidates ranked in registers by the select
constexpr int kLongMaxChunks = 4 * kTkThreads;  // chunks per row the select kernel can scan

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
  if (c0 >= n) return;  // past the visible chunks the select kernel reads
  const int cn = min(kLongChunk, n - c0);
  const int nvt = max(0, min(PER, cn - PER * tid));
  const int e0 = c0 + PER * tid;
  chunk_filter<NW, PER>(key, nvt, n, k, sh, ws + row * long_row_bytes(G), G, g,
                        [&](int j) { return e0 + j; });
}

__global__ __launch_bounds__(kTkThreads) void topk_long_select(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ seq_len, int T, int64_t qi0, int N, int m, int k, int G,
    int stride, int ordered, const uint8_t* __restrict__ ws, int32_t* __restrict__ idx) {
  // stride: entries per chunk of the chunks' first visible-range cut (chunk g holds visible
  // entries iff g * stride < n); ordered: segment order is index order
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
  const int Gn = min(G, (n + stride - 1) / stride);  // chunks holding visible entries
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
      // block-uniform: the candidate set holds the row's top k (and, for segments out of index
      // order, no tau-valued entry is left out, so no lowest-index choice is needed)
      if (tau >= f.tau_max && (ordered || cnt_eq == need)) {
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
// topk_stream: rows of up to 32768 entries (prefill), one 256-thread workgroup (4 waves) per
// row and several rows per CU; nothing of the row is held in registers, so the per-key work is
// a compare and, for the few candidates, an LDS store:
//  1. lo: a sample of 2048 keys (64 runs of 32 consecutive entries, one cache line each, spread
//     evenly over the row) and its r-th largest,
//     r = mu + 4 sigma + 8 with mu = 2048 k / n (select.h block_threshold); rows of at most
//     kStCap entries skip it (lo = the smallest key: every entry is a candidate).
//  2. One streaming pass: wave w scans the contiguous quarter w of the row, 6 loads of 16
//     bytes per lane in flight, and appends every score >= lo (order key and index) to its own
//     LDS segment in index order (a DPP prefix sum of the lanes' counts per 256 entries).
//  3. If every segment fits and together they hold at least k entries, they hold every one of
//     the top k: the threshold (tau, need) and the ranks come from the candidates alone (the
//     concatenated segments are in index order, so ties at tau go to the lowest indices), and
//     the selection is written in ascending index order.
//  4. Otherwise (an unlucky or adversarial sample, or heavy ties): stream_exact, a radix
//     select with 8-bit digits over the bits that vary in the row, each pass re-reading the row
//     from L2, then a counting pass and an ordered writing pass.
// ------------------------------------------------------------------------------------------
constexpr int kStThreads = 256;
constexpr int kStWaves = kStThreads / 64;
constexpr int kStSeg = 1024;                 // candidate slots per wave
constexpr int kStCap = kStWaves * kStSeg;    // 4096
constexpr int kStPC = kStCap / kStThreads;   // candidates per thread in the exact step
constexpr int kStSample = 2048;
constexpr int kStUnroll = 6;                 // 256-entry blocks a wave loads ahead

// Candidate indices are row-relative and below kLdsMaxN, so 16 bits hold them. The selection
// state shares its memory with the candidate keys: the sample's selection ends (barrier) before
// the streaming pass appends keys, and the exact step copies every key to registers (barrier)
// before its selection starts; the fallback's 256-bin histogram is the selection's first one.
// About 24 KB and 73 VGPRs: six rows per CU.
static_assert(kLdsMaxN <= 65536, "16-bit candidate indices");
struct __attribute__((aligned(16))) StShared {
  union {
    SelShared<kStWaves> sel;
    uint32_t ckey[kStCap];
  };
  uint16_t cidx[kStCap];
  uint32_t wcnt[kStWaves], weq[kStWaves];
  uint32_t bin, above, cnt;
  __device__ uint32_t* hist() { return &sel.hist[0][0]; }
};

__device__ __forceinline__ float key_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Entries [i0, i0 + 4) of row s as four floats (clamped to the row; the caller masks i >= n).
__device__ __forceinline__ f32x4_t load4(const float* __restrict__ s, int i0, int n, bool vec) {
  if (vec) return *reinterpret_cast<const f32x4_t*>(s + min(i0, (n - 1) & ~3));
  return f32x4_t{s[min(i0, n - 1)], s[min(i0 + 1, n - 1)], s[min(i0 + 2, n - 1)],
                 s[min(i0 + 3, n - 1)]};
}

// Keys per wave quarter: a multiple of 256, so every wave's blocks are whole 16-byte loads.
__device__ __forceinline__ int st_quarter(int n) { return ((n + 1023) >> 10) << 8; }

// f(i0, v) for every 256-entry block of this wave's range [r0, r1), in index order: lane l gets
// entries i0 = block + 4 l .. i0 + 3 (the caller masks i >= r1), with kStUnroll 16-byte loads
// per lane in flight.
template <typename F>
__device__ __forceinline__ void blocks_of(int b0, int r1, const f32x4_t (&v)[kStUnroll], F& f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kStUnroll; ++u) {
    if (b0 + 256 * u >= r1) break;  // wave-uniform
    f(b0 + 256 * u + 4 * lane, v[u]);
  }
}
__device__ __forceinline__ void load_blocks(const float* __restrict__ s, int n, bool vec, int b0,
                                            f32x4_t (&v)[kStUnroll]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kStUnroll; ++u) v[u] = load4(s, b0 + 256 * u + 4 * lane, n, vec);
}
template <typename F>
__device__ __forceinline__ void for_blocks(const float* __restrict__ s, int n, bool vec, int r0,
                                           int r1, F&& f) {
  for (int b0 = r0; b0 < r1; b0 += 256 * kStUnroll) {
    f32x4_t v[kStUnroll];
    load_blocks(s, n, vec, b0, v);
    blocks_of(b0, r1, v, f);
  }
}
// for_blocks with the first kStUnroll blocks already loaded (first, loaded at r0)
template <typename F>
__device__ __forceinline__ void for_blocks_from(const float* __restrict__ s, int n, bool vec,
                                                int r0, int r1, const f32x4_t (&first)[kStUnroll],
                                                F&& f) {
  if (r0 >= r1) return;
  blocks_of(r0, r1, first, f);
  for_blocks(s, n, vec, r0 + 256 * kStUnroll, r1, f);
}

// Exact whole-row select (step 4): tau and need by radix passes over the row re-read from L2,
// then the selection in ascending index order.
__device__ void stream_exact(const float* __restrict__ s, int n, int k, bool vec,
                             int32_t* __restrict__ out, StShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Lq = st_quarter(n), r0 = wv * Lq, r1 = min(n, r0 + Lq);
  uint32_t kand = 0xffffffffu, kor = 0u;
  for_blocks(s, n, vec, r0, r1, [&](int i0, const f32x4_t& v) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (i0 + j < r1) {
        const uint32_t u = order_key(v[j]);
        kand &= u;
        kor |= u;
      }
  });
  wave_and_or(kand, kor);
  if (lane == 0) {
    sh.sel.red_and[wv] = kand;
    sh.sel.red_or[wv] = kor;
  }
  __syncthreads();
  kand = 0xffffffffu;
  kor = 0u;
#pragma unroll
  for (int w = 0; w < kStWaves; ++w) {
    kand &= sh.sel.red_and[w];
    kor |= sh.sel.red_or[w];
  }
  const uint32_t diff = kand ^ kor;
  uint32_t prefix = kand, pmask = 0xffffffffu, need = (uint32_t)k;
  if (diff != 0) {
    const int top = 31 - __clz(diff);
    pmask = top == 31 ? 0u : (~0u << (top + 1));
    prefix = kand & pmask;
    for (int hi = top; hi >= 0; hi -= 8) {
      const int width = hi + 1 < 8 ? hi + 1 : 8;
      const int shift = hi + 1 - width;
      const uint32_t bmask = (1u << width) - 1u;
      sh.hist()[tid] = 0u;
      __syncthreads();
      for_blocks(s, n, vec, r0, r1, [&](int i0, const f32x4_t& v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t u = order_key(v[j]);
          if (i0 + j < r1 && (u & pmask) == prefix) atomicAdd(&sh.hist()[(u >> shift) & bmask], 1u);
        }
      });
      __syncthreads();
      // thread t holds bin 255 - t: an inclusive scan from the top finds the need-th key's bin
      const uint32_t c = sh.hist()[255 - tid];
      const uint32_t inc = wave_incl_scan(c);
      if (lane == 63) sh.sel.wtot[wv] = inc;
      __syncthreads();
      uint32_t before = 0;
#pragma unroll
      for (int w = 0; w < kStWaves; ++w) before += w < wv ? sh.sel.wtot[w] : 0u;
      const uint32_t hi_inc = before + inc;
      if (hi_inc >= need && hi_inc - c < need) {
        sh.bin = 255u - (uint32_t)tid;
        sh.above = hi_inc - c;
        sh.cnt = c;
      }
      __syncthreads();
      prefix |= sh.bin << shift;
      need -= sh.above;
      pmask |= bmask << shift;
      __syncthreads();  // sh.bin / sh.hist are rewritten by the next pass
    }
  }
  const uint32_t tau = prefix;
  // counts per wave quarter: entries above tau, entries equal to tau
  uint32_t gt = 0, eq = 0;
  for_blocks(s, n, vec, r0, r1, [&](int i0, const f32x4_t& v) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = order_key(v[j]);
      gt += (i0 + j < r1 && u > tau) ? 1u : 0u;
      eq += (i0 + j < r1 && u == tau) ? 1u : 0u;
    }
  });
  gt = wave_incl_scan(gt);
  eq = wave_incl_scan(eq);
  if (lane == 63) {
    sh.wcnt[wv] = gt;
    sh.weq[wv] = eq;
  }
  __syncthreads();
  uint32_t pos = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < kStWaves; ++w) {
    if (w < wv) {
      const uint32_t e = sh.weq[w];
      pos += sh.wcnt[w] + (e < need - min(need, eq_before) ? e : need - min(need, eq_before));
      eq_before += e;
    }
  }
  // ordered writes: every entry above tau, and tau-valued ones while fewer than need are taken
  for_blocks(s, n, vec, r0, r1, [&](int i0, const f32x4_t& v) {
    uint32_t take = 0, c = 0, e = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = order_key(v[j]);
      const bool in = i0 + j < r1;
      const bool isgt = in && u > tau, iseq = in && u == tau;
      take |= (uint32_t)isgt << j;
      take |= (uint32_t)iseq << (8 + j);
      e += iseq ? 1u : 0u;
    }
    const uint32_t e_inc = wave_incl_scan(e);
    uint32_t e_run = eq_before + e_inc - e;  // tau-valued entries of the row before this lane's
    uint32_t sel = take & 0xfu;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((take >> (8 + j)) & 1u) {
        if (e_run < need) sel |= 1u << j;
        ++e_run;
      }
    c = (uint32_t)__popc(sel);
    const uint32_t c_inc = wave_incl_scan(c);
    uint32_t o = pos + c_inc - c;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((sel >> j) & 1u) out[o++] = i0 + j;
    pos += (uint32_t)__builtin_amdgcn_readlane((int)c_inc, 63);
    eq_before += (uint32_t)__builtin_amdgcn_readlane((int)e_inc, 63);
  });
}

__global__ __launch_bounds__(kStThreads) void topk_stream(
    const float* __restrict__ scores, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ seq_len, int T, int64_t qi0, int N, int m, int k,
    int32_t* __restrict__ idx) {
  __shared__ StShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = blockIdx.x;
  const int n = n_visible(q_pos[qi0 + row], m, N, seq_len, (int)((qi0 + row) / T));
  int32_t* __restrict__ out = idx + row * (int64_t)k;
  const float* __restrict__ s = scores + row * (int64_t)N;
  if (n <= k) {
    for (int i = tid; i < k; i += kStThreads) out[i] = i < n ? i : -1;
    return;
  }
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(s) & 15) == 0;
  const int Lq = st_quarter(n), r0 = wv * Lq, r1 = min(n, r0 + Lq);
  // the streaming pass's first loads go out with the sample's, so their latency overlaps it
  f32x4_t first[kStUnroll];
  // 1. lo from the sample
  uint32_t lo = 0u;
  if (n <= kStCap) load_blocks(s, n, vec, r0, first);
  if (n > kStCap) {
    // 64 runs of 32 consecutive entries (one 128-byte line each, 8 KB in all) spread evenly
    // over the row; thread t reads 8 entries of run t / 4
    uint32_t sk[kStSample / kStThreads];
    static_assert(kStSample / kStThreads == 8, "two 16-byte loads per thread");
    const int run0 = (int)(((int64_t)(tid >> 2) * n) / 64) & ~31;
    const f32x4_t sv0 = load4(s, run0 + 8 * (tid & 3), n, vec);
    const f32x4_t sv1 = load4(s, run0 + 8 * (tid & 3) + 4, n, vec);
    load_blocks(s, n, vec, r0, first);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sk[j] = order_key(sv0[j]);
      sk[4 + j] = order_key(sv1[j]);
    }
    const float p = (float)k / (float)n;
    const float mu = p * (float)kStSample;
    const float rf = mu + 4.f * __builtin_sqrtf(mu * (1.f - p)) + 8.f;
    if (rf < (float)kStSample) {
      uint32_t need_s, eq_s;
      block_threshold<kStWaves, kStSample / kStThreads>(sk, kStSample / kStThreads,
                                                        (uint32_t)rf, sh.sel, lo, need_s, eq_s,
                                                        (uint32_t)kStSample);
    }
  }
  __syncthreads();  // the sample's selection state is about to hold candidate keys
  // keys up to order_key(-inf) are -inf or NaN images: lo there means "every entry"
  const float lo_f = lo <= 0x007fffffu ? -__builtin_huge_valf() : key_to_float(lo);
  // 2. the streaming pass: wave wv appends the candidates of its quarter in index order
  uint32_t wc = 0;
  uint32_t* ck = sh.ckey + wv * kStSeg;
  uint16_t* ci = sh.cidx + wv * kStSeg;
  for_blocks_from(s, n, vec, r0, r1, first, [&](int i0, const f32x4_t& v) {
    uint32_t bits = 0, c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool take = i0 + j < r1 && v[j] >= lo_f;
      bits |= (uint32_t)take << j;
      c += take ? 1u : 0u;
    }
    if (__ballot(c != 0) == 0) return;  // wave-uniform: no candidate in this block
    const uint32_t inc = wave_incl_scan(c);
    uint32_t o = wc + inc - c;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((bits >> j) & 1u) {
        if (o < (uint32_t)kStSeg) {
          ck[o] = order_key(v[j]);
          ci[o] = (uint16_t)(i0 + j);
        }
        ++o;
      }
    wc += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  });
  if (lane == 0) sh.wcnt[wv] = wc;
  __syncthreads();
  uint32_t total = 0, over = 0, off[kStWaves];
#pragma unroll
  for (int w = 0; w < kStWaves; ++w) {
    off[w] = total;
    total += sh.wcnt[w];
    over |= sh.wcnt[w] > (uint32_t)kStSeg ? 1u : 0u;
  }
  if (over == 0u && total >= (uint32_t)k) {  // block-uniform
    // 3. candidate c (concatenated order = index order) lives in wave segment w at c - off[w]
    uint32_t kc[kStPC];
    int phys[kStPC];
    const int c0 = kStPC * tid;
    const int nvc = max(0, min(kStPC, (int)total - c0));
#pragma unroll
    for (int j = 0; j < kStPC; ++j) {
      const uint32_t c = (uint32_t)min(c0 + j, (int)total - 1);
      int w = 0;
#pragma unroll
      for (int x = 1; x < kStWaves; ++x) w += c >= off[x] ? 1 : 0;
      phys[j] = w * kStSeg + (int)(c - off[w]);
      kc[j] = sh.ckey[phys[j]];
    }
    uint32_t tau, need, cnt_eq;
    __syncthreads();  // every candidate key is in registers before the selection state reuses them
    block_threshold<kStWaves, kStPC>(kc, nvc, (uint32_t)k, sh.sel, tau, need, cnt_eq, total);
    uint32_t base, take_eq, nsel;
    block_ranks<kStWaves, kStPC>(kc, nvc, tau, need, sh.sel, base, take_eq, nsel);
    const auto sel = select_mask<kStPC>(kc, nvc, tau, take_eq);
#pragma unroll
    for (int j = 0; j < kStPC; ++j)
      if ((sel >> j) & 1) out[base + sel_rank(sel, j)] = (int32_t)sh.cidx[phys[j]];
    return;
  }
  __syncthreads();  // the fallback rewrites the shared state
  stream_exact(s, n, k, vec, out, sh);
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
  if (s.N <= kLdsMaxN)
    return launch(topk_stream, grid, kStThreads, 0, st, scores, q_pos, seq_len, s.T, qi0, s.N,
                  s.m, s.top_k, idx);
  const int G = (s.N + kLongChunk - 1) / kLongChunk;
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (hipError_t e = launch(topk_long_filter, dim3((unsigned)G, (unsigned)nrows), kFiltThreads,
                            0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m, s.top_k, G, w))
    return e;
  return launch(topk_long_select, grid, kTkThreads, 0, st, scores, q_pos, seq_len, s.T, qi0, s.N, s.m,
                s.top_k, G, kLongChunk, 1, static_cast<const uint8_t*>(w), idx);
}

hipError_t launch_topk_segments(const Shape& s, int64_t qi0, int64_t nrows, const float* scores,
                                const int32_t* q_pos, const int32_t* seq_len, int stride,
                                int32_t* idx, const void* ws, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  const int G = (s.N + kLongChunk - 1) / kLongChunk;
  return launch(topk_long_select, dim3((unsigned)nrows), kTkThreads, 0, st, scores, q_pos, seq_len,
                s.T, qi0, s.N, s.m, s.top_k, G, stride, 0, static_cast<const uint8_t*>(ws), idx);
}

}  // namespace dsa
