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
// their order keys (common.h order_key) in registers. The selection is latency-bound (one row
// per block, a few thousand keys), so every step is built to need as few barriers as possible:
//  * block_threshold: the bits every visible key shares (block AND / OR) are skipped; the rest
//    are resolved 8 bits at a time into a shared 256-bin LDS histogram, three of them in
//    rotation so that clearing one never needs a barrier of its own. Each bin has four
//    counters in adjacent banks (lane & 3 picks one): the keys of a row concentrate in a few
//    bins of the first digit, and same-address atomics of one instruction serialise. After
//    the pass's barrier every wave finds the bin holding the need-th largest key itself (one
//    DPP prefix scan over the bins in descending order), so there is no broadcast step: one
//    barrier per pass. Once the bin holds at most kSelCand keys, they are copied to LDS, one
//    per lane, and every wave resolves the remaining bits one at a time with a ballot per bit.
//    Result: tau (the k-th largest key), need (how many tau-valued keys to take) and the count
//    of tau-valued keys.
//  * block_ranks: one block prefix scan of the packed (greater, equal) counts gives each thread
//    the rank, in ascending index order, of its first selected entry and how many of its
//    tau-valued entries it takes.
#pragma once

#include "common.h"

#include <type_traits>

namespace dsa {

constexpr int kSelCand = 64;  // boundary-bin size below which the candidates are ranked directly
static_assert(kSelCand == 64, "one candidate per lane of a wave");

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

// AND / OR over the 64 lanes of a wave without LDS: DPP swaps within rows of 16, then the
// permlane swaps across rows (16) and halves (32); every lane ends with the wave result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ void wave_and_or(uint32_t& a, uint32_t& o) {
  a &= dpp_u32<0xb1>(a);   // quad_perm 1,0,3,2
  o |= dpp_u32<0xb1>(o);
  a &= dpp_u32<0x4e>(a);   // quad_perm 2,3,0,1
  o |= dpp_u32<0x4e>(o);
  a &= dpp_u32<0x141>(a);  // row_half_mirror
  o |= dpp_u32<0x141>(o);
  a &= dpp_u32<0x140>(a);  // row_mirror
  o |= dpp_u32<0x140>(o);
  const auto a16 = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  const auto o16 = __builtin_amdgcn_permlane16_swap(o, o, false, false);
  a = a16[0] & a16[1];
  o = o16[0] | o16[1];
  const auto a32 = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  const auto o32 = __builtin_amdgcn_permlane32_swap(o, o, false, false);
  a = a32[0] & a32[1];
  o = o32[0] | o32[1];
}

template <int NW>
struct __attribute__((aligned(16))) SelShared {
  uint32_t hist[3][256 * 4];  // pass p counts into hist[p % 3]: bin b, copy c at 4b + c
  uint32_t cand[kSelCand];
  uint32_t wtot[NW < 4 ? 4 : NW];
  uint32_t red_and[NW], red_or[NW];
  uint32_t ncand;
};

// exclusive prefix sum over the block of v; also returns the block total. One barrier: sh.wtot
// must not be written again before the next barrier.
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
  total = tot;
  return before + inc - v;
}

// Threshold of the k largest among the valid keys (key[j], j < nv, of every thread), n > k.
template <int NW, int PER>
__device__ __forceinline__ void block_threshold(const uint32_t (&key)[PER], int nv, uint32_t k,
                                                SelShared<NW>& sh, uint32_t& tau,
                                                uint32_t& need, uint32_t& cnt_eq,
                                                uint32_t n) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // the histograms of passes 0 and 1 and the candidate count start at zero (ordered before
  // their first use by the reduction's barrier); pass p clears the histogram of pass p + 2
  for (int i = tid; i < 2 * 256; i += NW * 64)
    reinterpret_cast<u32x4_t*>(&sh.hist[0][0])[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (tid == 0) sh.ncand = 0u;
  uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < nv) {
      kand &= key[j];
      kor |= key[j];
    }
  }
  wave_and_or(kand, kor);
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
    int p = 0;
    for (int hi = top; hi >= 0; hi -= 8, ++p) {
      const int width = hi + 1 < 8 ? hi + 1 : 8;
      const int shift = hi + 1 - width;
      const uint32_t bmask = (1u << width) - 1u;
      uint32_t* h = sh.hist[p % 3];
      uint32_t* hc = h + (lane & 3);
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (j < nv && (key[j] & pmask) == prefix) atomicAdd(&hc[4 * ((key[j] >> shift) & bmask)], 1u);
      __syncthreads();
      // every wave: lane l holds bins 255-4l .. 252-4l, highest first; the lane whose range
      // reaches the need-th largest key owns the boundary bin
      const u32x4_t* hb = reinterpret_cast<const u32x4_t*>(h) + (252 - 4 * lane);
      const u32x4_t b0 = hb[0], b1 = hb[1], b2 = hb[2], b3 = hb[3];  // bins 252-4l .. 255-4l
      const uint32_t c[4] = {b3[0] + b3[1] + b3[2] + b3[3], b2[0] + b2[1] + b2[2] + b2[3],
                             b1[0] + b1[1] + b1[2] + b1[3], b0[0] + b0[1] + b0[2] + b0[3]};
      const uint32_t local = c[0] + c[1] + c[2] + c[3];
      const uint32_t inc = wave_incl_scan(local);  // keys in bins >= 252 - 4l
      const uint32_t excl = inc - local;
      const int leader = (int)(__builtin_ctzll(__ballot(inc >= need && excl < need)) & 63);
      uint32_t a = excl, jf = 3, af = 0, cf = 0;
      bool done = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool hit = !done && a + c[j] >= need;
        jf = hit ? (uint32_t)j : jf;
        af = hit ? a : af;
        cf = hit ? c[j] : cf;
        done = done || hit;
        a += c[j];
      }
      const uint32_t bin = 255u - 4u * (uint32_t)leader - __builtin_amdgcn_readlane(jf, leader);
      const uint32_t above = __builtin_amdgcn_readlane(af, leader);
      const uint32_t cnt = __builtin_amdgcn_readlane(cf, leader);
      // the histogram of pass p + 2 was last read in pass p - 1, before this pass's barrier
      for (int i = tid; i < 256; i += NW * 64)
        reinterpret_cast<u32x4_t*>(&sh.hist[(p + 2) % 3][0])[i] = u32x4_t{0u, 0u, 0u, 0u};
      prefix |= bin << shift;
      need -= above;
      pmask |= bmask << shift;
      cnt_eq = cnt;
      if (shift > 0 && cnt <= (uint32_t)kSelCand) {
        // the boundary bin's keys (cnt of them, need <= cnt) decide the remaining bits: one per
        // lane, then bit by bit from the top: when at least `need` of the candidates that match
        // the bits so far have the bit set, the need-th largest has it too; otherwise those are
        // all above it
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (j < nv && (key[j] & pmask) == prefix) sh.cand[atomicAdd(&sh.ncand, 1u)] = key[j];
        __syncthreads();
        const uint32_t ci = sh.cand[lane];
        const bool valid = lane < (int)cnt;
        for (int b = shift - 1; b >= 0; --b) {
          const uint32_t trial = prefix | (1u << b);
          const uint32_t mb = pmask | ((0xffffffffu << b) & ((1u << shift) - 1u));
          const uint32_t c1 = (uint32_t)__popcll(__ballot(valid && (ci & mb) == trial));
          if (c1 >= need) {
            prefix = trial;
          } else {
            need -= c1;
          }
        }
        cnt_eq = (uint32_t)__popcll(__ballot(valid && ci == prefix));
        break;
      }
    }
  }
  tau = prefix;
}

// Rank (in ascending index order) of this thread's first selected entry, how many of its
// tau-valued entries it takes and how many entries it selects; selected = key > tau, or
// key == tau among the first `need` tau-valued entries of the row. Counts fit 16 bits (rows of
// at most 32768 entries), so one scan carries both.
template <int NW, int PER>
__device__ __forceinline__ void block_ranks(const uint32_t (&key)[PER], int nv, uint32_t tau,
                                            uint32_t need, SelShared<NW>& sh, uint32_t& base,
                                            uint32_t& take_eq, uint32_t& nsel) {
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j < nv) {
      n_gt += key[j] > tau ? 1u : 0u;
      n_eq += key[j] == tau ? 1u : 0u;
    }
  }
  uint32_t tot;
  const uint32_t before = block_excl_scan<NW>((n_gt << 16) | n_eq, sh, tot);
  const uint32_t gt_before = before >> 16, eq_before = before & 0xffffu;
  // tau-valued entries of earlier threads that are taken; computed once and used by both
  // results (with the clamp written only inside base's expression, hipcc of ROCm 7.2 emitted
  // base = gt_before + eq_before without it)
  const uint32_t eq_taken = eq_before < need ? eq_before : need;
  take_eq = min(n_eq, need - eq_taken);
  base = gt_before + eq_taken;
  nsel = n_gt + take_eq;
}

// Bit j set: entry PER*t + j of this thread is selected (key > tau, or one of the first
// take_eq tau-valued entries of the thread). Straight-line masks instead of a running count, so
// the caller's stores of the selection are independent of each other.
template <int PER>
using SelMask = typename std::conditional<(PER > 32), uint64_t, uint32_t>::type;

template <int PER>
__device__ __forceinline__ SelMask<PER> select_mask(const uint32_t (&key)[PER], int nv,
                                                    uint32_t tau, uint32_t take_eq) {
  using M = SelMask<PER>;
  M gtm = 0, eqm = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    gtm |= (M)(j < nv && key[j] > tau) << j;
    eqm |= (M)(j < nv && key[j] == tau) << j;
  }
  M eqt = eqm;
  if (take_eq < (uint32_t)__popcll((unsigned long long)eqm)) {  // the thread at the tie cut
    eqt = 0;
    M m = eqm;
    for (uint32_t i = 0; i < take_eq; ++i) {
      eqt |= m & (~m + 1);  // lowest remaining tau-valued entry
      m &= m - 1;
    }
  }
  return gtm | eqt;
}

// position of selected entry j among this thread's selected entries
template <typename M>
__device__ __forceinline__ uint32_t sel_rank(M sel, int j) {
  return (uint32_t)__popcll((unsigned long long)(sel & (((M)1 << j) - 1)));
}

// ---- long rows: per-chunk candidate segments -------------------------------------------------
// A row longer than fits one workgroup is cut into G chunks. Each chunk keeps its own threshold
// tau_g = its r-th largest key, r = ceil(2k * cn / n) + 16 (about twice the chunk's fair share
// of the row's top k; cn = visible entries of the chunk, n = of the row), and writes every key
// >= tau_g with its index to the chunk's candidate segment, with its count and tau_g. A select
// over the concatenated segments is exact whenever its threshold tau >= tau_g for every chunk:
// an entry that is not a candidate lies below its chunk's tau_g <= tau.
constexpr int kLongChunk = 4096;  // entries per chunk
constexpr int kLongSeg = 1024;    // candidate slots per chunk

// Per-row workspace of the long-row path: counts[G], taus[G], cand_idx[G][kLongSeg],
// cand_key[G][kLongSeg]. A count of 0xffffffff marks an overflowed segment.
__host__ __device__ inline size_t long_row_bytes(int G) {
  return (size_t)G * (8 + 8 * (size_t)kLongSeg);
}

// The candidate segment of chunk g of a row whose workspace starts at rws: thread t holds the
// order keys key[0..nvt) (valid ones first) of entries index_of(j); n = the row's visible count
// (> k). Every thread of the block calls it.
template <int NW, int PER, typename IndexOf>
__device__ __forceinline__ void chunk_filter(const uint32_t (&key)[PER], int nvt, int n, int k,
                                             SelShared<NW>& sh, uint8_t* rws, int G, int g,
                                             IndexOf index_of) {
  uint32_t* counts = reinterpret_cast<uint32_t*>(rws);
  uint32_t* taus = counts + G;
  int32_t* cidx = reinterpret_cast<int32_t*>(taus + G) + (size_t)g * kLongSeg;
  uint32_t* ckey = reinterpret_cast<uint32_t*>(taus + G) + (size_t)G * kLongSeg + (size_t)g * kLongSeg;
  uint32_t cn;
  (void)block_excl_scan<NW>((uint32_t)nvt, sh, cn);
  __syncthreads();  // sh.wtot is written again below
  if (cn == 0u) {
    if (threadIdx.x == 0) {
      counts[g] = 0u;
      taus[g] = 0u;
    }
    return;
  }
  const int64_t r64 = (2 * (int64_t)k * cn + n - 1) / n + 16;
  uint32_t tau = 0u;  // every key >= 0: the whole chunk is a candidate
  if (r64 < (int64_t)cn) {
    uint32_t need, cnt_eq;
    block_threshold<NW, PER>(key, nvt, (uint32_t)r64, sh, tau, need, cnt_eq, cn);
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) cnt += (j < nvt && key[j] >= tau) ? 1u : 0u;
  uint32_t total;
  const uint32_t pos = block_excl_scan<NW>(cnt, sh, total);
  if (total <= (uint32_t)kLongSeg) {
    uint32_t o = pos;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (j < nvt && key[j] >= tau) {
        cidx[o] = index_of(j);
        ckey[o] = key[j];
        ++o;
      }
    }
  }
  if (threadIdx.x == 0) {
    counts[g] = total <= (uint32_t)kLongSeg ? total : 0xffffffffu;
    taus[g] = tau;
  }
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
