// attend.hip - sparse MQA-mode MLA attention over gathered entries on gfx950.
//
// ("DeepSeek-V3.2 sparse-attention principle and TPU adaptation", s1.3 fine-grained sparse
// attention: attention only over the top-k selected KV entries; s1.4: MLA in MQA mode, one
// latent row per entry shared by every query head; s2.2: one controllable sparse gather plus
// a much smaller dense matmul; s3 step 4: decode reads only the top-k KV. Tencent Cloud CSA
// snippets: sliding-window KV is concatenated with the compressed KV in one core attention.)
//
// For query row qi and head h, over E = {kv[b, idx[qi, i]] : idx >= 0} u {raw window rows}:
//   z_e = scale * q[qi,h,:] . K_e,  out[qi,h,:] = sum_e softmax(z)_e * K_e[:D_V],  lse = log sum exp z
//
// attend_mfma (bf16, D_K % 64 == 0, D_V % 16 == 0, H % 64 == 0): a workgroup = 4 waves = 64
// heads of one query over a split of its entry list. Per 32-entry tile the workgroup gathers the
// rows into LDS twice - row-major (the S^T = K Q^T A operand) and transposed for the first D_V
// columns (the P V B operand) - while the next tile's rows are already in flight in registers.
// Each wave owns 16 heads: q stays in registers (B operand of v_mfma_f32_16x16x32_bf16), the
// S^T accumulator layout is exactly the A-operand layout P needs, so P never leaves registers;
// online softmax in the exp2 domain, fp32 accumulators. Few-query calls split the entry list
// and merge the (m, l, O) partials in attend_combine.
// attend_generic: any dims, fp32 or bf16; one workgroup per (query, head), scalar fp32.
#include "../lightning_indexer_top_03_amd/csrc/common.h"
#include "../lightning_indexer_top_03_amd/csrc/launch.h"

#include <mutex>

namespace dsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kTile = 32;       // entries per tile
constexpr float kRefSlack = 8.f;  // log2 headroom of the lazily moved softmax reference
constexpr int kVtStride = 36;   // bf16 per transposed-V row (32 entries + pad): conflict-free b64 reads

// Source row of entry e of query (b, p); returns nullptr for a masked entry.
template <typename T>
__device__ __forceinline__ const T* entry_row(int e, const int32_t* __restrict__ idxrow, int top_k,
                                              const T* __restrict__ kv, int b, int N, int DK,
                                              const T* __restrict__ kv_raw, int64_t raw_base,
                                              int64_t n_raw, int p, int W) {
  if (e < top_k) {
    int j = idxrow[e];
    if (j < 0 || j >= N) return nullptr;
    return kv + ((size_t)b * N + j) * DK;
  }
  int64_t r = (int64_t)p - W + 1 + (e - top_k);
  if (r < 0 || r < raw_base || r >= raw_base + n_raw || kv_raw == nullptr) return nullptr;
  return kv_raw + ((size_t)b * n_raw + (r - raw_base)) * DK;
}

// Entry codes: >= 0 a row of kv (within the sequence), <= -2 a raw window row (-code-2 within
// kv_raw's rows of the sequence), -1 masked.
__device__ __forceinline__ int entry_code(int e, const int32_t* __restrict__ idxrow, int top_k,
                                          int N, int64_t raw_base, int64_t n_raw, int p, int W,
                                          bool has_raw) {
  if (e < top_k) {
    const int j = idxrow[e];
    return (j >= 0 && j < N) ? j : -1;
  }
  const int64_t r = (int64_t)p - W + 1 + (e - top_k);
  if (!has_raw || r < 0 || r < raw_base || r >= raw_base + n_raw) return -1;
  return -(int)(r - raw_base) - 2;
}

// ------------------------------------------------------------------------------------------
// attend_mfma_dma: same math as attend_mfma for D_K = 576, D_V = 512, but the gather goes
// straight from HBM into an NS-stage LDS ring with global_load_lds_dwordx4 (no register staging),
// and the P V B operand is read from the row-major tile with ds_read_b64_tr_b16 (no transposed
// copy of V). Per 32-entry tile and wave (8 rows): 8 row DMAs of the 1024-byte latent part (one
// row per instruction, fully coalesced) and one DMA of the 8 rows' 128-byte rope parts.
// LDS tile layout: latent rows at a 1040-byte stride (16-byte pad: conflict-free 16-byte reads by
// 8 consecutive rows), then the rope parts as [32 rows][8 chunks of 16 B] with the chunk slot
// XOR-swizzled by (row % 8). Waits are explicit (s_waitcnt vmcnt + s_barrier without a fence),
// so the DMAs of the next NS-1 tiles stay in flight while the current tile is computed.
//
// ds_read_b64_tr_b16, within each group of 16 lanes: if lane j reads the 4 bf16 M[j][0..3],
// lane 4a+b receives {M[a][b], M[a+4][b], M[a+8][b], M[a+12][b]}. Lane j of group g reading row
// 4g + j/4 at column 16*db + 4*(j%4) therefore receives, in lane n of the group, V[4g+0..3][16db+n]:
// the B-operand slots 0..3 of v_mfma_f32_16x16x32_bf16 for dim n (entries 4g..4g+3), which is the
// same slot -> entry map as the P operand taken from the S^T accumulators.
// ------------------------------------------------------------------------------------------
constexpr int kLatStride = 1040;                 // bytes per latent row in LDS
constexpr int kStageLat = kTile * kLatStride;    // 33280
constexpr int kStageRope = kTile * 128;          // 4096
constexpr int kStage = kStageLat + kStageRope;   // 37376

template <int N_>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N_) : "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// 16 ds_read_b64_tr_b16 for dim blocks d0 .. d0+7 (entry halves 4g.. and 16+4g..), waited for
// inside the same asm block. Written as asm because the builtin carries no memory operand, which
// makes the compiler wait for every LDS DMA still in flight before it.
#define DSA_TR(i, off) "ds_read_b64_tr_b16 %" #i ", %16 offset:" #off "\n"
#define DSA_TR_PAIR(i0, i1, D) DSA_TR(i0, (D) * 32) DSA_TR(i1, 16640 + (D) * 32)
#define DSA_TR_BLOCK(D0)                                                                        \
  case D0:                                                                                      \
    asm volatile(DSA_TR_PAIR(0, 1, D0) DSA_TR_PAIR(2, 3, D0 + 1) DSA_TR_PAIR(4, 5, D0 + 2)      \
                 DSA_TR_PAIR(6, 7, D0 + 3) DSA_TR_PAIR(8, 9, D0 + 4) DSA_TR_PAIR(10, 11, D0 + 5) \
                 DSA_TR_PAIR(12, 13, D0 + 6) DSA_TR_PAIR(14, 15, D0 + 7)                        \
                 "s_waitcnt lgkmcnt(0)"                                                         \
                 : "=&v"(tr[0]), "=&v"(tr[1]), "=&v"(tr[2]), "=&v"(tr[3]), "=&v"(tr[4]),         \
                   "=&v"(tr[5]), "=&v"(tr[6]), "=&v"(tr[7]), "=&v"(tr[8]), "=&v"(tr[9]),         \
                   "=&v"(tr[10]), "=&v"(tr[11]), "=&v"(tr[12]), "=&v"(tr[13]), "=&v"(tr[14]),    \
                   "=&v"(tr[15])                                                                \
                 : "v"(vaddr)                                                                   \
                 : "memory");                                                                   \
    break;
__device__ __forceinline__ void tr_read_block(u32x2_t* tr, uint32_t vaddr, int d0) {
  switch (d0) {
    DSA_TR_BLOCK(0) DSA_TR_BLOCK(8) DSA_TR_BLOCK(16) DSA_TR_BLOCK(24)
  }
}
#undef DSA_TR_BLOCK
#undef DSA_TR_PAIR
#undef DSA_TR

template <int NS>
__global__ __launch_bounds__(256, 1) void attend_mfma_dma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw, int64_t raw_base,
    int64_t n_raw, const int32_t* __restrict__ q_pos, int T, int N, int H, int top_k, int W,
    float scale_log2, int64_t qi0, int nsplit, int per_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int DK = 576, DV = 512, KK = DK / 32, DB = DV / 16;
  constexpr int DMAS = 9;  // DMA instructions per wave per tile
  __shared__ __attribute__((aligned(16))) char smem[NS * kStage];
  extern __shared__ int scode[];  // entry codes of this split, padded to whole tiles

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int64_t row = blockIdx.z;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T);
  const int p = q_pos[qi];
  const int split = blockIdx.x;
  const int h0 = blockIdx.y * 64 + wv * 16;
  const int E = top_k + W;
  const int e_begin = split * per_split;
  const int e_end = min(E, e_begin + per_split);
  const int ntiles = e_end > e_begin ? (e_end - e_begin + kTile - 1) / kTile : 0;
  const int32_t* __restrict__ idxrow = idx + row * (int64_t)top_k;
  const uint16_t* fallback = kv + (size_t)b * N * DK;  // any valid row; masked in the softmax

  u32x4_t qf[KK];
  {
    const uint16_t* qh = q + ((size_t)qi * H + h0 + n) * DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const u32x4_t*>(qh + 32 * kk);
    // complete the q loads here and make the values opaque: no wait for them inside the DMA
    // pipeline below, and no re-loading next to each use
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(qf[kk]));
  }
  // resolve the split's entries once: idx -> row code (masked rows keep a valid fallback address
  // for their DMA and are excluded in the softmax)
  for (int i = tid; i < ntiles * kTile; i += 256) {
    const int e = e_begin + i;
    scode[i] = e < e_end ? entry_code(e, idxrow, top_k, N, raw_base, n_raw, p, W, kv_raw != nullptr)
                         : -1;
  }
  __syncthreads();
  auto rowptr = [&](int code) -> const uint16_t* {
    if (code >= 0) return kv + ((size_t)b * N + code) * DK;
    if (code <= -2) return kv_raw + ((size_t)b * n_raw + (-code - 2)) * DK;
    return fallback;
  };

  f32x4_t acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // issue the DMAs of tile t (this wave's rows 8*wv .. 8*wv+7)
  auto issue = [&](int t) {
    const int stage = t % NS;
    // the DMA destination goes through an opaque wave-uniform integer: the waits for these
    // transfers are the explicit vmcnt waits of the pipeline below
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)(smem + stage * kStage));
    const int c0 = kTile * t + 8 * wv;  // this wave's first row in the code table
    // lane l resolves row l & 7 (latent DMAs, via readlane) and row l >> 3 (its rope chunk)
    const uint64_t pl = (uint64_t)(uintptr_t)rowptr(scode[c0 + (lane & 7)]);
    const uint16_t* pr = rowptr(scode[c0 + (lane >> 3)]);
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)pl, r8);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(pl >> 32), r8);
      const uint16_t* src = reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src + 8 * lane),
          (lds_void_t*)(uintptr_t)(sbase + (8 * wv + r8) * kLatStride), 16, 0, 0);
    }
    const int rr = lane >> 3;
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const void*>(pr + 512 + 8 * ((lane & 7) ^ rr)),
        (lds_void_t*)(uintptr_t)(sbase + kStageLat + wv * 1024), 16, 0, 0);
  };

  for (int t = 0; t < NS - 1 && t < ntiles; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    if (t + NS - 1 < ntiles) issue(t + NS - 1);
    const int later = min(NS - 1, ntiles - 1 - t);
    if (later >= 2) wait_vm<2 * DMAS>();
    else if (later == 1) wait_vm<DMAS>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();

    const int stage = t % NS;
    const char* sb = smem + stage * kStage;
    // S^T per 16-entry block: its 18 A-operand reads issued first, then two independent MFMA
    // chains (even / odd k-step)
    f32x4_t sp[2][2] = {};
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      const int R = eb * 16 + n;
      u32x4_t av[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const char* ap;
        if (kk < 16) {
          ap = sb + R * kLatStride + (32 * kk + 8 * g) * 2;
        } else {
          const int c = 4 * (kk - 16) + g;
          ap = sb + kStageLat + R * 128 + ((c ^ (R & 7)) * 16);
        }
        av[kk] = *reinterpret_cast<const u32x4_t*>(ap);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sp[eb][kk & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[kk]), as_bf16x8(qf[kk]),
                                                                 sp[eb][kk & 1], 0, 0, 0);
    }
    f32x4_t st[2] = {sp[0][0] + sp[0][1], sp[1][0] + sp[1][1]};
    float z[8];
    float mx = kNegInf;
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = eb * 16 + 4 * g + i;
        float v = scode[kTile * t + e] != -1 ? st[eb][i] * scale_log2 : kNegInf;
        z[eb * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazily moved softmax reference: m_run only moves (and the accumulators are rescaled) when
    // a head's tile maximum exceeds it by more than kRefSlack (log2 units), so p <= 2^kRefSlack
    // and the rescale of the 128 accumulators, which live in AGPRs, is rare.
    const bool grow = mx > m_run + kRefSlack;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      float ai[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[d][i] *= ai[i];
    }
    float psum = 0.f;
    uint32_t pk[4];
    {
      float pe[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // m_run == -inf only while every entry so far is masked (z == -inf as well)
        pe[i] = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(z[i] - m_run);
        psum += pe[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pe[2 * i], pe[2 * i + 1]);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    const bf16x8_t pa = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    // transposed V reads: rows 4g + n/4 (entries 4g..4g+3) and 16 + 4g + n/4, column 4*(n%4)
    const uint32_t vaddr = (uint32_t)(uintptr_t)(lds_void_t*)(sb + (4 * g + (n >> 2)) * kLatStride +
                                                             8 * (n & 3));
#pragma unroll
    for (int d0 = 0; d0 < DB; d0 += 8) {
      u32x2_t tr[16];
      tr_read_block(tr, vaddr, d0);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const u32x4_t bw = {tr[2 * d][0], tr[2 * d][1], tr[2 * d + 1][0], tr[2 * d + 1][1]};
        acc[d0 + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(bw), acc[d0 + d], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  float li[4], mi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    li[i] = __shfl(l_run, 4 * g + i, 64);
    mi[i] = __shfl(m_run, 4 * g + i, 64);
  }
  if (nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = li[i] > 0.f ? 1.f / li[i] : 0.f;
      uint16_t* orow = out + ((size_t)qi * H + h0 + 4 * g + i) * DV + n;
#pragma unroll
      for (int d = 0; d < DB; ++d) orow[16 * d] = f32_to_bf16(acc[d][i] * inv);
    }
    if (g == 0 && lse)
      lse[(size_t)qi * H + h0 + n] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t hrow = ((size_t)row * H + h0 + 4 * g + i) * nsplit + split;
      float* po = part_o + hrow * DV + n;
      for (int d = 0; d < DB; ++d) po[16 * d] = acc[d][i];
      if (n == 0) {
        part_ml[hrow * 2] = mi[i];
        part_ml[hrow * 2 + 1] = li[i];
      }
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// One workgroup of D_V/4 threads per (row, head); each thread owns 4 consecutive columns and
// reads every split's float4 (fully coalesced 2 KB per split).
template <typename OT>
__global__ __launch_bounds__(128) void attend_combine(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int64_t qi0, int H,
    int DV, int nsplit, OT* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x;
  const int64_t row = blockIdx.y;
  const size_t hrow = ((size_t)row * H + h) * nsplit;
  float M = kNegInf;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(hrow + s) * 2]);
  float L = 0.f;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  const int d = 4 * threadIdx.x;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = part_ml[(hrow + s) * 2];
    const float sc = ms == kNegInf ? 0.f : exp2f(ms - M);
    L += sc * part_ml[(hrow + s) * 2 + 1];
    if (d < DV) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(part_o + (hrow + s) * DV + d);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] += sc * v[i];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t orow = ((size_t)(qi0 + row) * H + h) * DV;
  if (d < DV) {
    if constexpr (sizeof(OT) == 2) {
      *reinterpret_cast<u32x2_t*>(out + orow + d) =
          u32x2_t{pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
    } else {
      *reinterpret_cast<f32x4_t*>(out + orow + d) = f32x4_t{a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv};
    }
  }
  if (threadIdx.x == 0 && lse)
    lse[(size_t)(qi0 + row) * H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// ---- generic scalar path ----
template <typename T>
__device__ __forceinline__ float ldv(const T* p, size_t i) {
  if constexpr (sizeof(T) == 2)
    return bf16_to_f32(p[i]);
  else
    return p[i];
}

template <typename T>
__global__ __launch_bounds__(256) void attend_generic(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ idx,
    const T* __restrict__ kv_raw, int64_t raw_base, int64_t n_raw,
    const int32_t* __restrict__ q_pos, int T_, int N, int H, int DK, int DV, int top_k, int W,
    float scale, int64_t qi0, T* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int E = top_k + W;
  float* sq = reinterpret_cast<float*>(smem);   // [DK]
  float* sz = sq + DK;                           // [E]
  const T** ssrc = reinterpret_cast<const T**>(sz + E + ((E & 1) ? 1 : 0));  // [E]
  __shared__ float red[256 / 64];
  const int h = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T_);
  const int p = q_pos[qi];
  const int32_t* idxrow = idx + row * (int64_t)top_k;
  for (int d = threadIdx.x; d < DK; d += blockDim.x) sq[d] = ldv(q, ((size_t)qi * H + h) * DK + d);
  __syncthreads();
  float mx = kNegInf;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const T* src = entry_row<T>(e, idxrow, top_k, kv, b, N, DK, kv_raw, raw_base, n_raw, p, W);
    ssrc[e] = src;
    float z = kNegInf;
    if (src) {
      float dot = 0.f;
      for (int d = 0; d < DK; ++d) dot += sq[d] * ldv(src, d);
      z = dot * scale;
    }
    sz[e] = z;
    mx = fmaxf(mx, z);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = kNegInf;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) mx = fmaxf(mx, red[i]);
  __syncthreads();
  float sum = 0.f;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float pe = (mx == kNegInf || sz[e] == kNegInf) ? 0.f : __expf(sz[e] - mx);
    sz[e] = pe;
    sum += pe;
  }
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  sum = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) sum += red[i];
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int d = threadIdx.x; d < DV; d += blockDim.x) {
    float a = 0.f;
    for (int e = 0; e < E; ++e)
      if (ssrc[e]) a += sz[e] * ldv(ssrc[e], d);
    a *= inv;
    if constexpr (sizeof(T) == 2)
      out[((size_t)qi * H + h) * DV + d] = f32_to_bf16(a);
    else
      out[((size_t)qi * H + h) * DV + d] = a;
  }
  if (threadIdx.x == 0 && lse) lse[(size_t)qi * H + h] = sum > 0.f ? mx + __logf(sum) : kNegInf;
}

bool mfma_ok(const Shape& s, int fmt) {
  return fmt == FMT_BF16 && s.D_K == 576 && s.D_V == 512 && s.H % 64 == 0;
}

}  // namespace

int attend_splits(const Shape& s, int64_t nrows, int fmt) {
  if (!mfma_ok(s, fmt) || nrows <= 0) return 1;
  const int64_t wgs = nrows * (s.H / 64);
  if (wgs >= 512) return 1;
  const int E = s.top_k + s.W;
  int64_t want = (512 + wgs - 1) / wgs;
  int64_t maxs = (E + 255) / 256;  // at least 256 entries per split
  int64_t ns = want < maxs ? want : maxs;
  if (ns > 8) ns = 8;
  return ns < 1 ? 1 : (int)ns;
}

size_t attend_ws_bytes(const Shape& s, int64_t nrows, int fmt) {
  const int ns = attend_splits(s, nrows, fmt);
  if (ns <= 1) return 0;
  return (size_t)nrows * s.H * ns * ((size_t)s.D_V + 2) * sizeof(float);
}

hipError_t launch_attend(const Shape& s, int64_t qi0, int64_t nrows, int fmt, const void* q,
                         const void* kv, const int32_t* idx, const void* kv_raw, int64_t raw_base,
                         int64_t n_raw, const int32_t* q_pos, float scale, void* out, float* lse,
                         void* ws, hipStream_t st, hipEvent_t between) {
  if (nrows <= 0) return hipSuccess;
  if (mfma_ok(s, fmt)) {
    const int ns = attend_splits(s, nrows, fmt);
    const int E = s.top_k + s.W;
    const int per = ((E + ns - 1) / ns + kTile - 1) / kTile * kTile;
    float* part_o = static_cast<float*>(ws);
    float* part_ml = ns > 1 ? part_o + (size_t)nrows * s.H * ns * s.D_V : nullptr;
    dim3 grid(ns, s.H / 64, (unsigned)nrows);
    const size_t code_bytes = sizeof(int) * (size_t)per;  // per is a multiple of the tile
    static std::once_flag once;  // the code table can take the block past 64 KB of LDS
    std::call_once(once, [] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_mfma_dma<2>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 48 * 1024);
    });
    attend_mfma_dma<2><<<grid, 256, code_bytes, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
        static_cast<const uint16_t*>(kv_raw), raw_base, n_raw, q_pos, s.T, s.N, s.H, s.top_k, s.W,
        scale * kLog2e, qi0, ns, per, static_cast<uint16_t*>(out), lse, part_o, part_ml);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    if (between) (void)hipEventRecord(between, st);
    attend_combine<uint16_t><<<dim3(s.H, (unsigned)nrows), 128, 0, st>>>(
        part_o, part_ml, qi0, s.H, s.D_V, ns, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
  }
  const int E = s.top_k + s.W;
  size_t shm = sizeof(float) * (s.D_K + E + 1) + sizeof(void*) * E + 16;
  dim3 grid(s.H, (unsigned)nrows);
  if (fmt == FMT_BF16)
    attend_generic<uint16_t><<<grid, 256, shm, st>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
        static_cast<const uint16_t*>(kv_raw), raw_base, n_raw, q_pos, s.T, s.N, s.H, s.D_K, s.D_V,
        s.top_k, s.W, scale, qi0, static_cast<uint16_t*>(out), lse);
  else
    attend_generic<float><<<grid, 256, shm, st>>>(
        static_cast<const float*>(q), static_cast<const float*>(kv), idx,
        static_cast<const float*>(kv_raw), raw_base, n_raw, q_pos, s.T, s.N, s.H, s.D_K, s.D_V,
        s.top_k, s.W, scale, qi0, static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace dsa
