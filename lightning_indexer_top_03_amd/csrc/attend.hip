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
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kTile = 32;       // entries per tile
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

template <int DK, int DV>
__global__ __launch_bounds__(256, 1) void attend_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw, int64_t raw_base,
    int64_t n_raw, const int32_t* __restrict__ q_pos, int T, int N, int H, int top_k, int W,
    float scale_log2, int64_t qi0, int nsplit, int per_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int KS = DK + 8;          // bf16 per row-major K row in LDS (16-byte pad)
  constexpr int CPR = DK / 8;         // 16-byte chunks per row
  constexpr int JPT = CPR / 8;        // chunks per thread per tile (8 threads per entry)
  constexpr int KK = DK / 32;         // MFMA k-steps for S
  constexpr int DB = DV / 16;         // 16-wide output column blocks
  __shared__ __attribute__((aligned(16))) uint16_t sK[kTile * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[DV * kVtStride];
  __shared__ int sValid[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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
  const int32_t* __restrict__ idxrow = idx + row * (int64_t)top_k;

  // q fragments: lane (head n, group g) holds q[h0+n][32kk + 8g .. +7]
  u32x4_t qf[KK];
  {
    const uint16_t* qh = q + ((size_t)qi * H + h0 + n) * DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const u32x4_t*>(qh + 32 * kk);
  }

  f32x4_t acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // gather mapping: thread handles entry r = tid & 31 of every tile, chunks cg + 8j
  const int r = tid & 31, cg = tid >> 5;
  u32x4_t pre[JPT];
  int pre_ok = 0;
  auto fetch = [&](int e0) {
    const int e = e0 + r;
    const uint16_t* src = e < e_end ? entry_row<uint16_t>(e, idxrow, top_k, kv, b, N, DK, kv_raw,
                                                          raw_base, n_raw, p, W)
                                    : nullptr;
    pre_ok = src != nullptr;
#pragma unroll
    for (int j = 0; j < JPT; ++j)
      pre[j] = src ? *reinterpret_cast<const u32x4_t*>(src + 8 * (cg + 8 * j))
                   : u32x4_t{0u, 0u, 0u, 0u};
  };

  if (e_begin < e_end) fetch(e_begin);
  for (int e0 = e_begin; e0 < e_end; e0 += kTile) {
    // commit the prefetched rows: row-major K and transposed V
#pragma unroll
    for (int j = 0; j < JPT; ++j) {
      const int cc = cg + 8 * j;
      *reinterpret_cast<u32x4_t*>(&sK[r * KS + 8 * cc]) = pre[j];
      if (8 * cc < DV) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t wd = pre[j][i];
          sVt[(8 * cc + 2 * i) * kVtStride + r] = (uint16_t)(wd & 0xffffu);
          sVt[(8 * cc + 2 * i + 1) * kVtStride + r] = (uint16_t)(wd >> 16);
        }
      }
    }
    if (cg == 0) sValid[r] = pre_ok;
    __syncthreads();
    if (e0 + kTile < e_end) fetch(e0 + kTile);

    // S^T[entry, head] for two 16-entry blocks
    f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&sK[(eb * 16 + n) * KS + 32 * kk + 8 * g]));
        st[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(qf[kk]), st[eb], 0, 0, 0);
      }
    }
    // lane (head n, g): st[eb][i] = entry eb*16 + 4g + i
    float z[8];
    float mx = kNegInf;
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = eb * 16 + 4 * g + i;
        float v = sValid[e] ? st[eb][i] * scale_log2 : kNegInf;
        z[eb * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    float alpha, psum = 0.f;
    uint32_t pk[4];
    if (m_new == kNegInf) {
      alpha = 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = 0u;
    } else {
      alpha = exp2f(m_run - m_new);
      float pe[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pe[i] = exp2f(z[i] - m_new);
        psum += pe[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pe[2 * i], pe[2 * i + 1]);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rows of acc are heads 4g + i: fetch their alpha from lane (4g + i)
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i, 64);
    const bf16x8_t pa = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[d][i] *= ai[i];
      const uint16_t* vrow = &sVt[(16 * d + n) * kVtStride];
      u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow + 4 * g);
      u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16 + 4 * g);
      bf16x8_t bv = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
      acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bv, acc[d], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue ----
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
#pragma unroll
      for (int d = 0; d < DB; ++d) po[16 * d] = acc[d][i];
      if (n == 0) {
        part_ml[hrow * 2] = mi[i];
        part_ml[hrow * 2 + 1] = li[i];
      }
    }
  }
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

// 8 ds_read_b64_tr_b16 for dim blocks d0 .. d0+3 (entry halves 4g.. and 16+4g..), waited for
// inside the same asm block. Written as asm because the builtin carries no memory operand, which
// makes the compiler wait for every LDS DMA still in flight before it.
#define DSA_TR(i, off) "ds_read_b64_tr_b16 %" #i ", %8 offset:" #off "\n"
#define DSA_TR_BLOCK(D0)                                                                        \
  case D0:                                                                                      \
    asm volatile(DSA_TR(0, D0 * 32) DSA_TR(1, 16640 + D0 * 32) DSA_TR(2, D0 * 32 + 32)          \
                 DSA_TR(3, 16640 + D0 * 32 + 32) DSA_TR(4, D0 * 32 + 64)                        \
                 DSA_TR(5, 16640 + D0 * 32 + 64) DSA_TR(6, D0 * 32 + 96)                        \
                 DSA_TR(7, 16640 + D0 * 32 + 96) "s_waitcnt lgkmcnt(0)"                         \
                 : "=&v"(tr[0]), "=&v"(tr[1]), "=&v"(tr[2]), "=&v"(tr[3]), "=&v"(tr[4]),         \
                   "=&v"(tr[5]), "=&v"(tr[6]), "=&v"(tr[7])                                     \
                 : "v"(vaddr)                                                                   \
                 : "memory");                                                                   \
    break;
__device__ __forceinline__ void tr_read_block(u32x2_t* tr, uint32_t vaddr, int d0) {
  switch (d0) {
    DSA_TR_BLOCK(0) DSA_TR_BLOCK(4) DSA_TR_BLOCK(8) DSA_TR_BLOCK(12)
    DSA_TR_BLOCK(16) DSA_TR_BLOCK(20) DSA_TR_BLOCK(24) DSA_TR_BLOCK(28)
  }
}
#undef DSA_TR_BLOCK
#undef DSA_TR

template <int NS>
__global__ __launch_bounds__(256, NS == 2 ? 2 : 1) void attend_mfma_dma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw, int64_t raw_base,
    int64_t n_raw, const int32_t* __restrict__ q_pos, int T, int N, int H, int top_k, int W,
    float scale_log2, int64_t qi0, int nsplit, int per_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int DK = 576, DV = 512, KK = DK / 32, DB = DV / 16;
  constexpr int DMAS = 9;  // DMA instructions per wave per tile
  __shared__ __attribute__((aligned(16))) char smem[NS * kStage];
  __shared__ int sValid[NS][kTile];

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
    const int e0 = e_begin + kTile * t + 8 * wv;
    const uint16_t* rp[8];
    uint32_t okm = 0;
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int e = e0 + r8;
      const uint16_t* src = e < e_end ? entry_row<uint16_t>(e, idxrow, top_k, kv, b, N, DK,
                                                            kv_raw, raw_base, n_raw, p, W)
                                      : nullptr;
      okm |= (src != nullptr ? 1u : 0u) << r8;
      rp[r8] = src ? src : fallback;
    }
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(rp[r8] + 8 * lane),
          (lds_void_t*)(uintptr_t)(sbase + (8 * wv + r8) * kLatStride), 16, 0, 0);
    const int rr = lane >> 3;  // row within the wave's 8
    const uint16_t* mine = rp[0];
#pragma unroll
    for (int r8 = 1; r8 < 8; ++r8) mine = rr == r8 ? rp[r8] : mine;
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const void*>(mine + 512 + 8 * ((lane & 7) ^ rr)),
        (lds_void_t*)(uintptr_t)(sbase + kStageLat + wv * 1024), 16, 0, 0);
    if (lane < 8) sValid[stage][8 * wv + lane] = (okm >> lane) & 1u;
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
    f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int eb = 0; eb < 2; ++eb) {
      const int R = eb * 16 + n;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const char* ap;
        if (kk < 16) {
          ap = sb + R * kLatStride + (32 * kk + 8 * g) * 2;
        } else {
          const int c = 4 * (kk - 16) + g;
          ap = sb + kStageLat + R * 128 + ((c ^ (R & 7)) * 16);
        }
        bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(ap));
        st[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(qf[kk]), st[eb], 0, 0, 0);
      }
    }
    float z[8];
    float mx = kNegInf;
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = eb * 16 + 4 * g + i;
        float v = sValid[stage][e] ? st[eb][i] * scale_log2 : kNegInf;
        z[eb * 4 + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    float alpha, psum = 0.f;
    uint32_t pk[4];
    if (m_new == kNegInf) {
      alpha = 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = 0u;
    } else {
      alpha = exp2f(m_run - m_new);
      float pe[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pe[i] = exp2f(z[i] - m_new);
        psum += pe[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = pack_bf16x2(pe[2 * i], pe[2 * i + 1]);
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    float ai[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ai[i] = __shfl(alpha, 4 * g + i, 64);
    const bf16x8_t pa = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    // transposed V reads: rows 4g + n/4 (entries 4g..4g+3) and 16 + 4g + n/4, column 4*(n%4)
    const uint32_t vaddr = (uint32_t)(uintptr_t)(lds_void_t*)(sb + (4 * g + (n >> 2)) * kLatStride +
                                                             8 * (n & 3));
#pragma unroll
    for (int d0 = 0; d0 < DB; d0 += 4) {
      u32x2_t tr[8];
      tr_read_block(tr, vaddr, d0);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[d0 + d][i] *= ai[i];
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
#pragma unroll
      for (int d = 0; d < DB; ++d) po[16 * d] = acc[d][i];
      if (n == 0) {
        part_ml[hrow * 2] = mi[i];
        part_ml[hrow * 2 + 1] = li[i];
      }
    }
  }
}

// Merge split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
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
  for (int s = 0; s < nsplit; ++s) {
    float ms = part_ml[(hrow + s) * 2];
    if (ms != kNegInf) L += exp2f(ms - M) * part_ml[(hrow + s) * 2 + 1];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const size_t orow = ((size_t)(qi0 + row) * H + h) * DV;
  for (int d = threadIdx.x; d < DV; d += blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      float ms = part_ml[(hrow + s) * 2];
      if (ms != kNegInf) a += exp2f(ms - M) * part_o[(hrow + s) * DV + d];
    }
    a *= inv;
    if constexpr (sizeof(OT) == 2)
      out[orow + d] = f32_to_bf16(a);
    else
      out[orow + d] = a;
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
    attend_mfma_dma<2><<<grid, 256, 0, st>>>(
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
