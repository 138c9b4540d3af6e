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
// attend_mfma_dma (bf16, D_K = 576, D_V = 512, H % 64 == 0): a workgroup = 8 waves = 64 heads
// of one query over a split of its entry list; tiles of 32 entries stream from HBM into an LDS
// ring by DMA, wave pairs split D_K for S = q K^T and D_V for P V (details at the kernel).
// attend_generic: any dims, fp32 or bf16; one workgroup per (query, head), scalar fp32.
#include "common.h"
#include "launch.h"
#include "select.h"

#include <algorithm>
#include <mutex>

namespace dsa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kTile = 32;       // entries per tile
// per (row, head, split) partial: m, l, then the fp16 scale c of each 128-column quarter
constexpr int kMlStride = 6;
constexpr float kRefSlack = 8.f;  // log2 headroom of the lazily moved softmax reference

// Joins an attention-sink logit s2 (log2 units; -inf = no sink) to a softmax state: m is the
// reference of the entries' exponentials (log2 units, -inf when there are none) and l their
// sum relative to it. Returns the reference M = max(m, s2) and the total L relative to M.
__device__ __forceinline__ void join_sink(float m, float l, float s2, float& M, float& L) {
  if (s2 == kNegInf) {
    M = m;
    L = l;
    return;
  }
  M = fmaxf(m, s2);
  L = (m == kNegInf ? 0.f : l * __builtin_amdgcn_exp2f(m - M)) + __builtin_amdgcn_exp2f(s2 - M);
}

// Source row of entry e of query (b, p); returns nullptr for a masked entry. idxrow == nullptr:
// every visible entry (entry e < top_k is entry e itself when e < lim = n_vis), else entries
// come from idxrow (lim = N).
template <typename T>
__device__ __forceinline__ const T* entry_row(int e, const int32_t* __restrict__ idxrow, int top_k,
                                              const T* __restrict__ kv, int b, int N, int DK,
                                              const T* __restrict__ kv_raw, int64_t raw_base,
                                              int64_t n_raw, int p, int W, int lim) {
  if (e < top_k) {
    int j = idxrow != nullptr ? idxrow[e] : e;
    if (j < 0 || j >= lim) return nullptr;
    return kv + ((size_t)b * N + j) * DK;
  }
  int64_t r = (int64_t)p - W + 1 + (e - top_k);
  if (r < 0 || r < raw_base || r >= raw_base + n_raw || kv_raw == nullptr) return nullptr;
  return kv_raw + ((size_t)b * n_raw + (r - raw_base)) * DK;
}

// Entry codes: >= 0 a row of kv (within the sequence), <= -2 a raw window row (-code-2 within
// kv_raw's rows of the sequence), -1 masked. idxrow == nullptr and lim as in entry_row.
__device__ __forceinline__ int entry_code(int e, const int32_t* __restrict__ idxrow, int top_k,
                                          int lim, int64_t raw_base, int64_t n_raw, int p, int W,
                                          bool has_raw) {
  if (e < top_k) {
    const int j = idxrow != nullptr ? idxrow[e] : e;
    return (j >= 0 && j < lim) ? j : -1;
  }
  const int64_t r = (int64_t)p - W + 1 + (e - top_k);
  if (!has_raw || r < 0 || r < raw_base || r >= raw_base + n_raw) return -1;
  return -(int)(r - raw_base) - 2;
}

// ------------------------------------------------------------------------------------------
// attend_mfma_dma (bf16, D_K = 576, D_V = 512, H % 64 == 0): one workgroup = 8 waves = 64 heads
// of one query over a split of its entry list, 32-entry tiles, software-pipelined across two
// kinds of wave so that every SIMD runs one of each:
//  * Gather: each tile goes straight from HBM into an NS-stage LDS ring with
//    global_load_lds_dwordx4 (no register staging), issued by the value waves only: one DMA per
//    row for the 1024-byte latent part (fully coalesced) and one per 8 rows for their 128-byte
//    rope parts. Latent rows sit at a 1056-byte stride: both the row-per-lane 16-byte reads of
//    S and the transposed 8-byte reads of P V are then free of bank conflicts. The rope parts
//    are [32 rows][8 chunks of 16 B], chunk c of row R at slot c ^ ((R >> 1) & 7), again
//    conflict-free for the row-per-lane reads.
//    Waits are explicit (s_waitcnt vmcnt + s_barrier, no fence).
//  * Score waves 0..3 (head block hb = wave): in iteration i, S^T = K Q^T for the 32 entries of
//    tile i (two 16-entry blocks, each over two accumulator chains of v_mfma_f32_16x16x32_bf16,
//    with q in registers as the B operand) and the online softmax (exp2 domain; the reference moves only
//    when a head's maximum grows by more than kRefSlack; head maxima reduced with
//    v_permlane16_swap / v_permlane32_swap). The S^T accumulator layout (lane: head n, entries
//    4g..4g+3) is the A-operand layout of P, so each lane hands its packed P (slots 0..3 =
//    entries 4g.., slots 4..7 = entries 16+4g..) to its value wave through LDS unchanged, with
//    the rescale factors when the reference moved.
//  * Value waves 4..7: in iteration i, P V for tile i-1; wave 4+v owns all 64 heads and value
//    columns 128*v .. +127, so each pair of transposed V reads feeds four MFMAs (32 MFMAs and
//    16 reads per tile). The B operands come straight from the row-major tile through
//    ds_read_b64_tr_b16: within each group of 16 lanes, if lane j reads M[j][0..3], lane 4a+b
//    receives {M[a][b], M[a+4][b], M[a+8][b], M[a+12][b]}. Lane j of group g reading entry
//    4g + j/4 at column c + 4*(j%4) therefore receives, in lane n, V[4g+0..3][c+n] (B slots 0..3
//    in P's order); a second read 16 rows further supplies slots 4..7. The reads of two column
//    blocks are issued ahead of the eight MFMAs of the two before them, inside one asm block
//    with its wait (pv_step2).
//  * The softmax runs on raw scores: maxima with v_max3, the scale folded into the exponent
//    (one fma per entry), and a finite stand-in reference while every entry so far is masked.
//  * Two barriers per iteration: after the first (tile i has landed) the score waves run the S
//    MFMAs of tile i alone on the matrix cores while the value waves issue the DMAs of the next
//    tile; after the second, the score waves' softmax (VALU) overlaps the value waves' P V MFMAs.
//    The two kinds of wave run separate loops with the same barrier count, so the register
//    allocator never holds q and the accumulators at once. The ring is 4 stages deep when the
//    split's entry table fits beside it (two tiles in flight ahead of the score waves), else 3.
//  * Few-query calls split the entry list and merge the (m, l, O) partials in attend_combine
//    (O as fp16 scaled per 128-column quarter).
//    Workgroups are numbered so that each XCD (workgroup id mod 8) gets a contiguous run of
//    (row, head group, split): the splits of a query share that XCD's L2 for q and the tiles.
// ------------------------------------------------------------------------------------------
constexpr int kLatStride = 1056;                 // bytes per latent row in LDS
constexpr int kStageLat = kTile * kLatStride;    // 33792
constexpr int kStageRope = kTile * 128;          // 4096
constexpr int kStage = kStageLat + kStageRope;   // 37888
constexpr int kAtWaves = 8;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int N_>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N_) : "memory");
}

// sum over the four 16-lane groups, on the VALU (permlane swaps exchange rows of 16 and halves
// of 32 lanes between two registers)
// Maxima without the canonicalising v_max x, x the compiler adds for values it cannot prove
// canonical (MFMA results): IEEE maximum of finite values and -inf. group_max_raw: over the
// four 16-lane groups.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float group_max_raw(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


#define DSA_PV_MFMAS2                                                                           \
  "v_mfma_f32_16x16x32_bf16 %0, %12, %16, %0\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %1, %13, %16, %1\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %2, %14, %16, %2\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %3, %15, %16, %3\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %4, %12, %17, %4\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %5, %13, %17, %5\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %6, %14, %17, %6\n"                                                 \
  "v_mfma_f32_16x16x32_bf16 %7, %15, %17, %7\n"
// Column blocks D, D+1 of P V on a value wave (four head blocks each): the transposed V reads
// of blocks D+2, D+3 (x0, x1: entries 4g.. / 16+4g.. of D+2; y0, y1: of D+3) are issued
// first and waited for at the end, so they run under the eight MFMAs (B operands b0, b1; A
// operands p0..p3). The MFMAs sit in the same asm block as the reads (a load's destination
// must not be reused before its wait); s_nop pads the VALU -> MFMA distance at the start and
// the MFMA -> VALU distance at the end of a tile.
template <int D>
__device__ __forceinline__ void pv_step2(f32x4_t* a, f32x4_t* b, const bf16x8_t* p,
                                         u32x4_t b0, u32x4_t b1, uint32_t vaddr, u32x2_t& x0,
                                         u32x2_t& x1, u32x2_t& y0, u32x2_t& y1) {
  if constexpr (D + 2 < 8) {
    asm volatile("ds_read_b64_tr_b16 %8, %18 offset:%19\n"
                 "ds_read_b64_tr_b16 %9, %18 offset:%20\n"
                 "ds_read_b64_tr_b16 %10, %18 offset:%21\n"
                 "ds_read_b64_tr_b16 %11, %18 offset:%22\n"
                 "s_nop 2\n" DSA_PV_MFMAS2 "s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                   "+v"(b[2]), "+v"(b[3]), "=&v"(x0), "=&v"(x1), "=&v"(y0), "=&v"(y1)
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(b0), "v"(b1), "v"(vaddr),
                   "n"((D + 2) * 32), "n"(16896 + (D + 2) * 32), "n"((D + 3) * 32),
                   "n"(16896 + (D + 3) * 32)
                 : "memory");
  } else {
    asm volatile("s_nop 2\n" DSA_PV_MFMAS2 "s_nop 7\ns_nop 7\ns_nop 7"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                   "+v"(b[2]), "+v"(b[3]), "=v"(x0), "=v"(x1), "=v"(y0), "=v"(y1)
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(b0), "v"(b1)
                 : "memory");
  }
}
#undef DSA_PV_MFMAS2
// the transposed reads of the first two column blocks, waited for
__device__ __forceinline__ void pv_first2(uint32_t vaddr, u32x2_t& x0, u32x2_t& x1, u32x2_t& y0,
                                          u32x2_t& y1) {
  asm volatile("ds_read_b64_tr_b16 %0, %4\n"
               "ds_read_b64_tr_b16 %1, %4 offset:16896\n"
               "ds_read_b64_tr_b16 %2, %4 offset:32\n"
               "ds_read_b64_tr_b16 %3, %4 offset:16928\n"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1), "=&v"(y0), "=&v"(y1)
               : "v"(vaddr)
               : "memory");
}

// max over the 16 lanes of a DPP row (lane groups of 16)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xb1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f32<0x4e>(x));   // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror: the other quad of the half row
  x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror: the other half row
  return x;
}

// PER == 0: the entries come from idx. PER > 0 (fused top-k): they come straight from the
// indexer scores; every workgroup of a row selects the row's top-k (block_threshold /
// block_ranks of select.h, PER entries per thread, in ascending index order) and keeps its own
// split's slice; the workgroup of split 0 / head group 0 also writes the row of idx_out.
// KVF: the entries' storage, 0 = bf16 rows, 8 = MXFP8 (e4m3 codes [B, N, 576]), 4 = MXFP4
// (e2m1 code pairs [B, N, 288], low nibble first); MX rows carry one E8M0 scale per 32 values.
template <int NS, int PER, int KVF>
__global__ __launch_bounds__(kAtWaves * 64, 1) void attend_mfma_dma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const uint16_t* __restrict__ kv_raw, int64_t raw_base,
    int64_t n_raw, const int32_t* __restrict__ q_pos, int T, int N, int H, int top_k, int W,
    float scale_log2, int64_t qi0, int nsplit, int per_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, f16x4_t* __restrict__ part_o, float* __restrict__ part_ml,
    int nitems, const float* __restrict__ scores, int m, int32_t* __restrict__ idx_out,
    const int32_t* __restrict__ seq_len, const float* __restrict__ sink,
    const uint8_t* __restrict__ kv_scale) {
  constexpr int DK = 576, DV = 512, KS = DK / 32, DB = DV / 16;
  constexpr bool KV8 = KVF != 0;             // low-precision entries, converted in the kernel
  constexpr int CB = KVF == 4 ? DK / 2 : DK;  // code bytes per entry
  __shared__ __attribute__((aligned(16))) char smem[NS * kStage];
  __shared__ __attribute__((aligned(16))) u32x4_t pbuf[2][4][64];  // P, per head block
  // rescale factor per head when the reference moved, and whether it moved (per head block)
  __shared__ __attribute__((aligned(16))) float abuf[2][4][16];
  __shared__ __attribute__((aligned(16))) uint32_t fbuf[2][4];
  __shared__ float sml[4][2][16];    // per head: [1] = the output multiplier (unsplit calls)
  extern __shared__ __attribute__((aligned(16))) int scode[];  // entry codes, whole tiles
  // MX entries: the codes of the next tile, CB bytes per row, staged by DMA one iteration
  // before they are converted into the ring
  static_assert(!KV8 || NS == 3, "the MX staging buffer fits beside a 3-stage ring only");
  __shared__ __attribute__((aligned(16))) char sf8[KV8 ? kTile * CB : 16];
  // ... and their E8M0 scale bytes, one per dword (a 1-byte DMA fills one dword per lane)
  __shared__ __attribute__((aligned(16))) uint32_t sf8s[KV8 ? kTile * 18 : 4];

  // all kernel arguments in one scalar round trip (the compiler otherwise loads them lazily,
  // in several dependent batches)
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  asm volatile(""
               : "+s"(bx), "+s"(by), "+s"(bz)
               : "s"(q), "s"(kv), "s"(idx), "s"(kv_raw), "s"(q_pos), "s"(qi0), "s"(raw_base),
                 "s"(n_raw), "s"(T), "s"(N), "s"(H), "s"(top_k), "s"(W), "s"(nsplit),
                 "s"(per_split), "s"(nitems));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wv < 4;
  const int hb = wv & 3;
  const int n = lane & 15, g = lane >> 4;
  const int HG = H / 64;
  const int item = xcd_item(bx + nsplit * (by + HG * bz), nitems);
  const int split = item % nsplit;
  const int hg = (item / nsplit) % HG;
  const int64_t row = item / (nsplit * HG);
  const int64_t qi = qi0 + row;
  const int b = (int)((uint32_t)qi / (uint32_t)T);  // query rows < 2^31
  const int h0 = hg * 64 + hb * 16;
  const int E = top_k + W;
  const int e_begin = split * per_split;
  const int e_end = min(E, e_begin + per_split);
  const int ntiles = e_end > e_begin ? (e_end - e_begin + kTile - 1) / kTile : 0;
  const int ncode = ntiles * kTile;
  // idx == nullptr: every visible entry takes part (dense attention over the compressed
  // sequence, no selection)
  const int32_t* __restrict__ idxrow = idx != nullptr ? idx + row * (int64_t)top_k : nullptr;

  // q fragments (score waves): lane (head n, group g) holds q[h0+n][32kk + 8g .. +7]
  u32x4_t qf[KS];
  auto load_q = [&]() {
    if (score_wave) {
      const uint16_t* qh = q + ((size_t)qi * H + h0 + n) * DK + 8 * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qf[kk] = *reinterpret_cast<const u32x4_t*>(qh + 32 * kk);
    }
  };
  // window entry e >= top_k: raw row p - W + 1 + (e - top_k) if held in kv_raw
  auto window_code = [&](int e, int p) -> int {
    const int64_t r = (int64_t)p - W + 1 + (e - top_k);
    if (kv_raw != nullptr && r >= 0 && r >= raw_base && r < raw_base + n_raw)
      return -(int)(r - raw_base) - 2;
    return -1;
  };
  if constexpr (PER == 0) {
    // Prologue: the idx reads of this thread's first two code slots (unconditional, clamped
    // address) and, on the score waves, the q loads are all issued before the first wait.
    int raw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      raw[j] = idxrow != nullptr ? idxrow[min(e_begin + tid + j * kAtWaves * 64, top_k - 1)]
                                 : e_begin + tid + j * kAtWaves * 64;
    load_q();
    const int p = q_pos[qi];
    const int lim = idxrow != nullptr ? N : n_visible(p, m, N, seq_len, b);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      asm volatile("" : "+v"(raw[j]));  // keep the reads above, not sunk into the branches below
      const int i = tid + j * kAtWaves * 64;
      const int e = e_begin + i;
      int code = -1;
      if (e < e_end) code = e < top_k ? ((raw[j] >= 0 && raw[j] < lim) ? raw[j] : -1) : window_code(e, p);
      if (i < ncode) scode[i] = code;
    }
    for (int i = tid + 2 * kAtWaves * 64; i < ncode; i += kAtWaves * 64) {
      const int e = e_begin + i;
      scode[i] = e < e_end ? entry_code(e, idxrow, top_k, lim, raw_base, n_raw, p, W, kv_raw != nullptr)
                           : -1;
    }
  } else {
    // Fused top-k: the row's scores (in flight with the q loads), its selection, this split's
    // slice of it. The selection's LDS scratch is the ring memory, idle until the first DMA.
    // The score loads do not wait for q_pos: they cover the whole row (addresses clamped to
    // N), and the visible count only trims them afterwards (one memory round trip fewer).
    int p = q_pos[qi];
    const float* __restrict__ srow = scores + row * (int64_t)N;
    uint32_t key[PER];
    load_keys<PER>(srow, N, N, key);
    asm volatile("" : "+v"(p));
    const int nvis = n_visible(p, m, N, seq_len, b);
    const int nv = nvis > top_k ? max(0, min(PER, nvis - PER * tid)) : 0;
    load_q();
    int32_t* __restrict__ orow =
        (idx_out != nullptr && split == 0 && hg == 0) ? idx_out + row * (int64_t)top_k : nullptr;
    // every slot first: window entries, keep-all rows (rank = index), -1 elsewhere; ranks of a
    // selected row are filled in below (after the selection's first barrier)
    for (int i = tid; i < ncode; i += kAtWaves * 64) {
      const int e = e_begin + i;
      int code = -1;
      if (e < e_end) code = e >= top_k ? window_code(e, p) : (nvis <= top_k && e < nvis ? e : -1);
      scode[i] = code;
    }
    if (nvis <= top_k) {
      if (orow)
        for (int i = tid; i < top_k; i += kAtWaves * 64) orow[i] = i < nvis ? i : -1;
    } else {
      SelShared<kAtWaves>& sh = *reinterpret_cast<SelShared<kAtWaves>*>(smem);
      uint32_t tau, need, cnt_eq;
      block_threshold<kAtWaves, PER>(key, nv, (uint32_t)top_k, sh, tau, need, cnt_eq, (uint32_t)nvis);
      uint32_t base, take_eq, nsel;
      block_ranks<kAtWaves, PER>(key, nv, tau, need, sh, base, take_eq, nsel);
      const int e0 = PER * tid;
      // only threads whose selected entries reach this split's slice (or that write idx_out)
      if (orow != nullptr || ((int)base < e_end && (int)(base + nsel) > e_begin)) {
        const auto sel = select_mask<PER>(key, nv, tau, take_eq);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          if ((sel >> j) & 1) {
            const int r = (int)(base + sel_rank(sel, j));
            if (r >= e_begin && r < e_end) scode[r - e_begin] = e0 + j;
            if (orow) orow[r] = e0 + j;
          }
        }
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  // per tile: whether any of its entries is masked (the softmax skips the masking otherwise)
  int* sflag = scode + per_split;
  for (int t = wv; t < ntiles; t += kAtWaves) {
    const int c = scode[kTile * t + (lane & 31)];
    const uint64_t bad = __ballot(c == -1);
    if (lane == 0) sflag[t] = bad != 0 ? 1 : 0;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();

  // row address of an entry code (masked entries read row 0 of the sequence; excluded in the
  // softmax)
  const uint16_t* kv_b = kv + (size_t)b * N * DK;
  const uint16_t* raw_b = kv_raw + (size_t)b * n_raw * DK;
  auto rowaddr = [&](int code) -> uint64_t {
    const uint64_t a = (uint64_t)(uintptr_t)(kv_b + (size_t)max(code, 0) * DK);
    const uint64_t r = (uint64_t)(uintptr_t)(raw_b + (size_t)max(-code - 2, 0) * DK);
    return code <= -2 ? r : a;
  };
  // DMAs of tile t, all issued by the value waves: wave 4 + v moves rows 8v .. 8v+7, one DMA
  // per 1024-byte latent part and one for the eight 128-byte rope parts (9 per tile). The
  // codes of the rows are read from LDS one tile ahead (fetch), so the issue never waits on
  // LDS. The CU's address unit takes a 1 KB DMA instruction in ~20 cycles and stalls the
  // issuing wave while its queue is full, so the DMAs go to the waves that are otherwise idle
  // while the score waves' S MFMAs run: the score waves issue no memory instruction in the loop.
  int nx_lat = -1, nx_rope = -1;
  const int vrow = 8 * (wv & 3);  // first tile row of a value wave's DMAs
  auto fetch = [&](int t) {
    if (!score_wave) {
      const int c0 = kTile * t + vrow;
      nx_lat = scode[c0 + (lane & 7)];
      nx_rope = scode[c0 + (lane >> 3)];
    }
  };
  uint32_t d_sbase = 0;
  uint64_t d_lat = 0;
  const uint16_t* d_rope = nullptr;
  int d_code = -1, d_rcode = -1;
  auto prep = [&](int t) {
    d_sbase = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)(smem + (t % NS) * kStage));
    d_lat = rowaddr(nx_lat);
    d_rope = reinterpret_cast<const uint16_t*>(rowaddr(nx_rope));
    d_code = nx_lat;
    d_rcode = nx_rope;
  };
  // DMA r of the prepared tile: r < 8 the latent part of row vrow + r, r == 8 the rope parts
  // of rows vrow .. vrow+7 (chunk c of row R at slot c ^ ((R >> 1) & 7)). With MXFP8 entries
  // only the raw window rows (bf16) come by DMA; the others are converted below.
  auto dma = [&](int r) {
    if (r < 8) {
      if (KV8 && __builtin_amdgcn_readlane(d_code, r) > -2) return;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)d_lat, r);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(d_lat >> 32), r);
      const uint16_t* src = reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src + 8 * lane),
          (lds_void_t*)(uintptr_t)(d_sbase + (vrow + r) * kLatStride), 16, 0, 0);
    } else {
      if (KV8 && d_rcode > -2) return;
      const int R = vrow + (lane >> 3);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(d_rope + 512 + 8 * ((lane & 7) ^ ((R >> 1) & 7))),
          (lds_void_t*)(uintptr_t)(d_sbase + kStageLat + vrow * 128), 16, 0, 0);
    }
  };
  constexpr int kDmas = 9;
  // MX entries (KV8): a value wave's 8 rows (8 CB code bytes, 144 scale bytes) come by DMA
  // into the staging buffers one iteration before they are needed (dma8); convert8 turns them
  // into bf16 in the ring stage, in the layout of the DMA'd rows.
  // Raw window rows (bf16) take the DMA above; masked entries convert row 0 (finite; P is 0).
  const uint8_t* kv8_b = reinterpret_cast<const uint8_t*>(kv) + (size_t)b * N * CB;
  const uint8_t* ksc_b = kv_scale + (size_t)b * N * (DK / 32);
  const uint32_t f8base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_void_t*)(sf8 + (KV8 ? vrow * CB : 0)));
  const uint32_t f8sbase = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_void_t*)(sf8s + (KV8 ? vrow * 18 : 0)));
  auto dma8 = [&](int codes) {  // lanes 0..7 of `codes`: the entry codes of rows vrow + 0..7
    constexpr int CPR = CB / 16, NCH = 8 * CPR;  // 16-byte chunks per row / per 8 rows
#pragma unroll
    for (int k = 0; k < (NCH + 63) / 64; ++k) {
      const int ch = 64 * k + lane, rr = ch / CPR, cc = ch - CPR * rr;
      const int code = __shfl(codes, min(rr, 7), 64);
      if (ch < NCH && code > -2)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(kv8_b + ((uint32_t)max(code, 0) * (uint32_t)CB + 16u * (uint32_t)cc)),
            (lds_void_t*)(uintptr_t)(f8base + 1024 * k), 16, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {  // 144 scale bytes, one dword each
      const int u = 64 * k + lane, rr = u / 18, sidx = u - 18 * rr;
      const int code = __shfl(codes, min(rr, 7), 64);
      if (u < 144 && code > -2)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(ksc_b + ((uint32_t)max(code, 0) * (uint32_t)(DK / 32) + (uint32_t)sidx)),
            (lds_void_t*)(uintptr_t)(f8sbase + 256 * k), 1, 0, 0);
    }
  };
  // d_code: the entry codes of the tile being converted (rows vrow + 0..7 in lanes 0..7).
  // Unit r < 8: the latent part of row vrow + r, lane l converting codes 8l .. 8l+7 (all
  // offsets are immediates off one lane base); then the rope parts, lane l converting codes
  // 512 + 8 (l & 7) .. of row vrow + (l >> 3). Eight e4m3 codes are 8 bytes, eight e2m1 codes
  // 4 (two per byte, low nibble first); either way 16 bytes of bf16.
  auto cvt8 = [&](const char* p, uint32_t e) -> u32x4_t {
    // E8M0 e -> 2^(e - 127) (e == 0 is the subnormal 2^-127)
    const float sc = __uint_as_float(e != 0u ? e << 23 : 0x00400000u);
    bf16x2_t p0, p1, p2, p3;
    if constexpr (KVF == 4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    } else {
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
      p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, false);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, true);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, false);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, true);
    }
    return u32x4_t{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                   __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
  };
  auto convert8 = [&](char* st) {
    constexpr int BPU = KVF == 4 ? 4 : 8;  // code bytes per unit of 8 codes
    const char* src = sf8 + (KV8 ? vrow * CB : 0);
    const uint32_t* ssrc = sf8s + (KV8 ? vrow * 18 : 0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (__builtin_amdgcn_readlane(d_code, r) > -2) {
        const uint32_t e = ssrc[r * 18 + (lane >> 2)] & 0xffu;
        *reinterpret_cast<u32x4_t*>(st + (vrow + r) * kLatStride + 16 * lane) =
            cvt8(src + r * CB + BPU * lane, e);
      }
    }
    {
      const int r = lane >> 3, c = lane & 7, R = vrow + r;
      if (__shfl(d_code, r, 64) > -2) {
        const uint32_t e = ssrc[r * 18 + 16 + (c >> 2)] & 0xffu;
        *reinterpret_cast<u32x4_t*>(st + kStageLat + R * 128 + 16 * (c ^ ((R >> 1) & 7))) =
            cvt8(src + r * CB + 64 * BPU + BPU * c, e);
      }
    }
    // the staging reads are done before the next dma8 overwrites the buffers
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto issue_all = [&]() {
    if (!score_wave)
#pragma unroll
      for (int r = 0; r < kDmas; ++r) dma(r);
  };
  // the ring runs NS-2 tiles ahead of the score waves: tiles 0 .. NS-3 now, tile i + NS - 2
  // during iteration i (into the stage the value waves finished with in iteration i-1)
#pragma unroll
  for (int t = 0; t < NS - 2; ++t)
    if (t < ntiles) {
      fetch(t);
      prep(t);
      issue_all();
      if constexpr (KV8)
        if (!score_wave) {
          dma8(d_code);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          convert8(smem + (t % NS) * kStage);
        }
    }
  if (NS - 2 < ntiles) fetch(NS - 2);
  if constexpr (KV8)
    if (!score_wave && NS - 2 < ntiles) dma8(nx_lat);  // the next tile's codes into staging
  // top of iteration i: wait until tile i has landed (tiles i+1 .. i+NS-3 may be in flight),
  // barrier, then form the addresses of tile i + NS - 2; returns whether its DMAs are due in
  // this iteration
  auto ring_top = [&](int i) -> bool {
    if (i < ntiles) {
      if (NS == 4 && i + 1 < ntiles && !score_wave) {
        wait_vm<kDmas>();
      } else {
        wait_vm<0>();
      }
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's P / flag writes
    }
    __builtin_amdgcn_s_barrier();
    if (i + NS - 2 < ntiles) {
      prep(i + NS - 2);
      if (i + NS - 1 < ntiles) fetch(i + NS - 1);
      return true;
    }
    return false;
  };
  // Each iteration is two phases split by a second barrier: first the score waves' S MFMAs
  // (alone on the matrix cores; the value waves issue their DMAs meanwhile), then the score
  // waves' softmax (VALU) overlapped with the value waves' P V MFMAs. Without it the two kinds
  // of MFMA interleave and the softmax runs after both, with the matrix cores idle.
  auto mid_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  if (score_wave) {
    // the score waves are the critical path of each iteration: their instructions (the S MFMAs
    // above all) issue ahead of the value waves', which fill the gaps
    __builtin_amdgcn_s_setprio(1);
    // complete the q loads here and make the values opaque: no wait for them inside the DMA
    // pipeline below, and no re-loading next to each use
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(qf[kk]));
    float m_run = kNegInf;  // per head n (same in the four lane groups)
    float l_run = 0.f;      // this lane's share: entries 4g.., 16+4g.. of every tile
    for (int i = 0; i <= ntiles; ++i) {
      ring_top(i);
      if (i == ntiles) {
        mid_barrier();
        break;
      }
      const char* sb = smem + (i % NS) * kStage;
      const i32x4_t cd0 = *reinterpret_cast<const i32x4_t*>(scode + kTile * i + 4 * g);
      const i32x4_t cd1 = *reinterpret_cast<const i32x4_t*>(scode + kTile * i + 16 + 4 * g);
      auto ld = [&](int R, int kk) -> u32x4_t {
        const char* ap;
        if (kk < 16) {
          ap = sb + R * kLatStride + 64 * kk + 16 * g;
        } else {
          const int c = 4 * (kk - 16) + g;
          ap = sb + kStageLat + R * 128 + ((c ^ ((R >> 1) & 7)) * 16);
        }
        return *reinterpret_cast<const u32x4_t*>(ap);
      };
      // S^T for entries 0..15 (sa) and 16..31 (sc), each over two accumulators (k-step parity)
      f32x4_t sa2[2], sc2[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) sa2[c] = sc2[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        constexpr int KB = 3;  // k-steps per block of reads, one block ahead of the MFMAs
        u32x4_t a0[KS], a1[KS];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          a0[kk] = ld(n, kk);
          a1[kk] = ld(16 + n, kk);
        }
#pragma unroll
        for (int blk = 0; blk < KS / KB; ++blk) {
          __builtin_amdgcn_sched_barrier(0);
          if (blk + 1 < KS / KB) {
#pragma unroll
            for (int kk = KB * blk + KB; kk < KB * blk + 2 * KB; ++kk) {
              a0[kk] = ld(n, kk);
              a1[kk] = ld(16 + n, kk);
            }
          }
#pragma unroll
          for (int kk = KB * blk; kk < KB * blk + KB; ++kk) {
            sa2[kk & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[kk]), as_bf16x8(qf[kk]), sa2[kk & 1], 0, 0, 0);
            sc2[kk & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[kk]), as_bf16x8(qf[kk]), sc2[kk & 1], 0, 0, 0);
          }
        }
      }
      mid_barrier();
      f32x4_t sa = sa2[0] + sa2[1], sc = sc2[0] + sc2[1];
      // lane (head n, g): raw scores of entries 4g+j (sa[j]) and 16+4g+j (sc[j]); masked
      // entries only in tiles whose flag says so (most tiles have none). The scale goes into
      // the exponent (one fma per entry); maxima are taken on the raw scores (scale > 0).
      if (__builtin_amdgcn_readfirstlane(sflag[i]) != 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sa[j] = cd0[j] != -1 ? sa[j] : kNegInf;
          sc[j] = cd1[j] != -1 ? sc[j] : kNegInf;
        }
      }
      float mx = vmax3(vmax3(sa[0], sa[1], sa[2]), vmax3(sa[3], sc[0], sc[1]), vmax(sc[2], sc[3]));
      mx = group_max_raw(mx) * scale_log2;
      // Lazily moved softmax reference: m_run only moves (and the value waves rescale their
      // accumulators) when a head's tile maximum exceeds it by more than kRefSlack (log2
      // units), so p <= 2^kRefSlack.
      const bool grow = mx > m_run + kRefSlack;
      const bool moved = __ballot(grow) != 0;
      if (moved) {
        const float m_new = grow ? mx : m_run;
        const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        if (g == 0) abuf[i & 1][hb][n] = alpha;
      }
      if (lane == 0) fbuf[i & 1][hb] = moved ? 1u : 0u;
      // m_run is -inf only while every entry so far is masked (all scores -inf): any finite
      // reference then gives exp2(-inf) = 0
      const float mneg = m_run == kNegInf ? 0.f : -m_run;
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float za = j < 2 ? sa[2 * j] : sc[2 * j - 4];
        const float zb = j < 2 ? sa[2 * j + 1] : sc[2 * j - 3];
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(za, scale_log2, mneg));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(zb, scale_log2, mneg));
        l_run += e0 + e1;
        pk[j] = pack_bf16x2(e0, e1);
      }
      pbuf[i & 1][hb][lane] = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
    }
    // final (m, l) per head for the value waves, and lse / the split's (m, l)
    const float l_head = group_sum(l_run);
    if (g == 0) {
      if (nsplit == 1) {
        // the sink logit joins the denominator (zero value vector); the value waves scale
        // their accumulators (relative to m_run) by 2^(m_run - M) / L
        float M, L;
        join_sink(m_run, l_head, sink != nullptr ? sink[h0 + n] * kLog2e : kNegInf, M, L);
        sml[hb][1][n] = (L > 0.f && m_run != kNegInf) ? __builtin_amdgcn_exp2f(m_run - M) / L : 0.f;
        if (lse) lse[(size_t)qi * H + h0 + n] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
      } else {
        const size_t hrow = ((size_t)row * H + h0 + n) * nsplit + split;
        part_ml[hrow * kMlStride] = m_run;
        part_ml[hrow * kMlStride + 1] = l_head;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    return;
  }

  // ---- value waves: wave 4 + v owns every head block (64 heads) and value columns
  // 128*v .. +127, so each pair of transposed V reads feeds four MFMAs ----
  const int vw = wv - 4;
  constexpr int DH = DB / 4;  // 8 column blocks of this wave
  f32x4_t acc[4][DH];         // [head block k][column block 8*vw + d]: heads 4g+j, col n
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[k][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // transposed V reads: entry 4g + n/4 (and 16 rows on), column 128*vw + 16d + 4*(n%4)
  const uint32_t voff = (4 * g + (n >> 2)) * kLatStride + 256 * vw + 8 * (n & 3);
  // KV8, iteration i (ring_top has waited for every DMA of this wave and prepared tile
  // i + NS - 2): convert that tile's staged codes into its stage, then stage the codes of the
  // tile after it (whose entry codes fetch() read into nx_lat)
  auto kv8_phase1 = [&](int i) {
    convert8(smem + ((i + NS - 2) % NS) * kStage);
    if (i + NS - 1 < ntiles) dma8(nx_lat);
  };
  for (int i = 0; i <= ntiles; ++i) {
    // the value waves issue their DMAs while the score waves' S MFMAs run; P, the moved flags
    // and the rescale factors are read first, so their LDS round trip hides under the issue
    const bool due = ring_top(i);
    if (i == 0) {
      if constexpr (KV8)
        if (due) kv8_phase1(i);
      if (due) issue_all();
      mid_barrier();
      continue;
    }
    const int t = i - 1;
    bf16x8_t pa[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pa[k] = as_bf16x8(pbuf[t & 1][k][lane]);
    const u32x4_t moved = *reinterpret_cast<const u32x4_t*>(&fbuf[t & 1][0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KV8)
      if (due) kv8_phase1(i);
    if (due) issue_all();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (__builtin_amdgcn_readfirstlane(moved[k]) != 0) {
        const f32x4_t alpha = *reinterpret_cast<const f32x4_t*>(&abuf[t & 1][k][4 * g]);
#pragma unroll
        for (int d = 0; d < DH; ++d) acc[k][d] *= alpha;
      }
    }
    mid_barrier();
    const uint32_t vaddr = (uint32_t)(uintptr_t)(lds_void_t*)(smem + (t % NS) * kStage) + voff;
    u32x2_t x0, x1, y0, y1;
    pv_first2(vaddr, x0, x1, y0, y1);
    // the transposed reads of blocks d+2, d+3 run under the MFMAs of blocks d, d+1
#define DSA_PV2(D)                                                                              \
    {                                                                                           \
      f32x4_t ca[4] = {acc[0][D], acc[1][D], acc[2][D], acc[3][D]};                             \
      f32x4_t cb[4] = {acc[0][D + 1], acc[1][D + 1], acc[2][D + 1], acc[3][D + 1]};             \
      u32x2_t nx0, nx1, ny0, ny1;                                                               \
      pv_step2<D>(ca, cb, pa, u32x4_t{x0[0], x0[1], x1[0], x1[1]},                              \
                  u32x4_t{y0[0], y0[1], y1[0], y1[1]}, vaddr, nx0, nx1, ny0, ny1);              \
      for (int k = 0; k < 4; ++k) {                                                             \
        acc[k][D] = ca[k];                                                                      \
        acc[k][D + 1] = cb[k];                                                                  \
      }                                                                                         \
      x0 = nx0; x1 = nx1; y0 = ny0; y1 = ny1;                                                   \
    }
    DSA_PV2(0) DSA_PV2(2) DSA_PV2(4) DSA_PV2(6)
#undef DSA_PV2
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();  // the score waves' final (m, l) are in sml
  if (nsplit == 1) {
    // normalise, round to bf16 and stage this wave's 64 x 128 block through the (idle) ring
    // memory (a region of its own) so that each output row is written with 16-byte stores
    uint16_t* so = reinterpret_cast<uint16_t*>(smem) + vw * 64 * (128 + 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float inv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) inv[j] = sml[k][1][4 * g + j];
#pragma unroll
      for (int d = 0; d < DH; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          so[(16 * k + 4 * g + j) * (128 + 8) + 16 * d + n] = f32_to_bf16(acc[k][d][j] * inv[j]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // 64 rows x 256 bytes: 16 chunks of 16 bytes per lane
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = lane + 64 * k, r = c >> 4, col = (c & 15) * 8;
      *reinterpret_cast<u32x4_t*>(out + ((size_t)qi * H + hg * 64 + r) * DV + 128 * vw + col) =
          *reinterpret_cast<const u32x4_t*>(so + r * (128 + 8) + col);
    }
  } else {
    // O partials (relative to this split's m) as fp16, each head's 128 columns divided by their
    // largest magnitude c (so every value lies in [-1, 1]; c goes beside the split's (m, l)), in
    // register order: [row][head group][split][slot 8][16 column blocks][64 lanes] x 4 heads
    // (4g..4g+3 of column 16d + n); slot = head block + 4 * (column half). 512-byte stores.
    f16x4_t* po = part_o + (((size_t)row * HG + hg) * nsplit + split) * 8 * 16 * 64 + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float c[4] = {0.f, 0.f, 0.f, 0.f}, inv[4];
#pragma unroll
      for (int d = 0; d < DH; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = fmaxf(c[j], fabsf(acc[k][d][j]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = row16_max(c[j]);  // over the 16 columns n of the lane group
        inv[j] = c[j] > 0.f ? 1.f / c[j] : 0.f;
      }
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        const f32x4_t a = acc[k][d] * f32x4_t{inv[0], inv[1], inv[2], inv[3]};
        po[((k + 4 * (vw >> 1)) * 16 + 8 * (vw & 1) + d) * 64] = __builtin_convertvector(a, f16x4_t);
      }
      if (n < 4) {
        const float cn = n == 0 ? c[0] : n == 1 ? c[1] : n == 2 ? c[2] : c[3];
        const size_t hrow = ((size_t)row * H + hg * 64 + k * 16 + 4 * g + n) * nsplit + split;
        part_ml[hrow * kMlStride + 2 + vw] = cn;
      }
    }
  }
}

// Merge split partials: out = sum_s w_s O_s, w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s,
// M = max_s m_s, with O_s = c_s x (its fp16 partial). One workgroup per (wave slot, column
// quarter, head group, row): 16 heads x 128 columns, a quarter of the block one value wave of
// attend_mfma_dma writes per split. Every partial is loaded before the first use (up to 32
// splits: 64 f16x4 per thread); the bf16 result goes through LDS so that each row of the output
// is written with 16-byte stores.
constexpr int kMaxSplits = 32;
__global__ __launch_bounds__(256) void attend_combine(
    const f16x4_t* __restrict__ part_o, const float* __restrict__ part_ml, int64_t qi0, int H,
    int nsplit, uint16_t* __restrict__ out, float* __restrict__ lse, int nitems,
    const float* __restrict__ sink) {
  constexpr int DV = 512;
  __shared__ float wsc[kMaxSplits][16];
  __shared__ __attribute__((aligned(16))) uint16_t sout[16][128 + 8];
  const int HG = H / 64;
  const int item = xcd_item(blockIdx.x + 16 * (blockIdx.y + HG * blockIdx.z), nitems);
  const int ws = (item & 15) >> 1, cq = item & 1, hg = (item >> 4) % HG;
  const int64_t row = item / (16 * HG);
  const int64_t qi = qi0 + row;
  const int h0 = hg * 64 + 16 * (ws & 3), c0 = 256 * (ws >> 2) + 128 * cq;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 4, n = lane & 15;
  // column blocks 8 cq + (tid >> 6) + 4 k of the wave slot's 256 columns
  const f16x4_t* base = part_o + (((size_t)row * HG + hg) * nsplit * 8 + ws) * 16 * 64;
  f16x4_t v[2][kMaxSplits];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int d = 8 * cq + (tid >> 6) + 4 * k;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      v[k][s] = s < nsplit ? base[(size_t)s * 8 * 16 * 64 + d * 64 + lane] : f16x4_t{0, 0, 0, 0};
  }
  // thread (head hh, sl) holds the (m, l, c) of splits sl and sl + 16
  const int hh = tid >> 4, sl = tid & 15;
  float ml_m[2] = {kNegInf, kNegInf}, ml_l[2] = {0.f, 0.f}, ml_c[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = sl + 16 * j;
    if (s < nsplit) {
      const size_t hrow = ((size_t)row * H + h0 + hh) * nsplit + s;
      ml_m[j] = part_ml[hrow * kMlStride];
      ml_l[j] = part_ml[hrow * kMlStride + 1];
      ml_c[j] = part_ml[hrow * kMlStride + 2 + 2 * (ws >> 2) + cq];  // scale of this column quarter
    }
  }
  // per head: M = max_s m_s, L = sum_s 2^(m_s - M) l_s, over the 16 lanes of each head
  float M = fmaxf(ml_m[0], ml_m[1]);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float wm[2], L = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    wm[j] = ml_m[j] == kNegInf ? 0.f : exp2f(ml_m[j] - M);
    L += wm[j] * ml_l[j];
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) L += __shfl_xor(L, o, 64);
  // the sink logit joins the denominator (zero value vector): reference M2, total L2
  float M2, L2;
  join_sink(M, L, sink != nullptr ? sink[h0 + hh] * kLog2e : kNegInf, M2, L2);
  const float shift = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - M2);
#pragma unroll
  for (int j = 0; j < 2; ++j) wsc[sl + 16 * j][hh] = L2 > 0.f ? wm[j] * shift / L2 * ml_c[j] : 0.f;
  if (sl == 0 && cq == 0 && lse)
    lse[(size_t)qi * H + h0 + hh] = L2 > 0.f ? (M2 + __log2f(L2)) * kLn2 : kNegInf;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int d = (tid >> 6) + 4 * k;  // column block within this quarter
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s < nsplit) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] += wsc[s][4 * g + i] * (float)v[k][s][i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sout[4 * g + i][16 * d + n] = f32_to_bf16(a[i]);
  }
  __syncthreads();
  // 16 rows x 256 bytes: one chunk of 16 bytes per thread
  {
    const int r = tid >> 4, col = (tid & 15) * 8;
    *reinterpret_cast<u32x4_t*>(out + ((size_t)qi * H + h0 + r) * DV + c0 + col) =
        *reinterpret_cast<const u32x4_t*>(&sout[r][col]);
  }
}

template <typename T>
__device__ __forceinline__ float ldv(const T* p, size_t i) {
  if constexpr (sizeof(T) == 2)
    return bf16_to_f32(p[i]);
  else
    return p[i];
}

// One OCP E4M3 (E4M3FN) code: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
// holds the subnormals m/8 * 2^-6; 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, mt = c & 7u;
  float v = e == 0u ? (float)mt * 0.001953125f                        // m/8 * 2^-6
                    : __uint_as_float(((e + 120u) << 23) | (mt << 20));  // (1 + m/8) 2^(e-7)
  if (e == 15u && mt == 7u) v = __builtin_nanf("");
  return (c & 0x80u) ? -v : v;
}

// One OCP E2M1 code (a nibble): sign, 2 exponent bits, 1 mantissa bit; magnitudes 0, 0.5, 1,
// 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, mt = c & 1u;
  const float v = e == 0u ? 0.5f * (float)mt : __uint_as_float(((e + 126u) << 23) | (mt << 22));
  return (c & 8u) ? -v : v;
}

// E8M0 scale byte e -> 2^(e - 127) (e == 0: the subnormal 2^-127; 0xFF is NaN)
__device__ __forceinline__ float e8m0_value(uint32_t e) {
  if (e == 255u) return __builtin_nanf("");
  return __uint_as_float(e != 0u ? e << 23 : 0x00400000u);
}

template <typename T>
__global__ __launch_bounds__(256) void attend_generic(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ idx,
    const T* __restrict__ kv_raw, int64_t raw_base, int64_t n_raw,
    const int32_t* __restrict__ q_pos, int T_, int N, int H, int DK, int DV, int top_k, int W,
    float scale, int64_t qi0, T* __restrict__ out, float* __restrict__ lse, int m,
    const int32_t* __restrict__ seq_len, const float* __restrict__ sink,
    const uint8_t* __restrict__ kv_scale, int kv4) {
  // kv_scale != nullptr: kv holds MX entries, e4m3 codes [B, N, DK] (kv4 == 0) or e2m1 code
  // pairs [B, N, DK / 2] (low nibble first), and E8M0 scales [B, N, DK / 32]; kv_raw rows stay
  // in T
  auto code_value = [&](size_t r8, int d) -> float {
    const uint8_t* kv8 = reinterpret_cast<const uint8_t*>(kv);
    return kv4 ? e2m1_value((uint32_t)(kv8[r8 * (DK / 2) + d / 2] >> (4 * (d & 1))) & 15u)
               : e4m3_value(kv8[r8 * DK + d]);
  };
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int E = top_k + W;
  float* sq = reinterpret_cast<float*>(smem);   // [DK]
  float* sz = sq + DK;                           // [E]
  const T** ssrc = reinterpret_cast<const T**>(sz + E + ((E & 1) ? 1 : 0));  // [E]
  int* srow8 = reinterpret_cast<int*>(ssrc + E);  // [E]: MX entry row, or -1
  __shared__ float red[256 / 64];
  const int h = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int64_t qi = qi0 + row;
  const int b = (int)(qi / T_);
  const int p = q_pos[qi];
  const int32_t* idxrow = idx != nullptr ? idx + row * (int64_t)top_k : nullptr;
  const int lim = idx != nullptr ? N : n_visible(p, m, N, seq_len, b);
  for (int d = threadIdx.x; d < DK; d += blockDim.x) sq[d] = ldv(q, ((size_t)qi * H + h) * DK + d);
  __syncthreads();
  float mx = kNegInf;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const T* src = entry_row<T>(e, idxrow, top_k, kv, b, N, DK, kv_raw, raw_base, n_raw, p, W, lim);
    int r8 = -1;
    if (kv_scale != nullptr && src != nullptr && e < top_k) {
      // an entry of kv: its row, read below as codes and scales
      r8 = (int)((src - kv) / DK);
      src = nullptr;
    }
    ssrc[e] = src;
    srow8[e] = r8;
    float z = kNegInf;
    if (src) {
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < DK; ++d) dot += sq[d] * ldv(src, d);  // 8 loads in flight at a time
      z = dot * scale;
    } else if (r8 >= 0) {
      const uint8_t* s8 = kv_scale + (size_t)r8 * (DK / 32);
      float dot = 0.f;
      for (int d0 = 0; d0 < DK; d0 += 32) {
        float blk = 0.f;
#pragma unroll 8
        for (int d = d0; d < d0 + 32; ++d) blk += sq[d] * code_value((size_t)r8, d);
        dot += blk * e8m0_value(s8[d0 / 32]);
      }
      z = dot * scale;
    }
    sz[e] = z;
    mx = fmaxf(mx, z);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  // the sink logit (zero value vector) joins the softmax
  const float sk = sink != nullptr ? sink[h] : kNegInf;
  mx = sk;
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
  sum = sk != kNegInf ? __expf(sk - mx) : 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) sum += red[i];
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int d = threadIdx.x; d < DV; d += blockDim.x) {
    float a = 0.f;
#pragma unroll 8
    for (int e = 0; e < E; ++e) {
      if (ssrc[e]) {
        a += sz[e] * ldv(ssrc[e], d);
      } else if (srow8[e] >= 0) {
        const size_t r8 = (size_t)srow8[e];
        a += sz[e] * (code_value(r8, d) * e8m0_value(kv_scale[r8 * (DK / 32) + d / 32]));
      }
    }
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
  // at least 256 entries per split (each workgroup's prologue is a fixed cost); 128, then 64,
  // when even that leaves most of the GPU idle (a handful of rows, as in long-context CSA
  // decode)
  const int min_per = wgs * ((E + 255) / 256) >= 256 ? 256 : wgs * ((E + 127) / 128) >= 256 ? 128 : 64;
  int64_t maxs = (E + min_per - 1) / min_per;
  int64_t ns = want < maxs ? want : maxs;
  if (ns > kMaxSplits) ns = kMaxSplits;
  return ns < 1 ? 1 : (int)ns;
}

size_t attend_ws_bytes(const Shape& s, int64_t nrows, int fmt) {
  const int ns = attend_splits(s, nrows, fmt);
  if (ns <= 1) return 0;
  // fp16 O partials, then (m, l, c_0 .. c_3) per split
  return (size_t)nrows * s.H * ns * ((size_t)s.D_V * 2 + kMlStride * sizeof(float));
}

// Dynamic LDS the attention kernels may take beside their static LDS (the ring and its
// buffers), set as each kernel's attribute on every device it runs on, once per device.
struct AttendLds {
  hipError_t err;
  size_t dyn4, dyn3, dyn3_kv8, dyn3_kv4;
};

static const AttendLds& attend_lds() {
  constexpr size_t kLdsMax = 160 * 1024;
  static AttendLds per_dev[64];
  static std::once_flag once[64];
  static const AttendLds bad{hipErrorInvalidDevice, 0, 0, 0, 0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return bad;
  std::call_once(once[dev], [dev] {
    AttendLds& r = per_dev[dev];
    r.err = hipSuccess;
    const void* k4[] = {reinterpret_cast<const void*>(&attend_mfma_dma<4, 0, 0>),
                        reinterpret_cast<const void*>(&attend_mfma_dma<4, 16, 0>),
                        reinterpret_cast<const void*>(&attend_mfma_dma<4, 64, 0>)};
    const void* k3[] = {reinterpret_cast<const void*>(&attend_mfma_dma<3, 0, 0>),
                        reinterpret_cast<const void*>(&attend_mfma_dma<3, 16, 0>),
                        reinterpret_cast<const void*>(&attend_mfma_dma<3, 64, 0>)};
    const void* k3x[] = {reinterpret_cast<const void*>(&attend_mfma_dma<3, 0, 8>),
                         reinterpret_cast<const void*>(&attend_mfma_dma<3, 16, 8>),
                         reinterpret_cast<const void*>(&attend_mfma_dma<3, 64, 8>)};
    const void* k3x4[] = {reinterpret_cast<const void*>(&attend_mfma_dma<3, 0, 4>),
                          reinterpret_cast<const void*>(&attend_mfma_dma<3, 16, 4>),
                          reinterpret_cast<const void*>(&attend_mfma_dma<3, 64, 4>)};
    auto room = [&](const void* const* ks, size_t& dyn) {
      dyn = kLdsMax;
      for (int j = 0; j < 3 && r.err == hipSuccess; ++j) {
        hipFuncAttributes fa;
        r.err = hipFuncGetAttributes(&fa, ks[j]);
        if (r.err == hipSuccess)
          dyn = fa.sharedSizeBytes < kLdsMax ? std::min(dyn, kLdsMax - fa.sharedSizeBytes) : 0;
      }
      for (int j = 0; j < 3 && r.err == hipSuccess; ++j)
        r.err = hipFuncSetAttribute(ks[j], hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    };
    room(k4, r.dyn4);
    room(k3, r.dyn3);
    room(k3x, r.dyn3_kv8);
    room(k3x4, r.dyn3_kv4);
  });
  return per_dev[dev];
}

// The MFMA attention for rows qi0 .. qi0+nrows-1 (+ the split merge). scores != nullptr selects
// the fused top-k variant (entries straight from the indexer scores, idx_out optional).
static hipError_t launch_attend_mfma(const Shape& s, int64_t qi0, int64_t nrows, const void* q,
                                     const void* kv, const uint8_t* kv_scale, int kv_fmt,
                                     const int32_t* idx, const float* scores,
                                     int32_t* idx_out, const void* kv_raw, int64_t raw_base,
                                     int64_t n_raw, const int32_t* q_pos,
                                     const int32_t* seq_len, const float* sink, float scale,
                                     void* out, float* lse, void* ws, hipStream_t st) {
  const int ns = attend_splits(s, nrows, FMT_BF16);
  const int E = s.top_k + s.W;
  const int per = ((E + ns - 1) / ns + kTile - 1) / kTile * kTile;
  f16x4_t* part_o = static_cast<f16x4_t*>(ws);
  float* part_ml = ns > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                     (size_t)nrows * s.H * ns * s.D_V * 2)
                          : nullptr;
  dim3 grid(ns, s.H / 64, (unsigned)nrows);
  // dynamic LDS: the entry codes (per is a multiple of the tile) and one flag per tile, beside
  // the static ring: a 4-stage ring when they fit in the 160 KB a workgroup can hold, else 3
  const size_t code_bytes = sizeof(int) * ((size_t)per + per / kTile);
  const AttendLds& lds = attend_lds();
  if (lds.err != hipSuccess) return lds.err;
  const int nitems = (int)(ns * (s.H / 64) * nrows);
  const int per_thread = scores == nullptr ? 0 : (s.N <= 16 * kAtWaves * 64 ? 16 : 64);
  if (scores != nullptr && s.N > 64 * kAtWaves * 64) return hipErrorInvalidValue;
  hipError_t e;
#define DSA_ATT2(NS_, PER_, KVF_)                                                                \
  e = launch(attend_mfma_dma<NS_, PER_, KVF_>, grid, kAtWaves * 64, code_bytes, st,              \
             static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,             \
             static_cast<const uint16_t*>(kv_raw), raw_base, n_raw, q_pos, s.T, s.N, s.H,        \
             s.top_k, s.W, scale * kLog2e, qi0, ns, per, static_cast<uint16_t*>(out), lse,       \
             part_o, part_ml, nitems, scores, s.m, idx_out, seq_len, sink, kv_scale)
#define DSA_ATT(NS_, PER_) DSA_ATT2(NS_, PER_, 0)
  if (kv_scale != nullptr && kv_fmt == FMT_MXFP4) {
    // MX entries: the 3-stage ring beside the code staging buffer
    if (code_bytes > lds.dyn3_kv4) return hipErrorInvalidValue;
    if (per_thread == 0) DSA_ATT2(3, 0, 4);
    else if (per_thread == 16) DSA_ATT2(3, 16, 4);
    else DSA_ATT2(3, 64, 4);
  } else if (kv_scale != nullptr) {
    if (code_bytes > lds.dyn3_kv8) return hipErrorInvalidValue;
    if (per_thread == 0) DSA_ATT2(3, 0, 8);
    else if (per_thread == 16) DSA_ATT2(3, 16, 8);
    else DSA_ATT2(3, 64, 8);
  } else if (code_bytes <= lds.dyn4) {
    if (per_thread == 0) DSA_ATT(4, 0);
    else if (per_thread == 16) DSA_ATT(4, 16);
    else DSA_ATT(4, 64);
  } else if (code_bytes <= lds.dyn3) {
    if (per_thread == 0) DSA_ATT(3, 0);
    else if (per_thread == 16) DSA_ATT(3, 16);
    else DSA_ATT(3, 64);
  } else {
    return hipErrorInvalidValue;
  }
#undef DSA_ATT
#undef DSA_ATT2
  if (e != hipSuccess || ns == 1) return e;
  return launch(attend_combine, dim3(16, s.H / 64, (unsigned)nrows), 256, 0, st, part_o, part_ml,
                qi0, s.H, ns, static_cast<uint16_t*>(out), lse, (int)(16 * (s.H / 64) * nrows),
                sink);
}

// Each of a row's workgroups (splits x head groups) repeats the row's selection in its
// prologue, which pays only while the separate top-k launch is a large share of the step: a
// few rows (decode), not a prefill chunk, where it would double the selection work.
constexpr int64_t kFusedMaxRows = 128;

bool attend_fused_ok(const Shape& s, int fmt, int64_t nrows) {
  return mfma_ok(s, fmt) && s.N <= 64 * kAtWaves * 64 && nrows <= kFusedMaxRows;
}

hipError_t launch_attend_fused(const Shape& s, int64_t qi0, int64_t nrows, const void* q,
                               const void* kv, const uint8_t* kv_scale, int kv_fmt,
                               const float* scores, int32_t* idx_out, const void* kv_raw,
                               int64_t raw_base,
                               int64_t n_raw, const int32_t* q_pos, const int32_t* seq_len,
                               const float* sink, float scale, void* out, float* lse, void* ws,
                               hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  if (!attend_fused_ok(s, FMT_BF16, nrows)) return hipErrorInvalidValue;
  return launch_attend_mfma(s, qi0, nrows, q, kv, kv_scale, kv_fmt, nullptr, scores, idx_out, kv_raw,
                            raw_base, n_raw, q_pos, seq_len, sink, scale, out, lse, ws, st);
}

hipError_t launch_attend(const Shape& s, int64_t qi0, int64_t nrows, int fmt, const void* q,
                         const void* kv, const uint8_t* kv_scale, int kv_fmt,
                         const int32_t* idx, const void* kv_raw, int64_t raw_base, int64_t n_raw,
                         const int32_t* q_pos, const int32_t* seq_len, const float* sink,
                         float scale, void* out, float* lse, void* ws, hipStream_t st) {
  if (nrows <= 0) return hipSuccess;
  if (mfma_ok(s, fmt))
    return launch_attend_mfma(s, qi0, nrows, q, kv, kv_scale, kv_fmt, idx, nullptr, nullptr, kv_raw,
                              raw_base, n_raw, q_pos, seq_len, sink, scale, out, lse, ws, st);
  const int E = s.top_k + s.W;
  size_t shm = sizeof(float) * (s.D_K + E + 1) + sizeof(void*) * E + sizeof(int) * E + 16;
  dim3 grid(s.H, (unsigned)nrows);
  if (fmt == FMT_BF16)
    return launch(attend_generic<uint16_t>, grid, 256, shm, st, static_cast<const uint16_t*>(q),
                  static_cast<const uint16_t*>(kv), idx, static_cast<const uint16_t*>(kv_raw),
                  raw_base, n_raw, q_pos, s.T, s.N, s.H, s.D_K, s.D_V, s.top_k, s.W, scale, qi0,
                  static_cast<uint16_t*>(out), lse, s.m, seq_len, sink, kv_scale,
                  kv_fmt == FMT_MXFP4 ? 1 : 0);
  return launch(attend_generic<float>, grid, 256, shm, st, static_cast<const float*>(q),
                static_cast<const float*>(kv), idx, static_cast<const float*>(kv_raw), raw_base,
                n_raw, q_pos, s.T, s.N, s.H, s.D_K, s.D_V, s.top_k, s.W, scale, qi0,
                static_cast<float*>(out), lse, s.m, seq_len, sink, kv_scale,
                kv_fmt == FMT_MXFP4 ? 1 : 0);
}

}  // namespace dsa
