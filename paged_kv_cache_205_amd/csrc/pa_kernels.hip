// pa_kernels.hip - gfx950 kernels for paged decode attention and the one-token
// KV append.  Host-side argument checks live in pa_api.cpp.
//
// Sources for what is computed (web pages describing the samir-vllm teaching
// engine):
//   [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
//            Inference - Start here" (memedata.com copy of the project README),
//            feature list: KV page pool item, paged decode attention item.
//   [ARCH]   "samir-vllm: Build LLM Inference From Scratch in C++ and CUDA"
//            (wpnews.pro), "Architecture walkthrough", KV cache paragraph.
//
// Pool plane layout: bf16 [num_pages][16 tokens][8 kv heads][64].  One token row
// of a page is 1 KiB; one (token, kv head) row is 128 contiguous bytes, so the
// K (or V) tile of one kv head in one page is 16 full 128-byte lines.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

#include <algorithm>
#include <atomic>

namespace pa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0): all LDS (and scalar) reads of this wave have returned.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Lane I of each quad of 4 lanes, to all 4 (DPP quad_perm [I, I, I, I]).
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), I * 0x55, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_read(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ---------------------------------------------------------------------------
// pa_append: one wave per sequence; each lane copies 16 bytes of the 1 KiB K
// row and 16 bytes of the 1 KiB V row of position L-1.

__global__ __launch_bounds__(256) void append_kernel(const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new,
                                                     uint16_t* __restrict__ k_pool,
                                                     uint16_t* __restrict__ v_pool,
                                                     const int32_t* __restrict__ block_table,
                                                     int max_blocks, const int32_t* __restrict__ seq_lens,
                                                     int B) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  const int L = seq_lens[b];
  if (L <= 0) return;
  const int pos = L - 1;
  const size_t page = (size_t)block_table[(size_t)b * max_blocks + (pos >> 4)];
  const size_t dst = (page * kPageTokens + (pos & 15)) * kRowElems + lane * 8;
  const size_t src = (size_t)b * kRowElems + lane * 8;
  *reinterpret_cast<u32x4*>(k_pool + dst) = ld16(k_new + src);
  *reinterpret_cast<u32x4*>(v_pool + dst) = ld16(v_new + src);
}

// ---------------------------------------------------------------------------
// pa_fill: a run of consecutive tokens per sequence into its pages.  Each wave
// moves 2 consecutive source rows (16 bytes of the K row and of the V row per
// lane), and the grid gives every pair of rows a wave of its own: on the
// 64 x 2047-row prompts that streams 7% faster than waves looping over 4 rows
// each on a grid of 8 workgroups per CU.  The run boundaries are staged in LDS
// and the sequence of a token found by binary search.  Rows whose position or
// page falls outside the table or the pool are skipped (the caller's contract
// excludes them).

constexpr int kFillRowsPerWave = 2;

__global__ __launch_bounds__(256) void fill_kernel(FillArgs a) {
  extern __shared__ int s_cu[];  // [B + 1]
  for (int i = threadIdx.x; i <= a.B; i += 256) s_cu[i] = a.cu_tokens[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int nchunk = (a.T + kFillRowsPerWave - 1) / kFillRowsPerWave;
  for (int c = blockIdx.x * 4 + (threadIdx.x >> 6); c < nchunk; c += gridDim.x * 4) {
    const int t0 = c * kFillRowsPerWave;
    int lo = 0, hi = a.B;  // largest b with cu[b] <= t0, for cu[0] = 0 <= t0 < cu[B] = T
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cu[mid] <= t0) lo = mid; else hi = mid;
    }
    int b = __builtin_amdgcn_readfirstlane(lo);
    u32x4 kr[kFillRowsPerWave], vr[kFillRowsPerWave];
    size_t dst[kFillRowsPerWave];
    bool ok[kFillRowsPerWave];
#pragma unroll
    for (int u = 0; u < kFillRowsPerWave; ++u) {
      const int t = t0 + u;
      ok[u] = false;
      dst[u] = 0;
      if (t < a.T) {
        while (b + 1 < a.B && s_cu[b + 1] <= t) ++b;  // runs may be empty
        const int pos = (a.start ? a.start[b] : 0) + (t - s_cu[b]);
        if (pos >= 0 && (pos >> 4) < a.max_blocks) {
          const int page = a.block_table[(size_t)b * a.max_blocks + (pos >> 4)];
          if (page >= 0 && page < a.num_pages) {
            ok[u] = true;
            dst[u] = ((size_t)page * kPageTokens + (pos & 15)) * kRowElems + lane * 8;
          }
        }
        kr[u] = ld16(a.k_src + (size_t)t * kRowElems + lane * 8);
        vr[u] = ld16(a.v_src + (size_t)t * kRowElems + lane * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kFillRowsPerWave; ++u)
      if (ok[u]) {
        __builtin_nontemporal_store(kr[u], reinterpret_cast<u32x4*>(a.k_pool + dst[u]));
        __builtin_nontemporal_store(vr[u], reinterpret_cast<u32x4*>(a.v_pool + dst[u]));
      }
  }
}

// ---------------------------------------------------------------------------
// pa_decode
//
// Work decomposition.  A sequence of npages pages is cut into
// nsplit = ceil(npages / part_pages) splits; split s owns the pages
// s, s + nsplit, s + 2*nsplit, ... (pages are dealt round-robin, so the
// workgroups of one sequence stream neighbouring pages at the same time).  The
// split count depends only on the sequence's own length.  One workgroup of 8
// waves handles one (sequence, split); wave g handles kv head g, i.e. query
// heads 4g..4g+3, so each page's K and V are read once for the 4 query heads
// that share them, and the 8 waves together read whole pages.
//
// Memory path.  Each wave streams its head's 2 KiB K tile and 2 KiB V tile of a
// page straight into its own LDS ring slot with global_load_lds_dwordx4
// (non-temporal): every load instruction covers 8 complete 128-byte lines.
// Inside a tile, token row tau keeps its eight 16-byte chunks in a permuted order
// (chunk C at position C ^ swz(tau)) so that the reads below are bank-conflict
// free.  kRing slots per wave keep kRing pages in flight.
//
// Arithmetic (per page, per wave).
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (two, for D = 64): A = K tile
//   (row = token), B = Q^T with the 4 query heads repeated over the 16 columns.
//   Lane l = 16c + t then holds, in result register r, the score of token
//   4c + r for query head t % 4.  BF16 x BF16 products are exact in FP32.
//   Online softmax in FP32 (base 2, log2(e) folded into the scale): a running
//   maximum per head, the same in every lane of that head, is raised only when
//   a score exceeds it (then the accumulators are rescaled).
//   PV on v_mfma_f32_16x16x16_bf16: A = the weights of the lane's 4 tokens for
//   its head, B = V transposed (read as 16-bit elements from the LDS tile).
//   The FP32 weight p is split into p_hi = bf16 truncation of p and
//   p_lo = bf16 truncation of (p - p_hi); two MFMAs accumulate p_hi V + p_lo V
//   in FP32, which represents p to about 2^-14 relative.  Result register r of
//   tile n holds out[head r][16n + t].
//
// Splits.  A single-split sequence writes out directly.  Otherwise each split
// stores its partial state (o = acc / l, m, l per query head) in the workspace,
// and for each KV head the last wave of the sequence's splits to finish (one
// atomic counter per sequence and KV head) merges that head's 4 query heads:
// out = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m).

#ifndef PA_RING_PAGES
#define PA_RING_PAGES 2
#endif
// Build-time switch for the PV product: 0 (default) MFMA with hi/lo bf16
// weights, 1 FP32 FMAs on the VALU (kept for the measured comparison).
#ifndef PA_DECODE_PV_VALU
#define PA_DECODE_PV_VALU 0
#endif
constexpr int kRing = PA_RING_PAGES;                     // LDS slots (pages in flight) per wave
constexpr int kTileBytes = kPageTokens * kHeadDim * 2;   // one head's K or V rows of a page
constexpr int kSlotBytes = 2 * kTileBytes;               // K tile then V tile

// Position permutation of the 16-byte chunks inside LDS token row tau.
__device__ __forceinline__ int swz(int tau) { return (tau & 7) ^ ((tau >> 3) << 1); }

// DMA addressing of one page tile: instruction i loads token rows 8i..8i+7;
// lane writes LDS bytes 16*lane of its 1 KiB, i.e. row 8i + lane/8, position
// lane%8, which holds chunk (lane%8) ^ swz(row).
struct DmaOffsets {
  uint32_t off0, off1;  // element offsets within a page for rows lane/8 and 8 + lane/8
};
__device__ __forceinline__ DmaOffsets dma_offsets(int lane, int g) {
  const int tau0 = lane >> 3;
  const int tau1 = 8 + (lane >> 3);
  return DmaOffsets{(uint32_t)(tau0 * kRowElems + g * kHeadDim + 8 * ((lane & 7) ^ swz(tau0))),
                    (uint32_t)(tau1 * kRowElems + g * kHeadDim + 8 * ((lane & 7) ^ swz(tau1)))};
}
// Starts the copy of head g's K and V tiles of one page into an LDS slot.
// Only token rows below `rows` are read (the last page of a sequence holds
// fewer tokens); the rows past them keep what the slot held, and attend_page
// masks them.  Every copy instruction is issued with at least one row (the
// second one keeps row 8), so each page counts as 4 loads in the waits.
__device__ __forceinline__ void issue_page(const DecodeArgs& a, unsigned char* dst, int32_t page, DmaOffsets o,
                                           int rows = kPageTokens) {
  const size_t base = (size_t)(uint32_t)page * (size_t)(kPageTokens * kRowElems);
  const uint16_t* kp = a.k_pool + base;
  const uint16_t* vp = a.v_pool + base;
  if (rows >= kPageTokens) {  // a full page (wave-uniform): no lane masks
    __builtin_amdgcn_global_load_lds(kp + o.off0, dst, 16, 0, 2);
    __builtin_amdgcn_global_load_lds(kp + o.off1, dst + 1024, 16, 0, 2);
    __builtin_amdgcn_global_load_lds(vp + o.off0, dst + kTileBytes, 16, 0, 2);
    __builtin_amdgcn_global_load_lds(vp + o.off1, dst + kTileBytes + 1024, 16, 0, 2);
    return;
  }
  const int row = (threadIdx.x & 63) >> 3;  // rows row and 8 + row of the two halves
  if (row < rows) {
    __builtin_amdgcn_global_load_lds(kp + o.off0, dst, 16, 0, 2);
    __builtin_amdgcn_global_load_lds(vp + o.off0, dst + kTileBytes, 16, 0, 2);
  }
  if (row == 0 || 8 + row < rows) {
    __builtin_amdgcn_global_load_lds(kp + o.off1, dst + 1024, 16, 0, 2);
    __builtin_amdgcn_global_load_lds(vp + o.off1, dst + kTileBytes + 1024, 16, 0, 2);
  }
}

// One page of a split: S^T = K Q^T on MFMA, the online-softmax update of the
// lane's head (running maximum m_lane and weight sum l_lane, base 2) and PV into
// acc.  j: the page's index in its sequence (tokens 16 j .. 16 j + 15), L: the
// sequence length (tokens past it are masked).
__device__ __forceinline__ void attend_page(const u32x4& k0, const u32x4& k1, s16x4 (&vb)[4], const bf16x8& qb0,
                                            const bf16x8& qb1, int j, int L, int c, float scale_log2,
                                            float& m_lane, float& l_lane, f32x4 (&acc)[4]) {
  const bool tail = (j + 1) * kPageTokens > L;
  f32x4 st = {0.f, 0.f, 0.f, 0.f};
  st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0), qb0, st, 0, 0, 0);
  st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1), qb1, st, 0, 0, 0);
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = (!tail || j * kPageTokens + 4 * c + r < L) ? st[r] * scale_log2 : -INFINITY;
  if (tail) {  // masked tokens: their V slots may hold anything (NaN included)
#pragma unroll
    for (int nn = 0; nn < 4; ++nn)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j * kPageTokens + 4 * c + q >= L) vb[nn][q] = 0;
  }

  const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__builtin_amdgcn_ballot_w64(xm > m_lane) != 0) {
    // page maximum of head t%4 over the 4 row groups, then rescale
    float pm = fmaxf(xm, __shfl_xor(xm, 16));
    pm = fmaxf(pm, __shfl_xor(pm, 32));
    const float mn = fmaxf(m_lane, pm);
    const float alpha = (mn == m_lane) ? 1.f : __builtin_amdgcn_exp2f(m_lane - mn);
    m_lane = mn;
    l_lane *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = lane_read(alpha, r);  // lane r holds head r
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) acc[nn][r] *= ar;
    }
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - m_lane);
  l_lane += (p[0] + p[1]) + (p[2] + p[3]);

#if PA_DECODE_PV_VALU
  // PV on the VALU in FP32 (the measured alternative to the MFMA below):
  // lane (t, c) adds its own 4 tokens 4c..4c+3 for all 4 heads, taking head
  // i's weights from lane i of its quad (lane t holds head t % 4); the row
  // groups c are summed once per split, in split_result.
  float pi[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    pi[0][q] = quad_bcast<0>(p[q]);
    pi[1][q] = quad_bcast<1>(p[q]);
    pi[2][q] = quad_bcast<2>(p[q]);
    pi[3][q] = quad_bcast<3>(p[q]);
  }
#pragma unroll
  for (int nn = 0; nn < 4; ++nn)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float v = __builtin_bit_cast(float, (unsigned)(unsigned short)vb[nn][q] << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nn][i] = __builtin_fmaf(pi[i][q], v, acc[nn][i]);
    }
#else
  unsigned hi[4], lo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = __builtin_bit_cast(unsigned, p[r]);
    lo[r] = __builtin_bit_cast(unsigned, p[r] - __builtin_bit_cast(float, hi[r] & 0xffff0000u));
  }
  // pack the upper halves (bf16 truncations) of two FP32 values into one dword
  const s16x4 ahi = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(hi[1], hi[0], 0x07060302u),
                                                    __builtin_amdgcn_perm(hi[3], hi[2], 0x07060302u)});
  const s16x4 alo = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(lo[1], lo[0], 0x07060302u),
                                                    __builtin_amdgcn_perm(lo[3], lo[2], 0x07060302u)});
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) {
    acc[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, vb[nn], acc[nn], 0, 0, 0);
    acc[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, vb[nn], acc[nn], 0, 0, 0);
  }
#endif
}

// End of a split: the per-head (l, m) and the lane's share of o.
struct SplitResult {
  f32x4 o;     // the lane's dims 16c + t of the 4 heads (unnormalised)
  f32x4 l, m;  // head r's weight sum and maximum in element r (the same in every lane)
};
// (acc passed by value: a reference would let the selection of the lane's
// tile below become an indexed access to memory)
__device__ __forceinline__ SplitResult split_result(f32x4 a0, f32x4 a1, f32x4 a2, f32x4 a3, float m_lane,
                                                    float l_lane, int c) {
#if PA_DECODE_PV_VALU
  // the four row groups' token sums, so that every lane holds the MFMA layout
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] += __shfl_xor(a0[i], 16);
    a0[i] += __shfl_xor(a0[i], 32);
    a1[i] += __shfl_xor(a1[i], 16);
    a1[i] += __shfl_xor(a1[i], 32);
    a2[i] += __shfl_xor(a2[i], 16);
    a2[i] += __shfl_xor(a2[i], 32);
    a3[i] += __shfl_xor(a3[i], 16);
    a3[i] += __shfl_xor(a3[i], 32);
  }
#endif
  SplitResult res;
  // l of head r: sum over the 4 row groups; lane r (r < 4) then holds head r.
  float lt = l_lane + __shfl_xor(l_lane, 16);
  lt += __shfl_xor(lt, 32);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    res.l[r] = lane_read(lt, r);
    res.m[r] = lane_read(m_lane, r);
  }
  // every row group holds the same tiles; lane (t, c) stores dim 16c + t of the 4 heads
  res.o = a0;
  if (c == 1) res.o = a1;
  if (c == 2) res.o = a2;
  if (c == 3) res.o = a3;
  return res;
}

// Table row and q of one sequence, loaded ahead of its item (b < 0: none).
struct ItemPrefetch {
  int b;
  int id0, id1;
  u32x4 q0, q1;
  u32x4 row;  // appended K (lanes 0-7) / V (lanes 8-15) row of the wave's head
};

// One work item: split s (of nsplit) of sequence b, whose length is L, n of its
// pages.  Called by all 8 waves of the workgroup with the same arguments; wave
// g handles KV head g, and the waves do not wait for one another.  A wave
// returns with no load in flight (its output stores may be).
template <bool kAppend, bool kRope>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int b, int s, int nsplit, int L, int n,
                                            const ItemPrefetch& pre, bool primed, DmaOffsets doff,
                                            unsigned char (*ring)[kRing][kSlotBytes]) {
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane index produced anew for every item, so that nothing derived from it is
  // hoisted out of the item loop and kept live across items
  int lane;
  asm volatile("v_and_b32 %0, 63, %1" : "=v"(lane) : "v"(threadIdx.x));
  const int t = lane & 15;
  const int c = lane >> 4;

  if (L <= 0) {  // empty sequence: zero its output rows
    wait_vmcnt<0>();  // returns, like the other paths, with no load in flight
    reinterpret_cast<f32x4*>(a.out + ((size_t)b * kQHeads + g * kGroup) * kHeadDim)[lane] =
        f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }

  // Block-table entries.  When the table row has at most 128 entries all of it
  // is loaded (lane i: entries i and 64 + i); otherwise the split's own entries.
  // Entries past the sequence are loaded but never used.
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
  const bool whole_row = a.max_blocks <= 128;
  const bool prefetched = whole_row && pre.b == b;
  int id0 = 0, id1 = 0;
  if (prefetched) {
    id0 = pre.id0;
    id1 = pre.id1;
  } else if (whole_row) {
    id0 = lane < a.max_blocks ? bt[lane] : 0;
    id1 = 64 + lane < a.max_blocks ? bt[64 + lane] : 0;
  }

  // The k-th page of this split is entry id_base + k * id_stride of (id0, id1).
  int id_base = s, id_stride = nsplit;
  if (!whole_row) {
    id0 = (lane < n) ? bt[s + lane * nsplit] : 0;
    id1 = (64 + lane < n) ? bt[s + (64 + lane) * nsplit] : 0;
    id_base = 0;
    id_stride = 1;
  }
  auto page_of = [&](int k) -> int32_t {  // k < n
    const int e = id_base + k * id_stride;
    return e < 64 ? __builtin_amdgcn_readlane(id0, e) : __builtin_amdgcn_readlane(id1, e - 64);
  };

  // Fused append (kAppend): position L-1 lives in page pa = (L-1)/16, owned by
  // split pa % nsplit at its page index pa / nsplit.  The wave of head g in that
  // workgroup stores the new K and V rows of head g to the pool (lanes 0-7: K,
  // 8-15: V, 16 bytes each) and later patches them into its LDS copy of the page,
  // so the attention sees exactly what pa_append would have written.
  int k_app = -1;
  int tau_app = 0;
  u32x4 new_row = {0u, 0u, 0u, 0u};
  f32x4 kc0, kc1, ks0, ks1;  // kRope: the table row of the new key's lanes
  if (kAppend) {
    const int pa = (L - 1) / kPageTokens;
    if (pa % nsplit == s) {
      k_app = pa / nsplit;
      tau_app = (L - 1) % kPageTokens;
      // RoPE of the new key at position L-1 (kRope): the table row is loaded
      // beside the key row, so that both arrive in one round trip.
      if (kRope) {
        const float* cs = a.cos_sin + (size_t)min(L - 1, a.max_pos - 1) * kHeadDim + 8 * (lane & 3);
        kc0 = *reinterpret_cast<const f32x4*>(cs);
        kc1 = *reinterpret_cast<const f32x4*>(cs + 4);
        ks0 = *reinterpret_cast<const f32x4*>(cs + 32);
        ks1 = *reinterpret_cast<const f32x4*>(cs + 36);
      }
      if (lane < 16) {
        const size_t head_off = ((size_t)b * kKvHeads + g) * kHeadDim + 8 * (lane & 7);
        new_row = prefetched ? pre.row : ld16((lane < 8 ? a.k_new : a.v_new) + head_off);
      }
      // With kRope the key is rotated and stored once the item's first page
      // copies are on their way (below): the workgroup patches the new row into
      // its own copy of the page, and no other split reads this slot.
      if (!kRope && lane < 16) {
        const size_t dst = ((size_t)(uint32_t)page_of(k_app) * kPageTokens + tau_app) * kRowElems + g * kHeadDim + 8 * (lane & 7);
        *reinterpret_cast<u32x4*>((lane < 8 ? a.k_pool_w : a.v_pool_w) + dst) = new_row;
      }
    }
  }

  // B operand of S^T = K Q^T: query head 4g + (t % 4), dims 8c..8c+7 and 32+8c..32+8c+7.
  const uint16_t* qrow = a.q + ((size_t)b * kQHeads + g * kGroup + (t & 3)) * kHeadDim;
  bf16x8 qb0 = __builtin_bit_cast(bf16x8, prefetched ? pre.q0 : ld16(qrow + 8 * c));
  bf16x8 qb1 = __builtin_bit_cast(bf16x8, prefetched ? pre.q1 : ld16(qrow + 32 + 8 * c));
  // RoPE of the query at position L-1 (kRope): the lane's two chunks, dims
  // 8c.. and 32 + 8c.., are 8 rotation pairs of one head.  The table row is
  // loaded here beside q; the rotation waits until the item's first page
  // copies are on their way.
  f32x4 qc0, qc1, qs0, qs1;
  if (kRope) {
    const float* cs = a.cos_sin + (size_t)min(L - 1, a.max_pos - 1) * kHeadDim + 8 * c;
    qc0 = *reinterpret_cast<const f32x4*>(cs);
    qc1 = *reinterpret_cast<const f32x4*>(cs + 4);
    qs0 = *reinterpret_cast<const f32x4*>(cs + 32);
    qs1 = *reinterpret_cast<const f32x4*>(cs + 36);
  }

  // the k-th page of the split is page s + k nsplit of the sequence
  auto issue = [&](int slot, int k, int32_t page) {
    issue_page(a, ring[g][slot], page, doff, min(kPageTokens, L - (s + k * nsplit) * kPageTokens));
  };
  // LDS read offsets: K (A operand) token t, chunks c and 4+c; V^T element
  // (token 4c+q, dim 16nn+t) lives in chunk 2nn + t/8 at element t%8.
  const int kr0 = t * 128 + 16 * (c ^ swz(t));
  const int kr1 = t * 128 + 16 * ((4 + c) ^ swz(t));
  int vr[4][4];
#pragma unroll
  for (int nn = 0; nn < 4; ++nn)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tau = 4 * c + q;
      vr[nn][q] = kTileBytes + tau * 128 + 16 * ((2 * nn + (t >> 3)) ^ swz(tau)) + 2 * (t & 7);
    }

  float m_lane = -INFINITY;  // running maximum (base-2 logits) of head t % 4
  float l_lane = 0.f;        // sum of this lane's weights (4 tokens per page)
  f32x4 acc[4];
#pragma unroll
  for (int nn = 0; nn < 4; ++nn) acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The appended row arrives with the table row it was loaded beside; waiting
  // for both here (the first copies need the table row anyway) spares the LDS
  // patch below a wait for every copy in flight.
  if (kAppend && !kRope) asm volatile("" ::"v"(id0), "v"(id1), "v"(new_row[0]), "v"(new_row[1]), "v"(new_row[2]),
                                      "v"(new_row[3]));
  if (!primed) {
#pragma unroll
    for (int u = 0; u < kRing; ++u)
      if (u < n) issue(u, u, page_of(u));
  }

  if (kRope) {
    const u32x4 x0 = __builtin_bit_cast(u32x4, qb0), x1 = __builtin_bit_cast(u32x4, qb1);
    const float cv[8] = {qc0[0], qc0[1], qc0[2], qc0[3], qc1[0], qc1[1], qc1[2], qc1[3]};
    const float sv[8] = {qs0[0], qs0[1], qs0[2], qs0[3], qs1[0], qs1[1], qs1[2], qs1[3]};
    u32x4 r0, r1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      unsigned o0[2], o1[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float lo = bf16_lo_hi(x0[m], e), hi = bf16_lo_hi(x1[m], e);
        o0[e] = bf16_rne(rope_term(lo, hi, cv[2 * m + e], sv[2 * m + e], false));
        o1[e] = bf16_rne(rope_term(hi, lo, cv[2 * m + e], sv[2 * m + e], true));
      }
      r0[m] = o0[0] | (o0[1] << 16);
      r1[m] = o1[0] | (o1[1] << 16);
    }
    qb0 = __builtin_bit_cast(bf16x8, r0);
    qb1 = __builtin_bit_cast(bf16x8, r1);
  }
  if (kRope && k_app >= 0) {
    // Lane j < 8 holds dims 8j..8j+7 of the new key, whose rotation partners
    // (32 dims away) lane j ^ 4 holds.  Every lane takes part in the swap;
    // lanes 8-15 keep the value row.
    u32x4 y;
#pragma unroll
    for (int m = 0; m < 4; ++m) y[m] = (unsigned)__shfl_xor((int)new_row[m], 4);
    const bool second = (lane & 4) != 0;
    const float cv[8] = {kc0[0], kc0[1], kc0[2], kc0[3], kc1[0], kc1[1], kc1[2], kc1[3]};
    const float sv[8] = {ks0[0], ks0[1], ks0[2], ks0[3], ks1[0], ks1[1], ks1[2], ks1[3]};
    u32x4 r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      unsigned o[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
        o[e] = bf16_rne(rope_term(bf16_lo_hi(new_row[m], e), bf16_lo_hi(y[m], e), cv[2 * m + e], sv[2 * m + e],
                                  second));
      r[m] = o[0] | (o[1] << 16);
    }
    if (lane < 8) new_row = r;
    if (lane < 16) {
      const size_t dst = ((size_t)(uint32_t)page_of(k_app) * kPageTokens + tau_app) * kRowElems + g * kHeadDim + 8 * (lane & 7);
      *reinterpret_cast<u32x4*>((lane < 8 ? a.k_pool_w : a.v_pool_w) + dst) = new_row;
    }
  }

  for (int kb = 0; kb < n; kb += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int k = kb + u;
      if (k >= n) break;
      // this slot's 4 loads have landed: younger loads are those of the next
      // kRing-1 pages, or none near the end of the split
      if (k + kRing - 1 < n)
        wait_vmcnt<4 * (kRing - 1)>();
      else
        wait_vmcnt<0>();
      unsigned char* tile = ring[g][u];
      if (kAppend && k == k_app && lane < 16)  // the new token's row, in the swizzled layout
        *reinterpret_cast<u32x4*>(tile + (lane < 8 ? 0 : kTileBytes) + tau_app * 128 +
                                  16 * ((lane & 7) ^ swz(tau_app))) = new_row;
      const u32x4 k0 = *reinterpret_cast<const u32x4*>(tile + kr0);
      const u32x4 k1 = *reinterpret_cast<const u32x4*>(tile + kr1);
      s16x4 vb[4];
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
#pragma unroll
        for (int q = 0; q < 4; ++q) vb[nn][q] = *reinterpret_cast<const short*>(tile + vr[nn][q]);
      wait_lgkmcnt0();  // slot fully read: refill it
      __builtin_amdgcn_sched_barrier(0);
      if (k + kRing < n) issue(u, k + kRing, page_of(k + kRing));

      attend_page(k0, k1, vb, qb0, qb1, s + k * nsplit, L, c, a.scale_log2, m_lane, l_lane, acc);
    }
  }
  const SplitResult sr = split_result(acc[0], acc[1], acc[2], acc[3], m_lane, l_lane, c);
  const f32x4 o = sr.o, lr = sr.l, mr = sr.m;
  const int d = 16 * c + t;
  if (nsplit == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a.out[((size_t)b * kQHeads + g * kGroup + r) * kHeadDim + d] = o[r] / lr[r];
    return;
  }
  // Partials are written and read with device-scope (sc1) accesses, which are
  // coherent across the XCDs' L2 caches without whole-cache write-back or
  // invalidation.  Each wave writes the partials of its own KV head's 4 query
  // heads and counts itself done on that (sequence, KV head)'s counter once its
  // stores have completed; the last wave of each head merges that head, so the
  // waves of a workgroup never wait for one another here.
  //
  // Ordering argument.  The counter update below is a relaxed atomic, so the
  // HIP memory model gives no happens-before edge from these stores to the
  // merging wave's loads; the order comes from how gfx950 executes agent-scope
  // relaxed accesses, and every step of it is explicit here:
  //  1. every partial word is stored as an agent-scope atomic (a global store
  //     with sc1: written through the XCD's L2 to the device coherence point,
  //     not left dirty in a non-coherent cache);
  //  2. s_waitcnt vmcnt(0) returns only when each of this wave's stores has
  //     been acknowledged by that point, before the wave's counter update;
  //  3. the counter update is an agent-scope atomic (executed at the coherence
  //     point, one modification order for all waves), so the wave whose update
  //     returns nsplit - 1 is ordered after every other split's update for the
  //     same head, hence after all of their acknowledged stores;
  //  4. the merging wave issues its loads only after that return value has
  //     come back, and they are agent-scope atomic loads (sc1), which do not
  //     hit in a non-coherent L1 or L2 line and read the coherence point.
  // This is what an agent-scope release/acquire pair would do for data written
  // and read only with agent-scope atomics, minus the whole-L2 write-back and
  // invalidate that a release or acquire fence adds for plain accesses (with
  // them in every workgroup the launch took three times as long).
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const size_t row = ((size_t)b * kQHeads + g * kGroup + r) * a.S + s;
    __hip_atomic_store(a.part_o + row * kHeadDim + d, o[r] / lr[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  {
    // m and l of the 4 heads in one store with every lane active: lane i
    // writes m (i & 4 clear) or l of head i & 3, and lanes that agree on
    // i & 7 write the same word with the same value.  (A store by lane 0
    // alone puts the stores in a branch, and the compiler then waits for
    // the first ones to complete before it issues the rest.)
    const int r = lane & 3;
    const float mv = r == 0 ? mr[0] : r == 1 ? mr[1] : r == 2 ? mr[2] : mr[3];
    const float lv = r == 0 ? lr[0] : r == 1 ? lr[1] : r == 2 ? lr[2] : lr[3];
    const size_t row = ((size_t)b * kQHeads + g * kGroup + r) * a.S + s;
    __hip_atomic_store((lane & 4) ? a.part_l + row : a.part_m + row, (lane & 4) ? lv : mv, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vmcnt<0>();

  // The last wave of this (sequence, KV head) to finish combines the head's
  // nsplit partial states (in split order, so the result does not depend on
  // which wave it is) and resets the counter for the next call.
  int prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(a.counters + (size_t)b * kKvHeads + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__builtin_amdgcn_readfirstlane(prev) != nsplit - 1) return;
  {
    const int h = lane >> 4;         // query head 4g + h
    const int d0 = (lane & 15) * 4;  // dims d0..d0+3
    const size_t row = ((size_t)b * kQHeads + g * kGroup + h) * a.S;
    auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
    // Up to 8 splits per round trip; rounds are combined online (for at most 8
    // splits this is exactly sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m)).
    float M = -INFINITY;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int c0 = 0; c0 < nsplit; c0 += 8) {
      float mv[8], lv[8];
      f32x4 ov[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (c0 + i < nsplit) {
          const size_t rs = row + c0 + i;
          const float* po = a.part_o + rs * kHeadDim + d0;
          mv[i] = ld(a.part_m + rs);
          lv[i] = ld(a.part_l + rs);
          ov[i] = f32x4{ld(po), ld(po + 1), ld(po + 2), ld(po + 3)};
        } else {
          mv[i] = -INFINITY;
          lv[i] = 0.f;
          ov[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      float cm = mv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) cm = fmaxf(cm, mv[i]);
      const float Mn = fmaxf(M, cm);
      const float carry = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      num *= carry;
      den *= carry;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float w = lv[i] * __builtin_amdgcn_exp2f(mv[i] - Mn);
        num += w * ov[i];
        den += w;
      }
      M = Mn;
    }
    *reinterpret_cast<f32x4*>(a.out + ((size_t)b * kQHeads + g * kGroup + h) * kHeadDim + d0) = num * (1.f / den);
  }
  if (lane == 0) __hip_atomic_store(a.counters + (size_t)b * kKvHeads + g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// ---------------------------------------------------------------------------
// Work plan.  Every workgroup builds the same plan in LDS from seq_lens:
//   pp      pages per split: a.part_pages if set, else ceil(total pages / n)
//           clamped to [m, 128], n = 192 when every sequence has the same page
//           count, and for mixed lengths 240 when sequences average 8 pages
//           or more, 384 below (about n items), m = 4 for batches of at most
//           64 sequences and 8 above;
//   nsplit  ceil(npages / pp) splits per sequence (1 for an empty sequence);
//   items   first every split of the multi-split sequences (sequence-major),
//           then the single-split sequences (longest first, by 16-page
//           bucket, when the queue is in use and items average 8 pages or more).
//           Workgroup w starts with item w; if there are more items than
//           workgroups the rest are handed out by an atomic queue.  Long
//           sequences' splits, the largest items, start first.
//   active  the workgroups that take items: the whole grid (two per CU) when
//           items average fewer than 8 pages, whose latency a second
//           workgroup per CU hides; else one per CU (a.narrow), which streams
//           pages faster and leaves the balancing to the queue.  The others
//           leave right after the plan.

constexpr int kTargetItems = 192;          // batches with one page count (and the host's guess)
constexpr int kLongItemPages = 8;          // items averaging this many pages run one workgroup per CU
constexpr int kTargetItemsMixed = 384;     // batches of mixed lengths (the queue takes what the active workgroups do not)
constexpr int kTargetItemsMixedLong = 240; // the same when sequences average kLongItemPages pages or more
constexpr int kAutoMinPages = 8;
constexpr int kMaxSplitPages = 128;
// Length buckets for handing out single-split items longest first: bucket k
// holds page counts down from kMaxSplitPages - 16k (the last one down to 0).
constexpr int kLenBuckets = 8;
__device__ __forceinline__ int len_bucket_of(int np) { return min(kLenBuckets - 1, (kMaxSplitPages - np) / 16); }

// Smallest automatic split: 4 pages for batches of at most 64 sequences (their
// items are few, so shorter ones cut the latency of each), 8 above.
__host__ __device__ __forceinline__ int auto_min_pages(int B) { return B <= 64 ? 4 : kAutoMinPages; }
__host__ __device__ __forceinline__ int auto_pages_per_split(int total_pages, int target = kTargetItems,
                                                             int minp = kAutoMinPages) {
  return min(kMaxSplitPages, max(minp, (total_pages + target - 1) / target));
}
// Items an automatic split aims at.  One page count: about 192, which suits
// streaming whole pages with one item per workgroup.  Mixed lengths: more,
// smaller items, so that long sequences are not left to a few workgroups at
// the end; about 384 when sequences are short on average (their items run two
// workgroups per CU), 240 when they average 8 pages or more (one workgroup per
// CU; on the fragmented workload 23-24 pages per split measured 631-633 us per
// step against 643-663 us at 15, 22 and 26-27 pages).
__host__ __device__ __forceinline__ int auto_target_items(bool uniform, int total_pages, int B) {
  return uniform ? kTargetItems : total_pages >= kLongItemPages * B ? kTargetItemsMixedLong : kTargetItemsMixed;
}

__device__ __forceinline__ int active_workgroups(int total_pages, int n_items, int narrow) {
  const int grid = (int)gridDim.x;
  return narrow > 0 && narrow < grid && total_pages >= kLongItemPages * n_items ? narrow : grid;
}

__device__ __forceinline__ int nsplit_of(int L, int pp) {
  if (L <= 0) return 1;
  const int np = (L + kPageTokens - 1) / kPageTokens;
  return (np + pp - 1) / pp;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16
// lanes through DPP, then the row totals added through readlane.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Maximum over the 64 lanes of a wave of values >= 0 (same pattern as the scan).
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
  return max(max(__builtin_amdgcn_readlane(v, 15), __builtin_amdgcn_readlane(v, 31)),
             max(__builtin_amdgcn_readlane(v, 47), __builtin_amdgcn_readlane(v, 63)));
}

// Largest b with pre[b] <= i, for a nondecreasing pre[0..B] with pre[0] = 0 <= i < pre[B].
__device__ __forceinline__ int owner_of(const int* pre, int B, int i) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

// The work plan, shared by the workgroup through LDS.
struct PlanLds {
  int wave_pages[8];   // pages per wave
  int wave_max[8];     // largest page count per wave
  int wave_min[8];     // kPageCap minus the smallest page count per wave
  int wave_multi[8];   // multi-split items per wave
  int wave_single[8];  // single-split items per wave
  int first[2];        // (sequence, split) of item blockIdx.x
  int pp;              // pages per split
  int uniform_ns;      // as in ItemPlan
  int by_length;       // single-split items are ordered longest first (sC holds the order)
  int active;          // workgroups that take items (see the plan above)
  int len_bucket[kLenBuckets][8];  // single-split sequences per length bucket and wave
};
struct ItemPlan {
  int pp, n_multi, n_items, active;
  int uniform_ns;     // > 0: every sequence has this many splits, item i is (i / ns, i % ns)
  int uniform_pages;  // with uniform_ns > 0: every sequence's page count
};
constexpr int kPageCap = 1 << 20;  // above any page count of a sequence

// Workgroup barrier for LDS data: waits for this wave's LDS accesses, not for
// its outstanding global loads or copies into LDS.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The plan is built in two steps so that the caller can start work between
// them: plan_lengths loads the lengths (thread t handles sequences
// [t*per, t*per + per)) into sL and sums their pages; plan_finish derives the
// items in LDS (sA / sC: exclusive prefixes of the multi-split and single-split
// item counts, pl->first: this workgroup's first item).  When every sequence
// has the same number of pages the items follow from the index alone and the
// plan ends after its first barrier.
struct PlanLengths {
  int pages, pmax, pmin_c;  // this thread's page sum, largest count, kPageCap - smallest count
};
constexpr int kLensPerThread = 8;  // lengths a thread of the plan handles, at most (B <= 4096)
static_assert(kMaxDecodeBatch <= 512 * kLensPerThread, "plan: lengths per thread");
__device__ __forceinline__ PlanLengths plan_lengths(int B, const int (&lens)[kLensPerThread], int* sL) {
  const int per = (B + 511) / 512;
  const int b0 = min(B, (int)threadIdx.x * per);
  PlanLengths x{0, 0, 0};
#pragma unroll
  for (int k = 0; k < kLensPerThread; ++k) {
    const int b = b0 + k;
    if (k >= per || b >= B) break;
    const int L = lens[k];
    sL[b] = L;
    const int np = L > 0 ? (L + kPageTokens - 1) / kPageTokens : 0;
    x.pages += np;
    x.pmax = max(x.pmax, np);
    x.pmin_c = max(x.pmin_c, kPageCap - np);
  }
  return x;
}

__device__ __forceinline__ ItemPlan plan_finish(PlanLengths x, int B, int part_pages, int narrow, int* sL, int* sA,
                                                int* sC, PlanLds* pl) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = (B + 511) / 512;
  const int b0 = min(B, (int)threadIdx.x * per), b1 = min(B, b0 + per);
  const int tp = wave_inclusive_scan(x.pages);
  const int pmax = wave_max_nonneg(x.pmax);
  const int pmin_c = wave_max_nonneg(x.pmin_c);
  if (lane == 63) {
    pl->wave_pages[w] = tp;
    pl->wave_max[w] = pmax;
    pl->wave_min[w] = pmin_c;
  }
  lds_barrier();
  int total_pages = 0, all_max = 0, all_min_c = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    total_pages += pl->wave_pages[v];
    all_max = max(all_max, pl->wave_max[v]);
    all_min_c = max(all_min_c, pl->wave_min[v]);
  }
  const bool uniform = kPageCap - all_min_c == all_max;
  const int pp = part_pages > 0 ? part_pages
                                : auto_pages_per_split(total_pages, auto_target_items(uniform, total_pages, B),
                                                       auto_min_pages(B));
  ItemPlan p;
  p.pp = pp;
  if (uniform) {
    const int ns = all_max > 0 ? (all_max + pp - 1) / pp : 1;
    p.uniform_ns = ns;
    p.uniform_pages = all_max;
    p.n_items = B * ns;
    p.n_multi = ns > 1 ? p.n_items : 0;
    p.active = active_workgroups(total_pages, p.n_items, narrow);
    // No barrier follows: every wave writes these (equal) values itself, so
    // that each wave's later reads see them.
    if ((threadIdx.x & 63) == 0) {
      pl->pp = pp;
      pl->uniform_ns = ns;
      pl->by_length = 0;
      pl->active = p.active;
      sA[B] = p.n_multi;
      sC[B] = p.n_items - p.n_multi;
    }
    return p;
  }
  int ca = 0, cc = 0;
  for (int b = b0; b < b1; ++b) {  // sL[b] was written by this thread
    const int ns = nsplit_of(sL[b], pp);
    ca += ns > 1 ? ns : 0;
    cc += ns > 1 ? 0 : 1;
  }
  const int ia = wave_inclusive_scan(ca), ic = wave_inclusive_scan(cc);
  if (lane == 63) {
    pl->wave_multi[w] = ia;
    pl->wave_single[w] = ic;
  }
  lds_barrier();
  int oa = ia - ca, oc = ic - cc, n_multi = 0, n_single = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int xa = pl->wave_multi[v], xc = pl->wave_single[v];
    oa += v < w ? xa : 0;
    oc += v < w ? xc : 0;
    n_multi += xa;
    n_single += xc;
  }
  const int i0 = blockIdx.x;
  const int active = active_workgroups(total_pages, n_multi + n_single, narrow);
  // When the queue hands out items and they are long on average (the batches
  // that run one workgroup per CU), the single-split items go longest first (by
  // 16-page length bucket, into sC), so that no long item starts late;
  // otherwise they keep sequence order.
  const bool by_length = n_multi + n_single > active && total_pages >= kLongItemPages * (n_multi + n_single);
  for (int b = b0; b < b1; ++b) {
    const int ns = nsplit_of(sL[b], pp);
    sA[b] = oa;
    sC[b] = oc;
    if (ns > 1 && i0 >= oa && i0 < oa + ns) {
      pl->first[0] = b;
      pl->first[1] = i0 - oa;
    }
    if (!by_length && ns == 1 && i0 == n_multi + oc) {
      pl->first[0] = b;
      pl->first[1] = 0;
    }
    oa += ns > 1 ? ns : 0;
    oc += ns > 1 ? 0 : 1;
  }
  if (threadIdx.x == 0) {
    sA[B] = n_multi;
    sC[B] = n_single;
    pl->pp = pp;
    pl->uniform_ns = 0;
    pl->by_length = by_length;
    pl->active = active;
  }
  if (by_length) {
    // Every workgroup must derive the same order, so it is a stable one: by
    // length bucket, and by sequence within a bucket (block-wide scans of the
    // per-thread bucket counts; no atomics).  Single-split sequences have at
    // most pp <= kMaxSplitPages pages.
    auto pages_of = [](int L) { return L > 0 ? (L + kPageTokens - 1) / kPageTokens : 0; };
    int cnt[kLenBuckets], incl[kLenBuckets];
#pragma unroll
    for (int k = 0; k < kLenBuckets; ++k) cnt[k] = 0;
    for (int b = b0; b < b1; ++b)
      if (nsplit_of(sL[b], pp) == 1) {
        const int kb = len_bucket_of(pages_of(sL[b]));
#pragma unroll
        for (int k = 0; k < kLenBuckets; ++k) cnt[k] += k == kb;
      }
#pragma unroll
    for (int k = 0; k < kLenBuckets; ++k) {
      incl[k] = wave_inclusive_scan(cnt[k]);
      if (lane == 63) pl->len_bucket[k][w] = incl[k];
    }
    lds_barrier();
    int next[kLenBuckets];  // this thread's next slot in each bucket
    int start = 0;
#pragma unroll
    for (int k = 0; k < kLenBuckets; ++k) {
      int before = 0, total = 0;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int x = pl->len_bucket[k][v];
        before += v < w ? x : 0;
        total += x;
      }
      next[k] = start + before + incl[k] - cnt[k];
      start += total;
    }
    for (int b = b0; b < b1; ++b)  // sC[0 .. n_single-1]: the order (sC[B] keeps the count)
      if (nsplit_of(sL[b], pp) == 1) {
        const int kb = len_bucket_of(pages_of(sL[b]));
        int slot = 0;
#pragma unroll
        for (int k = 0; k < kLenBuckets; ++k)
          if (k == kb) slot = next[k]++;
        sC[slot] = b;
      }
    lds_barrier();
    if (threadIdx.x == 0 && i0 >= n_multi && i0 < n_multi + n_single) {
      pl->first[0] = sC[i0 - n_multi];
      pl->first[1] = 0;
    }
  }
  lds_barrier();
  p.uniform_ns = 0;
  p.uniform_pages = 0;
  p.n_multi = n_multi;
  p.n_items = n_multi + n_single;
  p.active = active;
  return p;
}

template <bool kAppend, bool kRope>
__global__ __launch_bounds__(512) void decode_kernel(DecodeArgs a) {
  // Dynamic LDS: the page ring, then the plan's per-sequence arrays.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto ring = reinterpret_cast<unsigned char (*)[kRing][kSlotBytes]>(smem);
  int* plan_arrays = reinterpret_cast<int*>(smem + kKvHeads * kRing * kSlotBytes);
  __shared__ PlanLds plan_lds;
  __shared__ int next_item;
  const int B = a.B;
  int* sL = plan_arrays;  // [B] lengths
  int* sA = sL + B;       // [B+1] multi-split item prefix
  int* sC = sA + B + 1;   // [B+1] single-split item prefix


  // This thread's lengths for the plan (sequences t*per .. t*per + per - 1),
  // all loaded at once.
  const int per = (B + 511) / 512;
  int lens[kLensPerThread];
#pragma unroll
  for (int k = 0; k < kLensPerThread; ++k)
    lens[k] = k < per ? a.seq_lens[min((int)threadIdx.x * per + k, B - 1)] : 0;

  // While the plan is built, load the table row, q and the appended rows of
  // this workgroup's first item as it would be if every sequence filled its
  // table row (exact for a uniform full-context batch; otherwise unused).  The
  // loads are unconditional, with indices clamped into range, so that the
  // waits placed for them count exactly.
  const int ns_g = a.guess_ns;
  const int b_raw = ns_g > 1 ? (int)__umulhi(blockIdx.x, a.guess_magic) : (int)blockIdx.x;
  const int b_g = min(b_raw, B - 1);
  const int s_g = (int)blockIdx.x - b_raw * ns_g;
  const int n_g = ns_g > 1 ? (int)__umulhi((uint32_t)(a.max_blocks - s_g + ns_g - 1), a.guess_magic) : a.max_blocks;
  ItemPrefetch pre;
  pre.b = (a.max_blocks <= 128 && b_raw < B) ? b_raw : -1;
  {
    const int lane = threadIdx.x & 63, t = lane & 15, c = lane >> 4;
    const int g = threadIdx.x >> 6;
    const int32_t* bt = a.block_table + (size_t)b_g * a.max_blocks;
    // entries past the row are clamped to its last one (never used)
    pre.id0 = bt[min(lane, a.max_blocks - 1)];
    pre.id1 = bt[min(64 + lane, a.max_blocks - 1)];
    const uint16_t* qrow = a.q + ((size_t)b_g * kQHeads + g * kGroup + (t & 3)) * kHeadDim;
    pre.q0 = ld16(qrow + 8 * c);
    pre.q1 = ld16(qrow + 32 + 8 * c);
    pre.row = u32x4{0u, 0u, 0u, 0u};
    if (kAppend)  // lanes 16-63 repeat lanes 0-15
      pre.row = ld16(((lane & 8) ? a.v_new : a.k_new) + ((size_t)b_g * kKvHeads + g) * kHeadDim + 8 * (lane & 7));
  }
  const int L_g = a.seq_lens[b_g];
  __builtin_amdgcn_sched_barrier(0);

  // If the guessed sequence fills its table row, start the copies of the
  // guessed item's first pages now, so that the plan overlaps them.
  // They are used if the plan confirms the guess, else drained.
  const DmaOffsets doff = dma_offsets(threadIdx.x & 63, threadIdx.x >> 6);
  // the lengths and the table row are waited for here, so that no wait placed
  // for them later includes the copies
  asm volatile("" ::"v"(lens[0]), "v"(lens[1]), "v"(lens[2]), "v"(lens[3]), "v"(lens[4]), "v"(lens[5]),
               "v"(lens[6]), "v"(lens[7]), "v"(pre.id0), "v"(pre.id1));
  int prime_b = -1;
  if (pre.b >= 0 && (L_g + kPageTokens - 1) / kPageTokens == a.max_blocks) {
    const int g = threadIdx.x >> 6;
    int32_t pages[kRing];
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int e = min(s_g + u * ns_g, a.max_blocks - 1);
      pages[u] = e < 64 ? __builtin_amdgcn_readlane(pre.id0, e) : __builtin_amdgcn_readlane(pre.id1, e - 64);
    }
#pragma unroll
    for (int u = 0; u < kRing; ++u)
      if (u < n_g) issue_page(a, ring[g][u], pages[u], doff);
    prime_b = pre.b;
  }

  const PlanLengths pl_lens = plan_lengths(B, lens, sL);
  const ItemPlan plan = plan_finish(pl_lens, B, a.part_pages, a.narrow, sL, sA, sC, &plan_lds);
  // values read back from LDS are the same in every lane: keep them scalar
  const int ppu = __builtin_amdgcn_readfirstlane(plan.pp);
  const int uns = __builtin_amdgcn_readfirstlane(plan.uniform_ns);

  // Item blockIdx.x first.
  int b = -1, s = 0, L = 0, nsplit = 1, n = 0;
  if ((int)blockIdx.x < min(__builtin_amdgcn_readfirstlane(plan.n_items), __builtin_amdgcn_readfirstlane(plan.active))) {
    if (uns > 0 && pre.b >= 0 && __builtin_amdgcn_readfirstlane(plan.uniform_pages) == a.max_blocks &&
        ppu == a.guess_pp) {
      // every sequence fills its table row: the item is the guessed one
      b = pre.b;
      s = s_g;
      L = L_g;
      nsplit = ns_g;
      n = n_g;
    } else {
      if (uns > 0) {
        b = (int)blockIdx.x / uns;
        s = (int)blockIdx.x - b * uns;
      } else {
        b = __builtin_amdgcn_readfirstlane(plan_lds.first[0]);
        s = __builtin_amdgcn_readfirstlane(plan_lds.first[1]);
      }
      L = __builtin_amdgcn_readfirstlane(sL[b]);
      nsplit = nsplit_of(L, ppu);
      n = (L + kPageTokens - 1) / kPageTokens;
      n = (n - s + nsplit - 1) / nsplit;  // pages s, s + nsplit, ... of the split (n <= 128)
    }
  }
  bool primed = prime_b >= 0 && b == prime_b && s == s_g && nsplit == ns_g;
  if (prime_b >= 0 && !primed) wait_vmcnt<0>();  // unused copies land before their slots are reused

  // When there are more items than active workgroups, later items come from
  // a queue counter, so that workgroups busy with long splits take no further
  // work.  Nothing of the plan is kept in registers across an item: the next
  // item is derived from the plan in LDS.
  while (b >= 0) {
    if (s < nsplit) decode_item<kAppend, kRope>(a, b, s, nsplit, L, n, pre, primed, doff, ring);
    pre.b = -1;
    primed = false;
    b = -1;
    // no queue when every item had a workgroup of its own (item counts re-read from LDS)
    const int act = __builtin_amdgcn_readfirstlane(plan_lds.active);
    if (!a.queue || __builtin_amdgcn_readfirstlane(sA[B]) + __builtin_amdgcn_readfirstlane(sC[B]) <= act) break;
    // Wave 0 claims the next item as soon as it is done; the first barrier also
    // ensures every wave has read the previous next_item.  The barriers wait on
    // LDS only: the item's output stores need not complete before the claim
    // (a __syncthreads would wait for them, a round trip before the claim).
    int fetched = 0;
    if (threadIdx.x == 0)
      fetched = act + __hip_atomic_fetch_add(a.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    if (threadIdx.x == 0) next_item = fetched;
    lds_barrier();
    const int i = __builtin_amdgcn_readfirstlane(next_item);
    const int n_multi = __builtin_amdgcn_readfirstlane(sA[B]);
    const int n_items = n_multi + __builtin_amdgcn_readfirstlane(sC[B]);
    if (i < n_items) {
      const int pp = __builtin_amdgcn_readfirstlane(plan_lds.pp);
      const int ns_u = __builtin_amdgcn_readfirstlane(plan_lds.uniform_ns);
      if (ns_u > 0) {
        b = i / ns_u;
        s = i - b * ns_u;
      } else if (i < n_multi) {
        b = __builtin_amdgcn_readfirstlane(owner_of(sA, B, i));
        s = i - __builtin_amdgcn_readfirstlane(sA[b]);
      } else {
        b = __builtin_amdgcn_readfirstlane(plan_lds.by_length ? sC[i - n_multi] : owner_of(sC, B, i - n_multi));
        s = 0;
      }
      L = __builtin_amdgcn_readfirstlane(sL[b]);
      nsplit = nsplit_of(L, pp);
      n = (L + kPageTokens - 1) / kPageTokens;
      n = (n - s + nsplit - 1) / nsplit;
    }
  }
  // The last workgroup to leave (every workgroup of the grid counts itself)
  // resets the queue for the next call.
  if (a.queue && sA[B] + sC[B] > plan_lds.active && threadIdx.x == 0) {
    const int left = __hip_atomic_fetch_add(a.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left == (int)gridDim.x - 1) {
      __hip_atomic_store(a.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Plan once per step (pa_decode_plan) and decode from it (pa_decode_planned).
//
// The plan kernel is one workgroup.  It takes the lengths, chooses the pages per
// split exactly as the in-kernel plan does (so a sequence's splits, and thus its
// output bits, are the same under both), orders the (sequence, split) items
// (long ones by page count, longest first, with a counting sort over the counts
// 0..128 whose order among equal counts is not fixed; the output does not
// depend on it: an item's arithmetic depends only on its sequence and split,
// and splits are merged in split order; short ones as the in-kernel plan
// orders them, see plan_kernel), and deals them to the `active` workgroups:
//   - round 0 is fixed: workgroup w runs sorted item w (slot w);
//   - the items after it stay in sorted order in the following slots and are
//     claimed through the queue counter by the workgroups that finish first,
//     which balances what no cost model sees (when each workgroup starts, how
//     long its pages take to arrive); every workgroup copies this queued part of
//     the list into LDS at its start, so that a claim costs one atomic.
//   (The header's static_rounds allows more fixed rounds, in alternating
//   direction; with them the queue took longer on every workload measured.)
// A batch in which every sequence has the same page count keeps (sequence,
// split) order.

constexpr int kPlanThreads = 1024;
constexpr int kPlanKeys = kMaxSplitPages + 1;  // pages of a split: 0 .. 128
constexpr int kPlanMaxGrid = kPlanMaxBins;     // decode grids of planned launches (2 per CU) stay below

size_t plan_max_items(int B, int max_blocks, int part_pages) {
  const int minp = part_pages > 0 ? part_pages : auto_min_pages(B);
  const size_t all = (size_t)B * (size_t)((max_blocks + minp - 1) / minp);
  if (part_pages > 0) return all;
  // sum_b ceil(np_b / pp) < B + total / pp, and total / pp <= kTargetItemsMixed
  // unless pp is capped at kMaxSplitPages, when it is at most ceil(B * max_blocks / 128)
  const size_t capped = ((size_t)B * (size_t)max_blocks + kMaxSplitPages - 1) / kMaxSplitPages;
  const size_t bound = (size_t)B + (capped > (size_t)kTargetItemsMixed ? capped : (size_t)kTargetItemsMixed);
  return bound < all ? bound : all;
}

__device__ __forceinline__ int active_of(int total_pages, int n_items, int narrow, int grid) {
  return narrow > 0 && narrow < grid && total_pages >= kLongItemPages * n_items ? narrow : grid;
}

// Fixed rounds of a plan: round 0 (the rest goes through the queue).
__device__ __forceinline__ int static_rounds_of(int, int) { return 1; }

// Queued items a planned decode workgroup keeps in LDS beside the page ring (two
// workgroups still fit on a CU); claims past them read the slot from memory.
constexpr int kPlanStageItems = 960;
constexpr size_t kPlannedLdsBytes = (size_t)kKvHeads * kRing * kSlotBytes + (size_t)kPlanStageItems * 16;

// Slot of sorted item p: in the fixed rounds, r * act + the workgroup that runs
// it; after them, p itself.
__device__ __forceinline__ long slot_of(int p, int act, int static_rounds) {
  const int r = p / act;
  if (r >= static_rounds) return p;
  const int k = p - r * act;
  return (long)r * act + ((r & 1) ? act - 1 - k : k);
}

__device__ __forceinline__ void store_item(int* plan, long slot, int b, int s, int ns, int L) {
  reinterpret_cast<int4*>(reinterpret_cast<char*>(plan) + kPlanHeaderBytes)[slot] = int4{b, s, ns, L};
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seq_lens, int B,
                                                           int max_blocks, int part_pages, int narrow, int grid,
                                                           int* __restrict__ plan) {
  __shared__ int s_red[4];           // total pages, largest count, kPageCap - smallest count, items
  __shared__ int s_hist[kPlanKeys];  // items per split page count, then a cursor per count
  __shared__ int s_wsum[4];          // per-wave totals of the count scan below
  __shared__ int s_wm[kPlanThreads / 64], s_ws[kPlanThreads / 64];  // per-wave item totals
  __shared__ int s_len[kMaxDecodeBatch];
  const int t = threadIdx.x;
  const int lane = t & 63;
  if (t < 4) s_red[t] = 0;
  for (int k = t; k < kPlanKeys; k += kPlanThreads) s_hist[k] = 0;
  __syncthreads();
  int tp = 0, tmax = 0, tminc = 0;
  for (int b = t; b < B; b += kPlanThreads) {
    // lengths outside [0, 16 max_blocks] break the caller's contract; clamped
    // here so that the items never outgrow the plan buffer
    const int L = min(max(seq_lens[b], 0), kPageTokens * max_blocks);
    s_len[b] = L;
    const int np = L > 0 ? (L + kPageTokens - 1) / kPageTokens : 0;
    tp += np;
    tmax = max(tmax, np);
    tminc = max(tminc, kPageCap - np);
  }
  tp = wave_inclusive_scan(tp);
  tmax = wave_max_nonneg(tmax);
  tminc = wave_max_nonneg(tminc);
  if (lane == 63) {
    atomicAdd(&s_red[0], tp);
    atomicMax(&s_red[1], tmax);
    atomicMax(&s_red[2], tminc);
  }
  __syncthreads();
  const int total = s_red[0], all_max = s_red[1];
  const bool uniform = kPageCap - s_red[2] == all_max;
  const int pp = part_pages > 0 ? part_pages
                                : auto_pages_per_split(total, auto_target_items(uniform, total, B), auto_min_pages(B));
  PlanHeader h;
  h.magic = kPlanMagic;
  h.B = B;
  h.max_blocks = max_blocks;
  h.part_pages = part_pages;
  h.pp = pp;
  h.grid = grid;
  if (uniform) {
    const int ns = all_max > 0 ? (all_max + pp - 1) / pp : 1;
    const int n_items = B * ns;
    const int act = active_of(total, n_items, narrow, grid);
    const int srounds = static_rounds_of(n_items, act);
    for (int p = t; p < n_items; p += kPlanThreads) {
      const int b = p / ns;
      store_item(plan, slot_of(p, act, srounds), b, p - b * ns, ns, s_len[b]);
    }
    h.n_items = n_items;
    h.active = act;
    h.static_rounds = srounds;
    h.uniform_ns = ns;
    h.uniform_pages = all_max;
  } else {
    // Item order.  Long items (averaging kLongItemPages or more, which run one
    // workgroup per CU): by page count, longest first, so that no long item
    // starts late.  Short items: every split of the multi-split sequences
    // (sequence-major), then the single-split sequences in sequence order;
    // sorting these would give round 0 all the largest ones, whose workgroups
    // then finish and claim at the same moment.  Thread t counts the items of
    // sequences [t per, t per + per).
    const int per = (B + kPlanThreads - 1) / kPlanThreads;
    const int b0 = min(B, t * per), b1 = min(B, b0 + per);
    int cm = 0, cs = 0;
    for (int b = b0; b < b1; ++b) {
      const int ns = nsplit_of(s_len[b], pp);
      cm += ns > 1 ? ns : 0;
      cs += ns > 1 ? 0 : 1;
    }
    const int w = t >> 6;
    const int im = wave_inclusive_scan(cm), is = wave_inclusive_scan(cs);
    if (lane == 63) {
      s_wm[w] = im;
      s_ws[w] = is;
    }
    __syncthreads();
    int om = im - cm, os = is - cs, n_multi = 0, n_single = 0;
    for (int v = 0; v < kPlanThreads / 64; ++v) {
      om += v < w ? s_wm[v] : 0;
      os += v < w ? s_ws[v] : 0;
      n_multi += s_wm[v];
      n_single += s_ws[v];
    }
    const int n_items = n_multi + n_single;
    const int act = active_of(total, n_items, narrow, grid);
    const int srounds = static_rounds_of(n_items, act);
    if (total < kLongItemPages * n_items) {
      for (int b = b0; b < b1; ++b) {
        const int L = s_len[b];
        const int ns = nsplit_of(L, pp);
        if (ns > 1) {
          for (int sp = 0; sp < ns; ++sp) store_item(plan, slot_of(om++, act, srounds), b, sp, ns, L);
        } else {
          store_item(plan, slot_of(n_multi + os++, act, srounds), b, 0, 1, L);
        }
      }
    } else {
      // histogram of split page counts: a sequence of np pages in ns splits has
      // np % ns splits of np / ns + 1 pages and the rest of np / ns (split s
      // takes pages s, s + ns, ...); an empty sequence is one item of 0 pages
      for (int b = b0; b < b1; ++b) {
        const int L = s_len[b];
        const int ns = nsplit_of(L, pp);
        if (L <= 0) {
          atomicAdd(&s_hist[0], 1);
        } else {
          const int np = (L + kPageTokens - 1) / kPageTokens;
          const int q = np / ns, r = np - q * ns;
          if (r) atomicAdd(&s_hist[q + 1], r);
          atomicAdd(&s_hist[q], ns - r);
        }
      }
      __syncthreads();
      // first sorted position of each count, longest first: a prefix sum over
      // the counts taken from 128 down (three waves, 64 counts each)
      int incl = 0, mine = 0;
      if (w < 3) {
        const int key = kPlanKeys - 1 - t;
        mine = key >= 0 ? s_hist[key] : 0;
        incl = wave_inclusive_scan(mine);
        if (lane == 63) s_wsum[w] = incl;
      }
      __syncthreads();
      if (w < 3) {
        const int key = kPlanKeys - 1 - t;
        const int before = (w >= 1 ? s_wsum[0] : 0) + (w >= 2 ? s_wsum[1] : 0);
        if (key >= 0) s_hist[key] = before + incl - mine;  // s_hist now holds the cursors
      }
      __syncthreads();
      for (int b = b0; b < b1; ++b) {
        const int L = s_len[b];
        const int ns = nsplit_of(L, pp);
        const int np = L > 0 ? (L + kPageTokens - 1) / kPageTokens : 0;
        for (int sp = 0; sp < ns; ++sp) {
          const int key = L > 0 ? (np - sp + ns - 1) / ns : 0;
          const int p = atomicAdd(&s_hist[key], 1);
          store_item(plan, slot_of(p, act, srounds), b, sp, ns, L);
        }
      }
    }
    h.n_items = n_items;
    h.active = act;
    h.static_rounds = srounds;
    h.uniform_ns = 0;
    h.uniform_pages = 0;
  }
  if (t == 0) *reinterpret_cast<PlanHeader*>(plan) = h;
}

// Decode from a plan: the item code of decode_kernel, with the items read from
// the plan's slots instead of a plan built in every workgroup.  The header and
// this workgroup's first slot load together (no rows are loaded on a guess of
// the first item, as decode_kernel does: for mixed batches the guess misses,
// and its loads delayed the first item's own); the next fixed round's slot
// loads while an item runs; after the fixed rounds the workgroup claims the
// remaining items through the queue counter.
template <bool kAppend, bool kRope>
__global__ __launch_bounds__(512) void decode_planned_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto ring = reinterpret_cast<unsigned char (*)[kRing][kSlotBytes]>(smem);
  unsigned char* stage = smem + (size_t)kKvHeads * kRing * kSlotBytes;  // queued slots, 16 bytes each
  __shared__ int next_item;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x;
  const int4* slots = reinterpret_cast<const int4*>(reinterpret_cast<const char*>(a.plan) + kPlanHeaderBytes);
  const int hv = a.plan[min(lane, (int)(sizeof(PlanHeader) / sizeof(int)) - 1)];  // lane i: header word i
  int4 it = slots[w];
  ItemPrefetch pre = {};
  pre.b = -1;  // nothing prefetched
  const DmaOffsets doff = dma_offsets(lane, threadIdx.x >> 6);
  const int magic = __builtin_amdgcn_readlane(hv, 0);
  const int pB = __builtin_amdgcn_readlane(hv, 1);
  const int pmb = __builtin_amdgcn_readlane(hv, 2);
  const int ppart = __builtin_amdgcn_readlane(hv, 3);
  const int n_items = __builtin_amdgcn_readlane(hv, 4);
  const int act = __builtin_amdgcn_readlane(hv, 5);
  const int srounds = __builtin_amdgcn_readlane(hv, 6);
  const int pgrid = __builtin_amdgcn_readlane(hv, 11);
  if (magic != kPlanMagic || pB != a.B || pmb != a.max_blocks || ppart != a.part_pages || pgrid != (int)gridDim.x ||
      act <= 0 || act > (int)gridDim.x || srounds <= 0 || n_items <= 0) {
    // a plan built for other sizes: every output is NaN, so that the misuse shows
    const size_t n = (size_t)a.B * kQHeads * kHeadDim;
    for (size_t i = (size_t)blockIdx.x * 512 + threadIdx.x; i < n; i += (size_t)gridDim.x * 512)
      a.out[i] = __builtin_nanf("");
    return;
  }
  const int n_fixed = min(n_items, srounds * act);  // items in fixed slots
  const bool queued = n_items > n_fixed;
  const int n_stage = queued ? min(n_items - n_fixed, kPlanStageItems) : 0;
  if (w < act && n_stage > 0) {
    // copy the queued slots into LDS (64 per wave instruction); every wave
    // waits for its copies before the first claim's barrier
    const int wv = threadIdx.x >> 6;
    for (int c = wv; c * 64 < n_stage; c += kKvHeads) {
      const int i = min(c * 64 + lane, n_stage - 1);
      __builtin_amdgcn_global_load_lds(slots + n_fixed + i, stage + c * 64 * 16, 16, 0, 0);
    }
  }
  if (w < act) {
    for (int r = 0;;) {
      const int b = __builtin_amdgcn_readfirstlane(it.x);
      const int s = __builtin_amdgcn_readfirstlane(it.y);
      const int nsplit = __builtin_amdgcn_readfirstlane(it.z);
      const int L = __builtin_amdgcn_readfirstlane(it.w);
      const bool have = r < srounds ? (long)r * act + w < n_fixed : true;
      // the next fixed round's slot, loaded while this item runs
      if (r + 1 < srounds && (long)(r + 1) * act + w < n_fixed) it = slots[(size_t)(r + 1) * act + w];
      if (have && b >= 0 && b < a.B && s >= 0 && s < nsplit) {
        int n = L > 0 ? (L + kPageTokens - 1) / kPageTokens : 0;
        n = (n - s + nsplit - 1) / nsplit;
        decode_item<kAppend, kRope>(a, b, s, nsplit, L, n, pre, false, doff, ring);
      } else {
        wait_vmcnt<0>();  // what decode_item guarantees on return: no load in flight
      }
      pre.b = -1;
      ++r;
      if (r < srounds) {
        if ((long)r * act + w >= n_fixed) break;
        continue;
      }
      if (!queued) break;
      // claim one of the items after the fixed rounds (claiming while the item
      // still streams was slower: the workgroups of a round claim together).
      // Every wave's copies of the queued slots have landed: decode_item
      // returns with no load in flight, only its output stores, which the
      // claim does not wait for; the first barrier also ensures every wave
      // has read the previous next_item.  The barriers wait on LDS only (a
      // __syncthreads would wait for the stores, a round trip before the claim).
      int fetched = 0;
      if (threadIdx.x == 0)
        fetched = n_fixed + __hip_atomic_fetch_add(a.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_barrier();
      if (threadIdx.x == 0) next_item = fetched;
      lds_barrier();
      const int i = __builtin_amdgcn_readfirstlane(next_item);
      if (i >= n_items) break;
      it = i - n_fixed < n_stage ? *reinterpret_cast<const int4*>(stage + (size_t)(i - n_fixed) * 16) : slots[i];
    }
  }
  // The last workgroup of the grid to leave resets the queue for the next call.
  if (queued && threadIdx.x == 0) {
    const int left = __hip_atomic_fetch_add(a.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (left == (int)gridDim.x - 1) {
      __hip_atomic_store(a.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// merge: one thread per (sequence, query head, 4 dims).
//   out = sum_s w_s o_s / sum_s w_s,  w_s = l_s 2^(m_s - max_s m_s)

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int b = idx / (kQHeads * 16);
  if (b >= a.B) return;
  const int head = (idx >> 4) % kQHeads;
  const int d0 = (idx & 15) * 4;
  float* dst = a.out + ((size_t)b * kQHeads + head) * kHeadDim + d0;
  int live = a.S;
  if (a.seq_lens) {
    const int L = a.seq_lens[b];
    if (L <= 0) {
      if (!a.skip_single) *reinterpret_cast<f32x4*>(dst) = f32x4{0.f, 0.f, 0.f, 0.f};
      return;
    }
    live = min(a.S, (L + a.part_tokens - 1) / a.part_tokens);
    if (a.skip_single && live <= 1) return;  // pa_decode wrote this row directly
  }
  const size_t row = ((size_t)b * kQHeads + head) * a.S;
  float M = -INFINITY;
  for (int s = 0; s < live; ++s)
    if (a.part_l[row + s] > 0.f) M = fmaxf(M, a.part_m[row + s]);
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < live; ++s) {
      const float l = a.part_l[row + s];
      if (!(l > 0.f)) continue;
      const float w = l * __builtin_amdgcn_exp2f(a.part_m[row + s] - M);
      num += w * *reinterpret_cast<const f32x4*>(a.part_o + (row + s) * kHeadDim + d0);
      den += w;
    }
  }
  *reinterpret_cast<f32x4*>(dst) = den > 0.f ? num * (1.f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------------------
// clear: n ints set to zero (a kernel, not a memset, so that a captured graph
// replays it like any other node).

__global__ __launch_bounds__(256) void clear_kernel(int* p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// ---------------------------------------------------------------------------
// launchers (host)

hipError_t launch_clear(int* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int grid = std::min((n + 255) / 256, 1024);
  hipLaunchKernelGGL(clear_kernel, dim3(grid), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                         uint16_t* v_pool, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, int B, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3((B + 3) / 4), dim3(256), 0, stream, k_new, v_new, k_pool,
                     v_pool, block_table, max_blocks, seq_lens, B);
  return hipGetLastError();
}

// Dynamic LDS of a decode launch: the page ring and the plan's per-sequence arrays.
static size_t decode_dynamic_lds_bytes(int B) {
  return (size_t)kKvHeads * kRing * kSlotBytes + (3 * (size_t)B + 2) * sizeof(int);
}

size_t decode_lds_bytes(int B) { return decode_dynamic_lds_bytes(B) + sizeof(PlanLds) + 2 * sizeof(int); }

int auto_split_pages(long long total_pages, int B) {
  return auto_pages_per_split((int)(total_pages < (1 << 30) ? total_pages : (1 << 30)), kTargetItems,
                              auto_min_pages(B));
}

int auto_split_min_pages(int B) { return auto_min_pages(B); }

// Raises a decode kernel's dynamic LDS limit to what the largest batch needs,
// once per device (the attribute belongs to the device the call is made on).
static hipError_t allow_decode_lds(const void* kernel, int which, size_t bytes) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> done[6][kMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kMaxDevices && done[which][dev].load(std::memory_order_acquire)) return hipSuccess;
  err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess && dev >= 0 && dev < kMaxDevices) done[which][dev].store(1, std::memory_order_release);
  return err;
}

template <bool kAppend, bool kRope>
static hipError_t launch_decode_variant(const DecodeArgs& a, int grid, int which, hipStream_t stream) {
  const hipError_t attr = allow_decode_lds(reinterpret_cast<const void*>(decode_kernel<kAppend, kRope>), which,
                                           decode_dynamic_lds_bytes(kMaxDecodeBatch));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((decode_kernel<kAppend, kRope>), dim3(grid), dim3(64 * kKvHeads), decode_dynamic_lds_bytes(a.B),
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int grid, bool fused_append, bool rope, hipStream_t stream) {
  if (rope && !fused_append) return hipErrorInvalidValue;
  if (rope) return launch_decode_variant<true, true>(a, grid, 2, stream);
  if (fused_append) return launch_decode_variant<true, false>(a, grid, 1, stream);
  return launch_decode_variant<false, false>(a, grid, 0, stream);
}

hipError_t launch_plan(const int32_t* seq_lens, int B, int max_blocks, int part_pages, int narrow, int grid,
                       int* plan, hipStream_t stream) {
  if (B <= 0 || B > kMaxDecodeBatch || grid <= 0 || grid > kPlanMaxGrid) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, B, max_blocks, part_pages, narrow,
                     grid, plan);
  return hipGetLastError();
}

template <bool kAppend, bool kRope>
static hipError_t launch_planned_variant(const DecodeArgs& a, int grid, int which, hipStream_t stream) {
  const hipError_t attr = allow_decode_lds(reinterpret_cast<const void*>(decode_planned_kernel<kAppend, kRope>), which,
                                           kPlannedLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((decode_planned_kernel<kAppend, kRope>), dim3(grid), dim3(64 * kKvHeads), kPlannedLdsBytes, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_decode_planned(const DecodeArgs& a, int grid, bool fused_append, bool rope, hipStream_t stream) {
  if (rope && !fused_append) return hipErrorInvalidValue;
  if (grid <= 0 || grid > kPlanMaxGrid) return hipErrorInvalidValue;
  if (rope) return launch_planned_variant<true, true>(a, grid, 5, stream);
  if (fused_append) return launch_planned_variant<true, false>(a, grid, 4, stream);
  return launch_planned_variant<false, false>(a, grid, 3, stream);
}

hipError_t launch_fill(const FillArgs& a, hipStream_t stream) {
  const int nchunk = (a.T + kFillRowsPerWave - 1) / kFillRowsPerWave;
  const int grid = (nchunk + 3) / 4;  // 4 waves per workgroup, one chunk each
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(256), (a.B + 1) * sizeof(int), stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const unsigned threads = (unsigned)a.B * kQHeads * 16;
  hipLaunchKernelGGL(merge_kernel, dim3((threads + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
