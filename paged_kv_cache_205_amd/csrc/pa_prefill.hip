// Dense causal prefill attention with grouped-query heads (pa_prefill).
//
// Source: the pages' feature list ([README], "6 Hours of YouTube and 85
// handtyped pages of notes on LLM Inference - Start here"): dense causal
// prefill runs grouped-query attention in all 16 layers over the prompt's own
// K and V.  Position i of a prompt attends positions 0..i:
//   out[i][h] = sum_{j <= i} softmax_j(scale * q[i][h] . k[j][g]) v[j][g],  g = h / 4.
//
// Work: one workgroup of 4 waves per (64 query positions, KV head g).  Wave w
// owns positions r0 + 16w .. r0 + 16w + 15 for the 4 query heads of g, so each
// K/V tile staged in LDS serves 16 query rows x 4 heads per wave.  Per tile of
// 32 keys, for each head:
//   S^T = K Q^T        v_mfma_f32_16x16x32_bf16, A = K (16 keys x 32 dims from
//                      LDS), B = Q^T (registers); lane (t, c) gets keys
//                      4c..4c+3 (and 16 + 4c..) of query t;
//   O^T += V^T P^T     16x16x32 MFMA, B = P^T: the lane's 8 weights, in the
//                      order its scores arrived (keys 4c.., 16+4c..), so P needs
//                      no shuffle; A = V^T from transposing LDS reads in the
//                      same key order.  Two weight modes:
//                      bf16 pairs: each weight as a bf16 high part plus a bf16
//                      remainder (two bf16 MFMAs, at most 2^-16 relative error
//                      per weight), V in bf16, row sums added per lane;
//                      fp16: each weight rounded to fp16 (one f16 MFMA), V
//                      converted to fp16 in LDS once per tile by the
//                      workgroup, and the row sum taken over the same rounded
//                      weights by one more MFMA against a tile of ones.
// The softmax is the FP32 online one: a running maximum per (query, head),
// common to the 4 lanes that hold the query, raised (with a rescale) only when
// a tile exceeds it by more than 2^8 (the weights stay below 2^8).
// Keys before the query's prompt or after the query are masked (the tile is
// checked once per wave; only boundary tiles pay for the per-element mask).
// K and V tiles are copied into LDS by the DMA path (a ring of four stages,
// one workgroup barrier per tile), chunks of each 128-byte row XOR-swizzled so
// that the MFMA-layout reads are free of bank conflicts.  The scores of tile
// it + 1 are computed while tile it's weights are formed and applied.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"
#include "pa_prefill.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 64;       // query positions per workgroup
constexpr int kKeys = 32;       // keys per tile
constexpr int kTileBytes = kKeys * 128;  // one plane of a tile: 32 keys x 64 dims x bf16
constexpr int kStage = 2 * kTileBytes;   // K then V
constexpr int kStages = 4;               // LDS ring (a power of two)
constexpr float kSlack = 8.f;            // lazy-maximum slack, base-2 logits

// Position of 16-byte chunk C of LDS key row `key`: C ^ swz(key).
__device__ __forceinline__ int swz(int key) { return (key & 7) ^ ((key >> 3) << 1); }

// Key (within a 32-key tile) of element i of lane group c in the S^T result
// registers of the two 16-key halves, which is also MFMA k index 8c + i of O^T.
__device__ __forceinline__ constexpr int key_of(int c, int i) { return i < 4 ? 4 * c + i : 16 + 4 * c + (i - 4); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for LDS data only (not for outstanding global loads or copies).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Start of the prompt that packed row r belongs to: cu[b] for the largest b with cu[b] <= r.
__device__ __forceinline__ int prompt_start(const int32_t* cu, int B, int r) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid;
  }
  return cu[lo];
}

// Running state of one wave: O^T accumulators, per-(query, head) maximum and
// per-lane partial row sums.  The exponent offset and the raise threshold are
// kept beside the maximum, so a tile that does not raise it recomputes neither.
struct WaveState {
  f32x4 acc[4][4];  // [head][d tile]: O^T rows 16dt + 4c .. +3, query t
  float m[4];       // running maximum (base 2), the same in the 4 lanes of a query
  float nm[4];      // -m, or 0 while m is -inf: the exponent offset
  float thr[4];     // m + kSlack: a larger scaled score raises the maximum
  float l[4];       // bf16-pair weights: this lane's share of the row sum
  f32x4 lsum[4];    // fp16 weights: the row sum of the rounded weights (every register)
};

// K tile operand (A of S^T): key 16*sub + t, dims 8c.. and 32 + 8c..
__device__ __forceinline__ void load_k(u32x4 (&kreg)[2][2], const unsigned char* st, const int (&kofs)[2][2]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    kreg[sub][0] = *reinterpret_cast<const u32x4*>(st + kofs[sub][0]);
    kreg[sub][1] = *reinterpret_cast<const u32x4*>(st + kofs[sub][1]);
  }
}

// Raw scores S^T = K Q^T of one tile for the 4 heads: sv[h][i] is key
// key_of(c, i) of query t.
__device__ __forceinline__ void scores(float (&sv)[4][8], const u32x4 (&kreg)[2][2], const bf16x8 (&qb)[4][2]) {
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[0][0]), qb[h][0], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[1][0]), qb[h][0], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[0][1]), qb[h][1], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[1][1]), qb[h][1], s1, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[h][i] = s0[i];
      sv[h][4 + i] = s1[i];
    }
  }
}

// Per-tile geometry of the wave: first key, and whether some key of the tile is
// outside some row's range [s_r, r] (wave-uniform).
struct TileCtx {
  int j0;
  bool masked;
};

// Rows and ranges of the lane and the wave.
struct RowCtx {
  int c, r, s_r, s_min, w_last;
};

// The V plane of a tile, converted in place from bf16 to fp16 by the whole
// workgroup (thread i: bytes 16i .. 16i + 15).  Exact for the bf16 values within
// the fp16 range.
__device__ __forceinline__ void v_to_fp16(unsigned char* st) {
  u32x4* p = reinterpret_cast<u32x4*>(st + kTileBytes) + threadIdx.x;
  u32x4 w = *p;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = __builtin_bit_cast(unsigned, __builtin_convertvector(
               (f32x2){__builtin_bit_cast(float, w[j] << 16), __builtin_bit_cast(float, w[j] & 0xffff0000u)}, f16x2));
  *p = w;
}

// Softmax and O^T += V^T P^T for tile `st` with scores sv, and, when kNext,
// the scores of the next tile (K from st_next) into sn, whose MFMAs the
// compiler can interleave with this tile's exponentials.  Masked scores become
// -inf, which the exponential turns into exact zeros (c2 > 0).
template <bool kF16, bool kNext>
__device__ __forceinline__ void tile_step(WaveState& ws, float (&sv)[4][8], float (&sn)[4][8], const unsigned char* st,
                                          const unsigned char* st_next, const int (&kofs)[2][2], const int (&vofs)[2],
                                          const bf16x8 (&qb)[4][2], float c2, TileCtx tc, const RowCtx& rc) {
  // V^T by transposing LDS reads: read x of d tile dt gives lane (t, c) the 4
  // values V[key_of(c, 4x + k)][16dt + t], k = 0..3.  Issued as inline
  // assembly: the builtin makes the compiler wait for every outstanding copy
  // into LDS first, the next tiles' included.  LDS operations of one wave
  // complete in order, so the compiler's own lgkmcnt waits stay sufficient;
  // these results are waited for explicitly below.
  s16x4 vr[4][2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const unsigned base = (unsigned)(uintptr_t)st + (unsigned)vofs[x];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vr[dt][x]) : "v"(base ^ (32u * dt)));
  }
  u32x4 kn[2][2];
  if (kNext) load_k(kn, st_next, kofs);

  if (tc.masked) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = tc.j0 + key_of(rc.c, i);
      const bool keep = key <= rc.r && key >= rc.s_r;
#pragma unroll
      for (int h = 0; h < 4; ++h) sv[h][i] = keep ? sv[h][i] : -INFINITY;
    }
  }

  // the lanes' largest scaled scores (-inf where every key is masked)
  float xm[4];
  bool raise = false;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float x = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) x = fmaxf(x, sv[h][i]);
    xm[h] = x * c2;
    raise |= xm[h] > ws.thr[h];
  }
  // Lazy maximum: the running maximum moves only when a score exceeds it by
  // more than kSlack (base 2), so weights stay below 2^kSlack in between.
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float tm = fmaxf(xm[h], __shfl_xor(xm[h], 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mn = fmaxf(ws.m[h], tm);
      const float alpha = (mn == ws.m[h]) ? 1.f : __builtin_amdgcn_exp2f(ws.m[h] - mn);
      ws.m[h] = mn;
      ws.nm[h] = mn == -INFINITY ? 0.f : -mn;
      ws.thr[h] = mn + kSlack;
      if (kF16)
        ws.lsum[h] *= alpha;
      else
        ws.l[h] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ws.acc[h][dt] *= alpha;
    }
  }

  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(vr[0][0]), "+v"(vr[0][1]), "+v"(vr[1][0]), "+v"(vr[1][1]), "+v"(vr[2][0]), "+v"(vr[2][1]),
                 "+v"(vr[3][0]), "+v"(vr[3][1]));
  s16x8 vt[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      vt[dt][k] = vr[dt][0][k];
      vt[dt][4 + k] = vr[dt][1][k];
    }
  if (tc.masked) {
    // A key no row of the wave attends gets V = 0, so its zero weight adds an
    // exact zero whatever the row it was read from holds.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = tc.j0 + key_of(rc.c, i);
      const bool none = key > rc.w_last || key < rc.s_min;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vt[dt][i] = none ? (short)0 : vt[dt][i];
    }
  }
  if (kNext) scores(sn, kn, qb);

#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float nm = ws.nm[h];
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[h][i], c2, nm));
    if (kF16) {
      // p rounded to fp16 (2^-11 relative); the row sum is taken over the same
      // rounded weights, by an MFMA against a tile of ones
      u32x4 ph;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ph[i] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){p[2 * i], p[2 * i + 1]}, f16x2));
      const f16x8 pb = __builtin_bit_cast(f16x8, ph);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        ws.acc[h][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vt[dt]), pb, ws.acc[h][dt], 0, 0, 0);
      const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
      ws.lsum[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb, ws.lsum[h], 0, 0, 0);
    } else {
      ws.l[h] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // p = hi + lo: p rounded to bf16, and the rest (exact in FP32) rounded to
      // bf16; hi + lo is within 2^-16 of p, relatively
      u32x4 phi, plo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned hp = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){p[2 * i], p[2 * i + 1]}, bf16x2));
        const float r0 = p[2 * i] - __builtin_bit_cast(float, hp << 16);
        const float r1 = p[2 * i + 1] - __builtin_bit_cast(float, hp & 0xffff0000u);
        phi[i] = hp;
        plo[i] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){r0, r1}, bf16x2));
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, vt[dt]);
        ws.acc[h][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, phi), ws.acc[h][dt], 0, 0, 0);
        ws.acc[h][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, plo), ws.acc[h][dt], 0, 0, 0);
      }
    }
  }
}

template <bool kF16>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];  // [4 stages][K, V][32 keys][128 B]
  // Workgroup i takes KV head i % 8, so that the workgroups one XCD runs (every
  // eighth) share one head's K and V in that XCD's L2; the latest row blocks,
  // which have the most keys, start first.
  const int g = blockIdx.x & 7;
  const int nqb = gridDim.x >> 3;
  const int r0 = (nqb - 1 - (int)(blockIdx.x >> 3)) * kRows;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, t = lane & 15, c = lane >> 4;
  const int T = a.T;

  // The lane's query row and its prompt's first row, kept in [0, r] so that
  // every address below stays inside the inputs whatever cu_tokens holds.
  const int r = r0 + 16 * w + t;
  const bool row_ok = r < T;
  const int s_r = row_ok ? min(max(prompt_start(a.cu_tokens, a.B, r), 0), r) : T;
  // keys the workgroup reads: from its first row's prompt start to its last row
  const int k_lo = __builtin_amdgcn_readfirstlane(min(max(prompt_start(a.cu_tokens, a.B, r0), 0), r0));
  const int k_hi = min(r0 + kRows, T) - 1;
  const int ntiles = (k_hi - k_lo) / kKeys + 1;
  // The wave's rows: the first, the last one that exists, the earliest and the
  // latest prompt start among them.
  const int w_first = r0 + 16 * w;
  const int w_last = min(w_first + 15, T - 1);
  const bool w_rows = w_first < T;
  const int s_min = __builtin_amdgcn_readfirstlane(s_r);  // lane 0 holds row w_first
  int s_max = s_r;
  s_max = max(s_max, __shfl_xor(s_max, 1));
  s_max = max(s_max, __shfl_xor(s_max, 2));
  s_max = max(s_max, __shfl_xor(s_max, 4));
  s_max = max(s_max, __shfl_xor(s_max, 8));
  s_max = __builtin_amdgcn_readfirstlane(s_max);

  // Q^T operands: query row r, head 4g + h, dims 8c..8c+7 and 32 + 8c..  For
  // a negative scale the signs of q are flipped (exact) and |scale| is used; a
  // scale below 1e-30 acts as 1e-30 (every weight is then exactly 1, as for 0).
  const float c2 = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const unsigned qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  bf16x8 qb[4][2];
  {
    const uint16_t* qrow = a.q + ((size_t)(row_ok ? r : 0) * kQHeads + g * kGroup) * kHeadDim;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      qb[h][0] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + h * kHeadDim + 8 * c) ^ qsign);
      qb[h][1] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + h * kHeadDim + 32 + 8 * c) ^ qsign);
    }
    // take the queries in now, not behind the first tiles' copies
    asm volatile("" : "+v"(qb[0][0]), "+v"(qb[0][1]), "+v"(qb[1][0]), "+v"(qb[1][1]), "+v"(qb[2][0]), "+v"(qb[2][1]),
                 "+v"(qb[3][0]), "+v"(qb[3][1]));
  }

  // DMA: wave w copies keys 8w..8w+7 of a tile (lane: key 8w + lane/8, LDS
  // position lane%8, which holds chunk (lane%8) ^ swz(key)); keys past the last
  // row are read from the last row (and masked).
  const int dkey = 8 * w + (lane >> 3);
  const int dchunk = (lane & 7) ^ swz(dkey);
  auto issue = [&](int stage, int j0) {
    const int row = min(j0 + dkey, T - 1);
    const size_t off = ((size_t)row * kKvHeads + g) * kHeadDim + 8 * dchunk;
    unsigned char* dst = lds + stage * kStage + w * 1024;
    // cached loads: every row block of the prompt reads these rows again
    __builtin_amdgcn_global_load_lds(a.k + off, dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(a.v + off, dst + kTileBytes, 16, 0, 0);
  };

  // LDS read offsets.  K (A of S^T): key 16*sub + t, dims 8c.. (chunk c) and 32 + 8c.. (chunk 4 + c).
  int kofs[2][2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int key = 16 * sub + t;
    kofs[sub][0] = key * 128 + 16 * (c ^ swz(key));
    kofs[sub][1] = key * 128 + 16 * ((4 + c) ^ swz(key));
  }
  // V^T (A of O^T) by transposing reads (ds_read_b64_tr_b16): in each group of
  // 16 lanes (fixed c), lane t of read x supplies the address of the 4 dims
  // 16dt + 4(t%4) .. +3 of key key_of(c, 4x + t/4) and receives dim 16dt + t of
  // those 4 keys.  The dims sit in chunk 2dt + (t/2)%2, at position
  // 2dt ^ ((t/2)%2 ^ swz(key)); the other address bits hold no part of 32dt,
  // so the byte offset is vofs[x] ^ 32dt.
  int vofs[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int key = key_of(c, 4 * x + (t >> 2));
    vofs[x] = kTileBytes + key * 128 + 16 * (((t >> 1) & 1) ^ swz(key)) + 8 * (t & 1);
  }

  WaveState ws;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) ws.acc[h][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    ws.m[h] = -INFINITY;
    ws.nm[h] = 0.f;
    ws.thr[h] = -INFINITY;
    ws.l[h] = 0.f;
    ws.lsum[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Four LDS stages: at tile it the wave reads V of tile it and K of tile
  // it + 1, tile it + 2 is in flight and tile it + 3 is issued into the stage
  // of tile it - 1.  One barrier per tile publishes tile it + 1 and retires
  // tile it - 1.
  auto stage = [&](int it) { return lds + (it & (kStages - 1)) * kStage; };
  // In fp16 mode the workgroup converts tile it + 1's V in place at tile it
  // (tile 0's before the first tile), so each V element is converted once.
  for (int i = 0; i < 3 && i < ntiles; ++i) issue(i, k_lo + i * kKeys);
  if (kF16) {
    if (ntiles >= 3)
      wait_vmcnt<4>();  // this wave's copies of tile 0 have landed
    else if (ntiles == 2)
      wait_vmcnt<2>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    v_to_fp16(stage(0));
  }
  auto sync = [&](int it) {
    if (it + 2 < ntiles)
      wait_vmcnt<2>();  // this wave's copies of tiles <= it + 1 have landed (tile it + 2's may not)
    else
      wait_vmcnt<0>();
    lds_barrier();  // every wave's copies of tiles <= it + 1 have landed; tile it - 1 is done
    if (it + 3 < ntiles) issue((it + 3) & (kStages - 1), k_lo + (it + 3) * kKeys);
    if (kF16 && it + 1 < ntiles) v_to_fp16(stage(it + 1));  // read at tile it + 1, after the next barrier
  };
  auto ctx = [&](int it) {
    const int j0 = k_lo + it * kKeys;
    // masking unless every key of the tile is visible to every row of the wave
    return TileCtx{j0, !(j0 >= s_max && j0 + kKeys - 1 <= w_first)};
  };
  const RowCtx rc{c, r, s_r, s_min, w_last};
  // The tiles some row of the wave attends: keys from s_min to w_last.  Every
  // wave takes part in every tile's barrier (sync(it) once for each it, in
  // order); the accumulators live only through the middle part.
  const int t_lo = w_rows ? max(0, (s_min - k_lo) / kKeys) : ntiles;
  const int t_hi = w_rows ? min(ntiles - 1, (w_last - k_lo) / kKeys) : ntiles - 1;
  int it = 0;
  for (; it < t_lo; ++it) sync(it);
  if (t_lo <= t_hi) {
    float sa[4][8], sb[4][8];
    sync(it);
    {
      u32x4 k0[2][2];
      load_k(k0, stage(it), kofs);
      scores(sa, k0, qb);
    }
    // two tiles per trip, so the score arrays swap roles without copies
    for (; it + 1 < t_hi; it += 2) {
      tile_step<kF16, true>(ws, sa, sb, stage(it), stage(it + 1), kofs, vofs, qb, c2, ctx(it), rc);
      sync(it + 1);
      tile_step<kF16, true>(ws, sb, sa, stage(it + 1), stage(it + 2), kofs, vofs, qb, c2, ctx(it + 1), rc);
      sync(it + 2);
    }
    if (it < t_hi) {
      tile_step<kF16, true>(ws, sa, sb, stage(it), stage(it + 1), kofs, vofs, qb, c2, ctx(it), rc);
      sync(it + 1);
      ++it;
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) sa[h][i] = sb[h][i];
    }
    tile_step<kF16, false>(ws, sa, sb, stage(it), nullptr, kofs, vofs, qb, c2, ctx(it), rc);
    ++it;
  }
  for (; it < ntiles; ++it) sync(it);

  if (!row_ok) return;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float lt;
    if (kF16) {
      lt = ws.lsum[h][0];
    } else {
      lt = ws.l[h] + __shfl_xor(ws.l[h], 16);
      lt += __shfl_xor(lt, 32);
    }
    const float inv = 1.f / lt;
    float* orow = a.out + ((size_t)r * kQHeads + g * kGroup + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(orow + 16 * dt + 4 * c) = ws.acc[h][dt] * inv;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int nqb = (a.T + kRows - 1) / kRows;
  if (a.fp16_weights)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(nqb * kKvHeads), dim3(256), kStages * kStage, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(nqb * kKvHeads), dim3(256), kStages * kStage, stream, a);
  return hipGetLastError();
}

}  // namespace pa
