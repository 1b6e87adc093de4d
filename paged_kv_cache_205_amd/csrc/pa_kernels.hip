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
// 16 rows a kv head reads from a page are 16 full 128-byte lines.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// DPP row rotations (within each row of 16 lanes).
#define PA_DPP_ROR(n) (0x120 + (n))

template <int CTRL>
__device__ __forceinline__ float ror16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// All-reduce over the 16 lanes of a row: every lane ends with the row's max / sum.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, ror16<PA_DPP_ROR(8)>(x));
  x = fmaxf(x, ror16<PA_DPP_ROR(4)>(x));
  x = fmaxf(x, ror16<PA_DPP_ROR(2)>(x));
  x = fmaxf(x, ror16<PA_DPP_ROR(1)>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += ror16<PA_DPP_ROR(8)>(x);
  x += ror16<PA_DPP_ROR(4)>(x);
  x += ror16<PA_DPP_ROR(2)>(x);
  x += ror16<PA_DPP_ROR(1)>(x);
  return x;
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------------------
// pa_append: one wave per sequence; each lane copies 16 bytes of the 1 KiB K
// row and 16 bytes of the 1 KiB V row.

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
// pa_decode: one wave per work item (sequence b, kv head g, split s).
//
// Lane l = 16*c + t: token t (0..15) of the current page, dim chunk c (0..3).
// The lane loads 16 bytes of K (dims 8c..8c+7) and 16 bytes at +64 B (dims
// 32+8c..32+8c+7) of row (t, g), and the same 32 bytes of V.
//
// QK^T runs on the matrix cores: S^T tile via two v_mfma_f32_16x16x32_bf16,
// A = the 4 query heads of group g repeated to 16 rows (row i -> head i % 4),
// B = the K tile (column j = token j).  Lane l then holds s[h = r][t = l % 16]
// in result register r, in every row c, which is exactly the token this lane
// holds V for.  BF16 x BF16 products are exact in FP32; sums are FP32.
//
// Softmax is online (FP32): a running maximum per head, shared by the wave, is
// raised only when some score exceeds it (then acc and l are rescaled); the
// weights p = 2^(x - m) with x = scale*log2(e)*(q.k).  PV runs on the VALU in
// FP32: acc[h][i] += p[h] * V[t][dim i of chunk c].  Each lane accumulates its
// own tokens; the 16 lanes of a row are summed once per work item (DPP).

constexpr int kPrefetch = 2;  // pages loaded ahead of the one being consumed

struct PageRegs {
  u32x4 k0, k1, v0, v1;
};

__device__ __forceinline__ void load_page(PageRegs& r, const uint16_t* __restrict__ k_pool,
                                          const uint16_t* __restrict__ v_pool, int32_t page,
                                          uint32_t loff) {
  const size_t base = (size_t)(uint32_t)page * (size_t)(kPageTokens * kRowElems) + loff;
  r.k0 = ld16(k_pool + base);
  r.k1 = ld16(k_pool + base + 32);
  r.v0 = ld16(v_pool + base);
  r.v1 = ld16(v_pool + base + 32);
}

__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  // 1-D grid: blockIdx.x = (b * Hkv + g) * S + split
  const int split = blockIdx.x % a.S;
  const int bg = blockIdx.x / a.S;
  const int g = bg % kKvHeads;
  const int b = bg / kKvHeads;
  const int lane = threadIdx.x;
  const int t = lane & 15;
  const int c = lane >> 4;

  const int L = a.seq_lens[b];
  const int npages = (L + kPageTokens - 1) / kPageTokens;
  const int p0 = split * a.part_pages;
  if (p0 >= npages) {
    if (L <= 0 && split == 0) {  // empty sequence: zero output rows of this group
      float* o = a.out + ((size_t)b * kQHeads + g * kGroup) * kHeadDim;
      reinterpret_cast<f32x4*>(o)[lane] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int p1 = min(p0 + a.part_pages, npages);

  // A operand: query head 4g + (t % 4), dims 8c..8c+7 and 32+8c..32+8c+7.
  const uint16_t* qrow = a.q + ((size_t)b * kQHeads + g * kGroup + (t & 3)) * kHeadDim;
  const bf16x8 qa0 = __builtin_bit_cast(bf16x8, ld16(qrow + 8 * c));
  const bf16x8 qa1 = __builtin_bit_cast(bf16x8, ld16(qrow + 32 + 8 * c));

  const uint32_t loff = (uint32_t)(t * kRowElems + g * kHeadDim + 8 * c);
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks;
  const float c2 = a.scale_log2;

  float m[4], lsum[4], acc[4][16];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    lsum[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
  }

  PageRegs buf[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u)
    if (p0 + u < p1) load_page(buf[u], a.k_pool, a.v_pool, bt[p0 + u], loff);

  for (int jb = p0; jb < p1; jb += kPrefetch) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int j = jb + u;
      if (j >= p1) break;
      PageRegs cur = buf[u];
      if (j + kPrefetch < p1) load_page(buf[u], a.k_pool, a.v_pool, bt[j + kPrefetch], loff);

      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, __builtin_bit_cast(bf16x8, cur.k0), s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, __builtin_bit_cast(bf16x8, cur.k1), s, 0, 0, 0);

      float x[4];
      const bool tail = (j + 1) * kPageTokens > L;  // wave-uniform
      const bool valid = !tail || (j * kPageTokens + t) < L;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = valid ? s[r] * c2 : -INFINITY;
      if (tail && !valid) {
        cur.v0 = u32x4{0u, 0u, 0u, 0u};
        cur.v1 = u32x4{0u, 0u, 0u, 0u};
      }

      bool raise = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) raise |= x[r] > m[r];
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float mn = fmaxf(m[r], row_max16(x[r]));
          const float alpha = (mn == m[r]) ? 1.f : __builtin_amdgcn_exp2f(m[r] - mn);
          m[r] = mn;
          lsum[r] *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[r][i] *= alpha;
        }
      }

      float vf[16];
      const unsigned vw[8] = {cur.v0[0], cur.v0[1], cur.v0[2], cur.v0[3],
                              cur.v1[0], cur.v1[1], cur.v1[2], cur.v1[3]};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        vf[2 * w] = bf16_lo(vw[w]);
        vf[2 * w + 1] = bf16_hi(vw[w]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(x[r] - m[r]);
        lsum[r] += p;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] = fmaf(p, vf[i], acc[r][i]);
      }
    }
  }

  // Sum the 16 token lanes of each row; every lane of row c then holds the
  // totals for the dims of chunk c (rows hold the same l).
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lsum[r] = row_sum16(lsum[r]);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = row_sum16(acc[r][i]);
  }

  // Lane t of row c stores head h = t / 4, quarter qq = t % 4 of chunk c's 16 dims.
  const int h = t >> 2, qq = t & 3;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float lh = 0.f, mh = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (h == r) {
      lh = lsum[r];
      mh = m[r];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (qq == k) o = f32x4{acc[r][4 * k], acc[r][4 * k + 1], acc[r][4 * k + 2], acc[r][4 * k + 3]};
    }
  }
  const float inv = 1.f / lh;
  o *= inv;
  // dims of quarter qq of chunk c: qq 0,1 -> 8c + 4qq; qq 2,3 -> 32 + 8c + 4(qq-2)
  const int d0 = (qq < 2) ? (8 * c + 4 * qq) : (32 + 8 * c + 4 * (qq - 2));
  const int head = g * kGroup + h;
  if (npages <= a.part_pages) {
    float* dst = a.out + ((size_t)b * kQHeads + head) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = o;
  } else {
    const size_t row = ((size_t)b * kQHeads + head) * a.S + split;
    *reinterpret_cast<f32x4*>(a.part_o + row * kHeadDim + d0) = o;
    if (c == 0 && qq == 0) {
      a.part_m[row] = mh;
      a.part_l[row] = lh;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: one block of 512 threads per sequence; thread = (head, 4 dims).

__global__ __launch_bounds__(512) void merge_kernel(MergeArgs a) {
  const int b = blockIdx.x;
  const int head = threadIdx.x >> 4;
  const int d0 = (threadIdx.x & 15) * 4;
  int live = a.S;
  if (a.seq_lens) {
    const int L = a.seq_lens[b];
    if (L <= 0) {
      if (!a.skip_single)
        *reinterpret_cast<f32x4*>(a.out + ((size_t)b * kQHeads + head) * kHeadDim + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
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
      const f32x4 o = *reinterpret_cast<const f32x4*>(a.part_o + (row + s) * kHeadDim + d0);
      num += w * o;
      den += w;
    }
  }
  const f32x4 res = den > 0.f ? num * (1.f / den) : f32x4{0.f, 0.f, 0.f, 0.f};
  *reinterpret_cast<f32x4*>(a.out + ((size_t)b * kQHeads + head) * kHeadDim + d0) = res;
}

// ---------------------------------------------------------------------------
// launchers (host)

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                         uint16_t* v_pool, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, int B, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3((B + 3) / 4), dim3(256), 0, stream, k_new, v_new, k_pool,
                     v_pool, block_table, max_blocks, seq_lens, B);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(decode_kernel, dim3((unsigned)B * kKvHeads * a.S), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3(B), dim3(kQHeads * 16), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
