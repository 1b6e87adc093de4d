// pa_rope.hip - RoPE at the new token's absolute position, fused with the
// one-token KV append (pa_rope_append).
//
// Sources (web pages describing the samir-vllm teaching engine):
//   [README] "6 Hours of YouTube and 85 handtyped pages of notes on LLM
//            Inference - Start here" (memedata.com copy of the project README),
//            feature list: RoPE is applied to the projected queries and keys
//            before attention; KV page pool item: decode appends one new token
//            at its absolute RoPE position.
// The pages print no RoPE constants or pairing.  The caller's table gives, per
// position, 32 cosines then 32 sines (the base and any frequency scaling are
// in it), and dimension i turns with dimension i + 32:
//   x'[i]      = x[i] c_i - x[i + 32] s_i
//   x'[i + 32] = x[i + 32] c_i + x[i] s_i
// Each product and the sum are single FP32 operations (rope_term, with
// contraction off), rounded to BF16 to nearest, ties to even, by integer ops.
//
// Work: one wave per sequence.  A 64-wide BF16 head row is 128 bytes, 8 lanes
// of 16 bytes: lane l holds chunk j = l % 8 (dims 8j .. 8j + 7) of row l / 8,
// so one load moves 8 rows.  The rotation partner of chunk j (dims 32 away) is
// chunk j ^ 4, which lane l ^ 4 holds; it arrives by a lane swap.  Every lane
// loads the 8 cosines and 8 sines of its chunk once per sequence.  The 32 query
// rows are 4 loads, the 8 new key rows and value rows one each; all loads are
// issued before the first store, so q_out may be q itself.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"
#include "pa_rope.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// One 16-byte chunk (8 BF16 values) rotated: x is the lane's chunk, y its
// partner's; the first half of a row takes x c - y s, the second x c + y s.
__device__ __forceinline__ u32x4 rotate_chunk(u32x4 x, u32x4 y, const float (&c)[8], const float (&s)[8],
                                              bool second) {
  u32x4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    unsigned o[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      o[e] = bf16_rne(rope_term(bf16_lo_hi(x[m], e), bf16_lo_hi(y[m], e), c[2 * m + e], s[2 * m + e], second));
    r[m] = o[0] | (o[1] << 16);
  }
  return r;
}

__device__ __forceinline__ u32x4 partner(u32x4 x) {
  u32x4 y;
#pragma unroll
  for (int m = 0; m < 4; ++m) y[m] = (unsigned)__shfl_xor((int)x[m], 4);
  return y;
}

constexpr int kQLoads = kQHeads / 8;  // query rows per sequence / rows per load

__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= a.B) return;  // whole waves leave together
  const int j = lane & 7;
  const int row = lane >> 3;
  const bool second = j >= 4;
  // The rows need no length: they are loaded first, beside the length.  The
  // table row and the page entry depend only on the length and are loaded
  // together, so the chain is two round trips long.
  u32x4 xq[kQLoads];
#pragma unroll
  for (int p = 0; p < kQLoads; ++p) xq[p] = ld16(a.q + ((size_t)b * kQHeads + 8 * p + row) * kHeadDim + 8 * j);
  const size_t src = ((size_t)b * kKvHeads + row) * kHeadDim + 8 * j;
  const u32x4 xk = ld16(a.k_new + src);
  const u32x4 xv = ld16(a.v_new + src);
  const int L = a.seq_lens[b];
  const int pos = L - 1;
  if (L <= 0 || pos >= a.max_pos || (pos >> 4) >= a.max_blocks) return;
  const int page = a.block_table[(size_t)b * a.max_blocks + (pos >> 4)];
  const float* cs = a.cos_sin + (size_t)pos * kHeadDim + 8 * (j & 3);
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(cs + 32);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(cs + 36);
  if (page < 0 || page >= a.num_pages) return;
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};

#pragma unroll
  for (int p = 0; p < kQLoads; ++p)
    st16(a.q_out + ((size_t)b * kQHeads + 8 * p + row) * kHeadDim + 8 * j,
         rotate_chunk(xq[p], partner(xq[p]), c, s, second));
  const size_t dst = ((size_t)page * kPageTokens + (pos & (kPageTokens - 1))) * kRowElems + row * kHeadDim + 8 * j;
  st16(a.k_pool + dst, rotate_chunk(xk, partner(xk), c, s, second));
  st16(a.v_pool + dst, xv);
}

}  // namespace

hipError_t launch_rope_append(const RopeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(rope_append_kernel, dim3((a.B + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
