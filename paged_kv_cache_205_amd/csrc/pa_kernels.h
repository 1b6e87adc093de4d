// pa_kernels.h - internal interface between the C ABI (pa_api.cpp) and the
// gfx950 kernels (pa_kernels.hip).  Not installed; the public ABI is pa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kPageTokens = 16;
constexpr int kHeadDim = 64;
constexpr int kKvHeads = 8;
constexpr int kQHeads = 32;
constexpr int kGroup = kQHeads / kKvHeads;
constexpr int kRowElems = kKvHeads * kHeadDim;  // bf16 values in one token row of a page plane
constexpr int kMaxDecodeBatch = 4096;           // the work plan keeps 3 ints per sequence in LDS

struct DecodeArgs {
  // the fields read at the start of the kernel fill the first 64 bytes
  const int32_t* seq_lens;
  const int32_t* block_table;
  const uint16_t* q;
  const uint16_t* k_new;  // fused append only: [B][Hkv][D]
  const uint16_t* v_new;
  int B;
  int max_blocks;
  // The split plan of a batch in which every sequence fills its table row
  // (computed on the host from the sizes alone): splits per sequence,
  // ceil(2^32 / guess_ns) for dividing by it (guess_ns > 1), pages per split.
  int guess_ns;
  uint32_t guess_magic;
  int guess_pp;
  int part_pages;  // pages per split (<= 128); 0: chosen per call from the batch's total pages
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int S;             // row stride of the partials: an upper bound of any sequence's split count
  int narrow;        // workgroups to use when the items are long (one per CU); 0: all of the grid
  float scale_log2;  // scale * log2(e)
  uint16_t* k_pool_w;  // fused append only: the pools, writable
  uint16_t* v_pool_w;
  int* counters;  // [B][Hkv] split-completion counters, zero between calls
  int* queue;     // {next item, workgroups done}, zero between calls; NULL: one item per workgroup
  float* out;
  float* part_o;  // [B][Hq][S][D]
  float* part_m;  // [B][Hq][S]
  float* part_l;  // [B][Hq][S]
  const float* cos_sin;  // fused RoPE only: [max_pos][D], 32 cosines then 32 sines per position
  int max_pos;           // rows of cos_sin (positions past it read its last row; the host requires >= 16 max_blocks)
  const int* plan;       // planned decode only: a plan written by plan_kernel (PlanHeader, then the items)
};

// A decode plan: the work items of one batch, built once from seq_lens and read
// by every layer's decode launch of the step.  The header takes the first 256
// bytes; slot i is int4 {sequence, split, splits of that sequence, its length}
// at byte 256 + 16 i, in the plan's order (long items by pages, longest
// first; short ones multi-split sequences first, then sequence order; one page
// count for all: (sequence, split) order).  In the first static_rounds rounds
// (one, as built) workgroup w < active runs the item in slot r * active + w
// (later fixed rounds would alternate direction); the items after them are
// claimed in order through the workspace's queue counter.
struct PlanHeader {
  int magic;       // kPlanMagic once written
  int B;           // what the plan was built for
  int max_blocks;
  int part_pages;  // requested pages per split (0: automatic)
  int n_items;
  int active;         // workgroups that take items
  int static_rounds;  // rounds dealt to fixed slots
  int pp;             // pages per split chosen
  int uniform_ns;     // > 0: one page count for every sequence, this many splits each, items in order
  int uniform_pages;
  int reserved;
  int grid;  // the decode grid the plan was dealt for
};
constexpr int kPlanMagic = 0x504c414e;  // "PLAN"
constexpr size_t kPlanHeaderBytes = 256;
constexpr int kPlanMaxBins = 1024;  // workgroups a plan deals to; planned decode grids stay within it
// Items a plan can hold for these sizes (an upper bound for any lengths).
size_t plan_max_items(int B, int max_blocks, int part_pages);

// Writes the plan of a batch (one workgroup).  grid: the decode grid.
hipError_t launch_plan(const int32_t* seq_lens, int B, int max_blocks, int part_pages, int narrow, int grid,
                       int* plan, hipStream_t stream);
// Decode launch that takes its items from a.plan (the same kernels' item code).
hipError_t launch_decode_planned(const DecodeArgs& a, int grid, bool fused_append, bool rope, hipStream_t stream);

struct MergeArgs {
  int B;
  const float* part_o;
  const float* part_m;
  const float* part_l;
  const int32_t* seq_lens;  // may be NULL
  float* out;
  int part_tokens;
  int S;
  int skip_single;  // 1 inside pa_decode: rows with one split were written by the decode kernel
};

struct FillArgs {
  const uint16_t* k_src;  // [T][Hkv][D]
  const uint16_t* v_src;
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* block_table;  // [B][max_blocks]
  const int32_t* start;        // [B] first position of each run; NULL: all 0
  const int32_t* cu_tokens;    // [B+1] run b is rows cu_tokens[b] .. cu_tokens[b+1]-1
  int B;
  int max_blocks;
  int T;
  int num_pages;
};

hipError_t launch_fill(const FillArgs& a, hipStream_t stream);

// RoPE arithmetic shared by the RoPE kernels.  One output of a rotation pair
// (i, i + 32): x c - y s for the first half (second = false), x c + y s for the
// second, each product and the sum a single FP32 operation rounded to nearest
// (no fused multiply-add).
__device__ __forceinline__ float rope_term(float x, float y, float c, float s, bool second) {
#pragma clang fp contract(off)
  const float a = x * c;
  const float b = y * s;
  return second ? a + b : a - b;
}
// FP32 -> BF16 bits, to nearest with ties to even; a NaN keeps its sign and
// upper payload with the quiet bit set.
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __builtin_bit_cast(unsigned, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// BF16 element e (0 or 1) of a dword, as FP32.
__device__ __forceinline__ float bf16_lo_hi(unsigned w, int e) {
  return __builtin_bit_cast(float, e == 0 ? w << 16 : w & 0xffff0000u);
}

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                         uint16_t* v_pool, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, int B, hipStream_t stream);
size_t decode_lds_bytes(int B);
// Pages per split that the automatic plan picks for a batch with this many pages
// (all with the same page count), and its smallest split for a batch of B sequences.
int auto_split_pages(long long total_pages, int B);
int auto_split_min_pages(int B);
// rope: also rotate q and the new key by RoPE at position L-1 (needs fused_append).
hipError_t launch_decode(const DecodeArgs& a, int grid, bool fused_append, bool rope, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// Sets n ints at p to zero, with a kernel.
hipError_t launch_clear(int* p, int n, hipStream_t stream);

}  // namespace pa
