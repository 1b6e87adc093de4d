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

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_new;  // fused append only: [B][Hkv][D]
  const uint16_t* v_new;
  uint16_t* k_pool_w;     // fused append only: the pools, writable
  uint16_t* v_pool_w;
  int* counters;          // [B] split-completion counters, zero between calls
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* out;
  float* part_o;  // [B][Hq][S][D]
  float* part_m;  // [B][Hq][S]
  float* part_l;  // [B][Hq][S]
  int max_blocks;
  int part_pages;    // a sequence of npages pages has ceil(npages / part_pages) splits (part_pages <= 128)
  int S;             // splits per sequence in the grid = ceil(max_blocks / part_pages)
  float scale_log2;  // scale * log2(e)
};

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

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                         uint16_t* v_pool, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, int B, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int B, bool fused_append, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace pa
