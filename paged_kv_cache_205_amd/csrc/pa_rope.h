// pa_rope.h - internal interface between the C ABI (pa_api.cpp) and the RoPE +
// append kernel (pa_rope.hip).  Not installed; the public ABI is pa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pa {

struct RopeArgs {
  const uint16_t* q;         // [B][Hq][D]
  const uint16_t* k_new;     // [B][Hkv][D]
  const uint16_t* v_new;
  const float* cos_sin;      // [max_pos][D]: 32 cosines then 32 sines per position
  uint16_t* q_out;           // [B][Hq][D]
  uint16_t* k_pool;          // [num_pages][16][Hkv][D]
  uint16_t* v_pool;
  const int32_t* block_table;  // [B][max_blocks]
  const int32_t* seq_lens;     // [B]
  int B;
  int max_blocks;
  int max_pos;
  int num_pages;
};

hipError_t launch_rope_append(const RopeArgs& a, hipStream_t stream);

}  // namespace pa
