// pa_prefill.h - internal interface between the C ABI (pa_api.cpp) and the
// prefill attention kernel (pa_prefill.hip).  Not installed; the public ABI is pa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pa {

struct PrefillArgs {
  const uint16_t* q;           // [T][Hq][D]
  const uint16_t* k;           // [T][Hkv][D]
  const uint16_t* v;
  const int32_t* cu_tokens;    // [B+1] prompt b is rows cu_tokens[b] .. cu_tokens[b+1]-1
  int B;
  int T;
  float scale_log2;            // scale * log2(e)
  int fp16_weights;            // 0: weights as a bf16 pair with bf16 V; 1: fp16 weights and fp16 V
  float* out;                  // [T][Hq][D]
};

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
