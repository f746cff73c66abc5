// Internal launch interface shared by the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wan {

constexpr int kHeadDim = 128;
constexpr int kQuantBlock = 64;  // tokens per int8 scale block of Q and K

struct AttnShape {
  int64_t batch, heads, s_q, s_kv;
};

// bf16 flash-attention forward: q, k, v, o bf16 [b, s, H, 128].
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o,
                            const AttnShape& sh, hipStream_t stream);
// Key ranges per query tile for shapes with too few query tiles to fill the chip (1: none),
// the scratch bytes that split needs, and the split launch (attention over key ranges, then the
// combination of the ranges into o).
int attn_bf16_split(const AttnShape& sh);
size_t attn_bf16_split_bytes(const AttnShape& sh, int split);
hipError_t launch_attn_bf16_split(const void* q, const void* k, const void* v, void* o,
                                  const AttnShape& sh, int split, void* ws, hipStream_t stream);

// 8-bit path, stage 1: per-channel maxima into `chan_max` ([b, H, 3, 128] f32), then codes and
// scales (layouts documented in include/wan_attn.h).
hipError_t launch_attn8_quantize(const void* q, const void* k, const void* v, const AttnShape& sh,
                                 int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale,
                                 uint8_t* v_codes, float* v_scale, float* smooth, float* chan_max,
                                 hipStream_t stream);

// 8-bit path, stage 2.
hipError_t launch_attn8_fwd(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                            const float* k_scale, const uint8_t* v_codes, const float* v_scale,
                            void* o, const AttnShape& sh, hipStream_t stream);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace wan
