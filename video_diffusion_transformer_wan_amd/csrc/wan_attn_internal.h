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

// bf16 flash-attention forward: q, k, v, o bf16 [b, s, H, 128]; lse (optional, may be null) f32
// [b, H, s_q]: the row log-sum-exp of the scaled scores.
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            const AttnShape& sh, hipStream_t stream);
// Key ranges per query tile for shapes with too few query tiles to fill the chip (1: none),
// the scratch bytes that split needs, and the split launch (attention over key ranges, then the
// combination of the ranges into o).
int attn_bf16_split(const AttnShape& sh);
size_t attn_bf16_split_bytes(const AttnShape& sh, int split);
hipError_t launch_attn_bf16_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const AttnShape& sh, int split, void* ws, hipStream_t stream);

// bf16 attention backward.  Stage 1: the row statistics the gradient kernels read -- lse2 =
// lse * log2(e) and D = rowsum(dO * O), f32, per 64-row query tile [b*H][s_q_pad / 64][lse2 x 64 |
// D x 64] with s_q_pad = s_q rounded up to 64 (padding rows: lse2 = 1e30, D = 0).  Stage 2: dQ,
// then dK and dV (bf16, the layouts of q and k).
size_t attn_bwd_scratch_bytes(const AttnShape& sh);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                           const float* lse, void* dq, void* dk, void* dv, const AttnShape& sh,
                           void* scratch, hipStream_t stream);

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

// FP8 GEMM of the linear layers (layouts documented in include/wan_attn.h): per-token codes and
// scales of x [rows][cols], per-tensor codes and scale of w (the scale word doubles as the amax
// accumulator until the last kernel), and y [m][n] bf16 = (x~ w~^T) * x_scale[m] * w_scale.
hipError_t launch_fp8_quantize_rows(const void* x, int64_t rows, int64_t cols, void* codes, float* scales,
                                    hipStream_t stream);
hipError_t launch_fp8_quantize_tensor(const void* w, int64_t rows, int64_t cols, void* codes, float* scale,
                                      hipStream_t stream);
hipError_t launch_fp8_gemm(const void* x_codes, const float* x_scales, const void* w_codes, const float* w_scale,
                           void* y, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// Block-sparse (VSA-style) attention: the coarse stage (block means into `scratch`, then the
// top-keep key blocks of every query block into block_idx [b*H][n_qb][keep] int32) and the fine
// stage (attention over the listed key blocks).
size_t vsa_select_scratch_bytes(const AttnShape& sh);
int vsa_max_key_blocks();
hipError_t launch_vsa_select(const void* q, const void* k, const AttnShape& sh, int keep, int* block_idx,
                             void* scratch, hipStream_t stream);
hipError_t launch_vsa_attn(const void* q, const void* k, const void* v, const int* block_idx, int keep, void* o,
                           const AttnShape& sh, hipStream_t stream);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace wan
