// 8-bit attention, stage 1: quantisation of the bf16 Q, K, V (gfx950).
//
// The Wan 8-bit attention multiplies Q and K in int8 and runs the output-producing product in FP8
// with FP32 accumulation across KV blocks ("Wan 2.1: VBench 86.22% ..." explainer, section
// "干预与形式化"; "Wan模型是什么它能做什么" explainer, section 4.2).  The pages leave the
// granularity open; this stage produces, per (batch, head):
//   smooth[c] = sqrt(max_t|K[t,c]| / max_t|Q[t,c]|)  (1 if either is 0) -- an exact rebalancing of
//               the int8 range between Q and K (Q' = Q*smooth, K' = K/smooth keeps Q'K'^T = QK^T);
//   Q', K' int8 codes with one scale per 64-token block over all 128 channels;
//   V e4m3 codes with one scale per channel over all tokens, stored transposed per head.
// All decisions are fp32 with correctly rounded divide / sqrt and round-half-even, so the codes
// are fully determined by the inputs.  HBM-bound: each kernel streams its tensor once.

#include "wan_attn_internal.h"

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

constexpr int kThreads = 256;
constexpr int kChanChunk = 1024;   // tokens per workgroup of the channel-max pass

__device__ __forceinline__ float bf16_lo(unsigned x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(unsigned x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const u32x4_t& x, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(x[i]);
    f[2 * i + 1] = bf16_hi(x[i]);
  }
}

__global__ void fill_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// chan_max[bh][tensor][c] = max_t |X[b, t, h, c]| for X in (Q, K, V); float bits via atomicMax
// (non-negative floats order like their bit patterns, so the result is order-independent).
__global__ __launch_bounds__(kThreads) void chan_max_kernel(const uint16_t* q, const uint16_t* k,
                                                            const uint16_t* v, int heads, int s_q,
                                                            int s_kv, float* chan_max) {
  const int tensor = blockIdx.z;
  const int bh = blockIdx.y;
  const int b = bh / heads, h = bh - (bh / heads) * heads;
  const int s = tensor == 0 ? s_q : s_kv;
  const uint16_t* src = tensor == 0 ? q : (tensor == 1 ? k : v);
  const int t0 = blockIdx.x * kChanChunk;
  if (t0 >= s) return;
  const int t1 = min(t0 + kChanChunk, s);
  const int row = threadIdx.x >> 4, cs = threadIdx.x & 15;
  const int64_t tok_stride = (int64_t)heads * kHeadDim;
  const uint16_t* base = src + ((int64_t)b * s * heads + h) * kHeadDim + 8 * cs;
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mx[i] = 0.0f;
  for (int t = t0 + row; t < t1; t += 16) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(base + (int64_t)t * tok_stride);
    float f[8];
    unpack8(x, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) mx[i] = fmaxf(mx[i], fabsf(f[i]));
  }
  __shared__ float red[16][kHeadDim];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[row][8 * cs + i] = mx[i];
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, red[r][threadIdx.x]);
    unsigned* dst = reinterpret_cast<unsigned*>(chan_max) + ((int64_t)bh * 3 + tensor) * kHeadDim + threadIdx.x;
    atomicMax(dst, __builtin_bit_cast(unsigned, m));
  }
}

// sqrtf (not __fsqrt_rn, which maps to the bare v_sqrt_f32) is the correctly rounded square root
__device__ __forceinline__ float smooth_factor(float aq, float ak) {
  return (aq > 0.0f && ak > 0.0f) ? sqrtf(__fdiv_rn(ak, aq)) : 1.0f;
}

// Per (batch, head, channel), once: the smoothing factor and the V scale from the channel maxima,
// then the three per-channel multipliers the quantisation kernels apply, written over the maxima:
// chan_max[bh][0][c] <- smooth (Q), [1][c] <- 1/smooth (K), [2][c] <- 448/max|V| (V; 1 if 0).
__global__ __launch_bounds__(kThreads) void chan_factor_kernel(float* chan_max, float* smooth, float* v_scale,
                                                               int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // bh * 128 + c
  if (i >= n) return;
  const int bh = i / kHeadDim, c = i - bh * kHeadDim;
  float* cm = chan_max + (int64_t)bh * 3 * kHeadDim + c;
  const float aq = cm[0], ak = cm[kHeadDim], av = cm[2 * kHeadDim];
  const float a = smooth_factor(aq, ak);
  smooth[i] = a;
  v_scale[i] = av > 0.0f ? __fdiv_rn(av, 448.0f) : 1.0f;
  cm[0] = a;
  cm[kHeadDim] = __fdiv_rn(1.0f, a);
  cm[2 * kHeadDim] = av > 0.0f ? __fdiv_rn(448.0f, av) : 1.0f;
}

// One 64-token block of Q (blockIdx.z = 0) or K (1): scale by smooth (Q) or 1/smooth (K), block
// absmax, int8 codes, scale.  chan_max holds the multipliers of chan_factor_kernel.
__global__ __launch_bounds__(kThreads) void quant_qk_kernel(const uint16_t* q, const uint16_t* k,
                                                            int heads, int s_q, int s_kv,
                                                            const float* chan_max, int8_t* q_codes,
                                                            float* q_scale, int8_t* k_codes,
                                                            float* k_scale) {
  const int tensor = blockIdx.z;
  const int bh = blockIdx.y;
  const int blk = blockIdx.x;
  const int s = tensor == 0 ? s_q : s_kv;
  const int nb = (s + kQuantBlock - 1) / kQuantBlock;
  if (blk >= nb) return;
  const int b = bh / heads, h = bh - (bh / heads) * heads;
  const uint16_t* src = tensor == 0 ? q : k;
  int8_t* dst = tensor == 0 ? q_codes : k_codes;
  const int row = threadIdx.x >> 4, cs = threadIdx.x & 15;
  const int64_t tok_stride = (int64_t)heads * kHeadDim;
  const int64_t head_off = ((int64_t)b * s * heads + h) * kHeadDim + 8 * cs;

  float factor[8];
  const float* fac = chan_max + ((int64_t)bh * 3 + tensor) * kHeadDim + 8 * cs;
#pragma unroll
  for (int i = 0; i < 8; ++i) factor[i] = fac[i];

  float x[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = blk * kQuantBlock + it * 16 + row;
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (t < s) raw = *reinterpret_cast<const u32x4_t*>(src + head_off + (int64_t)t * tok_stride);
    float f[8];
    unpack8(raw, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[it][i] = __fmul_rn(f[i], factor[i]);
      amax = fmaxf(amax, fabsf(x[it][i]));
    }
  }
  // workgroup max
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));

  const float inv = amax > 0.0f ? __fdiv_rn(127.0f, amax) : 0.0f;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = blk * kQuantBlock + it * 16 + row;
    unsigned packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = __builtin_rintf(__fmul_rn(x[it][i], inv));
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      packed[i >> 2] |= ((unsigned)((int)c) & 0xffu) << (8 * (i & 3));
    }
    if (t < s) {
      const u32x2_t pv = {packed[0], packed[1]};
      *reinterpret_cast<u32x2_t*>(dst + head_off + (int64_t)t * tok_stride) = pv;
    }
  }
  if (threadIdx.x == 0) {
    float* sc = tensor == 0 ? q_scale : k_scale;
    sc[(int64_t)bh * nb + blk] = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 1.0f;
  }
}

__device__ __forceinline__ unsigned cvt_fp8x2(float a, float b) {
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// One 64-token block of V: e4m3 codes with the per-channel scale, written transposed to
// v_codes[bh][c][s_kv_pad]; tokens past s_kv get code 0.  chan_max holds the multipliers of
// chan_factor_kernel.  The transposing LDS tile has rows of 68 bytes: with 64 the 16 lanes that
// write one channel byte each (channels 8 apart) all hit one bank.
constexpr int kVRow = kQuantBlock + 4;
__global__ __launch_bounds__(kThreads) void quant_v_kernel(const uint16_t* v, int heads, int s_kv,
                                                           const float* chan_max, uint8_t* v_codes) {
  const int bh = blockIdx.y;
  const int blk = blockIdx.x;
  const int b = bh / heads, h = bh - (bh / heads) * heads;
  const int nb = (s_kv + kQuantBlock - 1) / kQuantBlock;
  const int64_t s_pad = (int64_t)nb * kQuantBlock;
  const int row = threadIdx.x >> 4, cs = threadIdx.x & 15;
  const int64_t tok_stride = (int64_t)heads * kHeadDim;
  const uint16_t* src = v + ((int64_t)b * s_kv * heads + h) * kHeadDim + 8 * cs;
  const float* cmv = chan_max + ((int64_t)bh * 3 + 2) * kHeadDim;

  float inv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) inv[i] = cmv[8 * cs + i];

  __shared__ __attribute__((aligned(16))) uint8_t tile[kHeadDim][kVRow];   // [channel][token]
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int tl = it * 16 + row;
    const int t = blk * kQuantBlock + tl;
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (t < s_kv) raw = *reinterpret_cast<const u32x4_t*>(src + (int64_t)t * tok_stride);
    float f[8];
    unpack8(raw, f);
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float a = fminf(fmaxf(__fmul_rn(f[i], inv[i]), -448.0f), 448.0f);
      const float c = fminf(fmaxf(__fmul_rn(f[i + 1], inv[i + 1]), -448.0f), 448.0f);
      const unsigned pk = cvt_fp8x2(a, c);
      tile[8 * cs + i][tl] = (uint8_t)(pk & 0xffu);
      tile[8 * cs + i + 1][tl] = (uint8_t)(pk >> 8);
    }
  }
  __syncthreads();
  // 128 channels x 64 bytes; thread writes 32 bytes of one channel (rows are 4-byte aligned)
  const int c = threadIdx.x >> 1, half = threadIdx.x & 1;
  const unsigned* srcrow = reinterpret_cast<const unsigned*>(&tile[c][32 * half]);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(v_codes + ((int64_t)bh * kHeadDim + c) * s_pad +
                                            (int64_t)blk * kQuantBlock + 32 * half);
  dst[0] = u32x4_t{srcrow[0], srcrow[1], srcrow[2], srcrow[3]};
  dst[1] = u32x4_t{srcrow[4], srcrow[5], srcrow[6], srcrow[7]};
}

}  // namespace

hipError_t launch_attn8_quantize(const void* q, const void* k, const void* v, const AttnShape& sh,
                                 int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale,
                                 uint8_t* v_codes, float* v_scale, float* smooth, float* chan_max,
                                 hipStream_t stream) {
  const int bh = (int)(sh.batch * sh.heads);
  const int n_cm = bh * 3 * kHeadDim;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n_cm + 255) / 256), dim3(256), 0, stream, chan_max, n_cm);
  const int64_t smax = sh.s_q > sh.s_kv ? sh.s_q : sh.s_kv;
  hipLaunchKernelGGL(chan_max_kernel, dim3((unsigned)ceil_div(smax, kChanChunk), bh, 3), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), (int)sh.heads, (int)sh.s_q, (int)sh.s_kv, chan_max);
  const int n_ch = bh * kHeadDim;
  hipLaunchKernelGGL(chan_factor_kernel, dim3((n_ch + kThreads - 1) / kThreads), dim3(kThreads), 0, stream,
                     chan_max, smooth, v_scale, n_ch);
  hipLaunchKernelGGL(quant_qk_kernel, dim3((unsigned)ceil_div(smax, kQuantBlock), bh, 2), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     (int)sh.heads, (int)sh.s_q, (int)sh.s_kv, chan_max, q_codes, q_scale, k_codes,
                     k_scale);
  hipLaunchKernelGGL(quant_v_kernel, dim3((unsigned)ceil_div(sh.s_kv, kQuantBlock), bh), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(v), (int)sh.heads, (int)sh.s_kv, chan_max,
                     v_codes);
  return hipGetLastError();
}

}  // namespace wan
