// 8-bit attention, stage 2: attention from the quantised operands of stage 1 (gfx950).
//
// The Wan 8-bit FlashAttention: int8 for QK^T, FP8 for the output-producing PV product, FP32
// accumulation across KV blocks ("Wan 2.1: VBench 86.22% ..." explainer, section "干预与形式化";
// "Wan模型是什么它能做什么" explainer, section 4.2).  Per (batch, head) and 64-key block:
//   S   = int32(q_code . k_code) * q_scale * k_scale / sqrt(128)        (v_mfma_i32_32x32x32_i8)
//   m'  = max(m, row max S);  alpha = exp(m - m');  p = exp(S - m')    (fp32)
//   P~  = e4m3(p * 2^8);  O = alpha*O + P~ . V~ (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulators)
//   l   = alpha*l + sum p;  out = bf16(O * v_scale[c] / (2^8 * l))
// The running max moves whenever a row's max grows (p * 2^8 <= 256 stays inside e4m3's range).
//
// Layout mirrors the bf16 kernel: 8 waves x 32 query rows per workgroup, S^T = K Q^T and
// O^T += V~^T P~^T so every lane owns one query row.  K code rows are placed in LDS in a fixed
// key permutation that makes the 32 P~ bytes a lane feeds to one fp8 MFMA belong to 32
// consecutive keys, so each V~^T operand is 32 contiguous bytes of a row of the pre-transposed
// V~ tile.  Both LDS tiles are 8 KB, double-buffered, XOR-swizzled against bank conflicts.

#include "wan_attn_internal.h"

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;          // 256 query rows per workgroup
constexpr int kBN = 64;                   // keys per tile == quantisation block
constexpr int kKBytes = kBN * kHeadDim;   // 8 KB of int8 K codes
constexpr int kVBytes = kHeadDim * kBN;   // 8 KB of e4m3 V^T codes
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr float kLog2eInvSqrtD = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr int kNegInt = -0x40000000;      // masked score (int accumulator domain)

struct Params {
  const int8_t* qc;
  const float* qs;
  const int8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  uint16_t* o;
  int heads, s_q, s_kv, nbq, nbk, q_tiles, total, per_xcd;
};

// LDS row of key kappa (0..63) of the tile: bits [h|kb|a1 a0|c1 c0] -> [kb|a1 a0|h|c1 c0]
__device__ __forceinline__ int krow_of_key(int kap) {
  return (((kap >> 4) & 1) << 5) | (((kap >> 2) & 3) << 3) | (((kap >> 5) & 1) << 2) | (kap & 3);
}
// and back: the key held in LDS row rho
__device__ __forceinline__ int key_of_krow(int rho) {
  return (((rho >> 2) & 1) << 5) | (((rho >> 5) & 1) << 4) | (((rho >> 3) & 3) << 2) | (rho & 3);
}
// K tile: 64 rows x 128 B; 16-byte chunk j of row r at j ^ ((r/2)%8)
__device__ __forceinline__ int k_off(int r, int j) { return r * 128 + ((j ^ ((r >> 1) & 7)) << 4); }
// V^T tile: 128 rows (channels) x 64 B; 16-byte chunk j of row d at j ^ ((d/4)%4)
__device__ __forceinline__ int v_off(int d, int j) { return d * 64 + ((j ^ ((d >> 2) & 3)) << 4); }

__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, r);
}

__global__ __launch_bounds__(kThreads, 1) void attn8_fwd_kernel(const Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];

  const int w = blockIdx.x;
  const int tile = (w & 7) * p.per_xcd + (w >> 3);
  if (tile >= p.total) return;
  const int qt = tile % p.q_tiles;
  const int bh = tile / p.q_tiles;
  const int bb = bh / p.heads;
  const int hh = bh - bb * p.heads;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int64_t tok_stride = (int64_t)p.heads * kHeadDim;
  const int8_t* qbase = p.qc + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;
  const int8_t* kbase = p.kc + ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim;
  const int64_t s_pad = (int64_t)p.nbk * kBN;
  const uint8_t* vbase = p.vc + (int64_t)bh * kHeadDim * s_pad;
  uint16_t* obase = p.o + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;

  // Q codes (B operand of S^T): query row l32 of this wave, channels 32c + 16h .. +15
  const int q_row = qt * kBM + wv * 32 + l32;
  const int q_rc = min(q_row, p.s_q - 1);
  i32x4_t qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qf[c] = *reinterpret_cast<const i32x4_t*>(qbase + (int64_t)q_rc * tok_stride + 32 * c + 16 * h);
  const float q_scale = p.qs[(int64_t)bh * p.nbq + q_rc / kBN];
  const float* kscale = p.ks + (int64_t)bh * p.nbk;

  // staging: threads 0-255 carry K (2 chunks of 16 B), threads 256-511 carry V^T (2 chunks)
  const bool k_loader = tid < 256;
  const int lt = tid & 255;
  u32x4_t stage[2];

  auto load_tile = [&](int j) {
    const int kv0 = j * kBN;
    if (k_loader) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int key = min(kv0 + (lt >> 3) + 32 * it, p.s_kv - 1);
        stage[it] = *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)key * tok_stride + 16 * (lt & 7));
      }
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int d = (lt >> 2) + 64 * it;
        stage[it] = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)d * s_pad + kv0 + 16 * (lt & 3));
      }
    }
  };
  auto store_tile = [&](unsigned char* ks, unsigned char* vts) {
    if (k_loader) {
#pragma unroll
      for (int it = 0; it < 2; ++it)
        *reinterpret_cast<u32x4_t*>(ks + k_off(krow_of_key((lt >> 3) + 32 * it), lt & 7)) = stage[it];
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it)
        *reinterpret_cast<u32x4_t*>(vts + v_off((lt >> 2) + 64 * it, lt & 3)) = stage[it];
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -1.0e30f;   // running max of S * log2(e), fp32
  float l = 0.0f;       // running sum of p * 2^8

  const int n_tiles = p.nbk;
  load_tile(0);
  for (int j = 0; j < n_tiles; ++j) {
    unsigned char* ks = smem + (j & 1) * kStageBytes;
    unsigned char* vts = ks + kKBytes;
    store_tile(ks, vts);
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);

    // S^T (int32) for the two 32-key blocks
    i32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const i32x4_t a = *reinterpret_cast<const i32x4_t*>(ks + k_off(32 * kb + l32, 2 * c + h));
        s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qf[c], s[kb], 0, 0, 0);
      }

    // keys past s_kv (last tile only): excluded from the max here, weighted by 0 below
    const int kv0 = j * kBN;
    const bool last = kv0 + kBN > p.s_kv;
    unsigned valid = 0xffffffffu;   // bit 16kb + r: key of S^T register (kb, r) exists
    if (last) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + key_of_krow(32 * kb + 8 * (r >> 2) + 4 * h + (r & 3));
          if (key >= p.s_kv) {
            s[kb][r] = kNegInt;
            valid &= ~(1u << (16 * kb + r));
          }
        }
    }

    // row max on the integer scores (the scale factor is positive)
    int mx = kNegInt;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = max(mx, max(s[kb][r], s[kb][r + 1]));
    mx = max(mx, __shfl_xor(mx, 32));
    const float f = q_scale * kscale[j] * kLog2eInvSqrtD;   // int score -> log2 units
    const float mnew = fmaxf(m, (float)mx * f);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }

    // exponent of p * 2^8 in log2 units
    const float bias = 8.0f - m;
    float t[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) t[kb][r] = __builtin_fmaf((float)s[kb][r], f, bias);
    if (last) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((valid >> (16 * kb + r)) & 1u)) t[kb][r] = -1.0e30f;
    }

    // P~ = e4m3(p * 2^8): B operand bytes 16kb + r  <->  S^T register r of key block kb
    unsigned pb[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int r = 4 * wd;
        const float p0 = __builtin_amdgcn_exp2f(t[kb][r]);
        const float p1 = __builtin_amdgcn_exp2f(t[kb][r + 1]);
        const float p2 = __builtin_amdgcn_exp2f(t[kb][r + 2]);
        const float p3 = __builtin_amdgcn_exp2f(t[kb][r + 3]);
        l += (p0 + p1) + (p2 + p3);
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
        pb[4 * kb + wd] = (unsigned)x;
      }
    const i32x8_t bop = {(int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3],
                         (int)pb[4], (int)pb[5], (int)pb[6], (int)pb[7]};

    // O^T += V~^T P~^T over all 64 keys: lane half h supplies keys 32h .. 32h+31
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + l32;
      const i32x4_t a0 = *reinterpret_cast<const i32x4_t*>(vts + v_off(d, 2 * h));
      const i32x4_t a1 = *reinterpret_cast<const i32x4_t*>(vts + v_off(d, 2 * h + 1));
      const i32x8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, o[db], 0, 0, 0, 0, 0, 0);
    }
  }

  // epilogue: out = O * v_scale[c] / l  (l carries the 2^8 of P~)
  const float lt_ = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt_;
  if (q_row < p.s_q) {
    uint16_t* dst = obase + (int64_t)q_row * tok_stride + 4 * h;
    const float* vsc = p.vs + (int64_t)bh * kHeadDim + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * db + 8 * g;
        u32x2_t x = {cvt_pk_bf16(o[db][4 * g] * vsc[c0] * inv, o[db][4 * g + 1] * vsc[c0 + 1] * inv),
                     cvt_pk_bf16(o[db][4 * g + 2] * vsc[c0 + 2] * inv, o[db][4 * g + 3] * vsc[c0 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(dst + c0) = x;
      }
  }
}

}  // namespace

hipError_t launch_attn8_fwd(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                            const float* k_scale, const uint8_t* v_codes, const float* v_scale,
                            void* o, const AttnShape& sh, hipStream_t stream) {
  Params p;
  p.qc = q_codes;
  p.qs = q_scale;
  p.kc = k_codes;
  p.ks = k_scale;
  p.vc = v_codes;
  p.vs = v_scale;
  p.o = static_cast<uint16_t*>(o);
  p.heads = (int)sh.heads;
  p.s_q = (int)sh.s_q;
  p.s_kv = (int)sh.s_kv;
  p.nbq = (int)ceil_div(sh.s_q, kQuantBlock);
  p.nbk = (int)ceil_div(sh.s_kv, kQuantBlock);
  p.q_tiles = (int)ceil_div(sh.s_q, kBM);
  p.total = (int)(p.q_tiles * sh.batch * sh.heads);
  p.per_xcd = (int)ceil_div(p.total, 8);
  hipLaunchKernelGGL(attn8_fwd_kernel, dim3((unsigned)(8 * p.per_xcd)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
