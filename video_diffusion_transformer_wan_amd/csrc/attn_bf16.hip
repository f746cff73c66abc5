// bf16 flash-attention forward for gfx950 (MI355X).
//
// Computes O = softmax(Q K^T / sqrt(128)) V per (batch, head), non-causal and unmasked: the full
// spatio-temporal self-attention of a Wan DiT block and its umT5 cross-attention ("Wan 2.1:
// VBench 86.22% ..." explainer of the Wan technical report, sections "先看现象" and
// "干预与形式化").  The result is reached by a tiled online softmax over 64-key blocks, exact in
// real arithmetic (a re-association of the definition).
//
// Design (one workgroup = 4 waves = 256 query rows of one (batch, head); 1 workgroup per CU):
//  * The products run transposed so that no operand ever needs a cross-lane shuffle:
//      S^T = K Q^T   (A = K tile from LDS, B = Q^T held in VGPRs for the whole kernel)
//      O^T += V^T P^T (A = V^T tile from LDS, B = P^T taken straight from the S^T accumulators)
//    With v_mfma_f32_32x32x16_bf16 every lane then owns one query row (lane % 32) of a 32-row
//    block, and lanes l and l+32 split the keys.  Row max / row sum are in-lane reductions plus
//    one exchange with lane l^32, and the per-row rescale of O multiplies a lane's own registers.
//  * K rows are placed in LDS with bits 2 and 3 of the key index swapped.  That makes the keys
//    held by a lane's S^T registers, in the order the PV product consumes them, 8 consecutive
//    keys -- so each V^T operand is one 16-byte LDS read.
//  * K and V tiles are double-buffered in LDS (2 x 32 KB); the next tile's global loads are in
//    flight in registers while the current tile computes; one barrier per tile.  V is transposed
//    on its way into LDS with byte permutes.  Both LDS tiles use XOR swizzles so the MFMA operand
//    reads are free of bank conflicts.
//  * Softmax in the exp2 domain with the scale folded in (one FMA + one v_exp_f32 per score);
//    the running max is only moved (and O rescaled) when some row's max grew by more than
//    2^8, since exponents against a stale max stay exact up to that factor; row sums come from
//    the bf16-rounded P through v_dot2 so numerator and denominator see the same weights.
//  * Workgroups are numbered so that the 32 CUs of one XCD work on consecutive query tiles of the
//    same head and share its K/V stream in their L2.

#include "wan_attn_internal.h"

#ifndef WAN_BF16_WAVES
#define WAN_BF16_WAVES 8
#endif
#ifndef WAN_BF16_QB
#define WAN_BF16_QB 1
#endif

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

constexpr int kBN = 64;                     // keys per tile
constexpr int kKBytes = kBN * kHeadDim * 2;      // K tile, 16 KB
constexpr int kVBytes = kHeadDim * kBN * 2;      // V^T tile, 16 KB
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr float kNeg = -1.0e30f;            // masked score (finite: keeps inf - inf out)
constexpr float kLazyLog2 = 8.0f;           // move the running max only past this growth
// log2(e) / sqrt(128): scores go straight into exp2
constexpr float kScaleLog2 = 0.12751743082459868f;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int heads;
  int s_q;
  int s_kv;
  int q_tiles;
  int total;      // q_tiles * batch * heads
  int per_xcd;    // ceil(total / 8)
};

__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}
// K tile: 64 rows (keys, permuted by swap23) x 256 B; 16-byte chunk j of row r sits at j ^ (r%16)
__device__ __forceinline__ int k_off(int r, int j) { return r * 256 + ((j ^ (r & 15)) << 4); }
// V^T tile: 128 rows (channels) x 128 B (64 keys); chunk j (keys 8j..8j+7) sits at j ^ ((d/2)%8)
__device__ __forceinline__ int vt_off(int d, int j) { return d * 128 + ((j ^ ((d >> 1) & 7)) << 4); }

__device__ __forceinline__ unsigned pack_lo(unsigned a, unsigned b) {   // {a.lo16, b.lo16}
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ unsigned pack_hi(unsigned a, unsigned b) {   // {a.hi16, b.hi16}
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, r);
}

// kWaves waves per workgroup, each owning kQB blocks of 32 query rows.
template <int kWaves, int kQB>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_fwd_bf16_kernel(const Params p) {
  constexpr int kThreads = kWaves * 64;
  constexpr int kBM = kWaves * 32 * kQB;
  static_assert(kWaves == 4 || kWaves == 8, "loader split assumes 4 or 8 waves");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStageBytes];

  // XCD-aware numbering: workgroup w runs on XCD w % 8; give each XCD a contiguous range.
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

  const int64_t tok_stride = (int64_t)p.heads * kHeadDim;   // elements between tokens
  const uint16_t* qbase = p.q + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;
  const uint16_t* kbase = p.k + ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim;
  const uint16_t* vbase = p.v + ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim;
  uint16_t* obase = p.o + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;

  // ---- Q^T operand: lane holds query row (l32) of block qb, channels 16c + 8h .. +7
  bf16x8_t qf[kQB][8];
  const int q0 = qt * kBM + wv * (32 * kQB);
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    // rows past s_q read the last row; their results are never stored
    const int row = min(q0 + qb * 32 + l32, p.s_q - 1);
    const uint16_t* src = qbase + (int64_t)row * tok_stride + 8 * h;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[qb][c] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(src + 16 * c));
  }

  // ---- global -> register staging of one K/V tile (256 threads each for K and for V; with 4
  // waves every thread does both, with 8 waves waves 0-3 take K and waves 4-7 take V)
  // K: thread covers rows it*16 + t/16 (it = 0..3), 16-byte chunk t%16
  // V: thread covers keys 4g..4g+3 (g = t/16) at channels 8s..8s+7 (s = t%16)
  const int lt = tid & 255;
  const bool k_loader = kWaves == 4 || tid < 256;
  const bool v_loader = kWaves == 4 || tid >= 256;
  const int kr_row = lt >> 4;
  const int kr_chunk = lt & 15;
  const int vg = lt >> 4;
  const int vs = lt & 15;
  u32x4_t kreg[4], vreg[4];

  auto load_tile = [&](int j) {
    const int kv0 = j * kBN;
    if (k_loader) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      // keys past s_kv read the last key: finite values whose scores are masked below
      const int key = min(kv0 + it * 16 + kr_row, p.s_kv - 1);
      kreg[it] = *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)key * tok_stride + 8 * kr_chunk);
    }
    }
    if (v_loader) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // past s_kv: finite values of the last key, weighted by an exact 0
      const int key = min(kv0 + 4 * vg + r, p.s_kv - 1);
      vreg[r] = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)key * tok_stride + 8 * vs);
    }
    }
  };

  auto store_tile = [&](unsigned char* ks, unsigned char* vts) {
    if (k_loader) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rho = swap23(it * 16 + kr_row);
      *reinterpret_cast<u32x4_t*>(ks + k_off(rho, kr_chunk)) = kreg[it];
    }
    }
    if (v_loader) {
    // transpose 4 keys x 8 channels into 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 8 * vs + 2 * i;
      u32x2_t lo = {pack_lo(vreg[0][i], vreg[1][i]), pack_lo(vreg[2][i], vreg[3][i])};
      u32x2_t hi = {pack_hi(vreg[0][i], vreg[1][i]), pack_hi(vreg[2][i], vreg[3][i])};
      *reinterpret_cast<u32x2_t*>(vts + vt_off(d0, vg >> 1) + ((vg & 1) << 3)) = lo;
      *reinterpret_cast<u32x2_t*>(vts + vt_off(d0 + 1, vg >> 1) + ((vg & 1) << 3)) = hi;
    }
    }
  };

  f32x16_t o[4][kQB];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.0f;
  float m[kQB], l[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m[qb] = kNeg;
    l[qb] = 0.0f;
  }
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  const int n_tiles = (p.s_kv + kBN - 1) / kBN;
  load_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    unsigned char* ks = smem + (j & 1) * kStageBytes;
    unsigned char* vts = ks + kKBytes;
    store_tile(ks, vts);
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);

    // ---- S^T = K Q^T for the 64 keys of this tile: [key block kb][query block qb]
    f32x16_t s[2][kQB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ks + k_off(32 * kb + l32, 2 * c + h));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][c], s[kb][qb], 0, 0, 0);
      }
    }

    // ---- keys past the end of the sequence (last tile only) contribute nothing
    const int kv0 = j * kBN;
    if (kv0 + kBN > p.s_kv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + swap23(32 * kb + 8 * (r >> 2) + 4 * h + (r & 3));
          if (key >= p.s_kv) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[kb][qb][r] = kNeg;
          }
        }
    }

    // ---- online softmax (per lane: one query row per block, 32 of this tile's 64 keys)
    float mnew[kQB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float mx = kNeg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[kb][qb][r], s[kb][qb][r + 1]));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      mnew[qb] = __builtin_fmaxf(m[qb], mx);
      grow |= (mnew[qb] - m[qb]) * kScaleLog2 > kLazyLog2;
    }
    if (__any(grow)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float alpha = __builtin_amdgcn_exp2f((m[qb] - mnew[qb]) * kScaleLog2);
        m[qb] = mnew[qb];
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
      }
    }

    unsigned pk[2][kQB][8];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float mc = m[qb] * kScaleLog2;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], kScaleLog2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r + 1], kScaleLog2, -mc));
          const unsigned pp = cvt_pk_bf16(p0, p1);
          pk[kb][qb][r >> 1] = pp;
          l[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), ones, l[qb], false);
        }
    }

    // ---- O^T += V^T P^T, 16 keys per MFMA: keys 16t .. 16t+15
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1;
      const int u = t & 1;
      bf16x8_t bop[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const u32x4_t x = {pk[kb][qb][4 * u], pk[kb][qb][4 * u + 1], pk[kb][qb][4 * u + 2],
                           pk[kb][qb][4 * u + 3]};
        bop[qb] = __builtin_bit_cast(bf16x8_t, x);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vts + vt_off(32 * db + l32, 2 * t + h));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[qb], o[db][qb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l -> bf16; lane owns channels 32db + 8g + 4h .. +3 of its query row
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const float inv = 1.0f / lt;
    const int row = q0 + qb * 32 + l32;
    if (row < p.s_q) {
      uint16_t* dst = obase + (int64_t)row * tok_stride + 4 * h;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2_t x = {cvt_pk_bf16(o[db][qb][4 * g] * inv, o[db][qb][4 * g + 1] * inv),
                       cvt_pk_bf16(o[db][qb][4 * g + 2] * inv, o[db][qb][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = x;
        }
    }
  }
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o,
                            const AttnShape& sh, hipStream_t stream) {
  Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.heads = (int)sh.heads;
  p.s_q = (int)sh.s_q;
  p.s_kv = (int)sh.s_kv;
  constexpr int kWaves = WAN_BF16_WAVES, kQB = WAN_BF16_QB;
  constexpr int kBM = kWaves * 32 * kQB;
  p.q_tiles = (int)ceil_div(sh.s_q, kBM);
  p.total = (int)(p.q_tiles * sh.batch * sh.heads);
  p.per_xcd = (int)ceil_div(p.total, 8);
  const dim3 grid((unsigned)(8 * p.per_xcd));
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<kWaves, kQB>), grid, dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
