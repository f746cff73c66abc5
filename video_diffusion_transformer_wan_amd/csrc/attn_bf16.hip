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
constexpr int kVBytes = kBN * kHeadDim * 2;      // V tile, 16 KB
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

__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, r);
}

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr unsigned kRsrcFlags = 0x00020000u;   // raw buffer, 32-bit dwords
constexpr short kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0), other counters untouched

// Buffer resource over [base, base + bytes); loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kRsrcFlags);
}


__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The V^T operands of one 16-key step t (keys 16t .. 16t+15) for the four 32-channel blocks:
// two transposed 64-bit LDS reads per block (keys +0..3 and +4..7 of the lane's half).  Written
// as one asm block that waits for its own reads, so the compiler never sees an output register
// before its data has landed, and the reads are not held back behind the in-flight direct loads
// of the next tile (which write the other LDS stage).
__device__ __forceinline__ void read_v_step(unsigned vs_lds, const int (&v_rd)[4], int t, u32x2_t (&r)[8]) {
  const unsigned a0 = vs_lds + v_rd[0] + 4096 * t, a1 = vs_lds + v_rd[1] + 4096 * t;
  const unsigned a2 = vs_lds + v_rd[2] + 4096 * t, a3 = vs_lds + v_rd[3] + 4096 * t;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:1024\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:1024\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// kWaves waves per workgroup, each owning kQB blocks of 32 query rows.
template <int kWaves, int kQB>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_fwd_bf16_kernel(const Params p) {
  constexpr int kBM = kWaves * 32 * kQB;
  static_assert(kWaves == 8, "K/V tile loads are split over exactly 8 waves");
  // [stage][K | V]: K rows permuted by swap23 and XOR-swizzled by (row % 16); V rows (keys) in
  // natural order, 16-byte chunks XOR-swizzled by 4 * (key % 4), read back transposed.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStageBytes];

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
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;   // bytes between tokens
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q) + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2;
  uint16_t* obase = p.o + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;
  const int64_t kv_bytes = (int64_t)(p.s_kv - 1) * stride + kHeadDim * 2;   // last key row ends here

  // ---- Q^T operand: lane holds query row (l32) of block qb, channels 16c + 8h .. +7
  // (rows past s_q read as zeros and are never stored)
  bf16x8_t qf[kQB][8];
  const int q0 = qt * kBM + wv * (32 * kQB);
  {
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(qbase + q0 * stride, (int64_t)(p.s_q - 1 - q0) * stride + kHeadDim * 2);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        qf[qb][c] = __builtin_bit_cast(
            bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, (unsigned)((qb * 32 + l32) * stride + 32 * c + 16 * h), 0, 0));
  }

  // ---- per-lane offsets of the direct global -> LDS tile loads: wave wv fills 1 KB blocks
  // m = 2wv and 2wv+1 of the K tile and of the V tile; lane i writes bytes 16i .. 16i+15.
  unsigned k_src[2], v_src[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int m = 2 * wv + it;
    const int row = 4 * m + (lane >> 4);
    const int pch = lane & 15;
    k_src[it] = (unsigned)(swap23(row) * stride + 16 * (pch ^ (row & 15)));
    v_src[it] = (unsigned)(row * stride + 16 * (pch ^ ((row & 3) << 2)));
  }
  auto issue_tile = [&](int j) {
    const int64_t off = (int64_t)j * kBN * stride;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + off, kv_bytes - off);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + off, kv_bytes - off);
    unsigned char* st = smem + (j & 1) * kStageBytes;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(st + 1024 * (2 * wv + it)), 16, k_src[it], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(st + kKBytes + 1024 * (2 * wv + it)), 16, v_src[it], 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets
  // K (A operand of S^T): row l32 (+32 for the second key block), chunk (2c + h) ^ (l32 % 16)
  int k_rd[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) k_rd[c] = l32 * 256 + 16 * ((2 * c + h) ^ (l32 & 15));
  // V (A operand of O^T, transposed read): within each 16-lane group, lane 4r + q addresses key
  // row r and channels 4q .. 4q+3 of its 16-channel slice; the read hands lane i channel i of
  // four consecutive keys.
  int v_rd[4];
  {
    const int g = lane >> 4, kq = (lane >> 2) & 3, q = lane & 3;
    const int x = 2 * (g & 1) + (q >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      v_rd[db] = (8 * (g >> 1) + kq) * 256 + 64 * (db ^ kq) + 16 * x + 8 * (q & 1);
  }

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
  issue_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    // tile j is in LDS once every wave's loads have landed; the barrier also tells every wave
    // that tile j-1's buffer is no longer read, so tile j+1 may overwrite it
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(j + 1);
    const unsigned char* ks = smem + (j & 1) * kStageBytes;
    const unsigned vs_lds = lds_addr(ks + kKBytes);

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
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(ks + k_rd[c] + 8192 * kb);
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
      u32x2_t vt[8];
      read_v_step(vs_lds, v_rd, t, vt);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x4_t cat = {vt[2 * db][0], vt[2 * db][1], vt[2 * db + 1][0], vt[2 * db + 1][1]};
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, cat);
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
      uint16_t* dst = obase + (int64_t)row * p.heads * kHeadDim + 4 * h;
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
