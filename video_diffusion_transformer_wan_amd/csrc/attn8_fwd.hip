// 8-bit attention, stage 2: attention from the quantised operands of stage 1 (gfx950).
//
// The Wan 8-bit FlashAttention: int8 for QK^T, FP8 for the output-producing PV product, FP32
// accumulation across KV blocks ("Wan 2.1: VBench 86.22% ..." explainer, section "干预与形式化";
// "Wan模型是什么它能做什么" explainer, section 4.2).  Per (batch, head) and 64-key block:
//   S   = int32(q_code . k_code) * q_scale * k_scale / sqrt(128)        (v_mfma_i32_32x32x32_i8)
//   m'  = max(m, row max S);  alpha = exp(m - m');  p = exp(S - m')    (fp32)
//   P~  = e4m3(p * 2^8);  O = alpha*O + P~ . V~ (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulators)
//   l   = alpha*l + sum P~;  out = bf16(O * v_scale[c] / l)     (l carries the 2^8 of P~)
// The normaliser sums the same FP8 weights that multiply V (the pages fix FP32 accumulation across
// KV blocks, not which P the normaliser adds), so it runs on the matrix core too: one more fp8 MFMA
// per tile with an all-ones A operand gives every query's sum of P~ over the tile's 64 keys.
// The running max moves whenever a row's max grows (p * 2^8 <= 256 stays inside e4m3's range).
//
// Design (the bf16 kernel's, with 8-bit operands): one workgroup = 8 waves = 256 query rows of
// one (batch, head), one workgroup per CU, persistent and XCD-aware.
//  * S^T = K Q^T and O^T += V~^T P~^T so every lane owns one query row.  K code rows sit in LDS
//    in a key permutation that makes the 32 P~ bytes a lane feeds to one fp8 MFMA belong to 32
//    consecutive keys, so each V~^T operand is 32 contiguous bytes of a row of the
//    pre-transposed V~ tile.
//  * The int32 accumulators of S^T start from the bit pattern of 1.5 * 2^23: the integer dot
//    product (|sum| <= 128 * 127^2 < 2^22) then lands in the fp32 binade [2^23, 2^24), whose
//    ulp is 1, so the int32 result read as fp32 is exactly 1.5 * 2^23 + sum.  One FMA per score
//    turns it into the exponent of p * 2^8 (no int-to-float conversion); the constant 1.5 * 2^23
//    * f it subtracts is rounded once per tile, an error below one integer unit of the sum.
//  * K and V~ tiles (8 KB each) go straight from HBM to LDS (buffer_load ... lds) into a 4-stage
//    ring, the XOR swizzles applied on the source side; operand reads are conflict-free.
//  * Ping-pong: waves 0-3 and 4-7 share the four SIMDs and run half a tile apart; in each
//    half-step one group issues MFMAs (S^T of tile j, PV of tile j-1) while the other runs the
//    softmax of its tile on the VALU.

#include <type_traits>

#include "wan_attn_internal.h"

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;          // 256 query rows per workgroup
constexpr int kBN = 64;                   // keys per tile == quantisation block
constexpr int kKBytes = kBN * kHeadDim;   // 8 KB of int8 K codes
constexpr int kVBytes = kHeadDim * kBN;   // 8 KB of e4m3 V^T codes
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr int kStages = 4;
constexpr float kLog2eInvSqrtD = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr int kMagicBits = 0x4B400000;    // 1.5 * 2^23 as fp32 bits
constexpr float kMagic = 12582912.0f;     // 1.5 * 2^23
constexpr float kNeg = -1.0e30f;          // masked score (finite: keeps inf - inf out)
constexpr unsigned kRsrcFlags = 0x00020000u;   // raw buffer, 32-bit dwords
constexpr short kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0), other counters untouched
constexpr short kWaitVm2 = 0x0F72;             // s_waitcnt vmcnt(2): one tile's two loads may stay in flight

struct Params {
  const int8_t* qc;
  const float* qs;
  const int8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  uint16_t* o;
  int heads, s_q, s_kv, nbq, nbk, q_tiles, total, per_xcd, n_slots;
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

// Values of lanes l and l^32 (the two halves of one query row), returned as (own, other).
__device__ __forceinline__ void pair_values(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup barrier without the release fence of __syncthreads(), which would make every wave
// wait for its in-flight direct-to-LDS loads; the kernel waits for those explicitly.  No wave
// has an LDS read in flight at a barrier (each half-step consumes its reads).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer resource over [base, base + bytes); loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kRsrcFlags);
}

__global__ __launch_bounds__(kThreads, 1) void attn8_fwd_kernel(const Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const bool first_group = wv < kWaves / 2;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t tok_stride = (int64_t)p.heads * kHeadDim;   // bytes between tokens of Q / K codes
  const int64_t s_pad = (int64_t)p.nbk * kBN;                // V~^T row length
  const int n_tiles = p.nbk;

  // ---- direct global -> LDS tile loads: wave wv fills 1 KB block wv of the K tile (LDS rows
  // 8wv .. 8wv+7) and of the V~^T tile (channels 16wv .. 16wv+15); lane i writes bytes
  // 16i .. 16i+15 of its block, i.e. the swizzled chunk position, and so reads the source chunk
  // that belongs there.
  unsigned k_src, v_src;
  {
    const int rho = 8 * wv + (lane >> 3);
    k_src = (unsigned)(key_of_krow(rho) * tok_stride + 16 * ((lane & 7) ^ ((rho >> 1) & 7)));
    const int d = 16 * wv + (lane >> 2);
    v_src = (unsigned)(d * s_pad + 16 * ((lane & 3) ^ ((d >> 2) & 3)));
  }
  // The seed of the S^T accumulators.  The empty asm hides its value, so it stays in 16 VGPRs
  // for the whole kernel instead of being rebuilt from a constant in every tile.
  i32x16_t magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                    kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits, kMagicBits,
                    kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  asm volatile("" : "+v"(magic));
  // A operand of the row-sum MFMA: 32 rows x 64 keys of e4m3 1.0 (code 0x38)
  i32x8_t ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                  0x38383838, 0x38383838, 0x38383838, 0x38383838};
  asm volatile("" : "+v"(ones));

  // Persistent, XCD-aware: workgroup w runs on XCD w % 8 and takes query tiles slot, slot +
  // n_slots, ... of that XCD's contiguous range, so the workgroups of one XCD sweep consecutive
  // query tiles of one head in lockstep and read each K/V tile through their shared L2.
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  for (int t_local = slot; t_local < p.per_xcd; t_local += p.n_slots) {
    const int tile = xcd * p.per_xcd + t_local;
    if (tile >= p.total) break;
    const int qt = tile % p.q_tiles;
    const int bh = tile / p.q_tiles;
    const int bb = bh / p.heads;
    const int hh = bh - bb * p.heads;

    const int8_t* qbase = p.qc + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;
    const int8_t* kbase = p.kc + ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim;
    const uint8_t* vbase = p.vc + (int64_t)bh * kHeadDim * s_pad;
    uint16_t* obase = p.o + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim;
    // k_scale of the head, read with scalar loads (constant address space): a vector load here
    // would be waited for with vmcnt, i.e. together with the tile loads in flight
    typedef __attribute__((address_space(4))) const float const_float_t;
    const_float_t* kscale = (const_float_t*)(p.ks + (int64_t)bh * p.nbk);
    float ks_next = kscale[0];   // k_scale of the tile the next softmax half-step works on

    // Q codes (B operand of S^T): query row l32 of this wave, channels 32c + 16h .. +15
    const int q_row = qt * kBM + wv * 32 + l32;
    const int q_rc = min(q_row, p.s_q - 1);
    i32x4_t qf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qf[c] = *reinterpret_cast<const i32x4_t*>(qbase + (int64_t)q_rc * tok_stride + 32 * c + 16 * h);
    const float q_scale = p.qs[(int64_t)bh * p.nbq + q_rc / kBN];
    auto issue_tile = [&](int j) __attribute__((always_inline)) {
      const int kv0 = j * kBN;
      const __amdgpu_buffer_rsrc_t kr =
          make_rsrc(kbase + (int64_t)kv0 * tok_stride, (int64_t)(p.s_kv - 1 - kv0) * tok_stride + kHeadDim);
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + kv0, kHeadDim * s_pad - kv0);
      unsigned char* st = smem + (j % kStages) * kStageBytes + 1024 * wv;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)st, 16, k_src, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(st + kKBytes), 16, v_src, 0, 0, 0);
    };

    f32x16_t o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = kNeg;     // running max of S in log2 units
    // running sum of P~ (= p * 2^8 in FP8) per query: every register of the row-sum MFMA's output holds
    // the query's sum; only register 0 is read (and rescaled), the others are left unscaled.
    f32x16_t lsum;
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum[r] = 0.0f;
    i32x16_t s[2];      // S^T of the newest tile per 32-key block, as 1.5 * 2^23 + integer sum
    unsigned pb[8];     // P~ of the tile awaiting its PV product: bytes 16kb + r <-> s[kb][r]

    // MFMA half-step: S^T of tile j (kQK), then the PV product of tile j-1 (kPV), as one stream
    // of 8 steps (4 S^T steps over 32 channels, 2 MFMAs each; 4 PV steps over 32 channels of
    // V~, 1 MFMA each).  The LDS operands of step i+1 are read while step i issues its MFMAs.
    auto mfma_phase = [&](int j, auto qk_tag, auto pv_tag) __attribute__((always_inline)) {
      constexpr bool kQK = decltype(qk_tag)::value;
      constexpr bool kPV = decltype(pv_tag)::value;
      const unsigned char* ks = smem + (j % kStages) * kStageBytes;
      const unsigned char* vts = smem + ((j + kStages - 1) % kStages) * kStageBytes + kKBytes;
      // this wave's share of the loads of tile j+2: its descriptor arithmetic is scalar work that
      // would otherwise sit on the softmax half-step's critical path
      const bool load_next = kQK && j + 2 < n_tiles;
      if (load_next) issue_tile(j + 2);
      __builtin_amdgcn_s_setprio(3);
      if constexpr (kPV) {
        const i32x8_t bop = {(int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3],
                             (int)pb[4], (int)pb[5], (int)pb[6], (int)pb[7]};
        lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, bop, lsum, 0, 0, 0, 0, 0, 0);
      }
      constexpr int kFirst = kQK ? 0 : 4;
      constexpr int kSteps = kPV ? 8 : 4;
      i32x4_t ring[2][2];
      auto read_step = [&](int i, i32x4_t (&f)[2]) {
        if (i < 4) {   // K rows 32kb + l32, channels 32i + 16h .. +15
          f[0] = *reinterpret_cast<const i32x4_t*>(ks + k_off(l32, 2 * i + h));
          f[1] = *reinterpret_cast<const i32x4_t*>(ks + k_off(32 + l32, 2 * i + h));
        } else {       // V~^T row 32(i-4) + l32, keys 32h .. 32h+31
          const int d = 32 * (i - 4) + l32;
          f[0] = *reinterpret_cast<const i32x4_t*>(vts + v_off(d, 2 * h));
          f[1] = *reinterpret_cast<const i32x4_t*>(vts + v_off(d, 2 * h + 1));
        }
      };
      read_step(kFirst, ring[0]);
#pragma unroll
      for (int i = kFirst; i < kSteps; ++i) {
        const int cur = (i - kFirst) & 1;
        if (i + 1 < kSteps) read_step(i + 1, ring[cur ^ 1]);
        if (i < 4) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ring[cur][kb], qf[i], i == 0 ? magic : s[kb], 0, 0, 0);
        } else {
          const i32x8_t a = {ring[cur][0][0], ring[cur][0][1], ring[cur][0][2], ring[cur][0][3],
                             ring[cur][1][0], ring[cur][1][1], ring[cur][1][2], ring[cur][1][3]};
          const i32x8_t bop = {(int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3],
                               (int)pb[4], (int)pb[5], (int)pb[6], (int)pb[7]};
          o[i - 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, o[i - 4], 0, 0, 0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // this wave's loads of tile j+1 (issued at the start of its previous MFMA half-step) must
      // have landed before the barrier that ends this half-step; those of tile j+2 may not have
      if (load_next) __builtin_amdgcn_s_waitcnt(kWaitVm2);
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
    };
    const std::true_type yes{};
    const std::false_type no{};

    // VALU half-step: the softmax of tile j (its S^T is in s), leaving P~ in pb.
    auto softmax_phase = [&](int j) __attribute__((always_inline)) {
      // (the whole vector is reinterpreted: __builtin_bit_cast of a single vector element read
      // element 0 whatever the index)
      f32x16_t sf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sf[kb] = __builtin_bit_cast(f32x16_t, s[kb]);
      const int kv0 = j * kBN;
      if (kv0 + kBN > p.s_kv) {   // keys past the end: S^T register (kb, r) holds key 32h + 16kb + r
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kv0 + 32 * h + 16 * kb + r >= p.s_kv) sf[kb][r] = kNeg;
      }
      float mx = kNeg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sf[kb][r]), sf[kb][r + 1]);
      float ma, mb;
      pair_values(mx, ma, mb);
      const float f = q_scale * ks_next * kLog2eInvSqrtD;   // one integer unit in log2 units
      ks_next = kscale[j + 1 < n_tiles ? j + 1 : j];
      const float mnew = __builtin_fmaxf(m, (__builtin_fmaxf(ma, mb) - kMagic) * f);
      if (__any(mnew > m)) {
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        lsum[0] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      // exponent of p * 2^8: (sf - 1.5 * 2^23) * f + 8 - m
      const float bias = 8.0f - m - kMagic * f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const int r = 4 * wd;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sf[kb][r], f, bias));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sf[kb][r + 1], f, bias));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sf[kb][r + 2], f, bias));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sf[kb][r + 3], f, bias));
          // both halves of the word are written, so the old value passed in is never kept (a
          // constant there would cost a v_mov per word)
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, (int)pb[4 * kb + wd], false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
          pb[4 * kb + wd] = (unsigned)x;
        }
    };

    // Schedule (B_k = k-th workgroup barrier of this query tile, B_0 the one after the prologue).
    // Every wave runs  MFMA(j) | barrier | softmax(j) | barrier  for j = 0 .. n-1, then the PV
    // product of tile n-1, waves 4-7 one barrier behind waves 0-3: group 1's MFMA(j) lies between
    // B_2j and B_2j+1, group 2's between B_2j+1 and B_2j+2.  Tile t is loaded into stage t % 4 at
    // the start of MFMA(t-2) -- after B_2t-4 (group 1) or B_2t-3 (group 2), so after the last
    // read of tile t-4, by group 2's PV product in MFMA(t-3), which ends at B_2t-4 -- and waited
    // for at the end of MFMA(t-1), before the barrier B_2t after which group 1 reads it.  The
    // prologue loads tiles 0 and 1 and waits for tile 0.
    issue_tile(0);
    if (n_tiles > 1) {
      issue_tile(1);
      __builtin_amdgcn_s_waitcnt(kWaitVm2);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    barrier();
    if (!first_group) barrier();
    mfma_phase(0, yes, no);
    barrier();
    softmax_phase(0);
    barrier();
    if (n_tiles > 1) {
      int j = 1;
      do {
        mfma_phase(j, yes, yes);
        barrier();
        softmax_phase(j);
        barrier();
      } while (++j < n_tiles);
    }
    mfma_phase(n_tiles, no, yes);
    if (first_group) barrier();
    barrier();   // every wave is done with the LDS ring before the next tile's loads

    // ---- epilogue: out = O * v_scale[c] / l  (l carries the 2^8 of P~); the lane's output
    // channels are 32db + 8g + 4h .. +3
    const float inv = 1.0f / lsum[0];
    if (q_row < p.s_q) {
      uint16_t* dst = obase + (int64_t)q_row * tok_stride + 4 * h;
      const float* vsc = p.vs + (int64_t)bh * kHeadDim + 4 * h;
      float vsv[4][4][4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) vsv[db][g][e] = vsc[32 * db + 8 * g + e];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float* vs4 = vsv[db][g];
          u32x2_t x = {cvt_pk_bf16(o[db][4 * g] * vs4[0] * inv, o[db][4 * g + 1] * vs4[1] * inv),
                       cvt_pk_bf16(o[db][4 * g + 2] * vs4[2] * inv, o[db][4 * g + 3] * vs4[3] * inv)};
          *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = x;
        }
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
  // one workgroup per CU (the registers allow no second one)
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8)
      cus = n;
    else
      cus = 256;
  }
  p.n_slots = (int)(p.per_xcd < cus / 8 ? p.per_xcd : cus / 8);
  hipLaunchKernelGGL(attn8_fwd_kernel, dim3((unsigned)(8 * p.n_slots)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
