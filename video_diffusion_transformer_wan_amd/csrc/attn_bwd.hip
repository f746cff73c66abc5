// bf16 attention backward for gfx950 (MI355X): dQ, dK and dV of O = softmax(Q K^T / sqrt(128)) V,
// non-causal, per (batch, head).  The backward of non-causal attention is the beta = 8 term of the
// DiT cost model and the bulk of training time at long sequences ("Wan 2.1: VBench 86.22% ..."
// explainer of the Wan technical report, section "先看现象").  With P = exp(S - lse) recomputed from
// the forward's row log-sum-exp, D_i = rowsum(dO_i * O_i) and dS = P * (dP - D):
//     dV = P^T dO,   dP = dO V^T,   dQ = dS K / sqrt(128),   dK = dS^T Q / sqrt(128)
// (the chain rule through the row softmax; D_i = sum_j P_ij dP_ij = dO_i . O_i).
//
// Kernels:
//  * attn_bwd_prep_kernel -- lse2 = lse * log2(e) - 15 and D * 2^-15 (D = rowsum(dO * O)) per
//    query row, f32, per 64-row query tile [b*H][s_q_pad / 64][lse2 x 64 | D x 64]; padding rows
//    get lse2 = 1e30 (so P = 0) and D = 0.  With these, exp2(S log2(e) / sqrt(128) - lse2) is
//    P * 2^15: the dQ kernel scales dQ back at the end, the dK/dV kernel dV and (through D) dS.
//  * attn_bwd_dq_kernel -- one workgroup = 8 waves = 256 query rows of one (batch, head); each lane
//    owns one query row (transposed products, as in the forward):
//        S^T = K Q^T,  dP^T = V dO^T   (A = K, V rows from LDS; B = Q^T, dO^T in VGPRs)
//        dQ^T += K^T dS^T               (A = K^T by transposing LDS reads; B = dS^T from VGPRs)
//    looping over 64-key tiles of K and V streamed through a 5-stage LDS ring, waves 0-3 and 4-7
//    in ping-pong (one group's S^T / dP^T products against the other's VALU work and dQ product).
//  * attn_bwd_dkdv_kernel -- one workgroup = 8 waves = 128 keys; each lane owns one key, and two
//    waves share each group of 32 keys (and a SIMD):
//        P wave:  S = Q K^T, P,             dV^T += dO^T P
//        dS wave: dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS   (P from the P wave through LDS)
//    (A = Q, dO rows and, by transposing LDS reads, dO^T, Q^T; B = K^T or V^T in VGPRs, P or dS
//    from VGPRs), looping over 64-query tiles of Q, dO and the row statistics (4-stage LDS ring);
//    the two waves of a pair alternate between MFMA and VALU phases, one tile per phase.
// Rows read as MFMA A operands go through a read-time permutation (bits 2 and 3 of the row index
// swapped inside each 32-row block) so that the 8 values a lane feeds a later MFMA from its
// accumulators belong to 8 consecutive rows; the transposing reads (ds_read_b64_tr_b16) hand
// each lane one channel of 4 consecutive rows.  Tiles are stored with 16-byte chunk c of row r at
// chunk c ^ sigma(r % 16), sigma swapping the two 2-bit fields: conflict-free for both the row
// reads and the transposing reads.

#include "wan_attn_internal.h"

#include <type_traits>

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kRows = 128;                     // keys per dK/dV workgroup
constexpr int kTile = 64;                      // rows per streamed LDS tile
constexpr int kTileBytes = kTile * kHeadDim * 2;   // 16 KB
constexpr int kStatBytes = 1024;               // lse2 and D of a query tile (512 bytes, loaded twice)
constexpr float kScaleLog2 = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr float kInvSqrtD = 0.08838834764831845f;    // 1 / sqrt(128)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPadLse2 = 1.0e30f;            // exp2(s * kScaleLog2 - kPadLse2) == 0
constexpr float kNeg = -1.0e30f;
// The row statistics carry P scaled by 2^15: lse2 is stored minus 15 and D times 2^-15, so that
// exp2(s * kScaleLog2 - lse2) gives P * 2^15 (at most 32768, and at least 2^-14, the smallest
// normal half, wherever P >= 2^-29), which the dK/dV kernel passes between waves as a half.
constexpr float kPScaleLog2 = 15.0f;
constexpr float kPScale = 32768.0f;
constexpr float kPUnscale = 1.0f / 32768.0f;
constexpr unsigned kRsrcFlags = 0x00020000u;   // raw buffer, 32-bit dwords

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* d_o;
  const float* lse;   // [b*H][s_q]
  float* stats;       // per 64-row query tile: lse2 - 15 of its rows, then D * 2^-15: [b*H][s_q_pad / 64][2][64]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int heads, s_q, s_kv, s_q_pad;
  int q_blocks;       // 256-row query blocks per (b, h)  (dQ kernel)
  int k_blocks;       // 128-key blocks per (b, h)        (dK/dV kernel)
};

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ __forceinline__ int sigma16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// byte offset of logical 16-byte chunk `chunk` of tile row `row`
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * 256 + 16 * (chunk ^ sigma16(row & 15)); }
// index of lse2 of query row i of (batch, head) bh in BwdParams::stats; D follows 64 floats later
__device__ __forceinline__ int64_t stat_index(int64_t bh, int s_q_pad, int i) {
  return bh * s_q_pad * 2 + (int64_t)(i >> 6) * 128 + (i & 63);
}

__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, r);
}
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
__device__ __forceinline__ unsigned cvt_pk_f16(float lo, float hi) {
  f16x2_t r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(unsigned, r);
}
// half (low or high 16 bits of x) times f32 t, one rounding (v_fma_mix_f32 with a zero addend)
__device__ __forceinline__ float mul_h_lo(unsigned x, float t) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(x), "v"(t));
  return r;
}
__device__ __forceinline__ float mul_h_hi(unsigned x, float t) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(x), "v"(t));
  return r;
}
__device__ __forceinline__ float bf16_lo(unsigned x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(unsigned x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

__device__ __forceinline__ int clamp_bytes(int64_t bytes) {
  return bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, clamp_bytes(bytes), (int)kRsrcFlags);
}
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const u32x4_t r = {(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, (unsigned)clamp_bytes(bytes), kRsrcFlags};
  return r;
}
// Direct global -> LDS load of 16 bytes per lane to lds_addr + 16 * lane (bytes past the buffer's
// end read as zeros).  Inline asm, so that the compiler adds no wait for it before unrelated LDS
// reads; every wait for these loads is explicit (the workgroup barrier at the end of a tile).
__device__ __forceinline__ void dma_b128(u32x4_t rsrc, unsigned lds_addr, unsigned voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}

// One row-major 64 x 128 bf16 tile from global memory (rows `stride` bytes apart, `bytes` readable
// from `base`) into LDS at `lds` by a workgroup of kW waves: wave wv writes 1 KB blocks
// (16 / kW) wv .. (16 / kW) (wv + 1) - 1, lane i the 16 bytes at block + 16 i, i.e. tile row
// 4 * block + i / 16, stored chunk i % 16, which holds logical chunk (i % 16) ^ sigma(row % 16).
template <int kW>
__device__ __forceinline__ void load_tile(const unsigned char* base, int64_t bytes, int64_t stride,
                                          unsigned lds, int wv, int lane) {
  constexpr int kPer = 16 / kW;
  const u32x4_t r = rsrc_words(base, bytes);
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int blk = kPer * wv + it;
    const int row = 4 * blk + (lane >> 4);
    const int chunk = (lane & 15) ^ sigma16(row & 15);
    dma_b128(r, lds + 1024 * blk, (unsigned)(row * stride + 16 * chunk));
  }
}

// A operand rows (32 x 16 channels) of MFMA step c for rows 32 rb .. 32 rb + 31 of a tile: lane
// reads tile row 32 rb + swap23(l32), channels 16c + 8h .. +7.
__device__ __forceinline__ bf16x8_t read_rows(const unsigned char* tile, int rb, int c, int l32, int h) {
  return *reinterpret_cast<const bf16x8_t*>(tile + tile_off(32 * rb + swap23(l32), 2 * c + h));
}

// A operand of a product that reduces over tile rows: 32 channels (32 db .. 32 db + 31) x 16 tile
// rows (16 t .. 16 t + 15), by two transposing reads.  Within each 16-lane group, lane 4 kq + q
// addresses row kq of 4 consecutive rows and channels 4q .. 4q+3 of the group's 16-channel slice;
// lane l32 receives channel 32 db + l32 of rows 16 t + 8 h + 4 e .. +3 (e = 0, 1).
__device__ __forceinline__ bf16x8_t read_cols(const unsigned char* tile, int t, int db, int lane) {
  const int g4 = lane >> 4, kq = (lane >> 2) & 3, q = lane & 3;
  i16x4_t part[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = 16 * t + 8 * (g4 >> 1) + 4 * e + kq;
    const int off = tile_off(row, 4 * db + 2 * (g4 & 1) + (q >> 1)) + 8 * (q & 1);
    part[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(tile + off));
  }
  return __builtin_bit_cast(bf16x8_t, part);
}

// Workgroup barrier without any wait (bare s_barrier): the kernels wait for their direct-to-LDS
// loads (s_waitcnt vmcnt) and their LDS writes (kWaitLgkm0) explicitly, where needed.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
constexpr short kWaitLgkm0 = (short)0xC07F;   // s_waitcnt lgkmcnt(0), other counters untouched

// ---------------------------------------------------------------------------------------------
// Stage 1: lse2 - 15 and D * 2^-15 per query row; 8 lanes per row (16 channels each), rows in
// [b*H][s_q_pad] order, written to the per-tile layout of BwdParams::stats.
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const BwdParams p, int64_t total) {
  const int64_t r = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int sub = threadIdx.x & 7;
  if (r >= total) return;   // the 8 lanes of a row leave together
  const int64_t bh = r / p.s_q_pad;
  const int i = (int)(r - bh * p.s_q_pad);
  float acc = 0.0f;
  if (i < p.s_q) {
    const int64_t b = bh / p.heads, h = bh - b * p.heads;
    const int64_t tok = ((b * p.s_q + i) * p.heads + h) * kHeadDim + 16 * sub;
    const u32x4_t* po = reinterpret_cast<const u32x4_t*>(p.o + tok);
    const u32x4_t* pg = reinterpret_cast<const u32x4_t*>(p.d_o + tok);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const u32x4_t a = po[w], g = pg[w];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(g[e]) + bf16_hi(a[e]) * bf16_hi(g[e]);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (sub == 0) {
    const int64_t x = stat_index(bh, p.s_q_pad, i);
    p.stats[x] = i < p.s_q ? p.lse[bh * p.s_q + i] * kLog2e - kPScaleLog2 : kPadLse2;
    p.stats[x + 64] = acc * kPUnscale;
  }
}

// ---------------------------------------------------------------------------------------------
// Stage 2a: dQ.  One workgroup = 8 waves = 256 query rows of one (batch, head); each lane owns one
// query row, and the products run transposed, as in the forward:
//     S^T = K Q^T,  dP^T = V dO^T   (A = K, V rows from LDS; B = Q^T, dO^T in VGPRs)
//     dQ^T += K^T dS^T               (A = K^T by transposing LDS reads; B = dS^T from VGPRs)
// Each wave's work on a 64-key tile is split into two half-steps between workgroup barriers:
// (1) S^T and dP^T of tile j; (2) the loads of tile j+3, dS of tile j and the dQ product.  Waves
// 0-3 and 4-7 share the four SIMDs and run one barrier apart, so each SIMD's matrix core takes one
// wave's S^T / dP^T products while the other wave runs its VALU work and then its dQ product.
// The dQ^T accumulators are MFMA builtins in VGPRs (256 per lane, no AGPRs): pinned to AGPRs by
// inline asm they would make the compiler split the register file 128 / 128, and the S^T, dP^T
// and operand registers would not fit in 128 VGPRs.  64-key tiles of K and V stream through a
// 5-stage LDS ring (all 160 KB of the CU's LDS): tile t is loaded at the start of half-step (2) of
// tile t-3 -- after every read of tile t-5, the last being the second group's dQ product of tile
// t-5, at least two barriers earlier -- and waited for at the end of half-step (1) of tile t-1,
// before the barrier after which the first group reads it (tile t+1 may still be in flight: the
// wait is counted).  The stage offsets rotate in scalar registers (computed as j % 5 they cost the
// loop 8 spilled VGPRs).  A 4-stage ring, loading two tiles ahead, was 0.65% slower per backward.
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;      // 256 query rows per workgroup
constexpr int kDqStage = 2 * kTileBytes;    // [K | V], 32 KB
constexpr int kDqRing = 5;

__global__ __launch_bounds__(kDqThreads, 1) void attn_bwd_dq_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kDqRing * kDqStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool first_group = wv < kDqWaves / 2;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int bh = blockIdx.x / p.q_blocks;
  const int qblk = blockIdx.x - bh * p.q_blocks;
  const int bb = bh / p.heads, hh = bh - bb * p.heads;
  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;
  const int q0 = qblk * kDqRows + 32 * wv;
  const int qrow = q0 + l32;
  const unsigned lds = (unsigned)(uintptr_t)(lds_void_t*)smem;

  // Q^T and dO^T operands: lane holds row qrow, channels 16c + 8h .. +7 (rows past s_q read zero)
  const int64_t qoff = ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2 + q0 * stride;
  const int64_t qbytes = (int64_t)(p.s_q - 1 - q0) * stride + kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(reinterpret_cast<const unsigned char*>(p.q) + qoff, qbytes);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(reinterpret_cast<const unsigned char*>(p.d_o) + qoff, qbytes);
  bf16x8_t qf[8], gf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const unsigned off = (unsigned)(l32 * stride + 32 * c + 16 * h);
    qf[c] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
    gf[c] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(gr, off, 0, 0));
  }
  const float lse2 = qrow < p.s_q ? p.stats[stat_index(bh, p.s_q_pad, qrow)] : kPadLse2;
  const float dsum = qrow < p.s_q ? p.stats[stat_index(bh, p.s_q_pad, qrow) + 64] * kPScale : 0.0f;
  // waited for here, before any direct-to-LDS load is issued: the compiler does not see those, and
  // would otherwise place its wait for these registers inside the tile loop
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int64_t kvoff = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + kvoff;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + kvoff;
  const int64_t kvbytes = (int64_t)(p.s_kv - 1) * stride + kHeadDim * 2;
  const int n_kt = (p.s_kv + kTile - 1) / kTile;
  auto issue_at = [&](int j, int stage_off) __attribute__((always_inline)) {
    const int64_t off = (int64_t)j * kTile * stride;
    const unsigned st = lds + (unsigned)stage_off;
    load_tile<kDqWaves>(kbase + off, kvbytes - off, stride, st, wv, lane);
    load_tile<kDqWaves>(vbase + off, kvbytes - off, stride, st + kTileBytes, wv, lane);
  };

  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  issue_at(0, 0);
  if (n_kt > 1) issue_at(1, kDqStage);
  if (n_kt > 2) issue_at(2, 2 * kDqStage);
  // tiles 0 and 1 have landed (tile 2 may be in flight: 4 loads per wave per tile)
  if (n_kt > 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  barrier();
  if (!first_group) barrier();
  int cur_off = 0;                  // stage of tile j
  int next_off = 3 * kDqStage;      // stage of tile j+3
  for (int j = 0; j < n_kt; ++j) {
    const unsigned char* ks = smem + cur_off;
    const unsigned char* vs = ks + kTileBytes;
    // (1) S^T and dP^T of tile j
    __builtin_amdgcn_s_setprio(3);
    f32x16_t s[2], dp[2];
    const f32x16_t zero = {};
    // one step = the 4 MFMAs of 16 channels; its LDS operands are read one step ahead
    bf16x8_t ring[2][4];
    auto read_step = [&](int c, bf16x8_t (&f)[4]) __attribute__((always_inline)) {
      f[0] = read_rows(ks, 0, c, l32, h);
      f[1] = read_rows(ks, 1, c, l32, h);
      f[2] = read_rows(vs, 0, c, l32, h);
      f[3] = read_rows(vs, 1, c, l32, h);
    };
    read_step(0, ring[0]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int cur = c & 1;
      if (c + 1 < 8) read_step(c + 1, ring[cur ^ 1]);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][0], qf[c], c == 0 ? zero : s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][1], qf[c], c == 0 ? zero : s[1], 0, 0, 0);
      dp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][2], gf[c], c == 0 ? zero : dp[0], 0, 0, 0);
      dp[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][3], gf[c], c == 0 ? zero : dp[1], 0, 0, 0);
      if (c + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // this wave's loads of tile j+1 (issued in half-step (2) of tile j-2) have landed; those of tile
    // j+2 may not have
    if (j + 2 < n_kt) __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    barrier();
    // (2) the loads of tile j+3; dS of tile j; dQ^T += K^T dS^T over the tile's 4 steps of 16 keys
    if (j + 3 < n_kt) issue_at(j + 3, next_off);
    cur_off = cur_off == (kDqRing - 1) * kDqStage ? 0 : cur_off + kDqStage;
    next_off = next_off == (kDqRing - 1) * kDqStage ? 0 : next_off + kDqStage;
    // register r of key block kb holds key 64 j + 32 kb + 16 (r / 8) + 8 h + r % 8 of this lane's row
    unsigned ds[2][8];
    const int kv0 = j * kTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float sa = s[kb][r], sb = s[kb][r + 1];
        if (kv0 + kTile > p.s_kv) {
          const int key = kv0 + 32 * kb + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key >= p.s_kv) sa = kNeg;
          if (key + 1 >= p.s_kv) sb = kNeg;
        }
        const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sa, kScaleLog2, -lse2));
        const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(sb, kScaleLog2, -lse2));
        ds[kb][r >> 1] = cvt_pk_bf16(pa * (dp[kb][r] - dsum), pb * (dp[kb][r + 1] - dsum));
      }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, u = t & 1;
      const u32x4_t x = {ds[kb][4 * u], ds[kb][4 * u + 1], ds[kb][4 * u + 2], ds[kb][4 * u + 3]};
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, x);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_cols(ks, t, db, lane), bop, acc[db], 0, 0, 0);
    }
    barrier();
  }
  if (first_group) barrier();

  // dQ = dQ^T * 2^-15 / sqrt(128) (dS carried the factor 2^15 of P); lane owns channels
  // 32 db + 8 g + 4 h .. +3 of row qrow
  if (qrow < p.s_q) {
    uint16_t* dst = p.dq + (((int64_t)bb * p.s_q + qrow) * p.heads + hh) * kHeadDim + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        constexpr float sc = kInvSqrtD * kPUnscale;
        const u32x2_t x = {cvt_pk_bf16(acc[db][4 * g] * sc, acc[db][4 * g + 1] * sc),
                           cvt_pk_bf16(acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc)};
        *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = x;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Stage 2b: dK and dV.  One workgroup = 8 waves = 128 keys of one (batch, head).  Waves w and
// w + 4 (w < 4) own keys 32 w .. 32 w + 31, one key per lane, and share a SIMD.  Wave w (the P
// wave) computes S = Q K^T, P and dV^T += dO^T P; wave w + 4 (the dS wave) computes dP = dO V^T,
// dS = P (dP - D) and dK^T += Q^T dS, taking P of each 64-query tile from the P wave through
// LDS.  The pair runs in opposite phases between workgroup barriers, one 64-query tile per phase:
// while one wave issues the 32 MFMAs of a tile (16 accumulating the previous tile, 16 for the
// new tile's product), the other runs the VALU work of a tile (P, or dS).  Per tile i:
//   2i    P wave: dV += tile i-1, S of tile i         dS wave: dS of tile i-1
//   2i+1  P wave: P of tile i (to LDS)                 dS wave: dK += tile i-1, dP of tile i
// then two more phases for tile n-1.  Q, dO and the row statistics of 64-query tiles stream
// through a 4-stage LDS ring: tile t is last read in phase 2t+3 (dK += t); each wave loads its
// share of tile u, into the stage of tile u-4, at the start of its VALU phase 2u-4 (dS wave) or
// 2u-3 (P wave), and waits for it at the end of phase 2u-1.
// P crosses from the P wave to the dS wave as a half: the row statistics carry the factor 2^15
// (kPScaleLog2), so the P wave computes P * 2^15, which a half holds to 11 bits wherever
// P >= 2^-29 (a bf16 copy of it, scaled back at the end, feeds dV).  Each wave holds one B operand
// (K^T or V^T), one accumulator set, the S or dP of a tile and the bf16 P or dS of the previous
// one: 227 VGPRs, so two waves fit on a SIMD.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvStage = 2 * kTileBytes + kStatBytes;   // [Q | dO | statistics], 33 KB
constexpr int kKvRing = 4;
constexpr int kPSlot = 4096;                            // half P * 2^15 of one tile per wave pair
constexpr int kPBuf = kKvRing * kKvStage;
constexpr int kKvLds = kPBuf + 4 * kPSlot;              // 148 KB
constexpr int kLoadsPerTile = 5;                        // direct-to-LDS loads per wave per tile
static_assert(kKvLds <= 160 * 1024, "LDS of one workgroup");

template <bool B> using bconst = std::integral_constant<bool, B>;

__global__ __launch_bounds__(kKvThreads, 1) void attn_bwd_dkdv_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kKvLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wv < 4;
  const int kw = wv & 3;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int bh = blockIdx.x / p.k_blocks;
  const int kblk = blockIdx.x - bh * p.k_blocks;
  const int bb = bh / p.heads, hh = bh - bb * p.heads;
  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;
  const int k0 = kblk * kRows + 32 * kw;
  const int krow = k0 + l32;
  const unsigned lds = (unsigned)(uintptr_t)(lds_void_t*)smem;

  const int64_t koff = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2 + k0 * stride;
  const int64_t kbytes = (int64_t)(p.s_kv - 1 - k0) * stride + kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t br =
      make_rsrc(reinterpret_cast<const unsigned char*>(pwave ? p.k : p.v) + koff, kbytes);
  bf16x8_t bf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    bf[c] = __builtin_bit_cast(
        bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(br, (unsigned)(l32 * stride + 32 * c + 16 * h), 0, 0));
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int64_t qoff = ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2;
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q) + qoff;
  const unsigned char* gbase = reinterpret_cast<const unsigned char*>(p.d_o) + qoff;
  const int64_t qbytes = (int64_t)(p.s_q - 1) * stride + kHeadDim * 2;
  const float* stats = p.stats + stat_index(bh, p.s_q_pad, 0);
  const int n_qt = p.s_q_pad / kTile;
  auto stage = [&](int i) __attribute__((always_inline)) { return smem + (i % kKvRing) * kKvStage; };
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int64_t off = (int64_t)i * kTile * stride;
    const unsigned st = lds + (unsigned)((i % kKvRing) * kKvStage);
    load_tile<kKvWaves>(qbase + off, qbytes - off, stride, st, wv, lane);
    load_tile<kKvWaves>(gbase + off, qbytes - off, stride, st + kTileBytes, wv, lane);
    dma_b128(rsrc_words(stats + (int64_t)i * 2 * kTile, 2 * kTile * 4), st + 2 * kTileBytes,
             (unsigned)(16 * (lane & 31)));
  };
  // tile i+2 into the stage of tile i-2 (last read in phase 2i-1), issued at the start of the
  // wave's VALU phase: 2i (dS wave) or 2i+1 (P wave; in its MFMA phase the loads measured 0.2%
  // slower)
  auto issue_at = [&](int i) __attribute__((always_inline)) {
    if (i + 2 < n_qt) issue(i + 2);
  };
  // end of phase 2i+1: tile i+1 has landed (s_waitcnt vmcnt, other counters untouched; tile i+2
  // may still be in flight)
  auto wait_next = [&](int i) __attribute__((always_inline)) {
    if (i + 2 < n_qt) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsPerTile);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  int rowoff[8], coloff[8];
  {
    const int g4 = lane >> 4, kq = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int c = 0; c < 8; ++c) rowoff[c] = tile_off(swap23(l32), 2 * c + h);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        coloff[2 * db + e] = tile_off(8 * (g4 >> 1) + 4 * e + kq, 4 * db + 2 * (g4 & 1) + (q >> 1)) + 8 * (q & 1);
    asm volatile("" : "+v"(rowoff[0]), "+v"(rowoff[1]), "+v"(rowoff[2]), "+v"(rowoff[3]), "+v"(rowoff[4]),
                 "+v"(rowoff[5]), "+v"(rowoff[6]), "+v"(rowoff[7]));
    asm volatile("" : "+v"(coloff[0]), "+v"(coloff[1]), "+v"(coloff[2]), "+v"(coloff[3]), "+v"(coloff[4]),
                 "+v"(coloff[5]), "+v"(coloff[6]), "+v"(coloff[7]));
  }
  auto rows = [&](const unsigned char* t, int qb, int c) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>((t + rowoff[c]) + 8192 * qb);
  };
  auto cols = [&](const unsigned char* t, int step, int db) __attribute__((always_inline)) {
    i16x4_t part[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      part[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((t + coloff[2 * db + e]) + 4096 * step));
    return __builtin_bit_cast(bf16x8_t, part);
  };
  unsigned char* pslot = smem + kPBuf + kPSlot * kw;

  // Register r of block qb of the S, P, dP or dS tile holds query 32 qb + 16 (r / 8) + 8 h + r % 8
  // (this lane's key); its statistics sit at rows 32 qb + 16 (i / 2) + 8 h + 4 (i % 2) .. +3.
  auto stat4 = [&](const unsigned char* st, int which, int qb, int i) __attribute__((always_inline)) {
    const float* x = reinterpret_cast<const float*>(st + 2 * kTileBytes) + 64 * which;
    return *reinterpret_cast<const f32x4_t*>(x + 32 * qb + 16 * (i >> 1) + 8 * h + 4 * (i & 1));
  };

  f32x16_t acc[4];          // dV^T (P wave) or dK^T (dS wave), 4 blocks of 32 channels
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  f32x16_t prod[2];         // S (P wave) or dP (dS wave) of the current tile, two 32-query blocks
  unsigned bop[16];         // bf16 P (P wave) or dS (dS wave) of the tile awaiting accumulation
  bf16x8_t pre[4];          // A operands of that accumulation's first step, read ahead
  f32x4_t sv[2][4];         // statistics of the tile in prod (lse2 - 15 or D * 2^-15)
  // bop is produced in the VALU phase: the empty volatile asm keeps the compiler from sinking its
  // conversions past the barrier into the MFMA phase that consumes it
  auto pin_bop = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(bop[0]), "+v"(bop[1]), "+v"(bop[2]), "+v"(bop[3]), "+v"(bop[4]), "+v"(bop[5]),
                 "+v"(bop[6]), "+v"(bop[7]));
    asm volatile("" : "+v"(bop[8]), "+v"(bop[9]), "+v"(bop[10]), "+v"(bop[11]), "+v"(bop[12]), "+v"(bop[13]),
                 "+v"(bop[14]), "+v"(bop[15]));
  };

  // MFMA phase: acc += sum over the 4 steps of 16 queries of (transposed A tile at `at`, step s)
  // x bop step s (if kAcc); prod[qb] = rows of the tile at pt x bf (if kProd) and the statistic
  // `which` of that tile for the VALU phase after it.  Eight groups of 4 MFMAs, the accumulation
  // steps alternating with pairs of product steps (one per block, so no MFMA follows the one it
  // depends on); each group's LDS operands are read while the group before it runs.
  auto mfma_phase = [&](auto acc_c, auto prod_c, const unsigned char* at, const unsigned char* st, int poff,
                        int which) __attribute__((always_inline)) {
    constexpr bool kAcc = decltype(acc_c)::value;
    constexpr bool kProd = decltype(prod_c)::value;
    const unsigned char* pt = st + poff;
    __builtin_amdgcn_s_setprio(3);
    // group sequence: kAcc && kProd: A0 P0 A1 P1 A2 P2 A3 P3; only kAcc: A0..A3; only kProd: P0..P3
    constexpr int kGroups = (kAcc ? 4 : 0) + (kProd ? 4 : 0);
    auto is_acc = [&](int g) __attribute__((always_inline)) { return kAcc && (!kProd || (g & 1) == 0); };
    auto gidx = [&](int g) __attribute__((always_inline)) { return (kAcc && kProd) ? (g >> 1) : g; };
    bf16x8_t ring[2][4];
    auto read_group = [&](int g, bf16x8_t (&f)[4]) __attribute__((always_inline)) {
      if (is_acc(g)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) f[db] = cols(at, gidx(g), db);
      } else {
        const int c2 = 2 * gidx(g);
        f[0] = rows(pt, 0, c2);
        f[1] = rows(pt, 1, c2);
        f[2] = rows(pt, 0, c2 + 1);
        f[3] = rows(pt, 1, c2 + 1);
      }
    };
    const f32x16_t zero = {};
    if constexpr (!kAcc) read_group(0, ring[0]);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int cur = g & 1;
      if (g + 1 < kGroups) read_group(g + 1, ring[cur ^ 1]);
      if (kProd && g == kGroups - 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[0][i] = stat4(st, which, 0, i);
      }
      if (is_acc(g)) {
        const int s = gidx(g);
        const u32x4_t x = {bop[4 * s], bop[4 * s + 1], bop[4 * s + 2], bop[4 * s + 3]};
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, x);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g == 0 ? pre[db] : ring[cur][db], b, acc[db], 0, 0, 0);
      } else {
        const int c2 = 2 * gidx(g);
        const bf16x8_t (&f)[4] = ring[cur];
        prod[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[0], bf[c2], c2 == 0 ? zero : prod[0], 0, 0, 0);
        prod[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[1], bf[c2], c2 == 0 ? zero : prod[1], 0, 0, 0);
        prod[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[2], bf[c2 + 1], prod[0], 0, 0, 0);
        prod[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[3], bf[c2 + 1], prod[1], 0, 0, 0);
      }
      if (g + 1 < kGroups) {
        if (is_acc(g + 1)) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      if (kProd && g == kGroups - 2) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  issue(0);
  if (n_qt > 1) issue(1);
  wait_next(-1);
  barrier();

  if (pwave) {
    // VALU phase: P * 2^15 of the tile at st from prod and lse2 - 15 (sv): bf16 to bop, half to the
    // pair's slot; the dO^T operands of the tile's first dV step and the statistics of the tile's
    // second block are read meanwhile
    auto valu_phase = [&](const unsigned char* st) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) pre[db] = cols(st + kTileBytes, 0, db);
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[1][i] = stat4(st, 0, 1, i);
      __builtin_amdgcn_sched_barrier(0);
      u32x2_t hp[8];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 2 * k;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(prod[qb][r], kScaleLog2, -sv[qb][r >> 2][r & 3]));
          const float p1 =
              __builtin_amdgcn_exp2f(__builtin_fmaf(prod[qb][r + 1], kScaleLog2, -sv[qb][r >> 2][(r & 3) + 1]));
          bop[8 * qb + k] = cvt_pk_bf16(p0, p1);
          hp[4 * qb + (k >> 1)][k & 1] = cvt_pk_f16(p0, p1);
        }
#pragma unroll
        for (int j = 2 * qb; j < 2 * qb + 2; ++j) {
          const u32x4_t x = {hp[2 * j][0], hp[2 * j][1], hp[2 * j + 1][0], hp[2 * j + 1][1]};
          *reinterpret_cast<u32x4_t*>(pslot + 16 * (64 * j + lane)) = x;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pin_bop();
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // P is in LDS before the barrier
    };
    mfma_phase(bconst<false>{}, bconst<true>{}, smem, stage(0), 0, 0);
    barrier();
    issue_at(0);
    valu_phase(stage(0));
    wait_next(0);
    barrier();
    for (int i = 1; i < n_qt; ++i) {
      mfma_phase(bconst<true>{}, bconst<true>{}, stage(i - 1) + kTileBytes, stage(i), 0, 0);
      barrier();
      issue_at(i);
      valu_phase(stage(i));
      wait_next(i);
      barrier();
    }
    mfma_phase(bconst<true>{}, bconst<false>{}, stage(n_qt - 1) + kTileBytes, smem, 0, 0);
    barrier();
    barrier();
  } else {
    // VALU phase: dS of the tile at st from prod (dP), the P wave's half P * 2^15 and D * 2^-15
    // (sv), to bop; the Q^T operands of the tile's first dK step and the statistics of its second
    // block are read meanwhile
    auto valu_phase = [&](const unsigned char* st) __attribute__((always_inline)) {
      u32x4_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pw[j] = *reinterpret_cast<const u32x4_t*>(pslot + 16 * (64 * j + lane));
#pragma unroll
      for (int db = 0; db < 4; ++db) pre[db] = cols(st, 0, db);
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[1][i] = stat4(st, 1, 1, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int r = 2 * k;
          const unsigned pk = pw[2 * qb + (k >> 2)][k & 3];
          // (dP - D) * 2^-15, exactly the fp32 dP - D scaled, times the half P * 2^15
          const float d0 = __builtin_fmaf(prod[qb][r], kPUnscale, -sv[qb][r >> 2][r & 3]);
          const float d1 = __builtin_fmaf(prod[qb][r + 1], kPUnscale, -sv[qb][r >> 2][(r & 3) + 1]);
          bop[8 * qb + k] = cvt_pk_bf16(mul_h_lo(pk, d0), mul_h_hi(pk, d1));
        }
      pin_bop();
    };
    issue_at(0);
    barrier();
    mfma_phase(bconst<false>{}, bconst<true>{}, smem, stage(0), kTileBytes, 1);
    wait_next(0);
    barrier();
    for (int i = 1; i < n_qt; ++i) {
      issue_at(i);
      valu_phase(stage(i - 1));
      barrier();
      mfma_phase(bconst<true>{}, bconst<true>{}, stage(i - 1), stage(i), kTileBytes, 1);
      wait_next(i);
      barrier();
    }
    valu_phase(stage(n_qt - 1));
    barrier();
    mfma_phase(bconst<true>{}, bconst<false>{}, stage(n_qt - 1), smem, 0, 1);
    barrier();
  }

  if (krow < p.s_kv) {
    // dV = dV^T; dK = dK^T * 1/sqrt(128); lane owns channels 32 db + 8 g + 4 h .. +3 of key krow
    const float scale = pwave ? kPUnscale : kInvSqrtD;
    uint16_t* dst = (pwave ? p.dv : p.dk) + (((int64_t)bb * p.s_kv + krow) * p.heads + hh) * kHeadDim + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t x = {cvt_pk_bf16(acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale),
                           cvt_pk_bf16(acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale)};
        *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = x;
      }
  }
}

}  // namespace

size_t attn_bwd_scratch_bytes(const AttnShape& sh) {
  const size_t s_q_pad = (size_t)ceil_div(sh.s_q, kTile) * kTile;
  return 2 * (size_t)sh.batch * sh.heads * s_q_pad * sizeof(float);
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                           const float* lse, void* dq, void* dk, void* dv, const AttnShape& sh,
                           void* scratch, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.d_o = static_cast<const uint16_t*>(d_o);
  p.lse = lse;
  p.heads = (int)sh.heads;
  p.s_q = (int)sh.s_q;
  p.s_kv = (int)sh.s_kv;
  p.s_q_pad = (int)(ceil_div(sh.s_q, kTile) * kTile);
  const int64_t bh = sh.batch * sh.heads;
  p.stats = static_cast<float*>(scratch);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.q_blocks = (int)ceil_div(sh.s_q, kDqRows);
  p.k_blocks = (int)ceil_div(sh.s_kv, kRows);
  const int64_t rows = bh * p.s_q_pad;
  hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)ceil_div(rows, 32)), dim3(256), 0, stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)(bh * p.q_blocks)), dim3(kDqThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)(bh * p.k_blocks)), dim3(kKvThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
