// bf16 attention backward for gfx950 (MI355X): dQ, dK and dV of O = softmax(Q K^T / sqrt(128)) V,
// non-causal, per (batch, head).  The backward of non-causal attention is the beta = 8 term of the
// DiT cost model and the bulk of training time at long sequences ("Wan 2.1: VBench 86.22% ..."
// explainer of the Wan technical report, section "先看现象").  With P = exp(S - lse) recomputed from
// the forward's row log-sum-exp, D_i = rowsum(dO_i * O_i) and dS = P * (dP - D):
//     dV = P^T dO,   dP = dO V^T,   dQ = dS K / sqrt(128),   dK = dS^T Q / sqrt(128)
// (the chain rule through the row softmax; D_i = sum_j P_ij dP_ij = dO_i . O_i).
//
// Kernels:
//  * attn_bwd_prep_kernel -- lse2 = lse * log2(e) and dsum = rowsum(dO * O) per query row, f32,
//    [b*H][s_q padded to 64]; padding rows get lse2 = 1e30 (so P = 0) and dsum = 0.
//  * attn_bwd_dq_kernel -- one workgroup = 4 waves = 128 query rows of one (batch, head); each lane
//    owns one query row (transposed products, as in the forward):
//        S^T = K Q^T,  dP^T = V dO^T   (A = K, V rows from LDS; B = Q^T, dO^T in VGPRs)
//        dQ^T += K^T dS^T               (A = K^T by transposing LDS reads; B = dS^T from VGPRs)
//    looping over 64-key tiles of K and V streamed through a 2-stage LDS ring.
//  * attn_bwd_dkdv_kernel -- one workgroup = 4 waves = 128 keys; each lane owns one key:
//        S = Q K^T,  dP = dO V^T        (A = Q, dO rows from LDS; B = K^T, V^T in VGPRs)
//        dV^T += dO^T P,  dK^T += Q^T dS  (A by transposing LDS reads; B = P, dS from VGPRs)
//    looping over 64-query tiles of Q, dO and the row statistics (3-stage LDS ring), software-
//    pipelined over 32-query blocks: S/dP products of block b+2, softmax of block b+1 and the
//    dV/dK accumulation of block b are issued together.
// Rows read as MFMA A operands go through a read-time permutation (bits 2 and 3 of the row index
// swapped inside each 32-row block) so that the 8 values a lane feeds a later MFMA from its
// accumulators belong to 8 consecutive rows; the transposing reads (ds_read_b64_tr_b16) hand
// each lane one channel of 4 consecutive rows.  Tiles are stored with 16-byte chunk c of row r at
// chunk c ^ sigma(r % 16), sigma swapping the two 2-bit fields: conflict-free for both the row
// reads and the transposing reads.

#include "wan_attn_internal.h"

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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;             // query rows (dQ kernel) or keys (dK/dV kernel) per workgroup
constexpr int kTile = 64;                      // rows per streamed LDS tile
constexpr int kTileBytes = kTile * kHeadDim * 2;   // 16 KB
constexpr int kStatBytes = 2048;               // lse2 (1 KB) and dsum (1 KB) of a query tile
constexpr float kScaleLog2 = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr float kInvSqrtD = 0.08838834764831845f;    // 1 / sqrt(128)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPadLse2 = 1.0e30f;            // exp2(s * kScaleLog2 - kPadLse2) == 0
constexpr float kNeg = -1.0e30f;
constexpr unsigned kRsrcFlags = 0x00020000u;   // raw buffer, 32-bit dwords

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* d_o;
  const float* lse;   // [b*H][s_q]
  float* lse2;        // [b*H][s_q_pad]
  float* dsum;        // [b*H][s_q_pad]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int heads, s_q, s_kv, s_q_pad;
  int q_blocks;       // 128-row query blocks per (b, h)  (dQ kernel)
  int k_blocks;       // 128-key blocks per (b, h)        (dK/dV kernel)
};

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
__device__ __forceinline__ int sigma16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// byte offset of logical 16-byte chunk `chunk` of tile row `row`
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * 256 + 16 * (chunk ^ sigma16(row & 15)); }

__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, r);
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
// from `base`) into LDS at `lds`: wave wv writes 1 KB blocks 4wv .. 4wv+3, lane i the 16 bytes at
// block + 16 i, i.e. tile row 4 * block + i / 16, stored chunk i % 16, which holds logical chunk
// (i % 16) ^ sigma(row % 16).
__device__ __forceinline__ void load_tile(const unsigned char* base, int64_t bytes, int64_t stride,
                                          unsigned lds, int wv, int lane) {
  const u32x4_t r = rsrc_words(base, bytes);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int blk = 4 * wv + it;
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

// Gradient accumulation on the matrix cores with the accumulators pinned to AGPRs: acc[i] +=
// a[i] * b (32x32x16 bf16 MFMAs), one asm block per step.  The accumulators live across the whole
// key or query sweep and only MFMAs touch them; written as builtins, the compiler would keep them
// in the same AGPRs as the S and dP products and copy them out and back every tile.  s_nop 2
// first: the B operand (and, at the first step, the zeroed accumulators) was just written by the
// VALU, and an MFMA may read a VGPR only 2 wait states after a VALU write to it.  After the sweep,
// settle_mfma() waits out the last accumulation before the VALU reads the accumulators.  The MFMA
// blocks are not volatile, so the compiler may interleave them with independent VALU work (a
// volatile asm statement would end its scheduling region).
__device__ __forceinline__ void mfma4_acc(f32x16_t (&acc)[4], const bf16x8_t (&a)[4], bf16x8_t b) {
  asm(
      "s_nop 2\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %5, %8, %1\n\t"
      "v_mfma_f32_32x32x16_bf16 %2, %6, %8, %2\n\t"
      "v_mfma_f32_32x32x16_bf16 %3, %7, %8, %3"
      : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b));
}
__device__ __forceinline__ void settle_mfma(f32x16_t (&acc)[4]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
}

// One step of two independent products with B operands held in AGPRs and the accumulators in
// VGPRs: c0 += a0 * b0, c1 += a1 * b1 (first step: c = a * b).  s_nop 1 first (an operand
// copied into place by the VALU may be read by an MFMA 2 wait states later; the nop issues while
// the matrix core is busy with the previous step).  The VALU may read c only after
// mfma_results_ready().
__device__ __forceinline__ void mfma2_first(f32x16_t& c0, f32x16_t& c1, bf16x8_t a0, bf16x8_t a1, bf16x8_t b0,
                                            bf16x8_t b1) {
  asm(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %3, %5, 0"
      : "=&v"(c0), "=&v"(c1)
      : "v"(a0), "v"(a1), "a"(b0), "a"(b1));
}
__device__ __forceinline__ void mfma2(f32x16_t& c0, f32x16_t& c1, bf16x8_t a0, bf16x8_t a1, bf16x8_t b0,
                                      bf16x8_t b1) {
  asm(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %3, %5, %1"
      : "+v"(c0), "+v"(c1)
      : "v"(a0), "v"(a1), "a"(b0), "a"(b1));
}
// 21 wait states between the last MFMA of a product and any VALU read of its results: the asm
// takes the results as operands, so it sits after that MFMA and before the reads.
__device__ __forceinline__ void mfma_results_ready(f32x16_t& c0, f32x16_t& c1) {
  asm("s_nop 15\n\ts_nop 4" : "+v"(c0), "+v"(c1));
}

// Wait for this wave's direct-to-LDS loads (the compiler does not track the inline-asm loads, so
// the wait is explicit: s_waitcnt vmcnt(0), other counters untouched), then the workgroup barrier:
// after it every wave's loads have landed and every wave is done with the tile it read before.
__device__ __forceinline__ void barrier_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// Stage 1: lse2 and dsum per query row; 8 lanes per row (16 channels each), rows in [b*H][s_q_pad]
// order.
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
    p.dsum[r] = acc;
    p.lse2[r] = i < p.s_q ? p.lse[bh * p.s_q + i] * kLog2e : kPadLse2;
  }
}

// ---------------------------------------------------------------------------------------------
// Stage 2a: dQ.
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dq_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * 2 * kTileBytes];   // [stage][K | V]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int bh = blockIdx.x / p.q_blocks;
  const int qblk = blockIdx.x - bh * p.q_blocks;
  const int bb = bh / p.heads, hh = bh - bb * p.heads;
  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;
  const int q0 = qblk * kRows + 32 * wv;
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
  const float lse2 = qrow < p.s_q ? p.lse2[(int64_t)bh * p.s_q_pad + qrow] : kPadLse2;
  const float dsum = qrow < p.s_q ? p.dsum[(int64_t)bh * p.s_q_pad + qrow] : 0.0f;

  const int64_t kvoff = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + kvoff;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + kvoff;
  const int64_t kvbytes = (int64_t)(p.s_kv - 1) * stride + kHeadDim * 2;
  const int n_kt = (p.s_kv + kTile - 1) / kTile;
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int64_t off = (int64_t)j * kTile * stride;
    const unsigned st = lds + (unsigned)((j & 1) * 2 * kTileBytes);
    load_tile(kbase + off, kvbytes - off, stride, st, wv, lane);
    load_tile(vbase + off, kvbytes - off, stride, st + kTileBytes, wv, lane);
  };

  f32x16_t acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

  issue(0);
  barrier_all();
  for (int j = 0; j < n_kt; ++j) {
    if (j + 1 < n_kt) issue(j + 1);   // stage (j+1) & 1: free since the barrier that ended tile j-1
    const unsigned char* ks = smem + (j & 1) * 2 * kTileBytes;
    const unsigned char* vs = ks + kTileBytes;
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows(ks, kb, c, l32, h), qf[c], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows(vs, kb, c, l32, h), gf[c], dp[kb], 0, 0, 0);
      }
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
    // dQ^T += K^T dS^T over the tile's 4 steps of 16 keys
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, u = t & 1;
      const u32x4_t x = {ds[kb][4 * u], ds[kb][4 * u + 1], ds[kb][4 * u + 2], ds[kb][4 * u + 3]};
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, x);
      bf16x8_t a[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) a[db] = read_cols(ks, t, db, lane);
      mfma4_acc(acc, a, bop);
    }
    barrier_all();   // tile j+1 has landed; every wave is done with stage j & 1
  }

  settle_mfma(acc);
  // dQ = dQ^T * 1/sqrt(128); lane owns channels 32 db + 8 g + 4 h .. +3 of row qrow
  if (qrow < p.s_q) {
    uint16_t* dst = p.dq + (((int64_t)bb * p.s_q + qrow) * p.heads + hh) * kHeadDim + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t x = {cvt_pk_bf16(acc[db][4 * g] * kInvSqrtD, acc[db][4 * g + 1] * kInvSqrtD),
                           cvt_pk_bf16(acc[db][4 * g + 2] * kInvSqrtD, acc[db][4 * g + 3] * kInvSqrtD)};
        *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = x;
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Stage 2b: dK and dV.
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dkdv_kernel(const BwdParams p) {
  constexpr int kStage = 2 * kTileBytes + kStatBytes;   // [Q | dO | stats]
  constexpr int kRing = 3;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRing * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int bh = blockIdx.x / p.k_blocks;
  const int kblk = blockIdx.x - bh * p.k_blocks;
  const int bb = bh / p.heads, hh = bh - bb * p.heads;
  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;
  const int k0 = kblk * kRows + 32 * wv;
  const int krow = k0 + l32;
  const unsigned lds = (unsigned)(uintptr_t)(lds_void_t*)smem;

  // K^T and V^T operands (B of S and dP, held in AGPRs): lane holds key krow, channels 16c + 8h .. +7
  const int64_t koff = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2 + k0 * stride;
  const int64_t kbytes = (int64_t)(p.s_kv - 1 - k0) * stride + kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(reinterpret_cast<const unsigned char*>(p.k) + koff, kbytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(reinterpret_cast<const unsigned char*>(p.v) + koff, kbytes);
  bf16x8_t kf[8], vf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const unsigned off = (unsigned)(l32 * stride + 32 * c + 16 * h);
    kf[c] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
    vf[c] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
  }

  const int64_t qoff = ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2;
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q) + qoff;
  const unsigned char* gbase = reinterpret_cast<const unsigned char*>(p.d_o) + qoff;
  const int64_t qbytes = (int64_t)(p.s_q - 1) * stride + kHeadDim * 2;
  const float* lse2 = p.lse2 + (int64_t)bh * p.s_q_pad;
  const float* dsum = p.dsum + (int64_t)bh * p.s_q_pad;
  const int n_qt = p.s_q_pad / kTile;
  auto stage = [&](int i) __attribute__((always_inline)) { return smem + (i % kRing) * kStage; };
  // Per-lane byte offsets of the operand reads within a tile (read_rows / read_cols with rows
  // 32 qb + ... and 16 step + ... taken out as immediates), computed once; the empty asm keeps
  // them in registers instead of being rebuilt from the lane index at every read.
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
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int64_t off = (int64_t)i * kTile * stride;
    const unsigned st = lds + (unsigned)((i % kRing) * kStage);
    load_tile(qbase + off, qbytes - off, stride, st, wv, lane);
    load_tile(gbase + off, qbytes - off, stride, st + kTileBytes, wv, lane);
    if (wv == 0) {   // 256 bytes of each statistic: lanes 16..63 repeat lanes 0..15
      dma_b128(rsrc_words(lse2 + i * kTile, kTile * 4), st + 2 * kTileBytes, (unsigned)(16 * (lane & 15)));
      dma_b128(rsrc_words(dsum + i * kTile, kTile * 4), st + 2 * kTileBytes + 1024, (unsigned)(16 * (lane & 15)));
    }
  };

  f32x16_t dka[4], dva[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[db][r] = dva[db][r] = 0.0f;

  // One pipeline step over blocks of 32 query rows (qb = 0, 1 of a tile in LDS at t):
  //   products S, dP of block b+2  (tile at pt, block pqb): 8 steps of 2 MFMAs -> s_out, d_out
  //   softmax of block b+1 (s_in, d_in; statistics of tile st, block sqb) -> pp_out, ds_out (VALU)
  //   accumulation of block b (pp_in, ds_in; tile at at, block aqb): dV^T, dK^T, 4 blocks of 4 MFMAs
  // written interleaved (MFMA blocks, each followed by a slice of the softmax) so that the VALU
  // work issues while the matrix core runs.  Register r of an S or dP block holds query
  // 32 qb + 16 (r / 8) + 8 h + r % 8 of its tile (this lane's key).
  auto step = [&](const unsigned char* pt, int pqb, f32x16_t& s_out, f32x16_t& d_out, const unsigned char* st,
                  int sqb, f32x16_t& s_in, f32x16_t& d_in, unsigned (&pp_out)[8], unsigned (&ds_out)[8],
                  const unsigned char* at, int aqb, const unsigned (&pp_in)[8], const unsigned (&ds_in)[8])
      __attribute__((always_inline)) {
    const float* st_lse2 = reinterpret_cast<const float*>(st + 2 * kTileBytes);
    const float* st_dsum = reinterpret_cast<const float*>(st + 2 * kTileBytes + 1024);
    f32x4_t lse[4], dsm[4];   // rows 32 sqb + 16 half + 8 h + 4 w .. +3 for (half, w) = (i / 2, i % 2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row0 = 32 * sqb + 16 * (i >> 1) + 8 * h + 4 * (i & 1);
      lse[i] = *reinterpret_cast<const f32x4_t*>(st_lse2 + row0);
      dsm[i] = *reinterpret_cast<const f32x4_t*>(st_dsum + row0);
    }
    // softmax slice k: S/dP registers 2k, 2k+1
    auto soft = [&](int k) __attribute__((always_inline)) {
      const int r = 2 * k;
      const float l0 = lse[r >> 2][r & 3], l1 = lse[r >> 2][(r & 3) + 1];
      const float d0 = dsm[r >> 2][r & 3], d1 = dsm[r >> 2][(r & 3) + 1];
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_in[r], kScaleLog2, -l0));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_in[r + 1], kScaleLog2, -l1));
      pp_out[k] = cvt_pk_bf16(p0, p1);
      ds_out[k] = cvt_pk_bf16(p0 * (d_in[r] - d0), p1 * (d_in[r + 1] - d1));
    };
    // operand rings, filled one MFMA block ahead of use (the MFMA blocks keep the source order)
    bf16x8_t rq[2], rg[2], ca[2][4];
    auto ld_rows = [&](int c) __attribute__((always_inline)) {
      rq[c & 1] = rows(pt, pqb, c);
      rg[c & 1] = rows(pt + kTileBytes, pqb, c);
    };
    // accumulation block m: (u, which) = (m / 2, m % 2): dV (which 0) or dK (which 1), rows 16 (2 aqb + u)
    auto ld_cols = [&](int m) __attribute__((always_inline)) {
      const int stp = 2 * aqb + (m >> 1);
#pragma unroll
      for (int db = 0; db < 4; ++db) ca[m & 1][db] = cols((m & 1) ? at : at + kTileBytes, stp, db);
    };
    auto acc = [&](int m) __attribute__((always_inline)) {
      const int u = m >> 1;
      const u32x4_t x = (m & 1) ? u32x4_t{ds_in[4 * u], ds_in[4 * u + 1], ds_in[4 * u + 2], ds_in[4 * u + 3]}
                                : u32x4_t{pp_in[4 * u], pp_in[4 * u + 1], pp_in[4 * u + 2], pp_in[4 * u + 3]};
      if (m & 1) mfma4_acc(dka, ca[m & 1], __builtin_bit_cast(bf16x8_t, x));
      else mfma4_acc(dva, ca[m & 1], __builtin_bit_cast(bf16x8_t, x));
    };
    auto prod = [&](int c) __attribute__((always_inline)) {
      if (c == 0) mfma2_first(s_out, d_out, rq[0], rg[0], kf[0], vf[0]);
      else mfma2(s_out, d_out, rq[c & 1], rg[c & 1], kf[c], vf[c]);
    };
    ld_rows(0); ld_cols(0);
    ld_rows(1); prod(0); soft(0);
    ld_cols(1); acc(0);
    ld_rows(2); prod(1); soft(1);
    ld_rows(3); prod(2); soft(2);
    ld_cols(2); acc(1);
    ld_rows(4); prod(3); soft(3);
    ld_rows(5); prod(4); soft(4);
    ld_cols(3); acc(2);
    ld_rows(6); prod(5); soft(5);
    ld_rows(7); prod(6); soft(6);
    acc(3);
    prod(7); soft(7);
    mfma_results_ready(s_out, d_out);
  };

  // Software pipeline over the blocks b = 2i + qb of query tile i: the step of block b issues the
  // products of block b+2, the softmax of block b+1 and the accumulation of block b.  Tile i sits in
  // stage i % 3; tile i+2 is loaded while tiles i and i+1 are read.  The products and softmax past
  // the last block read a stage holding an earlier tile (in bounds) and their results go unused;
  // the accumulation before block 0 runs on P = dS = 0 and adds nothing.
  issue(0);
  if (n_qt > 1) issue(1);
  barrier_all();
  f32x16_t sx, dx, sy, dy;
  unsigned px[8], gx[8], py[8], gy[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) py[k] = gy[k] = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) sx[r] = dx[r] = 0.0f;   // read by the first step's (discarded) softmax
  // prologue: products of blocks 0 and 1, softmax of block 0 (the accumulations add zeros)
  step(stage(0), 0, sy, dy, stage(0), 0, sx, dx, px, gx, stage(0), 0, py, gy);   // products of block 0
  step(stage(0), 1, sx, dx, stage(0), 0, sy, dy, px, gx, stage(0), 0, py, gy);   // block 1; softmax of block 0
  for (int i = 0; i < n_qt; ++i) {
    if (i + 2 < n_qt) issue(i + 2);   // stage (i+2) % 3, free since the barrier that ended tile i-1
    const unsigned char* cur = stage(i);
    const unsigned char* nxt = stage(i + 1);
    step(nxt, 0, sy, dy, cur, 1, sx, dx, py, gy, cur, 0, px, gx);   // products 2i+2, softmax 2i+1, acc 2i
    step(nxt, 1, sx, dx, nxt, 0, sy, dy, px, gx, cur, 1, py, gy);   // products 2i+3, softmax 2i+2, acc 2i+1
    barrier_all();   // tile i+2 has landed; every wave is done with stage i % 3
  }

  settle_mfma(dka);
  settle_mfma(dva);
  if (krow < p.s_kv) {
    const int64_t off = (((int64_t)bb * p.s_kv + krow) * p.heads + hh) * kHeadDim + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t xk = {cvt_pk_bf16(dka[db][4 * g] * kInvSqrtD, dka[db][4 * g + 1] * kInvSqrtD),
                            cvt_pk_bf16(dka[db][4 * g + 2] * kInvSqrtD, dka[db][4 * g + 3] * kInvSqrtD)};
        const u32x2_t xv = {cvt_pk_bf16(dva[db][4 * g], dva[db][4 * g + 1]),
                            cvt_pk_bf16(dva[db][4 * g + 2], dva[db][4 * g + 3])};
        *reinterpret_cast<u32x2_t*>(p.dk + off + 32 * db + 8 * g) = xk;
        *reinterpret_cast<u32x2_t*>(p.dv + off + 32 * db + 8 * g) = xv;
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
  p.lse2 = static_cast<float*>(scratch);
  p.dsum = p.lse2 + bh * p.s_q_pad;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.q_blocks = (int)ceil_div(sh.s_q, kRows);
  p.k_blocks = (int)ceil_div(sh.s_kv, kRows);
  const int64_t rows = bh * p.s_q_pad;
  hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)ceil_div(rows, 32)), dim3(256), 0, stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)(bh * p.q_blocks)), dim3(kThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)(bh * p.k_blocks)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
