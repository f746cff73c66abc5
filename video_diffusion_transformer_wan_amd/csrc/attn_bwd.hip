// bf16 attention backward for gfx950 (MI355X): dQ, dK and dV of O = softmax(Q K^T / sqrt(128)) V,
// non-causal, per (batch, head).  The backward of non-causal attention is the beta = 8 term of the
// DiT cost model and the bulk of training time at long sequences ("Wan 2.1: VBench 86.22% ..."
// explainer of the Wan technical report, section "先看现象").  With P = exp(S - lse) recomputed from
// the forward's row log-sum-exp, D_i = rowsum(dO_i * O_i) and dS = P * (dP - D):
//     dV = P^T dO,   dP = dO V^T,   dQ = dS K / sqrt(128),   dK = dS^T Q / sqrt(128)
// (the chain rule through the row softmax; D_i = sum_j P_ij dP_ij = dO_i . O_i).
//
// Kernels:
//  * attn_bwd_prep_kernel -- lse2 = lse * log2(e) and D = rowsum(dO * O) per query row, f32, per
//    64-row query tile [b*H][s_q_pad / 64][lse2 x 64 | D x 64]; padding rows get lse2 = 1e30 (so
//    P = 0) and D = 0.
//  * attn_bwd_dq_kernel -- one workgroup = 4 waves = 128 query rows of one (batch, head); each lane
//    owns one query row (transposed products, as in the forward):
//        S^T = K Q^T,  dP^T = V dO^T   (A = K, V rows from LDS; B = Q^T, dO^T in VGPRs)
//        dQ^T += K^T dS^T               (A = K^T by transposing LDS reads; B = dS^T from VGPRs)
//    looping over 64-key tiles of K and V streamed through a 2-stage LDS ring.
//  * attn_bwd_dkdv_kernel -- one workgroup = 8 waves = 128 keys; each lane owns one key, and two
//    waves share each group of 32 keys (and a SIMD):
//        P wave:  S = Q K^T, P,             dV^T += dO^T P
//        dS wave: dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS   (P from the P wave through LDS)
//    (A = Q, dO rows and, by transposing LDS reads, dO^T, Q^T; B = K^T or V^T in VGPRs, P or dS
//    from VGPRs), looping over 64-query tiles of Q, dO and the row statistics (4-stage LDS ring)
//    in 32-query blocks; the two waves of a pair alternate between MFMA and VALU phases.
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
constexpr int kStatBytes = 1024;               // lse2 and D of a query tile (512 bytes, loaded twice)
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
  float* stats;       // per 64-row query tile: lse2 of its rows, then D: [b*H][s_q_pad / 64][2][64]
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

// Wait for this wave's direct-to-LDS loads (the compiler does not track the inline-asm loads, so
// the wait is explicit: s_waitcnt vmcnt(0), other counters untouched), then the workgroup barrier:
// after it every wave's loads have landed and every wave is done with the tile it read before.
__device__ __forceinline__ void barrier_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}
// Workgroup barrier without any wait (bare s_barrier): the dK/dV kernel waits for its
// direct-to-LDS loads (s_waitcnt vmcnt) and its LDS writes (kWaitLgkm0) explicitly, where needed.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
constexpr short kWaitLgkm0 = (short)0xC07F;   // s_waitcnt lgkmcnt(0), other counters untouched

// ---------------------------------------------------------------------------------------------
// Stage 1: lse2 and D (dsum) per query row; 8 lanes per row (16 channels each), rows in
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
    p.stats[x] = i < p.s_q ? p.lse[bh * p.s_q + i] * kLog2e : kPadLse2;
    p.stats[x + 64] = acc;
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
  const float lse2 = qrow < p.s_q ? p.stats[stat_index(bh, p.s_q_pad, qrow)] : kPadLse2;
  const float dsum = qrow < p.s_q ? p.stats[stat_index(bh, p.s_q_pad, qrow) + 64] : 0.0f;

  const int64_t kvoff = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + kvoff;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + kvoff;
  const int64_t kvbytes = (int64_t)(p.s_kv - 1) * stride + kHeadDim * 2;
  const int n_kt = (p.s_kv + kTile - 1) / kTile;
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int64_t off = (int64_t)j * kTile * stride;
    const unsigned st = lds + (unsigned)((j & 1) * 2 * kTileBytes);
    load_tile<kWaves>(kbase + off, kvbytes - off, stride, st, wv, lane);
    load_tile<kWaves>(vbase + off, kvbytes - off, stride, st + kTileBytes, wv, lane);
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
// Stage 2b: dK and dV.  One workgroup = 8 waves = 128 keys of one (batch, head).  Waves w and
// w + 4 (w < 4) own keys 32 w .. 32 w + 31, one key per lane, and share a SIMD.  Wave w (the P
// wave) computes S = Q K^T, P and dV^T += dO^T P; wave w + 4 (the dS wave) computes dP = dO V^T,
// dS = P (dP - D) and dK^T += Q^T dS, taking the fp32 P of each block from the P wave through
// LDS.  Each wave holds one B operand (K^T or V^T) and one accumulator set, so two waves fit on a
// SIMD, and the pair runs in opposite phases between workgroup barriers: while one wave issues
// the MFMAs of a 32-query block, the other runs the VALU work of a block (P, or dS).  Per
// 64-query tile i (blocks 2i and 2i+1), phases 4i .. 4i+3:
//   4i    P wave: dV += block 2i-1, S of block 2i         dS wave: dS of block 2i-1
//   4i+1  P wave: P of block 2i (to LDS)                 dS wave: dK += block 2i-1, dP of block 2i
//   4i+2  P wave: dV += block 2i, S of block 2i+1        dS wave: dS of block 2i
//   4i+3  P wave: P of block 2i+1 (to LDS)               dS wave: dK += block 2i, dP of block 2i+1
// then two more phases for block 2n-1.  Q, dO and the row statistics of 64-query tiles stream
// through a 4-stage LDS ring: tile u is loaded at the start of phase 4u - 10, into the stage of
// tile u - 4 (last read in phase 4u - 11), and waited for at the end of phase 4u - 1.
constexpr int kKvWaves = 8;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvStage = 2 * kTileBytes + kStatBytes;   // [Q | dO | statistics], 33 KB
constexpr int kKvRing = 4;
constexpr int kPBuf = kKvRing * kKvStage;               // P of one 32-query block per wave pair, 4 KB each
constexpr int kKvLds = kPBuf + 4 * 4096;                // 148 KB
constexpr int kLoadsPerTile = 5;                        // direct-to-LDS loads per wave per tile

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

  // B operand of this wave's product: K^T (P wave) or V^T (dS wave); lane holds key krow,
  // channels 16c + 8h .. +7 (keys past s_kv read as zeros and are never stored)
  const int64_t koff = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2 + k0 * stride;
  const int64_t kbytes = (int64_t)(p.s_kv - 1 - k0) * stride + kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t br =
      make_rsrc(reinterpret_cast<const unsigned char*>(pwave ? p.k : p.v) + koff, kbytes);
  bf16x8_t bf[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
    bf[c] = __builtin_bit_cast(
        bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(br, (unsigned)(l32 * stride + 32 * c + 16 * h), 0, 0));
  // waited for here, before any direct-to-LDS load is issued: the compiler does not see those, and
  // would otherwise place its wait for these registers inside the tile loop
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int64_t qoff = ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2;
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q) + qoff;
  const unsigned char* gbase = reinterpret_cast<const unsigned char*>(p.d_o) + qoff;
  const int64_t qbytes = (int64_t)(p.s_q - 1) * stride + kHeadDim * 2;
  const float* stats = p.stats + stat_index(bh, p.s_q_pad, 0);
  const int n_qt = p.s_q_pad / kTile;
  auto stage = [&](int i) __attribute__((always_inline)) { return smem + (i % kKvRing) * kKvStage; };
  // tile i: Q and dO rows (2 + 2 blocks of 1 KB per wave) and the 512 bytes of statistics, which
  // every wave loads (lanes 32-63 repeating lanes 0-31, the same bytes to the same place) so that
  // all waves issue the same number of loads per tile
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int64_t off = (int64_t)i * kTile * stride;
    const unsigned st = lds + (unsigned)((i % kKvRing) * kKvStage);
    load_tile<kKvWaves>(qbase + off, qbytes - off, stride, st, wv, lane);
    load_tile<kKvWaves>(gbase + off, qbytes - off, stride, st + kTileBytes, wv, lane);
    dma_b128(rsrc_words(stats + (int64_t)i * 2 * kTile, 2 * kTile * 4), st + 2 * kTileBytes,
             (unsigned)(16 * (lane & 31)));
  };
  // wait until the tile issued before the last `after` tiles has landed (s_waitcnt vmcnt, other
  // counters untouched)
  auto wait_tile = [&](int after) __attribute__((always_inline)) {
    if (after >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kLoadsPerTile));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsPerTile);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  // per-lane byte offsets of the operand reads within a tile, computed once (the empty asm keeps
  // them in registers instead of being rebuilt from the lane index at every read)
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
  // A operand rows (read_rows) and transposed columns (read_cols) with the offsets above
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
  // this wave pair's P slot: chunk j (4 floats) of lane l at float 4 (64 j + l)
  float* pslot = reinterpret_cast<float*>(smem + kPBuf + 4096 * kw);

  // Register r of the S, P, dP or dS block holds query 32 qb + 16 (r / 8) + 8 h + r % 8 of its
  // tile (this lane's key); its statistics sit at rows 32 qb + 16 (i / 2) + 8 h + 4 (i % 2) .. +3.
  auto stat4 = [&](const unsigned char* st, int which, int qb, int i) __attribute__((always_inline)) {
    const float* x = reinterpret_cast<const float*>(st + 2 * kTileBytes) + 64 * which;
    return *reinterpret_cast<const f32x4_t*>(x + 32 * qb + 16 * (i >> 1) + 8 * h + 4 * (i & 1));
  };

  f32x16_t acc[4];          // dV^T (P wave) or dK^T (dS wave), 4 blocks of 32 channels
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  f32x16_t prod;            // S (P wave) or dP (dS wave) of the current block
  unsigned bop[8];          // bf16 P (P wave) or dS (dS wave) of the block awaiting accumulation
  bf16x8_t pre[4];          // A operands of that accumulation's first step, read ahead
#pragma unroll
  for (int k = 0; k < 8; ++k) bop[k] = 0u;

  f32x4_t sv[4];            // statistics of the block in prod (lse2 or D), read ahead for the VALU phase

  // MFMA phase: acc += (transposed A tile at at, half aq) x bop over the two 16-query steps of the
  // block awaiting accumulation (if `accum`), then prod = (rows of the tile at pt, half pq) x bf (if
  // `product`) and, for the VALU phase after it, statistic `which` of that block from stage st.
  // All operand reads are issued ahead, in groups that the scheduling barriers keep in this
  // order: the accumulation steps (whose operands are older) run first, while the product's rows
  // arrive, so no MFMA waits for a read issued just before it.
  auto mfma_phase = [&](bool accum, const unsigned char* at, int aq, bool product, const unsigned char* st,
                        int poff, int which, int pq) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(3);
    const unsigned char* pt = st + poff;
    bf16x8_t r0[4], r1[4], c1[4];
    if (accum) {
#pragma unroll
      for (int db = 0; db < 4; ++db) c1[db] = cols(at, 2 * aq + 1, db);
    }
    if (product) {
#pragma unroll
      for (int c = 0; c < 4; ++c) r0[c] = rows(pt, pq, c);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (accum) {
      const u32x4_t x = {bop[0], bop[1], bop[2], bop[3]};
      mfma4_acc(acc, pre, __builtin_bit_cast(bf16x8_t, x));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (product) {
#pragma unroll
      for (int c = 0; c < 4; ++c) r1[c] = rows(pt, pq, 4 + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = stat4(st, which, pq, i);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (accum) {
      const u32x4_t x = {bop[4], bop[5], bop[6], bop[7]};
      mfma4_acc(acc, c1, __builtin_bit_cast(bf16x8_t, x));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (product) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16_t zero = {};
        prod = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0[c], bf[c], c == 0 ? zero : prod, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < 4; ++c) prod = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1[c], bf[4 + c], prod, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  issue(0);
  if (n_qt > 1) issue(1);
  if (n_qt > 2) issue(2);
  wait_tile(min(n_qt - 1, 2));
  barrier();

  if (pwave) {
    // VALU phase: the dO^T operands of this block's first dV step; P of the block (tile at st,
    // half qb) from prod and its lse2 (sv): fp32 P to the pair's slot, bf16 P to bop
    auto valu_phase = [&](const unsigned char* st, int qb) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) pre[db] = cols(st + kTileBytes, 2 * qb, db);
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t pv[4];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 2 * k;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(prod[r], kScaleLog2, -sv[r >> 2][r & 3]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(prod[r + 1], kScaleLog2, -sv[r >> 2][(r & 3) + 1]));
        bop[k] = cvt_pk_bf16(p0, p1);
        pv[r >> 2][r & 3] = p0;
        pv[r >> 2][(r & 3) + 1] = p1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4_t*>(pslot + 4 * (64 * j + lane)) = pv[j];
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // P is in LDS before the barrier
    };
    for (int i = 0; i < n_qt; ++i) {
      const unsigned char* cur = stage(i);
      const unsigned char* prv = stage(i + 3);   // tile i - 1
      mfma_phase(i > 0, prv + kTileBytes, 1, true, cur, 0, 0, 0);
      barrier();
      valu_phase(cur, 0);
      barrier();
      if (i + 3 < n_qt) issue(i + 3);
      mfma_phase(true, cur + kTileBytes, 0, true, cur, 0, 0, 1);
      barrier();
      valu_phase(cur, 1);
      wait_tile(min(n_qt - 2 - i, 2));
      barrier();
    }
    mfma_phase(true, stage(n_qt - 1) + kTileBytes, 1, false, smem, 0, 0, 0);
    barrier();
    barrier();
  } else {
    // VALU phase: dS of the block (tile at st, half qb) from prod (dP), the P wave's fp32 P and D
    // (sv), to bop; the Q^T operands of this block's first dK step are read meanwhile
    auto valu_phase = [&](const unsigned char* st, int qb) __attribute__((always_inline)) {
      f32x4_t pv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[j] = *reinterpret_cast<const f32x4_t*>(pslot + 4 * (64 * j + lane));
#pragma unroll
      for (int db = 0; db < 4; ++db) pre[db] = cols(st, 2 * qb, db);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 2 * k;
        const float d0 = prod[r] - sv[r >> 2][r & 3], d1 = prod[r + 1] - sv[r >> 2][(r & 3) + 1];
        bop[k] = cvt_pk_bf16(pv[r >> 2][r & 3] * d0, pv[r >> 2][(r & 3) + 1] * d1);
      }
    };
    for (int i = 0; i < n_qt; ++i) {
      const unsigned char* cur = stage(i);
      const unsigned char* prv = stage(i + 3);   // tile i - 1
      if (i > 0) valu_phase(prv, 1);
      barrier();
      mfma_phase(i > 0, prv, 1, true, cur, kTileBytes, 1, 0);
      barrier();
      if (i + 3 < n_qt) issue(i + 3);
      valu_phase(cur, 0);
      barrier();
      mfma_phase(true, cur, 0, true, cur, kTileBytes, 1, 1);
      wait_tile(min(n_qt - 2 - i, 2));
      barrier();
    }
    valu_phase(stage(n_qt - 1), 1);
    barrier();
    mfma_phase(true, stage(n_qt - 1), 1, false, smem, 0, 1, 0);
    barrier();
  }

  settle_mfma(acc);
  if (krow < p.s_kv) {
    // dV = dV^T; dK = dK^T * 1/sqrt(128); lane owns channels 32 db + 8 g + 4 h .. +3 of key krow
    const float scale = pwave ? 1.0f : kInvSqrtD;
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
  p.q_blocks = (int)ceil_div(sh.s_q, kRows);
  p.k_blocks = (int)ceil_div(sh.s_kv, kRows);
  const int64_t rows = bh * p.s_q_pad;
  hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)ceil_div(rows, 32)), dim3(256), 0, stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)(bh * p.q_blocks)), dim3(kThreads), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)(bh * p.k_blocks)), dim3(kKvThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
