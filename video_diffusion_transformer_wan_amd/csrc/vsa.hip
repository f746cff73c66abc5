// Block-sparse attention in the style of Video Sparse Attention (VSA) for gfx950 (MI355X).  The
// FastWan / VSA article describes a coarse stage that finds the key blocks that matter and a fine
// block-sparse attention over them, with 64 x 64 blocks and 87.5% sparsity.  Blocks here are 64
// consecutive tokens; the coarse stage keeps, for every query block, the `keep` key blocks with
// the largest mean_q . mean_k / sqrt(128) (ties to the lower index); the fine stage is exact
// softmax attention over the selected keys only.
//
// Kernels:
//  * vsa_pool_kernel -- one workgroup per (batch*head, block, tensor): the fp32 mean of Q or K over
//    the block's real tokens, [bh][block][128].
//  * vsa_select_kernel -- one workgroup per 8 query blocks of one batch*head: their block scores
//    against all key blocks in fp32, and per query block a radix select of the top `keep` (larger
//    score first, then lower index), written in ascending index order.
//  * vsa_attn_kernel -- one workgroup = one wave pair = one query block (32 query rows per wave);
//    the pair streams the 32-key halves of its selected key blocks through a 2-stage LDS ring
//    (direct-to-LDS loads), with the bf16 forward's transposed products, LDS layouts and swizzles
//    (S^T = K Q^T; O^T += V^T P^T by transposing V reads) and an online softmax with a running row
//    max (the O accumulators rescaled only when some row's max grows).

#include "wan_attn_internal.h"

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
// Read-only data that every lane of a wave reads at the same index (the block lists), through the
// constant address space: the compiler loads it with scalar loads, whose completion counter is not
// the one the direct-to-LDS loads use, so reading an entry never waits for the K/V loads in flight.
typedef __attribute__((address_space(4))) const int const_int_t;

constexpr int kBlock = 64;
constexpr float kNeg = -1.0e30f;
constexpr float kScaleLog2 = 0.12751743082459868f;   // log2(e) / sqrt(128)
constexpr float kInvSqrtD = 0.08838834764831845f;    // 1 / sqrt(128)
constexpr unsigned kRsrcFlags = 0x00020000u;
constexpr short kWaitVm0 = 0x0F70;

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, r);
}

// Values of lanes l and l^32 (the two halves of one query row's keys).
__device__ __forceinline__ void pair_values(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Buffer resource over [base, base + bytes); loads past the end return zeros.
__device__ __forceinline__ unsigned clamp_bytes(int64_t bytes) {
  return bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (unsigned)bytes);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)clamp_bytes(bytes), (int)kRsrcFlags);
}
// The same descriptor as four words, for the inline-asm direct-to-LDS loads.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const u32x4_t r = {(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, clamp_bytes(bytes), kRsrcFlags};
  return r;
}

// Direct global -> LDS load of 16 bytes per lane (lane i's bytes land at lds_addr + 16 i).  Inline asm,
// so that the compiler does not make LDS reads of the other ring stage wait for it; the kernel waits
// for these loads itself (s_waitcnt vmcnt) before the barrier after which its waves read them.
__device__ __forceinline__ void dma_b128(u32x4_t rsrc, unsigned lds_addr, unsigned voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}

// Workgroup barrier without __syncthreads()'s release fence (which would wait for the loads in flight).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------------------
// Coarse stage 1: block means.  Workgroup x = (batch*head * nb_max + block) * 2 + tensor (0: q,
// 1: k); 4 waves, lane = 2 channels, wave w sums tokens 16w .. 16w+15 of the block in order, and
// the four partial sums are added in wave order.
__global__ __launch_bounds__(256) void vsa_pool_kernel(const uint16_t* q, const uint16_t* k, int heads, int s_q,
                                                       int s_kv, int nb_max, float* pooled_q, float* pooled_k) {
  __shared__ float2 part[3][64];
  const int which = blockIdx.x & 1;
  const int rest = blockIdx.x >> 1;
  const int bh = rest / nb_max, blk = rest - bh * nb_max;
  const int s = which == 0 ? s_q : s_kv;
  const int nb = (s + kBlock - 1) / kBlock;
  if (blk >= nb) return;   // uniform over the workgroup
  const uint16_t* x = which == 0 ? q : k;
  float* out = which == 0 ? pooled_q : pooled_k;
  const int b = bh / heads, h = bh - b * heads;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = blk * kBlock, t1 = min(t0 + kBlock, s);
  const int64_t stride = (int64_t)heads * (kHeadDim / 2);   // 32-bit words between tokens
  const unsigned* src = reinterpret_cast<const unsigned*>(x + ((int64_t)b * s * heads + h) * kHeadDim) + lane;
  unsigned v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = t0 + 16 * wv + i;
    v[i] = t < t1 ? src[(int64_t)t * stride] : 0u;
  }
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a0 += __builtin_bit_cast(float, v[i] << 16);
    a1 += __builtin_bit_cast(float, v[i] & 0xffff0000u);
  }
  if (wv > 0) part[wv - 1][lane] = make_float2(a0, a1);
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      a0 += part[w][lane].x;
      a1 += part[w][lane].y;
    }
    const float n = (float)(t1 - t0);
    float* dst = out + ((int64_t)bh * nb + blk) * kHeadDim + 2 * lane;
    *reinterpret_cast<float2*>(dst) = make_float2(__fdiv_rn(a0, n), __fdiv_rn(a1, n));
  }
}

// ---------------------------------------------------------------------------------------------
// Coarse stage 2: scores and the top-keep selection of kSelQB consecutive query blocks of one
// (batch, head) per workgroup (4 waves), so that each block mean of K is read once per kSelQB query
// blocks.
//  * Scores: 8 lanes per key block, 16 consecutive channels each (products summed in channel
//    order), then a 3-level butterfly over the 8 lanes; score[i][j] = sum / sqrt(128), in LDS.
//  * Selection of query block i (one wave): an order-preserving 32-bit key of each score (larger
//    score, larger key; -0 taken as +0), a radix select over 4 digits of 8 bits from the top finds
//    the keep-th largest key T and how many of the keys equal to T are taken; then one sweep in
//    index order takes every key above T and the first of those equal to T -- ties to the lower
//    index -- and writes their indices, ascending, by ballot prefix counts.
constexpr int kSelThreads = 256;
constexpr int kSelQB = 8;
constexpr int kMaxKeyBlocks = 4096;   // keys of kSelQB query blocks in LDS: 128 KB

__device__ __forceinline__ unsigned order_key(float f) {
  if (f == 0.0f) f = 0.0f;   // -0 and +0 compare equal
  const unsigned u = __builtin_bit_cast(unsigned, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kSelThreads) void vsa_select_kernel(const float* pooled_q, const float* pooled_k, int n_qb,
                                                                 int n_kb, int groups_per_bh, int keep, int* block_idx) {
  extern __shared__ unsigned sel_lds[];   // [kSelQB][n_kb] keys, then [4 waves][256] histograms
  unsigned* keys = sel_lds;
  unsigned* hist_all = sel_lds + kSelQB * n_kb;
  const int bh = blockIdx.x / groups_per_bh;
  const int qb0 = (blockIdx.x - bh * groups_per_bh) * kSelQB;
  const int nq = min(kSelQB, n_qb - qb0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int part = tid & 7;   // channels 16 part .. 16 part + 15
  const int sub = tid >> 3;   // key block within a pass of 32

  // ---- scores
  float qm[kSelQB][16];
#pragma unroll
  for (int i = 0; i < kSelQB; ++i) {
    const int qb = qb0 + (i < nq ? i : 0);
    const float4* src = reinterpret_cast<const float4*>(pooled_q + ((int64_t)bh * n_qb + qb) * kHeadDim + 16 * part);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 x = src[c];
      qm[i][4 * c] = x.x;
      qm[i][4 * c + 1] = x.y;
      qm[i][4 * c + 2] = x.z;
      qm[i][4 * c + 3] = x.w;
    }
  }
  const float* kmb = pooled_k + (int64_t)bh * n_kb * kHeadDim;
  for (int j0 = 0; j0 < n_kb; j0 += kSelThreads / 8) {
    const int j = j0 + sub;
    float km[16];
    const float4* kr = reinterpret_cast<const float4*>(kmb + (int64_t)(j < n_kb ? j : 0) * kHeadDim + 16 * part);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 x = kr[c];
      km[4 * c] = x.x;
      km[4 * c + 1] = x.y;
      km[4 * c + 2] = x.z;
      km[4 * c + 3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < kSelQB; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = __builtin_fmaf(qm[i][c], km[c], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      if (part == 0 && j < n_kb) keys[i * n_kb + j] = order_key(acc * kInvSqrtD);
    }
  }
  __syncthreads();

  // ---- selection, one query block per wave at a time
  unsigned* hist = hist_all + 256 * wv;
  const uint64_t lt_mask = (1ull << lane) - 1;
  for (int i = wv; i < nq; i += 4) {
    const unsigned* kk = keys + i * n_kb;
    unsigned prefix = 0, mask = 0;
    int need = keep;   // how many of the keys matching prefix/mask are still to be taken
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) hist[4 * lane + c] = 0;
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
      for (int j = lane; j < n_kb; j += 64) {
        const unsigned key = kk[j];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1u);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      // lane l owns digits 4l .. 4l+3; counts of larger digits: lanes above, then higher bins
      unsigned h4[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) h4[c] = hist[4 * lane + c];
      const unsigned mine = h4[0] + h4[1] + h4[2] + h4[3];
      unsigned inc = mine;   // inclusive suffix sum over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const unsigned y = __shfl_down(inc, d);
        if (lane + d < 64) inc += y;
      }
      const unsigned above = inc - mine;   // keys whose digit belongs to a higher lane
      int digit = -1, new_need = 0;
      unsigned acc = above;
#pragma unroll
      for (int c = 3; c >= 0; --c) {
        if (digit < 0 && acc < (unsigned)need && acc + h4[c] >= (unsigned)need) {
          digit = 4 * lane + c;
          new_need = need - (int)acc;
        }
        acc += h4[c];
      }
      const uint64_t found = __ballot(digit >= 0);
      const int src_lane = __builtin_ctzll(found);
      digit = __shfl(digit, src_lane);
      need = __shfl(new_need, src_lane);
      prefix |= (unsigned)digit << shift;
      mask |= 255u << shift;
    }
    // prefix is now the keep-th largest key T; take all keys > T and the first `need` equal to it
    int* dst = block_idx + ((int64_t)bh * n_qb + qb0 + i) * keep;
    int taken = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n_kb; j0 += 64) {
      const int j = j0 + lane;
      const unsigned key = j < n_kb ? kk[j] : 0u;
      const bool eq = j < n_kb && key == prefix;
      const uint64_t eqm = __ballot(eq);
      const int eq_rank = eq_seen + __popcll(eqm & lt_mask);
      const bool take = j < n_kb && (key > prefix || (eq && eq_rank < need));
      const uint64_t tm = __ballot(take);
      const int pos = taken + __popcll(tm & lt_mask);
      if (take && pos < keep) dst[pos] = j;   // exactly keep are taken; the bound only guards the list
      taken += __popcll(tm);
      eq_seen += __popcll(eqm);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Fine stage.  A workgroup is one wave pair serving one query block (32 query rows per wave), with
// its own 2-stage LDS ring of 32-key steps (32 KB): up to 5 workgroups per CU, each synchronising
// only its own two waves, so query blocks whose lists differ do not wait for each other.
constexpr int kAttnWaves = 2;
constexpr int kPairs = kAttnWaves / 2;
constexpr int kHalf = 32;                        // keys per step
constexpr int kKBytes = kHalf * kHeadDim * 2;    // K of one step, 8 KB
constexpr int kStageBytes = 2 * kKBytes;         // [K | V]
constexpr int kPairLds = 2 * kStageBytes;        // 2 stages per wave pair

struct VsaParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int* block_idx;   // [bh][n_qb][keep]
  uint16_t* o;
  int heads, s_q, s_kv, n_qb, n_kb, keep, groups_per_bh;
  int total;   // workgroups with work: batch*heads*groups_per_bh
};

// Workgroup numbering: workgroup w runs on XCD w % 8, and each run of 8 * kXcdChunk consecutive query
// blocks gives every XCD kXcdChunk consecutive ones.  All XCDs stay on about the same head (its K and
// V stay in the shared last-level cache), while each XCD's L2 serves neighbouring query blocks,
// whose selections overlap when the scores have locality.
constexpr int kXcdChunk = 64;

__global__ __launch_bounds__(64 * kAttnWaves, 1) void vsa_attn_kernel(const VsaParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kPairs * kPairLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wv >> 1, w2 = wv & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int round8 = slot / kXcdChunk;
  const int item = (8 * round8 + xcd) * kXcdChunk + (slot - round8 * kXcdChunk);
  if (item >= p.total) return;
  const int bh = item / p.groups_per_bh;
  const int qb = kPairs * (item - bh * p.groups_per_bh) + pair;
  const bool active = qb < p.n_qb;                  // wave-uniform
  const int bb = bh / p.heads, hh = bh - bb * p.heads;
  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;   // bytes between tokens
  unsigned char* ring = smem + pair * kPairLds;
  const unsigned lds_ring = (unsigned)(uintptr_t)(lds_void_t*)ring;

  // loads: wave w2 of the pair writes 1 KB blocks 4 w2 .. 4 w2 + 3 (4 key rows each) of the K and
  // of the V part of a stage; K rows permuted by swap23 and chunks XOR-swizzled by row % 16, V rows
  // in key order with chunks XOR-swizzled by 4 (row % 4) -- the bf16 forward's layouts
  unsigned k_src[4], v_src[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int m = 4 * w2 + it;
    const int row = 4 * m + (lane >> 4);
    const int pch = lane & 15;
    k_src[it] = (unsigned)(swap23(row) * stride + 16 * (pch ^ (row & 15)));
    v_src[it] = (unsigned)(row * stride + 16 * (pch ^ ((row & 3) << 2)));
  }
  const int k_rd0 = l32 * 256 + 16 * ((h ^ l32) & 1) + 32 * ((l32 >> 1) & 7);
  int v_rd0;
  {
    const int g = lane >> 4, kq = (lane >> 2) & 3, q = lane & 3;
    const int x = 2 * (g & 1) + (q >> 1);
    v_rd0 = kKBytes + (8 * (g >> 1) + kq) * 256 + 64 * kq + 16 * x + 8 * (q & 1);
  }

  const int64_t kv_head = ((int64_t)bb * p.s_kv * p.heads + hh) * kHeadDim * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + kv_head;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + kv_head;
  const const_int_t* list = (const const_int_t*)(p.block_idx + ((int64_t)bh * p.n_qb + (active ? qb : 0)) * p.keep);
  const int n_steps = 2 * p.keep;

  // Q^T operand: lane holds query row q0 + l32, channels 16c + 8h .. +7 (rows past s_q read zeros)
  const int q0 = qb * kBlock + 32 * w2;
  bf16x8_t qf[8];
  {
    const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q) +
                                 ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2 + (int64_t)q0 * stride;
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(qbase, active ? (int64_t)(p.s_q - 1 - q0) * stride + kHeadDim * 2 : 0);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[c] = __builtin_bit_cast(
          bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, (unsigned)(l32 * stride + 32 * c + 16 * h), 0, 0));
  }

  // first key of step t (-1: nothing to attend: an index outside [0, n_kb), a half past s_kv, or
  // an idle pair)
  auto step_key0 = [&](int t) __attribute__((always_inline)) {
    const int blk = list[t >> 1];
    const int kv0 = blk * kBlock + kHalf * (t & 1);
    return (active && blk >= 0 && blk < p.n_kb && kv0 < p.s_kv) ? kv0 : -1;
  };
  auto issue = [&](int t, int kv0) __attribute__((always_inline)) {
    const int64_t off = (int64_t)(kv0 >= 0 ? kv0 : 0) * stride;
    const int64_t bytes = kv0 >= 0 ? (int64_t)(p.s_kv - 1 - kv0) * stride + kHeadDim * 2 : 0;
    const u32x4_t kr = rsrc_words(kbase + off, bytes);
    const u32x4_t vr = rsrc_words(vbase + off, bytes);
    const unsigned st = lds_ring + (unsigned)((t & 1) * kStageBytes + 4096 * w2);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      dma_b128(kr, st + 1024 * it, k_src[it]);
      dma_b128(vr, st + kKBytes + 1024 * it, v_src[it]);
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = kNeg, l = 0.0f;

  int kv_next = step_key0(0);
  issue(0, kv_next);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  barrier();
  for (int t = 0; t < n_steps; ++t) {
    const int kv0 = kv_next;   // first key of this step, read when its loads were issued
    if (t + 1 < n_steps) {
      kv_next = step_key0(t + 1);
      issue(t + 1, kv_next);
    }
    if (kv0 >= 0) {
      const unsigned char* ks = ring + (t & 1) * kStageBytes;
      // S^T of the 32 keys: s holds key kv0 + swap23(8 (r / 4) + 4 h + r % 4) of the lane's row
      f32x16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8_t f0 = *reinterpret_cast<const bf16x8_t*>(ks + (k_rd0 ^ (64 * st)));
        const bf16x8_t f1 = *reinterpret_cast<const bf16x8_t*>(ks + (k_rd0 ^ (64 * st + 32)));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, qf[2 * st], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1, qf[2 * st + 1], s, 0, 0, 0);
      }
      if (kv0 + kHalf > p.s_kv) {   // keys past s_kv get a score that exp2 turns into 0
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kv0 + swap23(8 * (r >> 2) + 4 * h + (r & 3)) >= p.s_kv) s[r] = kNeg;
      }
      float mx = kNeg;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[r]);
      float ma, mb;
      pair_values(mx, ma, mb);
      const float m_new = __builtin_fmaxf(m, __builtin_fmaxf(ma, mb));
      if (__any(m_new > m)) {
        const float alpha = __builtin_amdgcn_exp2f((m - m_new) * kScaleLog2);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      m = m_new;
      const float mc = m * kScaleLog2;
      unsigned pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], kScaleLog2, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], kScaleLog2, -mc));
        pk[r >> 1] = cvt_pk_bf16(p0, p1);
        l += p0 + p1;
      }
      // O^T += V^T P^T over the step's 2 groups of 16 keys
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4_t x = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, x);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const unsigned char* vp = ks + (v_rd0 ^ (64 * db)) + 4096 * u;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vp));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vp + 1024));
          const i16x4_t cat[2] = {lo, hi};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cat), bop, o[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's loads of step t+1
    barrier();                              // step t+1 has landed; everyone is done with step t
  }

  if (active) {
    float la, lb;
    pair_values(l, la, lb);
    const float inv = 1.0f / (la + lb);
    const int row = q0 + l32;
    if (row < p.s_q) {
      uint16_t* dst = p.o + (((int64_t)bb * p.s_q + row) * p.heads + hh) * kHeadDim + 4 * h;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2_t x = {cvt_pk_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                             cvt_pk_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(dst + 32 * db + 8 * g) = x;
        }
    }
  }
}

}  // namespace

size_t vsa_select_scratch_bytes(const AttnShape& sh) {
  const int64_t nq = ceil_div(sh.s_q, kBlock), nk = ceil_div(sh.s_kv, kBlock);
  return (size_t)(sh.batch * sh.heads * (nq + nk) * kHeadDim) * sizeof(float);
}

int vsa_max_key_blocks() { return kMaxKeyBlocks; }

hipError_t launch_vsa_select(const void* q, const void* k, const AttnShape& sh, int keep, int* block_idx,
                             void* scratch, hipStream_t stream) {
  const int n_qb = (int)ceil_div(sh.s_q, kBlock), n_kb = (int)ceil_div(sh.s_kv, kBlock);
  if (n_kb > kMaxKeyBlocks) return hipErrorInvalidValue;
  const int64_t bh = sh.batch * sh.heads;
  float* pooled_q = static_cast<float*>(scratch);
  float* pooled_k = pooled_q + bh * n_qb * kHeadDim;
  const unsigned lds = (unsigned)(kSelQB * n_kb + 4 * 256) * 4;   // at most 132 KB
  hipError_t e;
  if (lds > 32768) {   // above the default dynamic LDS limit of some runtimes: raised once per device
    static bool raised[64] = {};
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!raised[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(vsa_select_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kSelQB * kMaxKeyBlocks + 4 * 256) * 4);
      if (e != hipSuccess) return e;
      raised[dev] = true;
    }
  }
  const int nb_max = n_qb > n_kb ? n_qb : n_kb;
  hipLaunchKernelGGL(vsa_pool_kernel, dim3((unsigned)(2 * bh * nb_max)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), (int)sh.heads, (int)sh.s_q,
                     (int)sh.s_kv, nb_max, pooled_q, pooled_k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int groups = (n_qb + kSelQB - 1) / kSelQB;
  hipLaunchKernelGGL(vsa_select_kernel, dim3((unsigned)(groups * bh)), dim3(kSelThreads), lds, stream, pooled_q,
                     pooled_k, n_qb, n_kb, groups, keep, block_idx);
  return hipGetLastError();
}

hipError_t launch_vsa_attn(const void* q, const void* k, const void* v, const int* block_idx, int keep, void* o,
                           const AttnShape& sh, hipStream_t stream) {
  VsaParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.block_idx = block_idx;
  p.o = static_cast<uint16_t*>(o);
  p.heads = (int)sh.heads;
  p.s_q = (int)sh.s_q;
  p.s_kv = (int)sh.s_kv;
  p.n_qb = (int)ceil_div(sh.s_q, kBlock);
  p.n_kb = (int)ceil_div(sh.s_kv, kBlock);
  p.keep = keep;
  p.groups_per_bh = (p.n_qb + kPairs - 1) / kPairs;
  p.total = (int)(sh.batch * sh.heads * p.groups_per_bh);
  const int64_t chunk8 = 8LL * kXcdChunk;
  const int64_t grid = (p.total + chunk8 - 1) / chunk8 * chunk8;
  hipLaunchKernelGGL(vsa_attn_kernel, dim3((unsigned)grid), dim3(64 * kAttnWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
