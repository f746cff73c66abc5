// bf16 flash-attention forward for gfx950 (MI355X).
//
// Computes O = softmax(Q K^T / sqrt(128)) V per (batch, head), non-causal and unmasked: the full
// spatio-temporal self-attention of a Wan DiT block and its umT5 cross-attention ("Wan 2.1:
// VBench 86.22% ..." explainer of the Wan technical report, sections "先看现象" and
// "干预与形式化").  The result is reached by a tiled softmax over 64-key blocks against a fixed
// per-row reference max, exact in real arithmetic (a re-association of the definition).
//
// Design (one workgroup = 8 waves = 256 query rows of one (batch, head); 1 workgroup per CU):
//  * The products run transposed so that no operand needs a cross-lane shuffle:
//      S^T = K Q^T    (A = K tile from LDS, B = Q^T held in VGPRs for the whole kernel)
//      O^T += V^T P^T (A = V^T from LDS via transposing reads, B = P^T straight from S^T)
//    With v_mfma_f32_32x32x16_bf16 every lane owns one query row (lane % 32) of its wave's
//    32 rows, and lanes l and l+32 split the keys.  Row max / row sum are in-lane reductions
//    plus one v_permlane32_swap.
//  * K rows sit in LDS with bits 2 and 3 of the key index swapped, which makes the 8 P values a
//    lane feeds to one PV MFMA belong to 8 consecutive keys.  V stays in natural [key][channel]
//    order and ds_read_b64_tr_b16 hands each lane 4 consecutive keys of one channel.
//  * K and V tiles go straight from HBM to LDS (buffer_load ... lds, out-of-range rows read as
//    zeros) into a 4-stage ring; both tiles are XOR-swizzled so operand reads are conflict-free.
//  * Ping-pong: waves 0-3 and waves 4-7 share the four SIMDs and run half a tile apart.  In each
//    half-step one group issues MFMAs (S^T of tile j and the PV product of tile j-1) while the
//    other runs the softmax of its tile on the VALU; a workgroup barrier between half-steps keeps
//    the two groups in opposite phases, so the matrix cores and the VALUs stay busy together.
//  * Softmax in the exp2 domain with the scale folded in (one FMA + one v_exp_f32 per score),
//    against a reference max per row that stays fixed for the whole sweep over the keys: the
//    max of the row's first 64 scores.  Softmax does not depend on the constant subtracted, so
//    the only risk is that a later, much larger score overflows P; then the row sum exceeds
//    2^64 (or is infinite), and the query tile is swept again -- once for the true row max
//    (S^T only), once for the result.  The loop carries no running max, no vote and no
//    rescaling of O.  Row sums add the fp32 P with v_add_f32: v_dot2_f32_bf16 on the packed P
//    would issue to the matrix-core pipe, where it waits behind the other wave's MFMAs (about
//    160 cycles each, against 6 on an idle pipe).
//  * Workgroups are numbered so that the 32 CUs of one XCD work on consecutive query tiles of the
//    same head and share its K/V stream in their L2.
//  * At a work-item boundary the O rows leave through LDS as whole rows and the next item's Q
//    arrives through LDS, both with the non-temporal hint (read or written once); for short key
//    sequences half the workgroups start late, so that the CUs do not all cross a boundary at once.

#include <type_traits>

#include "wan_attn_internal.h"

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;                 // 256 query rows per workgroup
constexpr int kBN = 64;                          // keys per tile
constexpr int kKBytes = kBN * kHeadDim * 2;      // K tile, 16 KB
constexpr int kVBytes = kBN * kHeadDim * 2;      // V tile, 16 KB
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr int kStages = 4;
constexpr float kNeg = -1.0e30f;            // masked score (finite: keeps inf - inf out)
// a row sum above this (P of some key above 2^64 / s_kv) sends the query tile to the exact
// two-sweep path
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64
// log2(e) / sqrt(128): scores go straight into exp2
constexpr float kScaleLog2 = 0.12751743082459868f;
constexpr float kInvSqrtD = 0.08838834764831845f;   // 1 / sqrt(128)
constexpr float kLn2 = 0.6931471805599453f;
constexpr unsigned kRsrcFlags = 0x00020000u;   // raw buffer, 32-bit dwords
constexpr short kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0), other counters untouched
constexpr short kWaitLgkm0 = (short)0xC07F;    // s_waitcnt lgkmcnt(0), other counters untouched

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int heads;
  int s_q;
  int s_kv;
  int q_tiles;
  int total;      // work items: q_tiles * batch * heads * split
  int per_xcd;    // ceil(total / 8): work items handled by each XCD
  int n_slots;    // workgroups per XCD (gridDim.x / 8)
  int split;      // key ranges per query tile (1: the whole key sequence)
  int split_tiles;   // 64-key tiles per key range
  float* ws;      // split > 1: partial results, [item][256][128] O then [item][256][2] (m, l)
  float* lse;     // optional (may be null): row log-sum-exp of the scaled scores, [b][H][s_q]
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

// Values of lanes l and l^32 (the two halves of one query row), returned as (own, other).
__device__ __forceinline__ void pair_values(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  a = __builtin_bit_cast(float, (unsigned)r[0]);
  b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup barrier without the release fence of __syncthreads(): the fence would make every
// wave wait here for its in-flight direct-to-LDS loads (vmcnt(0)), which this kernel waits for
// explicitly, one half-step later.  The memory clobber keeps the compiler from moving LDS reads
// across it.  LDS reads in flight at a barrier only target tiles that no load overwrites before
// the half-step after it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer resource over [base, base + bytes); loads past the end return zeros.
__device__ __forceinline__ int clamp_bytes(int64_t bytes) {
  return bytes <= 0 ? 0 : (bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, clamp_bytes(bytes), (int)kRsrcFlags);
}
// The same descriptor as four words, for the inline-asm loads below (bytes < 2^31).
__device__ __forceinline__ u32x4_t rsrc_words32(const void* base, unsigned bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const u32x4_t r = {(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, bytes, kRsrcFlags};
  return r;
}

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at LDS address
// lds_addr + 16 i.  Inline asm, because the compiler cannot tell the stages of the LDS ring apart
// and would make every LDS read after such a load wait for it -- among them the reads of the
// previous tile that the softmax half-step issues right after its loads.  The kernel waits for
// these loads itself (s_waitcnt vmcnt) before the barrier after which any wave reads their data.
__device__ __forceinline__ void dma_b128(u32x4_t rsrc, unsigned lds_addr, unsigned voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}
// The same with the non-temporal hint, for data read once (the next work item's Q): it streams
// past the caches instead of displacing the K/V tiles that the CUs of an XCD share in L2.
__device__ __forceinline__ void dma_b128_nt(u32x4_t rsrc, unsigned lds_addr, unsigned voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr));
}

// [stage][K | V]: K rows permuted by swap23 and XOR-swizzled by (row % 16); V rows (keys) in
// natural order, 16-byte chunks XOR-swizzled by 4 * (key % 4).
__shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
__shared__ int redo_flag[kWaves];

// The kernel's Params where the launch put them: its only argument, at the start of the
// kernel-argument segment.
typedef __attribute__((address_space(4))) const Params kernarg_params_t;

// The fields of *kp, loaded at this point of the program.  The zero index is hidden from the
// compiler, so it cannot hoist these loads to the kernel's start and hold every field in a scalar
// register for the whole kernel: the sweep over the keys needs those registers.
__device__ __forceinline__ Params load_params(kernarg_params_t* kp) {
  int z = 0;
  asm volatile("" : "+s"(z));
  kernarg_params_t& a = kp[z];
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.heads = a.heads;
  p.s_q = a.s_q;
  p.s_kv = a.s_kv;
  p.q_tiles = a.q_tiles;
  p.total = a.total;
  p.per_xcd = a.per_xcd;
  p.n_slots = a.n_slots;
  p.split = a.split;
  p.split_tiles = a.split_tiles;
  p.ws = a.ws;
  p.lse = a.lse;
  return p;
}

// Attention of one query tile (256 rows of one (batch, head)), run by the whole workgroup.
// kExact = false: one sweep against the max of the first 64 keys; writes O.  Returns kRedo when
// some row sum of the tile passed 2^64 (O, written regardless, is then invalid and the caller
// reruns the tile with kExact = true, which overwrites it).  When next_item >= 0 it also loads
// the next work item's Q tile into ring stages 2 and 3 once the sweep is done with the ring
// (the loads overlap this tile's epilogue and vote) and returns kQPrefetched; the caller then
// passes q_in_lds = true for that item, whose Q operands are read from LDS instead of HBM.
// kExact = true: one sweep for the row maxima, one softmax sweep against them; writes O.
// kSplit: work item `item` is key range item % split of query tile item / split; instead of O it
// writes the unnormalised O, the reference max m and the row sum l of that range to p.ws.
constexpr int kRedo = 1, kQPrefetched = 2;
template <bool kExact, bool kSplit>
__device__ __forceinline__ int attn_tile(kernarg_params_t* kp, const int item, const int next_item = -1,
                                         const bool q_in_lds = false) {
  const Params p = load_params(kp);
  const int tile = kSplit ? item / p.split : item;
  const int k0 = kSplit ? (item - tile * p.split) * p.split_tiles * kBN : 0;   // first key of the range
  const int s_kv = kSplit ? min(p.s_kv - k0, p.split_tiles * kBN) : p.s_kv;    // keys in the range
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const bool first_group = wv < kWaves / 2;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const unsigned lds_ring = (unsigned)(uintptr_t)(lds_void_t*)smem;   // LDS address of the ring
  const int64_t stride = (int64_t)p.heads * kHeadDim * 2;   // bytes between tokens
  const int n_tiles = (s_kv + kBN - 1) / kBN;

  // ---- direct global -> LDS tile loads: wave wv fills 1 KB blocks 2wv and 2wv+1 of the K tile
  // and of the V tile; lane i writes bytes 16i .. 16i+15 of its block.
  unsigned k_src[2], v_src[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int m = 2 * wv + it;
    const int row = 4 * m + (lane >> 4);
    const int pch = lane & 15;
    k_src[it] = (unsigned)(swap23(row) * stride + 16 * (pch ^ (row & 15)));
    v_src[it] = (unsigned)(row * stride + 16 * (pch ^ ((row & 3) << 2)));
  }

  // ---- per-lane LDS read offsets
  // K (A operand of S^T): row l32 (+32 for the second key block), 16-byte chunk
  // (2c + h) ^ (l32 % 16), i.e. byte offset k_rd0 ^ 32c (bits 5-7 carry c ^ ((l32 / 2) % 8))
  const int k_rd0 = l32 * 256 + 16 * ((h ^ l32) & 1) + 32 * ((l32 >> 1) & 7);
  // V (A operand of O^T, transposed read): within each 16-lane group, lane 4r + q addresses key
  // row r and channels 4q .. 4q+3 of its 16-channel slice; the read hands lane i channel i of
  // four consecutive keys.  Rows 16t + 8h + 4e (e = 0, 1) give the 8 keys of one MFMA.
  // Offset of channel block db: v_rd0 ^ 64db (bits 6-7 carry db ^ (row % 4)).
  int v_rd0;
  {
    const int g = lane >> 4, kq = (lane >> 2) & 3, q = lane & 3;
    const int x = 2 * (g & 1) + (q >> 1);
    v_rd0 = kKBytes + (8 * (g >> 1) + kq) * 256 + 64 * kq + 16 * x + 8 * (q & 1);
  }
  {
    const int qt = tile % p.q_tiles;
    const int bh = tile / p.q_tiles;
    const int bb = bh / p.heads;
    const int hh = bh - bb * p.heads;

    const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q) + ((int64_t)bb * p.s_q * p.heads + hh) * kHeadDim * 2;
    const int64_t kv_head = (((int64_t)bb * p.s_kv + k0) * p.heads + hh) * kHeadDim * 2;   // first key of the range
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + kv_head;
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v) + kv_head;
    const unsigned stride32 = (unsigned)stride;            // < 2^25: heads <= 65536
    const unsigned tile_bytes = kBN * stride32;             // bytes between consecutive key tiles

    // ---- Q^T operand: lane holds query row q0 + l32, channels 16c + 8h .. +7
    // (rows past s_q read as zeros and are never stored)
    bf16x8_t qf[8];
    const int q0 = qt * kBM + wv * 32;
    // Q rows staged in LDS by the previous work item (prefetch_q below): row r of the tile sits in
    // stage 2 (r < 128) or 3, row r % 128, its 16-byte chunk c at position c ^ (r % 16)
    const unsigned char* q_lds = smem + (2 + (wv >> 2)) * kStageBytes + (32 * (wv & 3) + l32) * 256;
    if (!q_in_lds) {
      const __amdgpu_buffer_rsrc_t qr =
          make_rsrc(qbase + q0 * stride, (int64_t)(p.s_q - 1 - q0) * stride + kHeadDim * 2);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        qf[c] = __builtin_bit_cast(
            bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qr, (unsigned)(l32 * stride + 32 * c + 16 * h), 0, 0));
    }

    // Tile j's descriptors start at its first key and end after its last valid key row, so rows
    // past s_kv read as zeros.  32-bit scalars only (a tile spans kBN * stride < 2^31 bytes): the
    // sweep loop's scalar registers are scarce.
    auto issue_tile = [&](int j) __attribute__((always_inline)) {
      const uint64_t off = (uint64_t)(unsigned)j * tile_bytes;
      const int rows = min(s_kv - j * kBN, kBN);
      const unsigned bytes = (unsigned)(rows - 1) * stride32 + kHeadDim * 2;
      const u32x4_t kr = rsrc_words32(kbase + off, bytes);
      const u32x4_t vr = rsrc_words32(vbase + off, bytes);
      const unsigned st = lds_ring + (unsigned)((j % kStages) * kStageBytes + 2048 * wv);
      dma_b128(kr, st, k_src[0]);
      dma_b128(kr, st + 1024, k_src[1]);
      dma_b128(vr, st + kKBytes, v_src[0]);
      dma_b128(vr, st + kKBytes + 1024, v_src[1]);
    };

    f32x16_t o[4];
    float m = kNeg, l = 0.0f;   // reference max of the lane's query row, lane's part of the row sum
    float m_run = kNeg;         // max-only sweep: largest score the lane has seen
    f32x16_t s[2];          // S^T of the newest tile, per 32-key block
    unsigned pk[2][8];      // bf16 P^T of the tile awaiting its PV product (pairs of S^T registers)

    // V^T operands of keys 16t .. 16t+15 of tile jj, the four 32-channel blocks
    auto read_v = [&](int jj, int t, bf16x8_t (&f)[4]) __attribute__((always_inline)) {
      const unsigned char* vst = smem + (jj % kStages) * kStageBytes;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const unsigned char* vp = vst + (v_rd0 ^ (64 * db)) + 4096 * t;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vp));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vp + 1024));
        const i16x4_t cat[2] = {lo, hi};
        f[db] = __builtin_bit_cast(bf16x8_t, cat);
      }
    };
    bf16x8_t pv_first[4];   // V^T operands of the first PV step, read ahead by the softmax half-step

    // MFMA half-step: S^T of tile j (kQK) and the PV product of tile j-1 (kPV), as one stream of
    // steps of 4 MFMAs (4 S^T steps over 32 channels each, 4 PV steps over 16 keys each).  A PV
    // step comes first because its operands (tile j-1) may be read before the barrier that opens
    // this half-step: the softmax half-step before it reads them, so the matrix core does not
    // wait for LDS at the start.  The LDS operands of step i+1 are read
    // while step i issues its MFMAs (two operand sets); the scheduling barriers keep that order,
    // and the register footprint, as written.
    auto mfma_phase = [&](int j, auto qk_tag, auto pv_tag) __attribute__((always_inline)) {
      constexpr bool kQK = decltype(qk_tag)::value;
      constexpr bool kPV = decltype(pv_tag)::value;
      const unsigned char* ks = smem + (j % kStages) * kStageBytes;
      // raised issue priority: the SIMD's other wave is in its softmax half-step, and its VALU
      // stream would otherwise delay these MFMAs
      __builtin_amdgcn_s_setprio(3);
      constexpr int kN = (kQK ? 4 : 0) + (kPV ? 4 : 0);
      // step at position i (0-3 S^T channel steps, 4-7 PV key steps): the first PV step, then
      // S^T (done early, so the softmax half-step after this one need not wait for it), then the
      // remaining PV steps
      auto step_at = [](int i) { return !kPV ? i : (!kQK ? i + 4 : (i == 0 ? 4 : (i <= 4 ? i - 1 : i))); };
      bf16x8_t ring[2][4];
      auto read_step = [&](int st, bf16x8_t (&f)[4]) {
        if (st < 4) {   // channels 32st .. 32st+31 (c = 2st, 2st+1) of both 32-key blocks
          const int o0 = k_rd0 ^ (64 * st), o1 = k_rd0 ^ (64 * st + 32);
          f[0] = *reinterpret_cast<const bf16x8_t*>(ks + o0);
          f[1] = *reinterpret_cast<const bf16x8_t*>(ks + o0 + 8192);
          f[2] = *reinterpret_cast<const bf16x8_t*>(ks + o1);
          f[3] = *reinterpret_cast<const bf16x8_t*>(ks + o1 + 8192);
        } else {
          read_v(j - 1, st - 4, f);
        }
      };
      if constexpr (kQK) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      }
      if constexpr (kPV) {
#pragma unroll
        for (int db = 0; db < 4; ++db) ring[0][db] = pv_first[db];
      } else {
        read_step(step_at(0), ring[0]);
      }
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int cur = i & 1;
        const int st = step_at(i);
        if (i + 1 < kN) read_step(step_at(i + 1), ring[cur ^ 1]);
        if (st < 4) {
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][0], qf[2 * st], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][1], qf[2 * st], s[1], 0, 0, 0);
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][2], qf[2 * st + 1], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][3], qf[2 * st + 1], s[1], 0, 0, 0);
        } else {
          // keys 16t .. 16t+15: S^T registers 8u .. 8u+7 of key block t/2
          const int t = st - 4, kb = t >> 1, u = t & 1;
          const u32x4_t x = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
          const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, x);
#pragma unroll
          for (int db = 0; db < 4; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[cur][db], bop, o[db], 0, 0, 0);
        }
        if (kQK && kPV && i == 0) {
          // the first step's order: two MFMAs, then the next step's four K reads two at a time
          // between the last two, so that they start as early as the pipe allows (left to
          // itself the scheduler can issue three MFMAs first, a wait of two MFMA slots)
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // this wave's loads of tile j+1 (issued at the start of its previous softmax half-step)
      // must have landed before the barrier that ends this half-step
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    };
    const std::true_type yes{};
    const std::false_type no{};

    // keys past the end of the sequence (last tile only) get a score that exp2 turns into 0
    auto mask_tile = [&](int j) __attribute__((always_inline)) {
      const int kv0 = j * kBN;
      if (kv0 + kBN > s_kv) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + swap23(32 * kb + 8 * (r >> 2) + 4 * h + (r & 3));
            if (key >= s_kv) s[kb][r] = kNeg;
          }
      }
    };

    // VALU half-step: this wave's share of the loads of tile j+2, then the softmax of tile j
    // (its S^T is in s) against the reference max, leaving bf16 P^T in pk.  set_ref: tile j = 0
    // of the first sweep, whose row max becomes the reference.
    auto softmax_phase = [&](int j, bool set_ref) __attribute__((always_inline)) {
      if (j + 2 < n_tiles) issue_tile(j + 2);
      mask_tile(j);
      if (set_ref) {
        float mx = kNeg;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[kb][r]), s[kb][r + 1]);
        float ma, mb;
        pair_values(mx, ma, mb);
        m = __builtin_fmaxf(ma, mb);
      }
      const float mc = m * kScaleLog2;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], kScaleLog2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], kScaleLog2, -mc));
          const unsigned pp = cvt_pk_bf16(p0, p1);
          pk[kb][r >> 1] = pp;
          l += p0 + p1;
        }
      // operands of the next half-step's first PV step (tile j, keys 0-15): tile j stays in its
      // stage until tile j+4 is loaded, well after that half-step
      read_v(j, 0, pv_first);
    };
    // VALU half-step of the max-only sweep: loads of tile j+2, row max of tile j
    auto max_phase = [&](int j) __attribute__((always_inline)) {
      if (j + 2 < n_tiles) issue_tile(j + 2);
      mask_tile(j);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) m_run = __builtin_fmaxf(__builtin_fmaxf(m_run, s[kb][r]), s[kb][r + 1]);
    };

    // One sweep over all keys (kExp: softmax and PV product; else S^T and row max only).
    // Schedule (B_k = k-th workgroup barrier of the sweep).  Every wave runs the same sequence
    // MFMA(j) | barrier | softmax(j) | barrier  for j = 0 .. n-1, then the PV product of tile
    // n-1, but waves 4-7 enter it one barrier later than waves 0-3, so between consecutive
    // barriers one group issues MFMAs while the other is on the VALU.  Tile t is loaded into
    // stage t % 4 at the start of softmax(t-2) -- after B_{2t-3} (group 1) or B_{2t-2} (group 2),
    // both after the last read of tile t-4 in group 2's MFMA(t-3) -- and waited for at the end
    // of MFMA(t-1), before the barrier B_{2t} after which group 1 reads it.
    auto sweep = [&](auto exp_tag, bool set_ref) __attribute__((always_inline)) {
      constexpr bool kExp = decltype(exp_tag)::value;
      if constexpr (kExp) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
        l = 0.0f;
      }
      issue_tile(0);
      if (n_tiles > 1) issue_tile(1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      barrier();
      if (q_in_lds && kExp && set_ref) {
        // the Q operands from stages 2 and 3, read before the barrier after which tile 2 is
        // loaded over them (the first softmax half-step of waves 0-3)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          qf[c] = *reinterpret_cast<const bf16x8_t*>(q_lds + 16 * ((2 * c + h) ^ (l32 & 15)));
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      }
      if (!first_group) barrier();
      mfma_phase(0, yes, no);
      barrier();
      if constexpr (kExp) softmax_phase(0, set_ref);
      else max_phase(0);
      barrier();
      if (n_tiles > 1) {
        int j = 1;
        do {
          mfma_phase(j, yes, exp_tag);
          barrier();
          if constexpr (kExp) softmax_phase(j, false);
          else max_phase(j);
          barrier();
        } while (++j < n_tiles);
      }
      if constexpr (kExp) mfma_phase(n_tiles, no, yes);
      if (first_group) barrier();
      barrier();   // every wave is done with the LDS ring before the next loads
    };

    if constexpr (!kExact) {
      sweep(yes, true);
    } else {
      m_run = kNeg;
      sweep(no, false);
      float ma, mb;
      pair_values(m_run, ma, mb);
      m = __builtin_fmaxf(ma, mb);
      sweep(yes, false);
    }

    // ---- epilogue: O / l -> bf16; lane owns channels 32db + 8g + 4h .. +3 of its query row.
    // Written before the overflow vote even on the fast path: when the vote sends the tile to the
    // exact path, that path rewrites every output written here (same threads, program order), and
    // O dies before the vote instead of living (spilled) across the exact path's call.
    float la, lb;
    pair_values(l, la, lb);
    const int row = q0 + l32;
    const Params pe = load_params(kp);   // the output fields, loaded after the sweep
    // Q of the next work item into ring stages 2 and 3 (the sweep's last barrier passed: no wave
    // reads the ring any more): wave wv loads its 32 rows, 4 rows of 256 bytes per direct-to-LDS
    // load, each lane the source chunk that belongs at its LDS position.  Rows past s_q read as
    // zeros (and are never stored).
    bool prefetched = false;
    if constexpr (!kExact) {
      if (next_item >= 0) {
        const int ntile = kSplit ? next_item / pe.split : next_item;
        const int nqt = ntile % pe.q_tiles;
        const int nbh = ntile / pe.q_tiles;
        const int nbb = nbh / pe.heads;
        const int nhh = nbh - nbb * pe.heads;
        const int nq0 = nqt * kBM;
        const unsigned char* nq = reinterpret_cast<const unsigned char*>(pe.q) +
                                  (((int64_t)nbb * pe.s_q + nq0) * pe.heads + nhh) * kHeadDim * 2;
        const u32x4_t qr = rsrc_words32(nq, (unsigned)(pe.s_q - 1 - nq0) * stride32 + kHeadDim * 2);
        const unsigned dst = lds_ring + (unsigned)((2 + (wv >> 2)) * kStageBytes + 32 * (wv & 3) * 256);
        const int sub = lane >> 4, pos = lane & 15;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 32 * wv + 4 * i + sub;   // row of the tile; its row in the stage is r % 128
          dma_b128_nt(qr, dst + 1024 * i, (unsigned)r * stride32 + 16 * (pos ^ (r & 15)));
        }
        prefetched = true;
      }
    }
    if constexpr (kSplit) {   // partial result of this key range (the combining kernel divides)
      if (row < pe.s_q) {
        const int64_t r = (int64_t)item * kBM + wv * 32 + l32;
        float* dst = pe.ws + r * kHeadDim + 4 * h;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4_t x = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
            *reinterpret_cast<f32x4_t*>(dst + 32 * db + 8 * g) = x;
          }
        if (h == 0) {
          const f32x2_t ml = {m, la + lb};
          *reinterpret_cast<f32x2_t*>(pe.ws + (int64_t)pe.total * kBM * kHeadDim + 2 * r) = ml;
        }
      }
    } else {
      const float inv = 1.0f / (la + lb);
      if (row < pe.s_q) {
        // log-sum-exp of the row's scaled scores: m / sqrt(128) + ln(sum of exp2((s - m) log2(e)/sqrt(128))),
        // the sum being >= 1 (the reference row max contributes 1 or more)
        if (pe.lse != nullptr && h == 0)
          pe.lse[((int64_t)bb * pe.heads + hh) * pe.s_q + row] = m * kInvSqrtD + __builtin_amdgcn_logf(la + lb) * kLn2;
      }
      // O rows through LDS (ring stages 0-1, free after the sweep; the vote's barriers separate these
      // reads from the next work item's tile loads there), so that each store writes four whole
      // 256-byte rows instead of 16 bytes of each of 32 rows.  Wave wv stages its 32 rows at
      // 8 KB * wv; the 16-byte chunk k of row r sits at position k ^ (r % 16).
      unsigned char* ost = smem + wv * 8192;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2_t x = {cvt_pk_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                       cvt_pk_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(ost + l32 * 256 + 16 * ((4 * db + g) ^ (l32 & 15)) + 8 * h) = x;
        }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the wave's own rows: no other wave reads them
      {
        const int sub = lane >> 4, pos = lane & 15;
        const int row0 = q0 + sub;
        uint16_t* obase_row = pe.o + (((int64_t)bb * pe.s_q + row0) * pe.heads + hh) * kHeadDim;
        const int64_t row_step = (int64_t)4 * pe.heads * kHeadDim;   // elements between rows 4 apart
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 4 * i + sub;   // row of the wave's 32
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(ost + r * 256 + 16 * pos);
          if (row0 + 4 * i < pe.s_q)
            // non-temporal: O is written once and not read back here
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(obase_row + i * row_step + 8 * (pos ^ (r & 15))));
        }
      }
      if constexpr (kExact) {
        // no vote follows the exact path: every wave has read its staged rows before the next
        // work item loads tiles into these stages
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        barrier();
      }
    }

    if constexpr (!kExact) {   // the overflow vote of the fast path
      const bool over = !(la + lb <= kSumLimit);
      // the ballot in converged code: inside the lane-0 branch it would count lane 0's row only
      const bool wave_over = __any(over);
      if (lane == 0) redo_flag[wv] = wave_over ? 1 : 0;
      // LDS-only synchronisation (lgkmcnt, then the barrier): a __syncthreads() fence would also
      // wait for the O stores just issued
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
      int redo = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) redo |= redo_flag[w];
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();   // every wave has read the flags before they are written again
      if (__builtin_amdgcn_readfirstlane(redo) != 0) return kRedo;
    }
    return prefetched ? kQPrefetched : 0;
  }
}

// The value of lane 0 (the same in every lane), as the compiler's uniform value.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ T* uniform(T* x) {
  const uint64_t u = reinterpret_cast<uint64_t>(x);
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)u);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return reinterpret_cast<T*>((hi << 32) | lo);
}

// The exact path, out of line: it runs only for query tiles whose scores outgrow the first 64
// keys' maximum by far, and keeping its code out of the kernel body keeps the common path's
// register allocation and schedule as they are.  Arguments of a device function arrive in
// VGPRs; both are made uniform again, so that the parameter loads and the buffer descriptors
// stay scalar.
template <bool kSplit>
__device__ __attribute__((noinline)) void attn_tile_exact(kernarg_params_t* kp, int item) {
  attn_tile<true, kSplit>(uniform(kp), uniform(item));
}

template <bool kSplit>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(const Params p) {
  // Persistent, XCD-aware: workgroup w runs on XCD w % 8 and takes work items slot, slot +
  // n_slots, ... of that XCD's contiguous range, so the workgroups of one XCD sweep consecutive
  // query tiles of one head in lockstep and read each K/V tile through their shared L2.
  kernarg_params_t* kp = (kernarg_params_t*)__builtin_amdgcn_kernarg_segment_ptr();
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  bool q_in_lds = false;   // this item's Q was loaded into LDS by the previous one
  // Short key sequences (at most 16 tiles: the text cross-attention): work items are short and all
  // of equal length, so every CU would load Q and store O at the same moments.  The odd slots start
  // about a quarter of a work item late (0.5 us per key tile on the 100 MHz real-time counter; the
  // wait is capped), so that the two halves of the CUs reach their item boundaries at different
  // times.
  if ((slot & 1) && p.split == 1 && p.s_kv <= 16 * kBN) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t d = 50ull * (uint64_t)((p.s_kv + kBN - 1) / kBN);
    for (int it = 0; it < 4096 && __builtin_amdgcn_s_memrealtime() - t0 < d; ++it) __builtin_amdgcn_s_sleep(4);
  }
  for (int t_local = slot; t_local < p.per_xcd; t_local += p.n_slots) {
    const int item = xcd * p.per_xcd + t_local;
    if (item >= p.total) break;
    const int next = (t_local + p.n_slots < p.per_xcd && item + p.n_slots < p.total) ? item + p.n_slots : -1;
    const int r = attn_tile<false, kSplit>(kp, item, next, q_in_lds);
    q_in_lds = (r & kQPrefetched) != 0;
    if (r & kRedo) {
      // the exact path reuses the whole ring: the next item loads its Q from HBM again
      attn_tile_exact<kSplit>(kp, item);
      q_in_lds = false;
    }
  }
}

// Combines the key ranges of a split run: for one query row (one wave, two channels per lane),
// O = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^((m_s - max_s m_s) log2(e)/sqrt(128)), the
// ranges' partial sums brought to a common reference max.  Lane s holds range s's (m, l) (at
// most 64 ranges), so max and sum are wave reductions; the O loads are unrolled to overlap.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, d));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}
__global__ __launch_bounds__(256) void attn_bf16_combine_kernel(const Params p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b*H + h) * s_q + i
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)(p.total / p.split) / p.q_tiles * p.s_q;   // b*H*s_q
  if (row >= rows) return;
  const int64_t bh = row / p.s_q;
  const int i = (int)(row - bh * p.s_q);
  const int64_t first = (bh * p.q_tiles + i / kBM) * p.split * kBM + i % kBM;   // range 0's row
  const float* ml = p.ws + (int64_t)p.total * kBM * kHeadDim;
  f32x2_t mine = {kNeg, 0.0f};
  if (lane < p.split) mine = *reinterpret_cast<const f32x2_t*>(ml + 2 * (first + (int64_t)lane * kBM));
  const float mx = wave_max(mine[0]);
  const float w = lane < p.split ? __builtin_amdgcn_exp2f((mine[0] - mx) * kScaleLog2) : 0.0f;
  const float total_l = wave_sum(w * mine[1]);
  const float inv = 1.0f / total_l;
  float a0 = 0.0f, a1 = 0.0f;
  // in groups of 8 ranges, the group's loads in flight together (the shuffles are convergent, so
  // the compiler does not unroll a loop of unknown trip count around them itself)
  for (int sp0 = 0; sp0 < p.split; sp0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = sp0 + u;
      const float ws = __shfl(w, sp & 63);
      if (sp < p.split) {
        const f32x2_t x = *reinterpret_cast<const f32x2_t*>(p.ws + (first + (int64_t)sp * kBM) * kHeadDim + 2 * lane);
        a0 += ws * x[0];
        a1 += ws * x[1];
      }
    }
  }
  const int64_t bb = bh / p.heads, hh = bh - bb * p.heads;
  *reinterpret_cast<unsigned*>(p.o + ((bb * p.s_q + i) * p.heads + hh) * kHeadDim + 2 * lane) =
      cvt_pk_bf16(a0 * inv, a1 * inv);
  if (p.lse != nullptr && lane == 0) p.lse[row] = mx * kInvSqrtD + __builtin_amdgcn_logf(total_l) * kLn2;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

Params make_params(const void* q, const void* k, const void* v, void* o, const AttnShape& sh, int split,
                   void* ws, float* lse) {
  Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.heads = (int)sh.heads;
  p.s_q = (int)sh.s_q;
  p.s_kv = (int)sh.s_kv;
  p.q_tiles = (int)ceil_div(sh.s_q, kBM);
  const int n_kt = (int)ceil_div(sh.s_kv, kBN);
  p.split = split;
  p.split_tiles = (int)ceil_div(n_kt, split);
  p.ws = static_cast<float*>(ws);
  p.lse = lse;
  p.total = (int)(p.q_tiles * sh.batch * sh.heads * split);
  p.per_xcd = (int)ceil_div(p.total, 8);
  // one workgroup per CU (the LDS ring and the registers allow no second one)
  const int cus = device_cus();
  p.n_slots = (int)(p.per_xcd < cus / 8 ? p.per_xcd : cus / 8);
  return p;
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            const AttnShape& sh, hipStream_t stream) {
  const Params p = make_params(q, k, v, o, sh, 1, nullptr, lse);
  hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, dim3((unsigned)(8 * p.n_slots)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

int attn_bf16_split(const AttnShape& sh) {
  // Too few query tiles to fill the chip: split each tile's keys into ranges of >= 2 tiles, aiming
  // at about two work items per CU.
  const int64_t tiles = ceil_div(sh.s_q, kBM) * sh.batch * sh.heads;
  const int64_t n_kt = ceil_div(sh.s_kv, kBN);
  const int64_t cus = device_cus();
  if (2 * tiles > cus || n_kt < 4) return 1;
  int64_t split = ceil_div(2 * cus, tiles);
  if (split > n_kt / 2) split = n_kt / 2;
  if (split > 64) split = 64;   // one wave combines all ranges of a row
  if (split < 2) return 1;
  return (int)ceil_div(n_kt, ceil_div(n_kt, split));   // no empty range
}

size_t attn_bf16_split_bytes(const AttnShape& sh, int split) {
  const int64_t items = ceil_div(sh.s_q, kBM) * sh.batch * sh.heads * split;
  return (size_t)items * kBM * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attn_bf16_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const AttnShape& sh, int split, void* ws, hipStream_t stream) {
  const Params p = make_params(q, k, v, o, sh, split, ws, lse);
  hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, dim3((unsigned)(8 * p.n_slots)), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = sh.batch * sh.heads * sh.s_q;
  hipLaunchKernelGGL(attn_bf16_combine_kernel, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
