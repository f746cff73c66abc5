// FP8 GEMM of the DiT linear layers for gfx950 (MI355X): Y = X W^T with e4m3fn operands, the
// activations X [M, K] quantised per token (row) and the weights W [N, K] per tensor, FP32
// accumulation on the matrix cores, Y [M, N] bf16 = (X~ W~^T) * scale_x[m] * scale_w.  The
// explainer of the Wan report ("Wan模型是什么它能做什么", section 4.2) runs every matrix
// multiplication of the linear layers in FP8 with exactly this split of scales (weights per
// tensor, activations per token); the quantisation rule itself (e4m3fn, scale = amax / 448,
// saturating round to nearest even) is the one of this library's 8-bit attention.
//
// Kernels:
//  * fp8_quant_rows_kernel -- one wave per row: amax, then codes = e4m3fn(clamp(x * 448/amax));
//    rows of up to 8,192 values are held in registers between the two (fp8_quant_rows_reg_kernel).
//  * fp8_amax_kernel, fp8_quant_tensor_kernel, fp8_finish_scale_kernel -- the per-tensor path:
//    the tensor's amax by an atomic max on the float bits (order-independent), the codes, and the
//    scale, all through the caller's scale word.
//  * fp8_gemm_kernel -- one workgroup = 8 waves = a 256 (tokens) x 256 (features) tile of Y.
//    The product runs transposed, Y^T = W~ X~^T with v_mfma_f32_16x16x128_f8f6f4 (A = 16 feature
//    rows of W~, B = 16 token rows of X~, 32 consecutive K bytes per lane each), so that a lane's
//    accumulators hold one token and 4 consecutive features per 16 x 16 block: the epilogue scales
//    them by scale_x[token] * scale_w and stores 4 bf16 at a time.  Wave (wm, wn) computes tokens
//    64 wm .. +63 and features 128 wn .. +127 (8 x 4 accumulators of 16 x 16).  One MFMA step
//    covers 128 K bytes: the step's W~ and X~ tiles (256 rows x 128 bytes each) stream from HBM
//    straight into a 5-slot LDS ring of operand tiles (buffer_load ... lds, 8 lanes per 128-byte
//    row, so every row is one whole line), one to two steps ahead, rows past M or N reading as
//    zeros.  Chunk c of tile row r sits at chunk c ^ swz(r), which keeps the operand reads free of
//    bank conflicts (the LDS serves the 16 lanes of a half-wave whose bits 2, 3 and 4 have the same
//    parity together; measured, not documented).  Persistent (one workgroup per CU) and XCD-aware:
//    the 32 CUs of one XCD share 4 token tiles and 8 feature tiles in their L2, and each workgroup
//    loads its next tile's first operand tiles behind its stores.

#include <type_traits>

#include "wan_attn_internal.h"

namespace wan {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr unsigned kRsrcFlags = 0x00020000u;   // raw buffer, 32-bit dwords
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ void unpack8(u32x4_t raw, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xffff0000u);
  }
}

// Four values -> four e4m3fn codes (saturating: clamped to +-448 first; round to nearest even).
__device__ __forceinline__ unsigned fp8x4(float a, float b, float c, float d) {
  const float lim = kE4m3Max;
  a = fminf(fmaxf(a, -lim), lim);
  b = fminf(fmaxf(b, -lim), lim);
  c = fminf(fmaxf(c, -lim), lim);
  d = fminf(fmaxf(d, -lim), lim);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// codes of 8 bf16 values (one 16-byte load) against inv -> 8 bytes
__device__ __forceinline__ u32x2_t quant8(u32x4_t raw, float inv) {
  float f[8];
  unpack8(raw, f);
  u32x2_t r;
  r[0] = fp8x4(__fmul_rn(f[0], inv), __fmul_rn(f[1], inv), __fmul_rn(f[2], inv), __fmul_rn(f[3], inv));
  r[1] = fp8x4(__fmul_rn(f[4], inv), __fmul_rn(f[5], inv), __fmul_rn(f[6], inv), __fmul_rn(f[7], inv));
  return r;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}

// ---------------------------------------------------------------------------------------------
// Per-token quantisation: one wave per row of x [rows][cols] (cols a multiple of 64).
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const uint16_t* x, int64_t rows, int cols,
                                                             uint8_t* codes, float* scales) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;   // whole waves leave together
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + row * cols);
  const int chunks = cols / 8;
  float amax = 0.0f;
  for (int c = lane; c < chunks; c += 64) {
    float f[8];
    unpack8(src[c], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  const float inv = amax > 0.0f ? __fdiv_rn(kE4m3Max, amax) : 1.0f;
  if (lane == 0) scales[row] = amax > 0.0f ? __fdiv_rn(amax, kE4m3Max) : 1.0f;
  u32x2_t* dst = reinterpret_cast<u32x2_t*>(codes + row * cols);
  for (int c = lane; c < chunks; c += 64) dst[c] = quant8(src[c], inv);
}

// The same for rows of at most 64 * kPer * 8 values: the row is read from HBM once into registers
// (kPer 16-byte chunks per lane, loads issued together), then its amax and its codes.
template <int kPer>
__global__ __launch_bounds__(256) void fp8_quant_rows_reg_kernel(const uint16_t* x, int64_t rows, int cols,
                                                                 uint8_t* codes, float* scales) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;   // whole waves leave together
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + row * cols);
  const int chunks = cols / 8;
  u32x4_t v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k;
    v[k] = c < chunks ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    float f[8];
    unpack8(v[k], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  const float inv = amax > 0.0f ? __fdiv_rn(kE4m3Max, amax) : 1.0f;
  if (lane == 0) scales[row] = amax > 0.0f ? __fdiv_rn(amax, kE4m3Max) : 1.0f;
  u32x2_t* dst = reinterpret_cast<u32x2_t*>(codes + row * cols);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int c = lane + 64 * k;
    if (c < chunks) dst[c] = quant8(v[k], inv);
  }
}
constexpr int kQuantRegChunks = 16;   // rows of up to 8,192 values take the register path

// ---------------------------------------------------------------------------------------------
// Per-tensor quantisation.  The caller's scale word first collects the bits of the tensor's amax
// (non-negative floats order like their bit patterns), then receives the scale.
__global__ void fp8_clear_kernel(unsigned* word) { *word = 0u; }

__global__ __launch_bounds__(256) void fp8_amax_kernel(const uint16_t* w, int64_t chunks, unsigned* amax_bits) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w);
  float amax = 0.0f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
    float f[8];
    unpack8(src[c], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __builtin_bit_cast(unsigned, amax));
}

__global__ __launch_bounds__(256) void fp8_quant_tensor_kernel(const uint16_t* w, int64_t chunks, uint8_t* codes,
                                                               const unsigned* amax_bits) {
  const float amax = __builtin_bit_cast(float, *amax_bits);
  const float inv = amax > 0.0f ? __fdiv_rn(kE4m3Max, amax) : 1.0f;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w);
  u32x2_t* dst = reinterpret_cast<u32x2_t*>(codes);
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256)
    dst[c] = quant8(src[c], inv);
}

__global__ void fp8_finish_scale_kernel(unsigned* word) {
  const float amax = __builtin_bit_cast(float, *word);
  *reinterpret_cast<float*>(word) = amax > 0.0f ? __fdiv_rn(amax, kE4m3Max) : 1.0f;
}

// ---------------------------------------------------------------------------------------------
// GEMM.
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kTM = 256;                 // tokens per workgroup tile
constexpr int kTN = 256;                 // features per workgroup tile
constexpr int kTK = 128;                 // K bytes per step (one MFMA step)
constexpr int kTileBytes = 256 * kTK;    // 32 KB per operand tile = one ring slot
constexpr int kSlots = 5;                // 160 KB of LDS
constexpr int kLoadsPerSlot = 4;         // direct-to-LDS loads per wave per slot
constexpr int kGroupM = 4;               // token tiles per group of consecutive work items

struct GemmParams {
  const uint8_t* x;       // [m][k] codes
  const float* xs;        // [m]
  const uint8_t* w;       // [n][k] codes
  const float* ws;        // [1]
  uint16_t* y;            // [m][n] bf16
  int64_t m, n;
  int k;
  int tiles_m, tiles_n, total, per_xcd, n_slots;
};

// 16-byte chunk c of tile row r sits at chunk c ^ swz(r) of the row's 128 bytes
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) * 1) ^ (((r >> 3) & 1) * 4); }

__device__ __forceinline__ u32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const unsigned nr = bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (unsigned)bytes);
  const u32x4_t r = {(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, nr, kRsrcFlags};
  return r;
}

// Direct global -> LDS load of 16 bytes per lane to lds_addr + 16 * lane from byte voff + soff of
// the buffer (offsets past the buffer's size read as zeros).  Inline asm: the compiler would otherwise
// wait for each of these loads before the next LDS read; the kernel waits for them itself
// (s_waitcnt vmcnt).
__device__ __forceinline__ void dma_b128(u32x4_t rsrc, unsigned lds_addr, unsigned voff, unsigned soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr), "s"(soff));
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__global__ __launch_bounds__(kGThreads, 1) void fp8_gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSlots * kTileBytes];
  // Persistent and XCD-aware: workgroup b runs on XCD b % 8 and takes work items (b % 8) * per_xcd +
  // b / 8 + i * n_slots of that XCD's contiguous range; items run token-tile-major in groups of
  // kGroupM token tiles, so the workgroups of one XCD share a few X and W tiles in L2.  The next
  // item's first five operand tiles are loaded at the end of each item, after its stores.
  const int xcd = blockIdx.x & 7;
  const int slot_id = blockIdx.x >> 3;
  auto item_tiles = [&](int t, int& mt, int& nt) __attribute__((always_inline)) {
    const int group = t / (kGroupM * p.tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(kGroupM, p.tiles_m - first_m);
    const int in_group = t - group * kGroupM * p.tiles_n;
    mt = first_m + in_group % gm;
    nt = in_group / gm;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int l16 = lane & 15, g = lane >> 4;
  const int K = p.k;
  const unsigned lds = (unsigned)(uintptr_t)(lds_void_t*)smem;

  // Loads.  The ring holds operand tiles: tile u = 2 s + o is step s's W~ tile (o = 0) or X~ tile
  // (o = 1), K bytes 128 s .. 128 s + 127 of 256 rows, in slot u % 5.  Wave wv writes 1 KB blocks
  // 4wv .. 4wv+3 of a tile (8 rows of 128 bytes per block), 8 lanes per row, lane i fetching the
  // logical chunk that belongs at physical chunk i % 8 of its row, so that the 8 lanes of a row read
  // one whole 128-byte line.  One descriptor per operand over its valid rows (rows past m or n read
  // as zeros); the K position is the scalar offset.  When k is an odd multiple of 64, the lanes of
  // the last step's upper 64 bytes point past the descriptor and read zeros.
  auto w_rsrc = [&](int nt) __attribute__((always_inline)) {
    const int64_t n0 = (int64_t)nt * kTN;
    return rsrc_words(p.w + n0 * K, min((int64_t)kTN, p.n - n0) * K);
  };
  auto x_rsrc = [&](int mt) __attribute__((always_inline)) {
    const int64_t m0 = (int64_t)mt * kTM;
    return rsrc_words(p.x + m0 * K, min((int64_t)kTM, p.m - m0) * K);
  };
  unsigned src_off[4];
  bool upper[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = 8 * (4 * wv + it) + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    src_off[it] = (unsigned)(row * K + 16 * chunk);
    upper[it] = chunk >= 4;
  }
  const int n_steps = (K + kTK - 1) / kTK;
  const int n_tiles = 2 * n_steps;
  const bool half_last = (K % kTK) != 0;
  auto issue_block_of = [&](const u32x4_t& wr, const u32x4_t& xr, int u, int it) __attribute__((always_inline)) {
    const int s = u >> 1;
    const u32x4_t rs = (u & 1) ? xr : wr;
    const unsigned koff = (unsigned)(s * kTK);
    const unsigned st = lds + (unsigned)((u % kSlots) * kTileBytes);
    const bool cut = half_last && s == n_steps - 1;
    dma_b128(rs, st + 1024 * (4 * wv + it), (cut && upper[it]) ? 0x80000000u : src_off[it], koff);
  };
  auto issue_of = [&](const u32x4_t& wr, const u32x4_t& xr, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 4; ++it) issue_block_of(wr, xr, u, it);
  };

  // Operands of v_mfma_f32_16x16x128_f8f6f4: a lane feeds row l16 of a 16-row block and the 32
  // K bytes 32 g .. 32 g + 31 of the step (logical chunks 2g, 2g+1).  A = 16 feature rows of W~,
  // B = 16 token rows of X~.  With the swizzle above, the 16 lanes the LDS serves together (one
  // half-wave, lanes whose bits 2, 3, 4 have the same parity) hit 16 distinct bank groups.
  const unsigned lane_off0 = (unsigned)(l16 * kTK + 16 * ((2 * g) ^ swz(l16)));
  const unsigned lane_off1 = (unsigned)(l16 * kTK + 16 * ((2 * g + 1) ^ swz(l16)));
  auto read_op = [&](unsigned base, int row0) __attribute__((always_inline)) {
    const unsigned char* p0 = smem + base + row0 * kTK;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(p0 + lane_off0);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(p0 + lane_off1);
    const i32x8_t r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
  };
  auto slot = [](int u) { return (unsigned)((u % kSlots) * kTileBytes); };
  // W rows 128 wn + 16 fi + l16 of slot 2s; X rows 64 wm + 16 ti + l16 of slot 2s+1
  auto read_a = [&](int s, int fi) __attribute__((always_inline)) { return read_op(slot(2 * s), 128 * wn + 16 * fi); };
  auto read_b = [&](int s, int ti) __attribute__((always_inline)) { return read_op(slot(2 * s + 1), 64 * wm + 16 * ti); };

  typedef __attribute__((ext_vector_type(4))) float f32x4_t;
  bool prefetched = false;   // this item's first operand tiles were loaded by the previous item
  for (int t_local = slot_id; t_local < p.per_xcd; t_local += p.n_slots) {
  const int t = xcd * p.per_xcd + t_local;
  if (t >= p.total) break;
  int mt, nt;
  item_tiles(t, mt, nt);
  const int64_t m0 = (int64_t)mt * kTM, n0 = (int64_t)nt * kTN;
  const u32x4_t wr = w_rsrc(nt), xr = x_rsrc(mt);
  auto issue_block = [&](int u, int it) __attribute__((always_inline)) { issue_block_of(wr, xr, u, it); };
  auto issue = [&](int u) __attribute__((always_inline)) { issue_of(wr, xr, u); };
  f32x4_t acc[8][4];
#pragma unroll
  for (int fi = 0; fi < 8; ++fi)
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) acc[fi][ti] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Pipeline over steps s (tiles 2s, 2s+1).  Tiles 0..4 are loaded up front; the rest two per step,
  // into the slots step s has finished reading: tile 2s+5 (-> slot of 2s) right after the barrier M_s
  // in the middle of step s, tile 2s+6 (-> slot of 2s+1, needed two steps later) spread over the rows
  // of step s+1, so that no wave issues all of a step's loads in one burst (a burst of 8 measured 6%
  // slower).  Before M_s every wave has waited for its own loads of tiles 2s+2, 2s+3 (only those of
  // 2s+4, all issued during step s, may still be in flight) and for its own operand reads of step s;
  // after it, it reads step s+1's B operands and first A.
  if (!prefetched)
    for (int u = 0; u < min(kSlots, n_tiles); ++u) issue(u);
  // tiles 0 and 1 landed; n_tiles is even, so 0, 2 or 3 tiles may still be in flight (the previous
  // item's stores, issued before these loads, only make the count larger)
  if (n_tiles >= kSlots) __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * kLoadsPerSlot));
  else if (n_tiles == 4) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kLoadsPerSlot));
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  barrier();
  i32x8_t bop[4], aop[2];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) bop[ti] = read_b(0, ti);
  aop[0] = read_a(0, 0);
  int pend = -1;   // tile whose loads are spread over the rows of this step
  for (int s = 0; s < n_steps; ++s) {
#pragma unroll
    for (int fi = 0; fi < 7; ++fi) {
      // the 4 loads of the tile issued last are spread over rows 1, 3, 5, 6 of the next step
      constexpr int kSpread[7] = {-1, 0, -1, 1, -1, 2, 3};
      if (kSpread[fi] >= 0 && pend >= 0) issue_block(pend, kSpread[fi]);
      aop[(fi + 1) & 1] = read_a(s, fi + 1);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        acc[fi][ti] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[fi & 1], bop[ti], acc[fi][ti], 0, 0, 0, 0,
                                                                       0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // M_s
    if (s + 1 < n_steps && 2 * s + 4 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsPerSlot);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's reads of step s are done
    barrier();
    if (2 * s + 5 < n_tiles) issue(2 * s + 5);
    pend = 2 * s + 6 < n_tiles ? 2 * s + 6 : -1;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      acc[7][ti] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop[1], bop[ti], acc[7][ti], 0, 0, 0, 0, 0, 0);
      // (after the last step this reads a stale slot whose values go unused: no branch around it)
      bop[ti] = read_b(s + 1, ti);
    }
    aop[0] = read_a(s + 1, 0);
  }

  // Epilogue: lane owns token m0 + 64 wm + 16 ti + l16 and features n0 + 128 wn + 16 fi + 4 g .. +3
  const float sw = *p.ws;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    const int64_t m = m0 + 64 * wm + 16 * ti + l16;
    if (m >= p.m) continue;
    const float sc = p.xs[m] * sw;
    uint16_t* yrow = p.y + m * p.n;
#pragma unroll
    for (int fi = 0; fi < 8; ++fi) {
      const int64_t n = n0 + 128 * wn + 16 * fi + 4 * g;
      if (n >= p.n) continue;
      bf16x2_t a, c;
      a[0] = (__bf16)(acc[fi][ti][0] * sc);
      a[1] = (__bf16)(acc[fi][ti][1] * sc);
      c[0] = (__bf16)(acc[fi][ti][2] * sc);
      c[1] = (__bf16)(acc[fi][ti][3] * sc);
      const u32x2_t v = {__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, c)};
      *reinterpret_cast<u32x2_t*>(yrow + n) = v;
    }
  }
  // The next item's first operand tiles, after this item's stores (so that the next item's counted
  // waits for them stay exact).  Every wave finished its reads of this item's operands before the
  // barrier of the last step (what it read after that was a stale slot, unused).
  prefetched = false;
  if (t_local + p.n_slots < p.per_xcd && t + p.n_slots < p.total) {
    int nmt, nnt;
    item_tiles(t + p.n_slots, nmt, nnt);
    const u32x4_t nwr = w_rsrc(nnt), nxr = x_rsrc(nmt);
    for (int u = 0; u < min(kSlots, n_tiles); ++u) issue_of(nwr, nxr, u);
    prefetched = true;
  }
  }
}

}  // namespace

hipError_t launch_fp8_quantize_rows(const void* x, int64_t rows, int64_t cols, void* codes, float* scales,
                                    hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(rows, 4));
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  uint8_t* cs = static_cast<uint8_t*>(codes);
  const int64_t per = ceil_div(cols / 8, 64);   // 16-byte chunks per lane
  if (per <= 2)
    hipLaunchKernelGGL(fp8_quant_rows_reg_kernel<2>, grid, dim3(256), 0, stream, xs, rows, (int)cols, cs, scales);
  else if (per <= 4)
    hipLaunchKernelGGL(fp8_quant_rows_reg_kernel<4>, grid, dim3(256), 0, stream, xs, rows, (int)cols, cs, scales);
  else if (per <= 8)
    hipLaunchKernelGGL(fp8_quant_rows_reg_kernel<8>, grid, dim3(256), 0, stream, xs, rows, (int)cols, cs, scales);
  else if (per <= kQuantRegChunks)
    hipLaunchKernelGGL(fp8_quant_rows_reg_kernel<kQuantRegChunks>, grid, dim3(256), 0, stream, xs, rows, (int)cols,
                       cs, scales);
  else
    hipLaunchKernelGGL(fp8_quant_rows_kernel, grid, dim3(256), 0, stream, xs, rows, (int)cols, cs, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_tensor(const void* w, int64_t rows, int64_t cols, void* codes, float* scale,
                                      hipStream_t stream) {
  unsigned* word = reinterpret_cast<unsigned*>(scale);
  const int64_t chunks = rows * cols / 8;
  const int64_t blocks = ceil_div(chunks, 256);
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(fp8_clear_kernel, dim3(1), dim3(1), 0, stream, word);
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint16_t*>(w), chunks, word);
  hipLaunchKernelGGL(fp8_quant_tensor_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint16_t*>(w),
                     chunks, static_cast<uint8_t*>(codes), word);
  hipLaunchKernelGGL(fp8_finish_scale_kernel, dim3(1), dim3(1), 0, stream, word);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const void* x_codes, const float* x_scales, const void* w_codes, const float* w_scale,
                           void* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  GemmParams p;
  p.x = static_cast<const uint8_t*>(x_codes);
  p.xs = x_scales;
  p.w = static_cast<const uint8_t*>(w_codes);
  p.ws = w_scale;
  p.y = static_cast<uint16_t*>(y);
  p.m = m;
  p.n = n;
  p.k = (int)k;
  p.tiles_m = (int)ceil_div(m, kTM);
  p.tiles_n = (int)ceil_div(n, kTN);
  p.total = p.tiles_m * p.tiles_n;
  p.per_xcd = (int)ceil_div(p.total, 8);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 8)
    cus = 256;
  p.n_slots = p.per_xcd < cus / 8 ? p.per_xcd : cus / 8;   // one workgroup per CU
  hipLaunchKernelGGL(fp8_gemm_kernel, dim3((unsigned)(8 * p.n_slots)), dim3(kGThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
