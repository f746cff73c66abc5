// FP8 GEMM of the DiT linear layers for gfx950 (MI355X): Y = X W^T with e4m3fn operands, the
// activations X [M, K] quantised per token (row) and the weights W [N, K] per tensor, FP32
// accumulation on the matrix cores, Y [M, N] bf16 = (X~ W~^T) * scale_x[m] * scale_w.  The
// explainer of the Wan report ("Wan模型是什么它能做什么", section 4.2) runs every matrix
// multiplication of the linear layers in FP8 with exactly this split of scales (weights per
// tensor, activations per token); the quantisation rule itself (e4m3fn, scale = amax / 448,
// saturating round to nearest even) is the one of this library's 8-bit attention.
//
// Kernels:
//  * fp8_quant_rows_kernel -- one wave per row: amax, then codes = e4m3fn(clamp(x * 448/amax)).
//  * fp8_amax_kernel, fp8_quant_tensor_kernel, fp8_finish_scale_kernel -- the per-tensor path:
//    the tensor's amax by an atomic max on the float bits (order-independent), the codes, and the
//    scale, all through the caller's scale word.
//  * fp8_gemm_kernel -- one workgroup = 8 waves = a 256 (tokens) x 256 (features) tile of Y.
//    The product runs transposed, Y^T = W~ X~^T with v_mfma_f32_32x32x64_f8f6f4 (A = 32 feature
//    rows of W~, B = 32 token rows of X~, 32 consecutive K bytes per lane each), so that a lane's
//    accumulators hold one token and 4 consecutive features per group: the epilogue scales them
//    by scale_x[token] * scale_w and stores 4 bf16 at a time.  Wave (wm, wn) computes tokens
//    64 wm .. +63 and features 128 wn .. +127 (4 x 2 accumulators of 32 x 32).  W~ and X~ tiles of
//    64 K bytes stream from HBM straight into a 5-stage LDS ring (buffer_load ... lds), four
//    stages ahead, rows past M or N reading as zeros; each step's operands are read into
//    registers during the step before (two register sets); 16-byte chunk c of tile row r sits at chunk
//    c ^ sigma(r), sigma(r) = ((r >> 1) ^ (r >> 2)) & 3, so that the operand reads (16 rows, one
//    chunk, per 16 lanes; or 8 rows per 8 lanes) hit distinct banks.  Workgroups are numbered so
//    that the 32 CUs of one XCD share 4 token tiles and 8 feature tiles in their L2.

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
constexpr int kTK = 64;                  // K bytes per stage (one MFMA step)
constexpr int kTileBytes = 256 * kTK;    // 16 KB per operand tile
constexpr int kStage = 2 * kTileBytes;   // [W | X]
constexpr int kStages = 5;               // 160 KB of LDS
constexpr int kLoadsPerStage = 4;        // direct-to-LDS loads per wave per stage
constexpr int kGroupM = 4;               // token tiles per group of consecutive work items

struct GemmParams {
  const uint8_t* x;       // [m][k] codes
  const float* xs;        // [m]
  const uint8_t* w;       // [n][k] codes
  const float* ws;        // [1]
  uint16_t* y;            // [m][n] bf16
  int64_t m, n;
  int k;
  int tiles_m, tiles_n, total, per_xcd;
};

__device__ __forceinline__ int sigma4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ u32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const unsigned nr = bytes <= 0 ? 0u : (bytes >= 0x7fffffffLL ? 0x7fffffffu : (unsigned)bytes);
  const u32x4_t r = {(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, nr, kRsrcFlags};
  return r;
}

// Direct global -> LDS load of 16 bytes per lane to lds_addr + 16 * lane from byte voff + soff of
// the buffer (rows past the buffer's end read as zeros).  Inline asm: the compiler would otherwise
// wait for each of these loads before the next LDS read; the kernel waits for them itself
// (s_waitcnt vmcnt, counted).
__device__ __forceinline__ void dma_b128(u32x4_t rsrc, unsigned lds_addr, unsigned voff, unsigned soff) {
  asm volatile("buffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr), "s"(soff));
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__global__ __launch_bounds__(kGThreads, 1) void fp8_gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStage];
  // XCD-aware numbering: workgroup b runs on XCD b % 8 and takes work item (b % 8) * per_xcd +
  // b / 8; items run token-tile-major in groups of kGroupM token tiles, so the workgroups of one
  // XCD share a few X and W tiles in L2.
  const int b = blockIdx.x;
  const int t = (b & 7) * p.per_xcd + (b >> 3);
  if (t >= p.total) return;
  const int group = t / (kGroupM * p.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(kGroupM, p.tiles_m - first_m);
  const int in_group = t - group * kGroupM * p.tiles_n;
  const int mt = first_m + in_group % gm;
  const int nt = in_group / gm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)mt * kTM, n0 = (int64_t)nt * kTN;
  const int K = p.k;
  const unsigned lds = (unsigned)(uintptr_t)(lds_void_t*)smem;

  // loads: wave wv writes 1 KB blocks 2wv, 2wv+1 of each 16 KB tile (16 rows of 64 bytes per
  // block); lane i fetches the logical chunk that belongs at physical chunk i % 4 of its row
  // one descriptor per operand tile, over its valid rows (rows past m or n read as zeros: their
  // offset row * K + chunk is past valid rows * K); the K position of a stage is the scalar offset
  const u32x4_t wr = rsrc_words(p.w + n0 * K, min((int64_t)kTN, p.n - n0) * K);
  const u32x4_t xr = rsrc_words(p.x + m0 * K, min((int64_t)kTM, p.m - m0) * K);
  unsigned src_off[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int row = 16 * (2 * wv + it) + (lane >> 2);
    src_off[it] = (unsigned)(row * K + 16 * ((lane & 3) ^ sigma4(row)));
  }
  const int n_k = K / kTK;
  auto issue = [&](int kk) __attribute__((always_inline)) {
    const unsigned koff = (unsigned)(kk * kTK);
    const unsigned st = lds + (unsigned)((kk % kStages) * kStage);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      dma_b128(wr, st + 1024 * (2 * wv + it), src_off[it], koff);
      dma_b128(xr, st + kTileBytes + 1024 * (2 * wv + it), src_off[it], koff);
    }
  };
  // wait until the stage issued before the last `after` stages has landed
  auto wait_stage = [&](int after) __attribute__((always_inline)) {
    if (after >= 3) __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * kLoadsPerStage));
    else if (after == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kLoadsPerStage));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | kLoadsPerStage);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  // operand read offsets: row r, bytes 32h .. 32h+31 = logical chunks 2h and 2h+1
  int aoff[4][2], boff[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
      const int r = 128 * wn + 32 * fi + l32;
      aoff[fi][e] = r * kTK + 16 * ((2 * h + e) ^ sigma4(r));
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int r = 64 * wm + 32 * ti + l32;
      boff[ti][e] = kTileBytes + r * kTK + 16 * ((2 * h + e) ^ sigma4(r));
    }
  }
  auto read8 = [&](const unsigned char* st, const int (&off)[2]) __attribute__((always_inline)) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(st + off[0]);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(st + off[1]);
    const i32x8_t r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return r;
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fi][ti][r] = 0.0f;

  // Pipeline: stage s is loaded at step s - 4 (into the slot of stage s - 5, whose operands every
  // wave read during step s - 6 and fed to its MFMAs during step s - 5), waited for at step s - 1,
  // when its operands are read into registers, and multiplied at step s.  The barrier of step kk
  // comes after every wave's MFMAs of step kk - 1.
  i32x8_t aop[2][4], bop[2][2];
  auto read_ops = [&](int kk, int buf) __attribute__((always_inline)) {
    const unsigned char* st = smem + (kk % kStages) * kStage;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) bop[buf][ti] = read8(st, boff[ti]);
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) aop[buf][fi] = read8(st, aoff[fi]);
  };
  for (int s0 = 0; s0 < 4; ++s0)
    if (s0 < n_k) issue(s0);
  wait_stage(min(n_k - 1, 3));
  barrier();
  read_ops(0, 0);
  // one step; the register set is a compile-time index (the loop runs two steps per iteration)
  auto step = [&](int kk, auto cur_tag) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_tag)::value;
    if (kk + 1 < n_k) wait_stage(min(n_k - 2 - kk, 2));
    barrier();   // stage kk+1 has landed everywhere; every wave is done with step kk-1
    if (kk + 4 < n_k) issue(kk + 4);
    // (on the last step this reads a stale slot whose values go unused: no branch around the reads)
    read_ops(kk + 1, cur ^ 1);
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
        acc[fi][ti] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop[cur][fi], bop[cur][ti], acc[fi][ti], 0, 0,
                                                                       0, 0, 0, 0);
    // the next step's 12 operand reads spread between these 8 MFMAs (one MFMA, two reads), not
    // issued as one burst that fills the LDS queue while the matrix core waits for this wave
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };
  for (int kk = 0; kk < n_k; kk += 2) {
    step(kk, std::integral_constant<int, 0>{});
    if (kk + 1 < n_k) step(kk + 1, std::integral_constant<int, 1>{});
  }

  // epilogue: lane owns token m0 + 64 wm + 32 ti + l32 and features n0 + 128 wn + 32 fi + 8 g + 4 h .. +3
  const float sw = *p.ws;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int64_t m = m0 + 64 * wm + 32 * ti + l32;
    if (m >= p.m) continue;
    const float s = p.xs[m] * sw;
    uint16_t* yrow = p.y + m * p.n;
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + 128 * wn + 32 * fi + 8 * g + 4 * h;
        if (n >= p.n) continue;
        bf16x2_t a, c;
        a[0] = (__bf16)(acc[fi][ti][4 * g] * s);
        a[1] = (__bf16)(acc[fi][ti][4 * g + 1] * s);
        c[0] = (__bf16)(acc[fi][ti][4 * g + 2] * s);
        c[1] = (__bf16)(acc[fi][ti][4 * g + 3] * s);
        const u32x2_t v = {__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, c)};
        *reinterpret_cast<u32x2_t*>(yrow + n) = v;
      }
  }
}

}  // namespace

hipError_t launch_fp8_quantize_rows(const void* x, int64_t rows, int64_t cols, void* codes, float* scales,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(fp8_quant_rows_kernel, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), rows, (int)cols, static_cast<uint8_t*>(codes), scales);
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
  hipLaunchKernelGGL(fp8_gemm_kernel, dim3((unsigned)(8 * p.per_xcd)), dim3(kGThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace wan
