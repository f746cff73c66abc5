// Sustained matrix-core rate of gfx950 under its power limit: a measurement kernel, not part of the
// attention library.  One workgroup of 4 waves per compute unit, one wave per SIMD; every wave issues
// a long stream of independent MFMAs whose operands come from registers and change from one
// instruction to the next (random data from the caller, four operand sets in rotation), so the
// matrix core runs as busy as the instruction stream allows and the chip settles at the clock its
// power limit gives that load.  The rate it reaches is the practical ceiling of any kernel built
// from the same instruction.
//
// libwan_mfma_ceiling.so exports
//   int wan_mfma_ceiling_run(int kind, const void* operands, float* out, int n_workgroups,
//                            int iters, hipStream_t stream);
// kind: 0 = v_mfma_f32_32x32x16_bf16, 1 = v_mfma_f32_16x16x32_bf16, 2 = v_mfma_f32_32x32x64_f8f6f4
// (e4m3 operands), 3 = v_mfma_i32_32x32x32_i8, 4 = v_mfma_f32_16x16x128_f8f6f4 (e4m3),
// 5 = v_mfma_i32_16x16x64_i8.  operands: device buffer of 64 lanes x 8 x 32 bytes
// (16 KiB), read once per wave.  out: device buffer of n_workgroups * 4 floats, written with a sum
// of each wave's accumulators (keeps the work alive).  96 KiB of LDS per workgroup keeps one workgroup per
// compute unit.  Per wave and iteration the kernel issues
// 8 MFMAs of kinds 0, 2, 3 and 16 of kinds 1, 4, 5, i.e. 8 * 32768, 16 * 16384, 8 * 131072, 8 * 65536,
// 16 * 65536, 16 * 32768 operations.  Returns 0, or 1 on a bad argument, or 2 when the launch fails.

#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

constexpr int kWaves = 4;

template <int Kind>
__global__ __launch_bounds__(256, 1) void mfma_ceiling_kernel(const i32x8_t* __restrict__ operands,
                                                              float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // 8 operand registers of 32 bytes per lane: sets 0-3 feed A, 4-7 feed B
  i32x8_t r[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = operands[lane * 8 + s];
  float sum = 0.f;
  if constexpr (Kind == 0 || Kind == 1) {
    constexpr int kAcc = Kind == 0 ? 8 : 16;
    typedef typename std::conditional<Kind == 0, f32x16_t, f32x4_t>::type acc_t;
    acc_t acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = acc_t{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kAcc; ++j) {
        const i32x8_t& ra = r[j & 3];
        const i32x8_t& rb = r[4 + ((j + (j >> 2)) & 3)];
        // the low and high 16 bytes of a 32-byte register set alternate between instructions
        i32x4_t a4 = (j & 1) ? i32x4_t{ra[4], ra[5], ra[6], ra[7]} : i32x4_t{ra[0], ra[1], ra[2], ra[3]};
        i32x4_t b4 = (j & 2) ? i32x4_t{rb[4], rb[5], rb[6], rb[7]} : i32x4_t{rb[0], rb[1], rb[2], rb[3]};
        bf16x8_t a = __builtin_bit_cast(bf16x8_t, a4);
        bf16x8_t b = __builtin_bit_cast(bf16x8_t, b4);
        if constexpr (Kind == 0)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
      for (int e = 0; e < (Kind == 0 ? 16 : 4); ++e) sum += acc[j][e];
  } else if constexpr (Kind == 2) {
    f32x16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x16_t{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        // cbsz = blgp = 0: both operands e4m3
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(r[j & 3], r[4 + ((j + (j >> 2)) & 3)], acc[j],
                                                                 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[j][e];
  } else if constexpr (Kind == 4) {
    f32x4_t acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x4_t{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r[j & 3], r[4 + ((j + (j >> 2)) & 3)], acc[j],
                                                                  0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += acc[j][e];
  } else if constexpr (Kind == 5) {
    i32x4_t acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = i32x4_t{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const i32x8_t& ra = r[j & 3];
        const i32x8_t& rb = r[4 + ((j + (j >> 2)) & 3)];
        i32x4_t a = (j & 1) ? i32x4_t{ra[4], ra[5], ra[6], ra[7]} : i32x4_t{ra[0], ra[1], ra[2], ra[3]};
        i32x4_t b = (j & 2) ? i32x4_t{rb[4], rb[5], rb[6], rb[7]} : i32x4_t{rb[0], rb[1], rb[2], rb[3]};
        acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += (float)acc[j][e];
  } else {
    i32x16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = i32x16_t{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const i32x8_t& ra = r[j & 3];
        const i32x8_t& rb = r[4 + ((j + (j >> 2)) & 3)];
        i32x4_t a = (j & 1) ? i32x4_t{ra[4], ra[5], ra[6], ra[7]} : i32x4_t{ra[0], ra[1], ra[2], ra[3]};
        i32x4_t b = (j & 2) ? i32x4_t{rb[4], rb[5], rb[6], rb[7]} : i32x4_t{rb[0], rb[1], rb[2], rb[3]};
        acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += (float)acc[j][e];
  }
  // 96 KiB of LDS, allocated but only touched on a path no launch takes (iters > 0 is checked by the
  // host), so that no two workgroups share a compute unit whatever the register count
  __shared__ float hold[96 * 1024 / 4];
  if (iters < 0) {
    hold[threadIdx.x] = sum;
    __syncthreads();
    sum = hold[255 - threadIdx.x];
  }
  sum += __shfl_xor(sum, 32);
  if (lane == 0) out[blockIdx.x * kWaves + wave] = sum;
}

}  // namespace

extern "C" int wan_mfma_ceiling_run(int kind, const void* operands, float* out, int n_workgroups, int iters,
                                    hipStream_t stream) {
  if (operands == nullptr || out == nullptr || n_workgroups <= 0 || iters <= 0 || kind < 0 || kind > 5) return 1;
  const dim3 grid(n_workgroups), block(64 * kWaves);
  const i32x8_t* src = static_cast<const i32x8_t*>(operands);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_ceiling_kernel<0>, grid, block, 0, stream, src, out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_ceiling_kernel<1>, grid, block, 0, stream, src, out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_ceiling_kernel<2>, grid, block, 0, stream, src, out, iters); break;
    case 3: hipLaunchKernelGGL(mfma_ceiling_kernel<3>, grid, block, 0, stream, src, out, iters); break;
    case 4: hipLaunchKernelGGL(mfma_ceiling_kernel<4>, grid, block, 0, stream, src, out, iters); break;
    default: hipLaunchKernelGGL(mfma_ceiling_kernel<5>, grid, block, 0, stream, src, out, iters); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
