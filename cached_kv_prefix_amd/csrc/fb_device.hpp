// Device helpers for the gfx950 kernels: bfloat16 conversion, MFMA operand types,
// base-2 transcendentals and wave-level butterflies.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// exp2 that maps -inf to 0 and stays finite for the operands produced here.
__device__ __forceinline__ float exp2_or_zero(float x) {
  return x == kNegInf ? 0.0f : fast_exp2(x);
}

// Max / sum of a lane's value with the value of the lane 32 away, through
// v_permlane32_swap (a VALU lane swap, no LDS round trip).  With x in both operands the
// two results hold, in every lane l, x[l & 31] and x[(l & 31) + 32]; max and + of two
// operands are commutative, so every lane gets exactly fmax(x[l], x[l ^ 32]) and
// x[l] + x[l ^ 32].
__device__ __forceinline__ float wave_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Inclusive scan of one value per thread over a 256-thread block: a shuffle scan inside
// each wave, then the wave totals through LDS (tmp holds 4 ints).  Every thread gets its
// inclusive prefix; *total receives the block sum.
__device__ __forceinline__ int block_incl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += tmp[i];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return v + before;
}

}  // namespace fb
