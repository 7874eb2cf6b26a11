// Measured ceilings: a streaming read of a device buffer and a loop of bf16 matrix FMAs,
// the two rates the attention kernels are bound by (HBM reads for the prefix pass, the
// matrix units for a long block's pass), measured on this chip under its own power and
// clock limits; and how far the matrix work of one wave and the vector work of another
// overlap on one SIMD.  Built into libfb_ceiling.so, apart from the attention library.
#include <hip/hip_runtime.h>

#include "fb_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadUnroll = 4;   // 16-byte loads in flight per lane
constexpr int kMfmaAcc = 4;      // independent accumulators per wave, enough to cover the MFMA latency
constexpr int64_t kMaxIters = 262144;
constexpr int32_t kMaxWorkgroups = 65536;

// Grid-stride read: in every pass, lane t of workgroup g reads words
// (g * 256 * U + t + 256 u) for u < U; the passes step by the whole grid.  Each word is read
// by exactly one lane, and the XOR of the words a workgroup read goes to its sink entry.
// NT: loads carry the non-temporal hint (`nt` on gfx950), the form the streaming attention
// pass uses for K/V it reads once.
template <bool NT>
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ p, int64_t n16, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256 * kReadUnroll;
  for (int64_t i = (int64_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; i < n16; i += stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const u32x4* a = p + i + u * 256;
      v[u] = i + u * 256 < n16 ? (NT ? __builtin_nontemporal_load(a) : *a) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] ^= (uint32_t)__shfl_xor((int)acc[c], o);
  }
  __shared__ u32x4 part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Register-only MFMA loop: the operands come from kernel arguments, so nothing can be folded
// at compile time, and the accumulators are written out, so nothing can be dropped.
__global__ void __launch_bounds__(256) mfma_loop_kernel(float a, float b, int64_t iters, float* sink) {
  bf16x8 va, vb;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    va[j] = (__bf16)a;
    vb[j] = (__bf16)b;
  }
  f32x16 acc[kMfmaAcc];
#pragma unroll
  for (int k = 0; k < kMfmaAcc; ++k) acc[k] = f32x16{};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kMfmaAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaAcc; ++k) s += acc[k][0];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// Matrix and vector work on one SIMD.  A workgroup of 8 waves puts waves w and w + 4 on the
// same SIMD (waves are placed on the 4 SIMDs of a CU in turn).  MODE 0: waves 0-3 run the
// MFMA stream alone; MODE 1: waves 0-3 run the vector stream alone; MODE 2: waves 0-3 the
// MFMA stream and waves 4-7 the vector stream, side by side; MODE 3: waves 0-3 each
// interleave the two.  The MFMA stream is 8 v_mfma_f32_32x32x16_bf16 per round (two on
// each of 4 accumulators); the vector stream is K operations per MFMA on 8 independent
// chains, half v_exp_f32 and half v_fma_f32, the mix of an attention softmax.  Each chain
// takes x -> 2^x then x -> x * one - one in turn, so from x = 0 it returns to 0 every two
// operations and its final value is exactly 0 when `one` is 1.
template <int MODE, int K>
__global__ void __launch_bounds__(512) mfma_valu_kernel(float one, int64_t rounds, float* sink) {
  bf16x8 va;
#pragma unroll
  for (int j = 0; j < 8; ++j) va[j] = (__bf16)one;
  f32x16 acc[kMfmaAcc];
#pragma unroll
  for (int k = 0; k < kMfmaAcc; ++k) acc[k] = f32x16{};
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = (one - 1.0f) * (float)(c + 1);   // 0, as 8 distinct expressions
  const int w = threadIdx.x >> 6;
  const bool mfma = MODE == 0 || MODE == 3 || (MODE == 2 && w < 4);
  const bool valu = MODE == 1 || MODE == 3 || (MODE == 2 && w >= 4);
  // one round: 8 MFMA slots, K vector operations after each; operation n of the round goes
  // to chain n % 8 and is an exp when (n / 8) is even, so every chain alternates exp, fma.
  auto vec = [&](int slot) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int n = slot * K + j;
      if ((n / 8) % 2 == 0) x[n % 8] = __builtin_amdgcn_exp2f(x[n % 8]);
      else x[n % 8] = __builtin_fmaf(x[n % 8], one, -one);
    }
  };
  if (MODE == 3) {
    for (int64_t i = 0; i < rounds; ++i) {
#pragma unroll
      for (int slot = 0; slot < 8; ++slot) {
        acc[slot % kMfmaAcc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, va, acc[slot % kMfmaAcc], 0, 0, 0);
        vec(slot);
      }
    }
  } else if (mfma) {
    for (int64_t i = 0; i < rounds; ++i) {
#pragma unroll
      for (int slot = 0; slot < 8; ++slot)
        acc[slot % kMfmaAcc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, va, acc[slot % kMfmaAcc], 0, 0, 0);
    }
  } else if (valu) {
    for (int64_t i = 0; i < rounds; ++i) {
#pragma unroll
      for (int slot = 0; slot < 8; ++slot) vec(slot);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaAcc; ++k) s += acc[k][0];
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 8 + w] = s;
}

template <int MODE>
void launch_mfma_valu(int k, int32_t workgroups, int64_t rounds, float one, float* sink, hipStream_t stream) {
  const dim3 grid((unsigned)workgroups), block(MODE == 2 ? 512 : 256);
  switch (k) {
    case 0: hipLaunchKernelGGL((mfma_valu_kernel<MODE, 0>), grid, block, 0, stream, one, rounds, sink); break;
    case 2: hipLaunchKernelGGL((mfma_valu_kernel<MODE, 2>), grid, block, 0, stream, one, rounds, sink); break;
    case 4: hipLaunchKernelGGL((mfma_valu_kernel<MODE, 4>), grid, block, 0, stream, one, rounds, sink); break;
    default: hipLaunchKernelGGL((mfma_valu_kernel<MODE, 8>), grid, block, 0, stream, one, rounds, sink); break;
  }
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 5; }

}  // namespace

extern "C" int fbc_stream_read(const void* buf, int64_t bytes, int32_t workgroups, int32_t nontemporal, void* sink,
                               hipStream_t stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > kMaxWorkgroups) return 1;
  if (nontemporal != 0 && nontemporal != 1) return 1;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 16 != 0) return 1;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)workgroups), dim3(256), 0, stream,
                       static_cast<const u32x4*>(buf), bytes / 16, static_cast<u32x4*>(sink));
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)workgroups), dim3(256), 0, stream,
                       static_cast<const u32x4*>(buf), bytes / 16, static_cast<u32x4*>(sink));
  return launch_status();
}

extern "C" int fbc_mfma_loop(int32_t workgroups, int64_t iters, float a, float b, float* sink, hipStream_t stream) {
  if (!sink || workgroups < 1 || workgroups > kMaxWorkgroups || iters < 1 || iters > kMaxIters) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, a, b, iters, sink);
  return launch_status();
}

extern "C" int fbc_mfma_valu(int32_t mode, int32_t valu_per_mfma, int32_t workgroups, int64_t rounds, float one,
                             float* sink, hipStream_t stream) {
  if (!sink || mode < 0 || mode > 3 || workgroups < 1 || workgroups > kMaxWorkgroups || rounds < 1 ||
      rounds > kMaxIters)
    return 1;
  if (valu_per_mfma != 2 && valu_per_mfma != 4 && valu_per_mfma != 8 && !(valu_per_mfma == 0 && mode == 0)) return 1;
  switch (mode) {
    case 0: launch_mfma_valu<0>(valu_per_mfma, workgroups, rounds, one, sink, stream); break;
    case 1: launch_mfma_valu<1>(valu_per_mfma, workgroups, rounds, one, sink, stream); break;
    case 2: launch_mfma_valu<2>(valu_per_mfma, workgroups, rounds, one, sink, stream); break;
    default: launch_mfma_valu<3>(valu_per_mfma, workgroups, rounds, one, sink, stream); break;
  }
  return launch_status();
}
