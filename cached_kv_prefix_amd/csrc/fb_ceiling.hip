// Measured ceilings: a streaming read of a device buffer and a loop of bf16 matrix FMAs,
// the two rates the attention kernels are bound by (HBM reads for the prefix pass, the
// matrix units for a long block's pass), measured on this chip under its own power and
// clock limits.  Built into libfb_ceiling.so, apart from the attention library.
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
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ p, int64_t n16, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256 * kReadUnroll;
  for (int64_t i = (int64_t)blockIdx.x * 256 * kReadUnroll + threadIdx.x; i < n16; i += stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = i + u * 256 < n16 ? p[i + u * 256] : u32x4{0u, 0u, 0u, 0u};
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

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 5; }

}  // namespace

extern "C" int fbc_stream_read(const void* buf, int64_t bytes, int32_t workgroups, void* sink, hipStream_t stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > kMaxWorkgroups) return 1;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 16 != 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<u32x4*>(sink));
  return launch_status();
}

extern "C" int fbc_mfma_loop(int32_t workgroups, int64_t iters, float a, float b, float* sink, hipStream_t stream) {
  if (!sink || workgroups < 1 || workgroups > kMaxWorkgroups || iters < 1 || iters > kMaxIters) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, a, b, iters, sink);
  return launch_status();
}
