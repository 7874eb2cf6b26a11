// Block lifecycle kernels: append a finished block's K/V to the packed prefix, the row map
// of the multi-branch pass, and the small fills the block driver needs (kernels rather than
// memset nodes, so a captured step sequence holds kernel nodes only).
//
// "FlashBlock: Attention Caching for Efficient Long-Context Block Diffusion", abstract:
// block-wise causal inference over a KV cache that grows block by block.  Once a block's
// steps are done, its B tokens follow the sequence's prefix.
#include "fb_device.hpp"
#include "fb_internal.hpp"

namespace fb {

// One thread per PIECE-byte piece of an output token row.  Grid: (token pieces, batch).
// Token t of sequence b comes from the old prefix (t < N_b) or from the block.
template <typename PIECE>
__global__ void __launch_bounds__(256) append_kernel(const AppendArgs a) {
  const int b = blockIdx.y;
  if (a.cu_out && blockIdx.x == 0 && b == 0) {
    for (int i = threadIdx.x; i <= a.batch; i += 256)
      a.cu_out[i] = (a.cu ? a.cu[i] : i * a.n_uniform) + i * a.B;
  }
  const int64_t pieces = a.row_bytes / (int64_t)sizeof(PIECE);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n = a.cu ? a.cu[b + 1] - a.cu[b] : a.n_uniform;
  const int64_t seq0 = a.cu ? a.cu[b] : (int64_t)b * a.n_uniform;
  const int64_t t = (a.tail_only ? n : 0) + idx / pieces;   // in place: only the block rows
  const int64_t pc = idx % pieces;
  if (t >= (int64_t)n + a.B) return;
  const int64_t dst0 = seq0 + (int64_t)b * a.B;   // every earlier sequence grew by B
  const PIECE* sk;
  const PIECE* sv;
  if (t < n) {
    sk = (const PIECE*)((const char*)a.k + (seq0 + t) * a.row_bytes);
    sv = (const PIECE*)((const char*)a.v + (seq0 + t) * a.row_bytes);
  } else {
    const int64_t r = (int64_t)b * a.B + (t - n);
    sk = (const PIECE*)((const char*)a.k_blk + r * a.row_bytes);
    sv = (const PIECE*)((const char*)a.v_blk + r * a.row_bytes);
  }
  ((PIECE*)((char*)a.k_out + (dst0 + t) * a.row_bytes))[pc] = sk[pc];
  ((PIECE*)((char*)a.v_out + (dst0 + t) * a.row_bytes))[pc] = sv[pc];
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  const bool wide = a.row_bytes % 16 == 0;
  const int64_t pieces = a.row_bytes / (wide ? 16 : 4);
  const int64_t tokens = a.tail_only ? a.B : (int64_t)a.max_len + a.B;
  const int64_t n = tokens * pieces;
  if (n <= 0 || a.batch == 0) return hipSuccess;
  if ((n + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + 255) / 256), a.batch);
  if (wide)
    hipLaunchKernelGGL(append_kernel<u32x4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(append_kernel<uint32_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Multi-branch prefix pass ("Resumen Técnico: BlockBatch", system optimisation: the query
// positions of all branches in one variable-length buffer): the row map the attention
// kernels read queries through.  Rows past a branch's block repeat its last query (their
// results are not written out); an empty branch points at row 0.
__global__ void varlen_rows_kernel(const int32_t* cu_q, int batch, int b_max, int total_q, int32_t* row_tok) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * b_max) return;
  const int b = idx / b_max, i = idx % b_max;
  const int q0 = cu_q[b], nb = cu_q[b + 1] - q0;
  const int r = q0 + min(i, nb - 1);
  row_tok[idx] = nb > 0 ? max(0, min(r, total_q - 1)) : 0;
}

hipError_t launch_varlen_rows(const int32_t* cu_q, int32_t batch, int32_t b_max, int32_t total_q, int32_t* row_tok,
                              hipStream_t st) {
  const int64_t n = (int64_t)batch * b_max;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cu_q, batch, b_max,
                     total_q, row_tok);
  return hipGetLastError();
}

__global__ void fill_u8_kernel(uint8_t* p, int64_t n, uint8_t value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}


hipError_t launch_fill_u8(uint8_t* p, int64_t n, uint8_t value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}


}  // namespace fb
