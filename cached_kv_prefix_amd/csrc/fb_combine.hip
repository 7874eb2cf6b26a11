// Split reduction + merge kernel (row logic in fb_combine_row.hpp), the standalone
// log-space merge, the reuse masks and the head cosine.
#include "fb_combine_row.hpp"

namespace fb {

// One wave per output row (b, i, h); lanes own dims lane + 64 e.
template <int E, int UP, int UB, bool DECIDE>
__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs C) {
  const int lane = threadIdx.x & 63;
  const int rowid = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (rowid >= C.batch * C.B * C.h_q) return;
  RowState<E, UP, UB> st;
  row_issue<E, UP, UB, DECIDE>(C, rowid, lane, st);
  if (st.valid) row_finish<E, UP, UB>(C, lane, st);
}

template <int E, int UP, int UR, int UB>
__global__ void __launch_bounds__(256) combine_residual_kernel(const CombineArgs C) {
  const int lane = threadIdx.x & 63;
  const int rowid = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (rowid >= C.batch * C.B * C.h_q) return;
  residual_row<E, UP, UR, UB>(C, rowid, lane);
}

template <int E>
__global__ void __launch_bounds__(256) lse_merge_kernel(int64_t rows, int d, const float* ao_, const float* lo_,
                                                        const float* ai_, const float* li_, void* af_,
                                                        int out_bf16, float* lf_) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float ao[E], ai[E], af[E], lf;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int dd = lane + 64 * e;
    ao[e] = dd < d ? ao_[r * d + dd] : 0.f;
    ai[e] = dd < d ? ai_[r * d + dd] : 0.f;
  }
  merge_row<E>(ao, lo_[r], ai, li_[r], af, lf);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int dd = lane + 64 * e;
    if (dd >= d) continue;
    if (out_bf16)
      ((uint16_t*)af_)[r * d + dd] = f32_to_bf16(af[e]);
    else
      ((float*)af_)[r * d + dd] = af[e];
  }
  if (lf_ && lane == 0) lf_[r] = lf;
}

// Debug check of the cache rows a step would reuse: *bad = 1 if any of them holds NaN in
// cache_l (never written), else 0.  One workgroup scans every row, so the flag needs no
// clearing beforehand.
__global__ void __launch_bounds__(256) cache_check_kernel(const float* cache_l, int batch, int B, int h_q,
                                                          const uint8_t* mask, const int32_t* m_upd, int tau,
                                                          int all_rows, int32_t* bad) {
  const int64_t rows = (int64_t)batch * B * h_q;
  int found = 0;
  for (int64_t r = threadIdx.x; r < rows; r += 256) {
    const int h = (int)(r % h_q);
    const int b = (int)(r / ((int64_t)B * h_q));
    const bool reused = all_rows || (m_upd ? m_upd[b] < tau : mask ? mask[b * h_q + h] != 0 : false);
    found |= reused && __builtin_isnan(cache_l[r]);
  }
  found = __syncthreads_or(found);
  if (threadIdx.x == 0) *bad = found ? 1 : 0;
}

__global__ void mask_threshold_kernel(const int32_t* m, int tau, int batch, int h_q, uint8_t* mask) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * h_q) return;
  mask[idx] = m[idx / h_q] < tau ? 1 : 0;
}

__global__ void mask_similarity_kernel(const float* sim, float gamma, int64_t n, uint8_t* mask) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  mask[idx] = sim[idx] > gamma ? 1 : 0;
}

// One workgroup per (b, h): fp64 partial sums in a fixed order, then a fixed tree.
__global__ void __launch_bounds__(256) head_cosine_kernel(int B, int h_q, int d, const float* x,
                                                          const float* y, float* sim) {
  __shared__ double red[3][256];
  const int bh = blockIdx.x;
  const int h = bh % h_q, b = bh / h_q;
  double sxy = 0.0, sxx = 0.0, syy = 0.0;
  const int64_t n = (int64_t)B * d;
  for (int64_t e = threadIdx.x; e < n; e += 256) {
    const int i = e / d, dd = e % d;
    const int64_t off = (((int64_t)b * B + i) * h_q + h) * d + dd;
    const double xv = x[off], yv = y[off];
    sxy += xv * yv;
    sxx += xv * xv;
    syy += yv * yv;
  }
  red[0][threadIdx.x] = sxy;
  red[1][threadIdx.x] = sxx;
  red[2][threadIdx.x] = syy;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      red[0][threadIdx.x] += red[0][threadIdx.x + s];
      red[1][threadIdx.x] += red[1][threadIdx.x + s];
      red[2][threadIdx.x] += red[2][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double nx = sqrt(red[1][0]), ny = sqrt(red[2][0]);
    sim[bh] = (nx == 0.0 || ny == 0.0) ? 0.f : (float)(red[0][0] / (nx * ny));
  }
}

// One thread per (b, h): the head's rows in order, then the cosine (0 for a zero vector);
// with next_mask, also the per-head rule for the next step (sim > gamma, fp32).
__global__ void sim_reduce_kernel(int batch, int B, int h_q, const double* parts, float* sim, float gamma,
                                  uint8_t* next_mask) {
  const int64_t bh = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= (int64_t)batch * h_q) return;
  const int h = bh % h_q, b = bh / h_q;
  double xy = 0.0, xx = 0.0, yy = 0.0;
  const double* base = parts + ((int64_t)b * B * h_q + h) * 3;
  const int64_t step = (int64_t)h_q * 3;
  int i = 0;
  for (; i + 8 <= B; i += 8) {   // eight rows' loads in flight, then added in row order
    double v[8][3];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < 3; ++c) v[u][c] = base[(i + u) * step + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      xy += v[u][0];
      xx += v[u][1];
      yy += v[u][2];
    }
  }
  for (; i < B; ++i) {
    xy += base[i * step + 0];
    xx += base[i * step + 1];
    yy += base[i * step + 2];
  }
  const float s = (xx == 0.0 || yy == 0.0) ? 0.f : (float)(xy / (sqrt(xx) * sqrt(yy)));
  sim[bh] = s;
  if (next_mask) next_mask[bh] = s > gamma ? 1 : 0;
}

hipError_t launch_sim_reduce(int32_t batch, int32_t B, int32_t h_q, const double* parts, float* sim,
                             float gamma, uint8_t* next_mask, hipStream_t st) {
  const int64_t n = (int64_t)batch * h_q;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(sim_reduce_kernel, dim3((unsigned)((n + 63) / 64)), dim3(64), 0, st, batch, B, h_q, parts, sim,
                     gamma, next_mask);
  return hipGetLastError();
}

constexpr int64_t kCombineDecideRows = 16384;

hipError_t launch_combine(const CombineArgs& c, hipStream_t st) {
  const int64_t rows = (int64_t)c.batch * c.B * c.h_q;
  if (rows == 0) return hipSuccess;
  if (rows > INT32_MAX - 4) return hipErrorInvalidValue;   // row indices are 32-bit
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (c.mode == kModeResidual) {   // chunk loads issued at once: up to 16 selected, 32 residual, 1 block
    if (c.d <= 64)
      hipLaunchKernelGGL((combine_residual_kernel<1, 16, 32, 1>), grid, dim3(256), 0, st, c);
    else if (c.d <= 128)
      hipLaunchKernelGGL((combine_residual_kernel<2, 16, 32, 1>), grid, dim3(256), 0, st, c);
    else
      hipLaunchKernelGGL((combine_residual_kernel<4, 8, 8, 1>), grid, dim3(256), 0, st, c);
    return hipGetLastError();
  }
  // chunk loads issued up front: as many as the plan has (d = 128), else 8
  const int up = c.p_splits <= 1 ? 1 : c.p_splits <= 2 ? 2 : c.p_splits <= 4 ? 4 : 8;
  const bool ub1 = c.b_splits <= 1;
  // a large step combine is bound by its bytes: the rows read the reuse decision first (or
  // know it, with no mask and no count) and load only what they use; a small one is bound
  // by latency and loads everything at once
  const bool decide = c.mode == kModeStep && rows > kCombineDecideRows;
  if (c.d <= 64) {
    hipLaunchKernelGGL((combine_kernel<1, 8, 8, false>), grid, dim3(256), 0, st, c);
  } else if (c.d <= 128) {
#define FB_COMBINE_UB(UP)                                                                    \
  if (ub1 && decide)                                                                         \
    hipLaunchKernelGGL((combine_kernel<2, UP, 1, true>), grid, dim3(256), 0, st, c);         \
  else if (ub1)                                                                              \
    hipLaunchKernelGGL((combine_kernel<2, UP, 1, false>), grid, dim3(256), 0, st, c);        \
  else                                                                                       \
    hipLaunchKernelGGL((combine_kernel<2, UP, 8, false>), grid, dim3(256), 0, st, c);
    if (up == 1) {
      FB_COMBINE_UB(1)
    } else if (up == 2) {
      FB_COMBINE_UB(2)
    } else if (up == 4) {
      FB_COMBINE_UB(4)
    } else {
      FB_COMBINE_UB(8)
    }
#undef FB_COMBINE_UB
  } else {
    hipLaunchKernelGGL((combine_kernel<4, 8, 8, false>), grid, dim3(256), 0, st, c);
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(int64_t rows, int32_t d, const float* ao, const float* lo, const float* ai,
                            const float* li, void* af, int out_bf16, float* lf, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (d <= 64)
    hipLaunchKernelGGL(lse_merge_kernel<1>, grid, dim3(256), 0, st, rows, d, ao, lo, ai, li, af, out_bf16, lf);
  else if (d <= 128)
    hipLaunchKernelGGL(lse_merge_kernel<2>, grid, dim3(256), 0, st, rows, d, ao, lo, ai, li, af, out_bf16, lf);
  else
    hipLaunchKernelGGL(lse_merge_kernel<4>, grid, dim3(256), 0, st, rows, d, ao, lo, ai, li, af, out_bf16, lf);
  return hipGetLastError();
}

hipError_t launch_cache_check(const float* cache_l, int32_t batch, int32_t B, int32_t h_q, const uint8_t* mask,
                              const int32_t* m_upd, int32_t tau, bool all_rows, int32_t* bad, hipStream_t st) {
  hipLaunchKernelGGL(cache_check_kernel, dim3(1), dim3(256), 0, st, cache_l, batch, B, h_q, mask, m_upd, tau,
                     all_rows ? 1 : 0, bad);
  return hipGetLastError();
}

hipError_t launch_mask_threshold(const int32_t* m, int32_t tau, int32_t batch, int32_t h_q, uint8_t* mask,
                                 hipStream_t st) {
  const int64_t n = (int64_t)batch * h_q;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_threshold_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, m, tau, batch,
                     h_q, mask);
  return hipGetLastError();
}

hipError_t launch_mask_similarity(const float* sim, float gamma, int64_t n, uint8_t* mask, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_similarity_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sim, gamma, n,
                     mask);
  return hipGetLastError();
}

hipError_t launch_head_cosine(int32_t batch, int32_t B, int32_t h_q, int32_t d, const float* a0, const float* a1,
                              float* sim, hipStream_t st) {
  const int64_t n = (int64_t)batch * h_q;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(head_cosine_kernel, dim3((unsigned)n), dim3(256), 0, st, B, h_q, d, a0, a1, sim);
  return hipGetLastError();
}

}  // namespace fb
