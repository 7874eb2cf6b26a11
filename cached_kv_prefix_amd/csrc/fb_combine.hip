// Split reduction, log-space merge, cache write/reuse, reuse masks and the head cosine.
//
// Merge ("Resumo Técnico: FlashBlock", §2 Mecanismo Central, merge equation):
//   m = max(L_out, L_in); A = (e^{L_out-m} A_out + e^{L_in-m} A_in) / (e^{L_out-m} + e^{L_in-m})
// Reuse ("Resumo Técnico: FlashBlock", §2 Estratégias de Reutilização Adaptativa): a row
// whose head reuses reads the cached (A_out, L_out) and leaves it untouched; a recomputed
// row reduces its prefix chunks, writes the cache and merges the very values it wrote, so
// reuse and recompute on unchanged inputs give bit-identical outputs.
// LoSA ("LoSA", §2 steps 2 and 4): active rows take the sparse prefix result into the
// cache; stable rows reuse their cached statistics; every row merges with the block part.
#include "fb_device.hpp"
#include "fb_internal.hpp"

namespace fb {

namespace {

// Partial results of one row, loaded before anything is known about which of them are
// valid: the statistics of chunk `lane` and the O rows of the first U chunks.  Every load
// stays inside the workspace region of its group (chunk indices are clamped to the plan's
// split count), so stale slots are read but never used: the reduction selects by the
// valid count.  Issuing all loads at once turns the combine from a chain of dependent
// round trips into one.
template <int E, int U>
struct RowPartials {
  float m, l;
  float x[U][E];
};

template <int E, int U>
__device__ __forceinline__ void issue_partials(const float* po, const float* pml, int64_t slot0, int rows,
                                               int row, int nmax, int d, int lane, RowPartials<E, U>& P) {
  const int sl = lane < nmax ? lane : 0;
  const float* ml = pml + ((slot0 + sl) * rows + row) * 2;
  P.m = ml[0];
  P.l = ml[1];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = (slot0 + (u < nmax ? u : nmax - 1)) * rows + row;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      P.x[u][e] = dd < d ? po[r * d + dd] : 0.f;
    }
  }
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Reduce the first n (<= nmax) chunks of one row: base-2 (m, l, O) partials -> normalised
// A and natural-log L.  The O sum runs over the chunks in ascending order; the order
// depends on the shape only, so results are deterministic.
template <int E, int U>
__device__ __forceinline__ void reduce_chunks(const RowPartials<E, U>& P, const float* po, const float* pml,
                                              int64_t slot0, int rows, int row, int n, int d, int lane,
                                              float (&a)[E], float& L) {
  float M = kNegInf, l = 0.f, Mu;
  if (n <= U) {   // uniform: the statistics of the first U chunks are read lane by lane
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n) M = fmaxf(M, lane_value(P.m, u));
    Mu = M == kNegInf ? 0.f : M;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n) l += exp2_or_zero(lane_value(P.m, u) - Mu) * lane_value(P.l, u);
  } else {
    M = lane < n ? P.m : kNegInf;
    for (int s = lane + 64; s < n; s += 64) M = fmaxf(M, pml[((slot0 + s) * rows + row) * 2]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    Mu = M == kNegInf ? 0.f : M;
    l = lane < n ? exp2_or_zero(P.m - Mu) * P.l : 0.f;
    for (int s = lane + 64; s < n; s += 64) {
      const float* ml = pml + ((slot0 + s) * rows + row) * 2;
      l += exp2_or_zero(ml[0] - Mu) * ml[1];
    }
    l = wave_sum(l);
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < n) {   // uniform
      const float f = exp2_or_zero(lane_value(P.m, u) - Mu);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += f * P.x[u][e];
    }
  }
  for (int s = U; s < n; ++s) {
    const int64_t r = (slot0 + s) * rows + row;
    const float f = exp2_or_zero(pml[r * 2] - Mu);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      acc[e] += f * (dd < d ? po[r * d + dd] : 0.f);
    }
  }
  if (l > 0.f) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = acc[e] * inv;
    L = (M + fast_log2(l)) * kLn2;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = 0.f;
    L = kNegInf;
  }
}

// Two-way log-space merge of one row (natural-log L).  Both sides empty gives 0 / -inf.
template <int E>
__device__ __forceinline__ void merge_row(const float (&ao)[E], float lo, const float (&ai)[E],
                                          float li, float (&af)[E], float& lf) {
  const float m = fmaxf(lo, li);
  if (m == kNegInf) {
#pragma unroll
    for (int e = 0; e < E; ++e) af[e] = 0.f;
    lf = kNegInf;
    return;
  }
  const float wo = lo == kNegInf ? 0.f : fast_exp2((lo - m) * kLog2e);
  const float wi = li == kNegInf ? 0.f : fast_exp2((li - m) * kLog2e);
  const float den = wo + wi;
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < E; ++e) af[e] = (wo * ao[e] + wi * ai[e]) * inv;
  lf = m + fast_log2(den) * kLn2;
}

__device__ __forceinline__ int n_chunks(int n_keys, int chunk) { return (n_keys + chunk - 1) / chunk; }

}  // namespace

// One wave per output row (b, i, h); lanes own dims lane + 64 e.  The row indices are
// wave-uniform, so the reuse inputs (flag, sequence length, active list) are scalar loads,
// which do not wait behind vector loads; every partial load of the row (prefix, block,
// cached row) is issued before the reuse decision is known.
template <int E>
__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs C) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  const int rowid = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nrows = C.batch * C.B * C.h_q;
  if (rowid >= nrows) return;
  const int h = rowid % C.h_q;
  const int i = (rowid / C.h_q) % C.B;
  const int b = rowid / (C.h_q * C.B);
  const int hk = h / C.G, jg = h % C.G;
  const int d = C.d;
  const int64_t roff = (int64_t)rowid * d;
  const bool has_prefix = C.mode != kModeBlockOnly;

  // --- the LoSA active list decides which partial row to read ----------------------------
  int prow = jg * C.B + i;
  bool fresh = true;
  if (C.mode == kModeLosa) {
    int pos = -1;
    for (int a = 0; a < C.n_active; ++a)
      if (C.active[b * C.n_active + a] == i) pos = a;
    fresh = pos >= 0;
    prow = jg * C.n_active + (pos < 0 ? 0 : pos);
  }

  // --- every partial load ----------------------------------------------------------------
  const int64_t pslot0 = (int64_t)(b * C.h_kv + hk) * C.p_splits;
  const int64_t bslot0 = (int64_t)(b * C.h_kv + hk) * C.b_splits;
  RowPartials<E, U> PP, PB;
  float cached[E], cached_l = kNegInf;
  if (has_prefix && C.p_splits > 0) issue_partials<E, U>(C.po, C.pml, pslot0, C.p_rows, prow, C.p_splits, d, lane, PP);
  if (C.mode != kModePrefixOnly && C.b_splits > 0)
    issue_partials<E, U>(C.bo, C.bml, bslot0, C.b_rows, jg * C.B + i, C.b_splits, d, lane, PB);
  if (has_prefix && C.mode != kModePrefixOnly) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      cached[e] = dd < d ? C.cache_a[roff + dd] : 0.f;
    }
    cached_l = C.cache_l[rowid];
  }

  // --- reuse inputs, read while the partials are in flight -------------------------------
  if (C.mode != kModeLosa) {
    if (C.m_upd)
      fresh = C.m_upd[b] >= C.tau;
    else if (C.mask)
      fresh = C.mask[b * C.h_q + h] == 0;
  }
  int nk = C.n_uniform;
  if (C.page_count)
    nk = C.page_count[b * C.h_kv + hk] * C.page_size;
  else if (C.cu)
    nk = C.cu[b + 1] - C.cu[b];

  float ao[E], ai[E], af[E];
  float lo = kNegInf, li = kNegInf, lf;

  // --- block-external part ---------------------------------------------------------------
  if (has_prefix) {
    if (fresh) {
      const int n = C.p_splits > 0 ? min(n_chunks(nk, C.p_chunk), C.p_splits) : 0;
      reduce_chunks<E, U>(PP, C.po, C.pml, pslot0, C.p_rows, prow, n, d, lane, ao, lo);
      float* ca = C.cache_a + roff;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int dd = lane + 64 * e;
        if (dd < d) ca[dd] = ao[e];
      }
      if (lane == 0) C.cache_l[rowid] = lo;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) ao[e] = cached[e];
      lo = cached_l;
    }
    if (C.mode == kModePrefixOnly) return;
  }

  // --- block-internal part ---------------------------------------------------------------
  {
    const int n = C.b_splits > 0 ? min(n_chunks(C.B, C.b_chunk), C.b_splits) : 0;
    reduce_chunks<E, U>(PB, C.bo, C.bml, bslot0, C.b_rows, jg * C.B + i, n, d, lane, ai, li);
  }
  if (C.mode == kModeBlockOnly) {
    float* pa = C.ain + roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) pa[dd] = ai[e];
    }
    if (lane == 0) C.lin[rowid] = li;
    return;
  }

  merge_row<E>(ao, lo, ai, li, af, lf);
  if (C.out_bf16) {
    uint16_t* out = (uint16_t*)C.a_full + roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) out[dd] = f32_to_bf16(af[e]);
    }
  } else {
    float* out = (float*)C.a_full + roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) out[dd] = af[e];
    }
  }
  if (C.l_full && lane == 0) C.l_full[rowid] = lf;
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

hipError_t launch_combine(const CombineArgs& c, hipStream_t st) {
  const int64_t rows = (int64_t)c.batch * c.B * c.h_q;
  if (rows == 0) return hipSuccess;
  if (rows > INT32_MAX - 4) return hipErrorInvalidValue;   // row indices are 32-bit
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (c.d <= 64)
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, st, c);
  else if (c.d <= 128)
    hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(256), 0, st, c);
  else
    hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, st, c);
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
