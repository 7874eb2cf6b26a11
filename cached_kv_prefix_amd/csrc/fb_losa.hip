// LoSA-style selection ("LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion
// Language Models", §2 "El Algoritmo LoSA"):
//   step 1  locality pruning: per-token mean squared change of the queries between two
//           denoising steps; the |A| largest form the active set (ties: lower index);
//   step 3  a QUEST-like page selector for the active queries only, then the union of the
//           selected pages per KV head (§1: the memory cost is the size of that union).
// The page score is the maximum of q.k over the page's per-dimension key box,
//   S = sum_d max(q_d kmin_d, q_d kmax_d) = sum_d q_d * (q_d >= 0 ? kmax_d : kmin_d).
// Every decision is taken in fp64 with sums in a fixed left-to-right order (per head
// over dims, then over heads, for the locality score; over dims for the page score) and
// without fused multiply-add, so the selected indices are exactly reproducible.
#include "fb_device.hpp"
#include "fb_internal.hpp"

#pragma clang fp contract(off)

namespace fb {

namespace {

__device__ __forceinline__ double load_elem(const void* p, int64_t idx, int bf16) {
  return bf16 ? (double)bf16_to_f32(((const uint16_t*)p)[idx]) : (double)((const float*)p)[idx];
}

__device__ __forceinline__ void seq_of(const LosaArgs& a, int b, int& seq0, int& n) {
  if (a.cu) {
    seq0 = a.cu[b];
    n = a.cu[b + 1] - seq0;
  } else {
    seq0 = b * a.n_uniform;
    n = a.n_uniform;
  }
}

// Order-preserving map of an fp64 score to uint64 (larger score -> larger key); -0 is
// folded into +0 first.
__device__ __forceinline__ uint64_t order_key(double s) {
  s = s + 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive scan of one value per thread (blockDim.x == 256) through LDS.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp) {
  tmp[threadIdx.x] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) {
      const int x = tmp[t];
      tmp[t] = run;
      run += x;
    }
    tmp[256] = run;
  }
  __syncthreads();
  const int r = tmp[threadIdx.x];
  return r;
}

}  // namespace

// kmin/kmax layout [batch][h_kv][d/8][max_pages][8]: consecutive pages of one 8-dim chunk
// are adjacent, so the score kernel reads them with unit-stride 16-byte (bf16) loads.
__global__ void __launch_bounds__(256) page_meta_kernel(const LosaArgs a, const void* k, void* kmin, void* kmax) {
  const int b = blockIdx.z, hk = blockIdx.y;
  const int nc = a.d / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)nc * a.max_pages) return;
  const int c = idx / a.max_pages, p = idx % a.max_pages;
  int seq0, n;
  seq_of(a, b, seq0, n);
  const int t0 = p * a.page_size;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + a.page_size);
  float mn[8], mx[8];
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  for (int t = t0; t < t1; ++t) {
    const int64_t base = ((int64_t)(seq0 + t) * a.h_kv + hk) * a.d + c * 8;
    for (int e = 0; e < 8; ++e) {
      const float x = (float)load_elem(k, base + e, a.bf16);
      mn[e] = fminf(mn[e], x);
      mx[e] = fmaxf(mx[e], x);
    }
  }
  const int64_t out = ((((int64_t)b * a.h_kv + hk) * nc + c) * a.max_pages + p) * 8;
  for (int e = 0; e < 8; ++e) {
    if (a.bf16) {
      ((uint16_t*)kmin)[out + e] = (uint16_t)(__float_as_uint(mn[e]) >> 16);
      ((uint16_t*)kmax)[out + e] = (uint16_t)(__float_as_uint(mx[e]) >> 16);
    } else {
      ((float*)kmin)[out + e] = mn[e];
      ((float*)kmax)[out + e] = mx[e];
    }
  }
}

// One workgroup (1024 threads) per sequence.  Heads are processed in groups whose
// per-(token, head) sums fit in LDS; each group's sums are added to the token totals in
// head order.
__global__ void __launch_bounds__(1024) locality_kernel(const LosaArgs a, const void* qc, const void* qp,
                                                        int32_t* active) {
  constexpr int kLdsDoubles = 6144;
  __shared__ double inner[kLdsDoubles];
  __shared__ double total[1024];
  __shared__ int sel[1024];
  const int b = blockIdx.x;
  const int B = a.B, H = a.h_q, d = a.d;
  for (int i = threadIdx.x; i < B; i += blockDim.x) total[i] = 0.0;
  const int hg = max(1, min(H, kLdsDoubles / B));
  for (int h0 = 0; h0 < H; h0 += hg) {
    const int nh = min(hg, H - h0);
    __syncthreads();
    for (int w = threadIdx.x; w < B * nh; w += blockDim.x) {
      const int i = w / nh, hh = w % nh;
      const int64_t base = (((int64_t)b * B + i) * H + h0 + hh) * d;
      double s = 0.0;
      for (int j = 0; j < d; ++j) {
        const double df = load_elem(qc, base + j, a.bf16) - load_elem(qp, base + j, a.bf16);
        s = s + df * df;
      }
      inner[i * nh + hh] = s;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
      double t = total[i];
      for (int hh = 0; hh < nh; ++hh) t = t + inner[i * nh + hh];
      total[i] = t;
    }
  }
  __syncthreads();
  const double inv = 1.0 / (double)(H * d);
  for (int i = threadIdx.x; i < B; i += blockDim.x) total[i] = total[i] * inv;
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const double si = total[i];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const double sj = total[j];
      rank += (sj > si || (sj == si && j < i)) ? 1 : 0;
    }
    sel[i] = rank < a.n_active ? 1 : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    if (!sel[i]) continue;
    int pos = 0;
    for (int j = 0; j < i; ++j) pos += sel[j];
    active[b * a.n_active + pos] = i;
  }
}

// grid (page blocks of 256, h_kv, batch); a thread scores one page for every active row of
// the KV head's query heads, eight rows at a time, summing over d left to right.
__global__ void __launch_bounds__(256) quest_score_kernel(const LosaArgs a, const void* qc, const int32_t* active,
                                                          const void* kmin, const void* kmax, double* scores) {
  __shared__ double qs[8][256];
  const int b = blockIdx.z, hk = blockIdx.y;
  const int p = blockIdx.x * 256 + threadIdx.x;
  int seq0, n;
  seq_of(a, b, seq0, n);
  const int P = (n + a.page_size - 1) / a.page_size;
  const int d = a.d, nc = d / 8;
  const int R = a.G * a.n_active;
  for (int r0 = 0; r0 < R; r0 += 8) {
    const int nr = min(8, R - r0);
    __syncthreads();
    for (int w = threadIdx.x; w < nr * d; w += 256) {
      const int rr = w / d, j = w % d;
      const int r = r0 + rr;
      const int h = hk * a.G + r / a.n_active;
      const int tok = active[b * a.n_active + r % a.n_active];
      qs[rr][j] = load_elem(qc, (((int64_t)b * a.B + tok) * a.h_q + h) * d + j, a.bf16);
    }
    __syncthreads();
    if (p >= P) continue;
    double acc[8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) acc[rr] = 0.0;
    const int64_t mbase = (((int64_t)b * a.h_kv + hk) * nc) * a.max_pages * 8;
    for (int c = 0; c < nc; ++c) {
      const int64_t off = mbase + ((int64_t)c * a.max_pages + p) * 8;
      double kn[8], kx[8];
      if (a.bf16) {
        const u16x8 vn = *(const u16x8*)((const uint16_t*)kmin + off);
        const u16x8 vx = *(const u16x8*)((const uint16_t*)kmax + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kn[e] = (double)bf16_to_f32(vn[e]);
          kx[e] = (double)bf16_to_f32(vx[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kn[e] = (double)((const float*)kmin)[off + e];
          kx[e] = (double)((const float*)kmax)[off + e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          const double qv = qs[rr][c * 8 + e];
          acc[rr] = acc[rr] + qv * (qv >= 0.0 ? kx[e] : kn[e]);
        }
    }
    for (int rr = 0; rr < nr; ++rr) {
      const int r = r0 + rr;
      const int h = hk * a.G + r / a.n_active;
      const int ai = r % a.n_active;
      scores[(((int64_t)b * a.h_q + h) * a.n_active + ai) * a.max_pages + p] = acc[rr];
    }
  }
}

// One workgroup per (b, h, active row): exact top-k by (score desc, page asc) with an
// 8-pass MSB-first radix select on order-preserving 64-bit keys held in LDS; ties at the
// threshold go to the lowest page indices; output ascending, padded with -1.
__global__ void __launch_bounds__(256) topk_kernel(const LosaArgs a, const double* scores, int32_t* topk_pages) {
  __shared__ uint64_t key[16384];
  __shared__ int hist[257];
  __shared__ int scan[257];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  const int rid = blockIdx.x;                   // (b * h_q + h) * n_active + ai
  const int b = rid / (a.h_q * a.n_active);
  int seq0, n;
  seq_of(a, b, seq0, n);
  const int P = (n + a.page_size - 1) / a.page_size;
  const int K = a.topk;
  int32_t* out = topk_pages + (int64_t)rid * K;
  if (P <= K) {
    for (int t = threadIdx.x; t < K; t += 256) out[t] = t < P ? t : -1;
    return;
  }
  const double* sc = scores + (int64_t)rid * a.max_pages;
  for (int p = threadIdx.x; p < P; p += 256) key[p] = order_key(sc[p]);
  if (threadIdx.x == 0) {
    s_prefix = 0;
    s_need = K;
  }
  uint64_t pmask = 0;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int t = threadIdx.x; t < 256; t += 256) hist[t] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix;
    for (int p = threadIdx.x; p < P; p += 256)
      if ((key[p] & pmask) == prefix) atomicAdd(&hist[(key[p] >> shift) & 255], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
      int need = s_need, above = 0, dg = 255;
      for (; dg > 0; --dg) {
        if (above + hist[dg] >= need) break;
        above += hist[dg];
      }
      s_need = need - above;
      s_prefix = prefix | ((uint64_t)dg << shift);
    }
    pmask |= (uint64_t)255 << shift;
    __syncthreads();
  }
  const uint64_t T = s_prefix;
  const int need_eq = s_need;                    // keys equal to T to take, lowest pages first
  const int per = (P + 255) / 256;
  const int p0 = min(P, (int)threadIdx.x * per), p1 = min(P, p0 + per);
  int eq = 0, gt = 0;
  for (int p = p0; p < p1; ++p) {
    eq += key[p] == T;
    gt += key[p] > T;
  }
  const int eq_before = block_excl_scan(eq, scan);
  const int take_eq = max(0, min(eq, need_eq - eq_before));
  __syncthreads();
  int pos = block_excl_scan(gt + take_eq, scan);
  int te = take_eq;
  for (int p = p0; p < p1; ++p) {
    if (key[p] > T) {
      out[pos++] = p;
    } else if (key[p] == T && te > 0) {
      out[pos++] = p;
      --te;
    }
  }
}

// One workgroup per (b, h_kv): LDS bitmap of the group's selected pages, then an ascending
// compaction.
__global__ void __launch_bounds__(256) union_kernel(const LosaArgs a, const int32_t* topk_pages,
                                                    int32_t* union_pages, int32_t* union_count) {
  __shared__ uint32_t bits[16384 / 32];
  __shared__ int scan[257];
  const int b = blockIdx.x / a.h_kv, hk = blockIdx.x % a.h_kv;
  const int nw = (a.max_pages + 31) / 32;
  for (int t = threadIdx.x; t < nw; t += 256) bits[t] = 0u;
  __syncthreads();
  const int per_head = a.n_active * a.topk;
  const int32_t* src = topk_pages + ((int64_t)b * a.h_q + (int64_t)hk * a.G) * per_head;
  for (int t = threadIdx.x; t < a.G * per_head; t += 256) {
    const int p = src[t];
    if (p >= 0) atomicOr(&bits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  const int per = (nw + 255) / 256;
  const int w0 = min(nw, (int)threadIdx.x * per), w1 = min(nw, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  int pos = block_excl_scan(cnt, scan);
  const int total = scan[256];
  int32_t* out = union_pages + ((int64_t)b * a.h_kv + hk) * a.max_union;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      out[pos++] = w * 32 + bit;
    }
  }
  if (threadIdx.x == 0) union_count[b * a.h_kv + hk] = total;
}

hipError_t launch_page_meta(const LosaArgs& a, const void* k, void* kmin, void* kmax, hipStream_t st) {
  const int64_t n = (int64_t)(a.d / 8) * a.max_pages;
  dim3 grid((unsigned)((n + 255) / 256), a.h_kv, a.batch);
  hipLaunchKernelGGL(page_meta_kernel, grid, dim3(256), 0, st, a, k, kmin, kmax);
  return hipGetLastError();
}

hipError_t launch_locality(const LosaArgs& a, const void* qc, const void* qp, int32_t* active, hipStream_t st) {
  hipLaunchKernelGGL(locality_kernel, dim3(a.batch), dim3(1024), 0, st, a, qc, qp, active);
  return hipGetLastError();
}

hipError_t launch_quest_scores(const LosaArgs& a, const void* qc, const int32_t* active, const void* kmin,
                               const void* kmax, double* scores, hipStream_t st) {
  dim3 grid((unsigned)((a.max_pages + 255) / 256), a.h_kv, a.batch);
  hipLaunchKernelGGL(quest_score_kernel, grid, dim3(256), 0, st, a, qc, active, kmin, kmax, scores);
  return hipGetLastError();
}

hipError_t launch_topk(const LosaArgs& a, const double* scores, int32_t* topk_pages, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(a.batch * a.h_q * a.n_active)), dim3(256), 0, st, a, scores,
                     topk_pages);
  return hipGetLastError();
}

hipError_t launch_union(const LosaArgs& a, const int32_t* topk_pages, int32_t* union_pages, int32_t* union_count,
                        hipStream_t st) {
  hipLaunchKernelGGL(union_kernel, dim3((unsigned)(a.batch * a.h_kv)), dim3(256), 0, st, a, topk_pages,
                     union_pages, union_count);
  return hipGetLastError();
}

}  // namespace fb
