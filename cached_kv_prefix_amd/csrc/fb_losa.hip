// LoSA-style selection ("LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion
// Language Models", §2 "El Algoritmo LoSA"):
//   step 1  locality pruning: per-token mean squared change of the queries between two
//           denoising steps; the |A| largest form the active set (ties: lower index);
//   step 3  a QUEST-like page selector for the active queries only, then the union of the
//           selected pages per KV head (§1: the memory cost is the size of that union).
// The page score is the maximum of q.k over the page's per-dimension key box,
//   S = sum_d max(q_d kmin_d, q_d kmax_d) = sum_d q_d * (q_d >= 0 ? kmax_d : kmin_d).
// Every decision is taken in fp64 with sums in a fixed left-to-right order (per head
// over dims, then over heads, for the locality score; over dims for the page score), and
// the compiler may not contract a multiply and an add into one rounding, so the selected
// indices are exactly reproducible.  The page score's explicit two-FMA step is the one
// exception, and it rounds exactly as the plain sum does (see quest_score_kernel).
#include "fb_device.hpp"
#include "fb_internal.hpp"
#include <type_traits>

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


}  // namespace

// kmin/kmax layout [batch][h_kv][d/8][max_pages][8]: consecutive pages of one 8-dim chunk
// are adjacent, so the score kernel reads them with unit-stride 16-byte (bf16) loads.
// tail > 0: only the pages that hold one of the last `tail` tokens of each sequence (the
// grid covers `span` pages from the first of them); tail == 0: every page (span = max_pages).
__global__ void __launch_bounds__(256) page_meta_kernel(const LosaArgs a, const void* k, void* kmin, void* kmax,
                                                        int tail, int span) {
  const int b = blockIdx.z, hk = blockIdx.y;
  const int nc = a.d / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)nc * span) return;
  int seq0, n;
  seq_of(a, b, seq0, n);
  const int c = idx / span;
  const int p = (tail > 0 ? max(0, n - tail) / a.page_size : 0) + (int)(idx % span);
  const int t0 = p * a.page_size;
  if (p >= a.max_pages || t0 >= n) return;
  const int t1 = min(n, t0 + a.page_size);
  float mn[8], mx[8];
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_inff();
    mx[e] = -__builtin_inff();
  }
  for (int t = t0; t < t1; ++t) {
    const int64_t base = ((int64_t)(seq0 + t) * a.h_kv + hk) * a.d + c * 8;
    float x[8];
    if (a.bf16) {
      const u16x8 v = *(const u16x8*)((const uint16_t*)k + base);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ((const float*)k)[base + e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = fminf(mn[e], x[e]);
      mx[e] = fmaxf(mx[e], x[e]);
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

// Locality score, part 1: one wave per (sequence, token).  Lane h forms its head's sum
// over d, left to right, of the squared query change in fp64 (both queries are exact in
// fp64 and so is their difference); the heads' sums are then added in head order and the
// total is divided by H d, exactly as the definition is written.
__global__ void __launch_bounds__(64) locality_kernel(const LosaArgs a, const void* qc, const void* qp,
                                                      double* loc) {
  __shared__ double inner[1024];
  const int i = blockIdx.x, b = blockIdx.y;
  const int H = a.h_q, d = a.d, lane = threadIdx.x;
  for (int h = lane; h < H; h += 64) {
    const int64_t base = (((int64_t)b * a.B + i) * H + h) * d;
    double acc = 0.0;
    if (a.bf16 && d <= 128) {
      // the whole row of both queries in flight at once
      u16x8 xc[16], xp[16];
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if (8 * c < d) {
          xc[c] = *(const u16x8*)((const uint16_t*)qc + base + 8 * c);
          xp[c] = *(const u16x8*)((const uint16_t*)qp + base + 8 * c);
        }
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if (8 * c < d)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double df = (double)bf16_to_f32(xc[c][e]) - (double)bf16_to_f32(xp[c][e]);
            acc = acc + df * df;
          }
    } else {
      for (int j = 0; j < d; ++j) {
        const double df = load_elem(qc, base + j, a.bf16) - load_elem(qp, base + j, a.bf16);
        acc = acc + df * df;
      }
    }
    inner[h] = acc;
  }
  __syncthreads();
  if (lane == 0) {
    double t = 0.0;
    for (int h = 0; h < H; ++h) t = t + inner[h];
    loc[(int64_t)b * a.B + i] = t / (double)(H * d);
  }
}

// Locality score, part 2: the active set of sequence b, the n_active largest scores (ties
// to the lower token), listed ascending.  A workgroup of 256 threads ranks every score
// against all B of them; sc and sel are LDS arrays of at least B entries.  The list goes to
// act_lds (LDS, when set) and to active (global, when set).  Ends with a barrier.
__device__ __forceinline__ void rank_active(const LosaArgs& a, const double* loc, int b, double* sc, int* sel,
                                            int* act_lds, int32_t* active) {
  const int B = a.B;
  if (B <= 64) {   // one score per lane; every wave ranks them alike and wave 0 writes the list
    const int lane = threadIdx.x & 63;
    const double si = lane < B ? loc[(int64_t)b * B + lane] : 0.0;
    const int64_t bits = __builtin_bit_cast(int64_t, si);
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int lo = __builtin_amdgcn_readlane((int)(uint32_t)bits, j);
      const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)bits >> 32), j);
      const double sj = __builtin_bit_cast(double, ((int64_t)hi << 32) | (uint32_t)lo);
      rank += (sj > si || (sj == si && j < lane)) ? 1 : 0;
    }
    const bool take = lane < B && rank < a.n_active;
    const uint64_t m = __ballot(take);
    const int pos = __popcll(m & ((1ull << lane) - 1));
    if (take && threadIdx.x < 64) {
      if (act_lds) act_lds[pos] = lane;
      if (active) active[b * a.n_active + pos] = lane;
    }
    __syncthreads();
    return;
  }
  for (int i = threadIdx.x; i < B; i += 256) sc[i] = loc[(int64_t)b * B + i];
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += 256) {
    const double si = sc[i];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const double sj = sc[j];
      rank += (sj > si || (sj == si && j < i)) ? 1 : 0;
    }
    sel[i] = rank < a.n_active ? 1 : 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += 256) {
    if (!sel[i]) continue;
    int pos = 0;
    for (int j = 0; j < i; ++j) pos += sel[j];
    if (act_lds) act_lds[pos] = i;
    if (active) active[b * a.n_active + pos] = i;
  }
  __syncthreads();
}

// Blocks of more than kRankInQuest tokens: the active sets in a launch of their own.
__global__ void __launch_bounds__(256) active_kernel(const LosaArgs a, const double* loc, int32_t* active) {
  __shared__ double sc[1024];
  __shared__ int sel[1024];
  rank_active(a, loc, blockIdx.x, sc, sel, nullptr, active);
}

// QUEST page scores.  grid (page blocks of 128 * kQpp, h_kv, batch), 256 threads.  Lane l
// of wave w scores pages ((blockIdx.x * 4 + w) * 32 + (l & 31)) * kQpp + 0 .. kQpp-1 for rows
// 4 (l >> 5) .. 4 (l >> 5) + 3 of the current chunk of 8 active rows, so the two halves of a
// wave read the same metadata (one fetch) and each fp64 pair of q read from LDS feeds
// 2 kQpp FMAs.  With q+ = max(q, 0) and q- = min(q, 0) (held in LDS as fp64 pairs),
//   acc + q * (q >= 0 ? kmax : kmin) == fma(q-, kmin, fma(q+, kmax, acc))
// exactly: one of the two products is zero, the other is exact in fp64 and rounds once, as
// in the left-to-right fp64 sum over d of the definition.
constexpr int kQpp = 2;   // pages per thread: 114 VGPRs, 4 waves per SIMD (4 pages: 202, 2 waves, 4 us slower per step)
constexpr int kRankInQuest = 256;   // blocks up to this size rank their active set inside the QUEST launch
constexpr int kQRow = 257;   // LDS row stride (pairs): the two half-waves' rows fall in different banks
template <bool BF16>
// With loc set (blocks of at most kRankInQuest tokens), every workgroup ranks its
// sequence's locality scores itself, and workgroup (0, 0, b) writes the active list, which
// the later launches of the step read; otherwise `active` holds the list already.
__global__ void __launch_bounds__(256) quest_score_kernel(const LosaArgs a, const void* qc, const double* loc,
                                                          int32_t* active, const void* kmin, const void* kmax,
                                                          double* scores) {
  __shared__ __attribute__((aligned(16))) double qpn[8][kQRow][2];
  __shared__ double rank_sc[kRankInQuest];
  __shared__ int rank_sel[kRankInQuest], act_lds[kRankInQuest];
  const int b = blockIdx.z, hk = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, rg = lane >> 5;
  const int p0 = ((blockIdx.x * 4 + w) * 32 + (lane & 31)) * kQpp;
  int seq0, n;
  seq_of(a, b, seq0, n);
  const int P = (n + a.page_size - 1) / a.page_size;
  const int d = a.d, nc = d / 8;
  const int R = a.G * a.n_active;
  const int64_t mbase = (((int64_t)b * a.h_kv + hk) * nc) * a.max_pages * 8;
  // Metadata of chunk c for this thread's pages (clamped to the last page: always in range),
  // kept raw (bf16: one 16-byte vector per page) and widened where it is used.
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  typedef typename std::conditional<BF16, u32x4, f32x8>::type Raw;
  auto load_meta = [&](const void* m, int c, int u) -> Raw {
    const int64_t off = mbase + ((int64_t)c * a.max_pages + min(p0 + u, P - 1)) * 8;
    if constexpr (BF16)
      return *(const u32x4*)((const uint16_t*)m + off);
    else
      return *(const f32x8*)((const float*)m + off);
  };
  auto elem = [&](const Raw& x, int e) -> double {
    if constexpr (BF16)
      return (double)__uint_as_float((e & 1) ? (x[e >> 1] & 0xffff0000u) : (x[e >> 1] << 16));
    else
      return (double)x[e];
  };
  // The first chunk's metadata does not depend on the rows: it is in flight while the
  // active set is ranked and the first rows of q are staged.
  Raw mn[kQpp], mx[kQpp];
  auto load_first = [&]() {
#pragma unroll
    for (int u = 0; u < kQpp; ++u) {
      mn[u] = load_meta(kmin, 0, u);
      mx[u] = load_meta(kmax, 0, u);
    }
  };
  if (p0 < P) load_first();
  if (loc) rank_active(a, loc, b, rank_sc, rank_sel, act_lds, blockIdx.x == 0 && blockIdx.y == 0 ? active : nullptr);
  for (int r0 = 0; r0 < R; r0 += 8) {
    const int nr = min(8, R - r0);
    __syncthreads();
    for (int t = threadIdx.x; t < 8 * d; t += 256) {
      const int rr = t / d, j = t % d;
      double q = 0.0;
      if (rr < nr) {
        const int r = r0 + rr;
        const int h = hk * a.G + r / a.n_active;
        const int tok = loc ? act_lds[r % a.n_active] : active[b * a.n_active + r % a.n_active];
        q = load_elem(qc, (((int64_t)b * a.B + tok) * a.h_q + h) * d + j, a.bf16);
      }
      qpn[rr][j][0] = q > 0.0 ? q : 0.0;
      qpn[rr][j][1] = q < 0.0 ? q : 0.0;
    }
    __syncthreads();
    if (p0 >= P) continue;
    double acc[kQpp][4];
#pragma unroll
    for (int u = 0; u < kQpp; ++u)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[u][rr] = 0.0;
    if (r0 > 0) load_first();
    for (int c = 0; c < nc; ++c) {
      Raw cn[kQpp], cx[kQpp];
#pragma unroll
      for (int u = 0; u < kQpp; ++u) {
        cn[u] = mn[u];
        cx[u] = mx[u];
      }
      if (c + 1 < nc) {   // the next chunk's metadata is in flight while this one is scored
#pragma unroll
        for (int u = 0; u < kQpp; ++u) {
          mn[u] = load_meta(kmin, c + 1, u);
          mx[u] = load_meta(kmax, c + 1, u);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double kn[kQpp], kx[kQpp];
#pragma unroll
        for (int u = 0; u < kQpp; ++u) {
          kn[u] = elem(cn[u], e);
          kx[u] = elem(cx[u], e);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const double qp_ = qpn[4 * rg + rr][c * 8 + e][0], qn_ = qpn[4 * rg + rr][c * 8 + e][1];
#pragma unroll
          for (int u = 0; u < kQpp; ++u) acc[u][rr] = __builtin_fma(qn_, kn[u], __builtin_fma(qp_, kx[u], acc[u][rr]));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kQpp; ++u) {
      if (p0 + u >= P) continue;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        if (4 * rg + rr >= nr) continue;
        const int r = r0 + 4 * rg + rr;
        const int h = hk * a.G + r / a.n_active;
        const int ai = r % a.n_active;
        scores[(((int64_t)b * a.h_q + h) * a.n_active + ai) * a.max_pages + p0 + u] = acc[u][rr];
      }
    }
  }
}

__device__ __forceinline__ uint64_t wave_and64(uint64_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, o), hi = __shfl_xor((uint32_t)(x >> 32), o);
    x &= ((uint64_t)hi << 32) | lo;
  }
  return x;
}
__device__ __forceinline__ uint64_t wave_or64(uint64_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, o), hi = __shfl_xor((uint32_t)(x >> 32), o);
    x |= ((uint64_t)hi << 32) | lo;
  }
  return x;
}

// Exact top-k by (score desc, page asc) with an MSB-first radix select (8-bit digits) on
// order-preserving 64-bit keys.  Thread t holds keys t + 256 j, j < N, of which those below
// `limit` are real (at least K of them).
// Leading bytes common to all keys are skipped; each remaining pass builds a 256-bucket
// histogram of the keys that match the prefix so far, and a block scan over the buckets
// (highest digit first) picks the digit of the k-th largest key.  The passes stop as soon
// as the bucket holding it is exactly what is still needed.  On return: the selected keys
// are those with (key & pmask) > prefix, plus `need` of those with (key & pmask) == prefix
// (lowest pages first).
struct TopkShared {
  int hist[256];
  int tmp[4];
  int digit, above, count;
  unsigned long long kand, kor;
};

template <int N>
__device__ __forceinline__ void radix_select(const uint64_t (&key)[N], int limit, int K, TopkShared& sh,
                                             uint64_t& prefix_out, uint64_t& pmask_out, int& need_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) {
    sh.kand = ~0ull;
    sh.kor = 0ull;
  }
  __syncthreads();
  {
    uint64_t ka = ~0ull, ko = 0ull;
#pragma unroll
    for (int j = 0; j < N; ++j)
      if (tid + 256 * j < limit) {
        ka &= key[j];
        ko |= key[j];
      }
    ka = wave_and64(ka);
    ko = wave_or64(ko);
    if (lane == 0) {
      atomicAnd(&sh.kand, (unsigned long long)ka);
      atomicOr(&sh.kor, (unsigned long long)ko);
    }
  }
  __syncthreads();
  const uint64_t diff = sh.kand ^ sh.kor;
  int pass0 = 0;
  while (pass0 < 8 && ((diff >> (56 - 8 * pass0)) & 255) == 0) ++pass0;
  uint64_t pmask = pass0 == 0 ? 0ull : (pass0 == 8 ? ~0ull : ~0ull << (64 - 8 * pass0));
  uint64_t prefix = sh.kand & pmask;
  int need = K;
  for (int pass = pass0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    sh.hist[tid] = 0;
    __syncthreads();
    // when every matching lane of a wave has the same digit (common in the leading
    // passes) the wave adds its count with one atomic
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const bool match = tid + 256 * j < limit && (key[j] & pmask) == prefix;
      const int dg = (int)((key[j] >> shift) & 255);
      const uint64_t m = __ballot(match);
      if (m) {
        const int leader = __ffsll((unsigned long long)m) - 1;
        const int ldg = __builtin_amdgcn_readlane(dg, leader);
        if (__ballot(match && dg == ldg) == m) {
          if (lane == leader) atomicAdd(&sh.hist[ldg], (int)__popcll(m));
        } else if (match) {
          atomicAdd(&sh.hist[dg], 1);
        }
      }
    }
    __syncthreads();
    // thread t looks at digit 255 - t: inclusive count of keys with a digit >= 255 - t
    const int c = sh.hist[255 - tid];
    int total;
    const int cum = block_incl_scan(c, sh.tmp, &total);
    if (cum >= need && cum - c < need) {
      sh.digit = 255 - tid;
      sh.above = cum - c;
      sh.count = c;
    }
    __syncthreads();
    need -= sh.above;
    prefix |= (uint64_t)sh.digit << shift;
    pmask |= (uint64_t)255 << shift;
    const bool whole = sh.count == need;          // the bucket is exactly what is still needed
    __syncthreads();
    if (whole) break;
  }
  prefix_out = prefix;
  pmask_out = pmask;
  need_out = need;
}

// One workgroup per (b, h, active row).  Thread t holds the keys of pages t + 256 j in
// registers (coalesced loads).
//   * Fast path (k <= 256): the radix select first runs over the per-thread maxima, one
//     key per thread, and T is the prefix it settles on with its lower bits clear.  T is
//     at most the k-th largest maximum, which is at most the k-th largest key (k distinct
//     maxima are at least as large), so every selected key, ties included, is >= T.  The
//     keys >= T (a few hundred on most inputs) are gathered in LDS and the radix select
//     runs again over at most 4 per thread.  Both of its runs touch far fewer keys than
//     one pass over all of them, whose LDS histogram atomics dominate the full path.
//   * Otherwise (or when more than kTopkCap keys are >= T, as with many equal scores) the
//     radix select runs over all the keys.
// The selection is then two LDS bitmaps over the pages (keys above the selected bucket,
// keys equal to it): equal keys are taken lowest pages first, and the result is compacted
// in ascending page order.  Fewer than k pages: all of them, padded with -1.
constexpr int kTopkCap = 1024;
template <int KPT>
__global__ void __launch_bounds__(256) topk_kernel(const LosaArgs a, const double* scores, int32_t* topk_pages) {
  constexpr int NW = 4 * KPT;                   // 64-page words of the bitmaps
  constexpr int KC = kTopkCap / 256;            // candidate slots per thread
  __shared__ TopkShared sh;
  __shared__ uint64_t gt_bits[NW], eq_bits[NW];
  __shared__ uint64_t c_key[kTopkCap];
  __shared__ int c_page[kTopkCap];
  const int rid = blockIdx.x;                   // (b * h_q + h) * n_active + ai
  const int b = rid / (a.h_q * a.n_active);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int seq0, n;
  seq_of(a, b, seq0, n);
  const int P = (n + a.page_size - 1) / a.page_size;
  const int K = a.topk;
  int32_t* out = topk_pages + (int64_t)rid * K;
  if (P <= K) {
    for (int t = tid; t < K; t += 256) out[t] = t < P ? t : -1;
    return;
  }
  const double* sc = scores + (int64_t)rid * a.max_pages;
  uint64_t key[KPT];
  // unconditional loads (clamped index), so that all of them are in flight at once
  double raw[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) raw[j] = sc[min(tid + 256 * j, P - 1)];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = tid + 256 * j < P ? order_key(raw[j]) : 0ull;
  for (int i = tid; i < NW; i += 256) {
    gt_bits[i] = 0ull;
    eq_bits[i] = 0ull;
  }

  // ---- fast path: candidates >= T ----------------------------------------------------
  bool fast = false;
  uint64_t prefix = 0, pmask = 0;
  int need = 0;
  if (K <= 256) {
    // thread t has keys iff t < P, and P > K: at least K maxima
    uint64_t mt[1] = {0ull};
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (tid + 256 * j < P) mt[0] = key[j] > mt[0] ? key[j] : mt[0];
    uint64_t tprefix, tmask;
    int tneed;
    radix_select<1>(mt, P < 256 ? P : 256, K, sh, tprefix, tmask, tneed);
    {
      const uint64_t T = tprefix;   // the bits below tmask are clear
      int c = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) c += tid + 256 * j < P && key[j] >= T ? 1 : 0;
      int total;
      int o = block_incl_scan(c, sh.tmp, &total) - c;
      if (total <= kTopkCap) {   // uniform
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (tid + 256 * j < P && key[j] >= T) {
            c_key[o] = key[j];
            c_page[o] = tid + 256 * j;
            ++o;
          }
        __syncthreads();
        uint64_t ck[KC];
        int cpg[KC];
#pragma unroll
        for (int i = 0; i < KC; ++i) {
          const int idx = tid + 256 * i;
          ck[i] = idx < total ? c_key[idx] : 0ull;
          cpg[i] = idx < total ? c_page[idx] : 0;
        }
        radix_select<KC>(ck, total, K, sh, prefix, pmask, need);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
          if (tid + 256 * i >= total) continue;
          const uint64_t km = ck[i] & pmask;
          const unsigned long long bit = 1ull << (cpg[i] & 63);
          if (km > prefix) atomicOr((unsigned long long*)&gt_bits[cpg[i] >> 6], bit);
          else if (km == prefix) atomicOr((unsigned long long*)&eq_bits[cpg[i] >> 6], bit);
        }
        fast = true;
      }
    }
  }
  if (!fast) {
    // ---- all keys -----------------------------------------------------------------------
    radix_select<KPT>(key, P, K, sh, prefix, pmask, need);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = tid + 256 * j < P;
      const uint64_t km = key[j] & pmask;
      const uint64_t g = __ballot(ok && km > prefix), e = __ballot(ok && km == prefix);
      if (lane == 0) {
        gt_bits[4 * j + w] = g;
        eq_bits[4 * j + w] = e;
      }
    }
  }
  __syncthreads();
  // word t (pages 64 t ..): equal keys before it, then this word's share of them
  const int wi = tid < NW ? tid : 0;
  const uint64_t eqw = tid < NW ? eq_bits[wi] : 0ull;
  int total;
  const int eq_before = block_incl_scan(__popcll(eqw), sh.tmp, &total) - __popcll(eqw);
  uint64_t take = 0ull;
  {
    int left = need - eq_before;
    uint64_t m = eqw;
    while (left > 0 && m) {
      const uint64_t low = m & (~m + 1);
      take |= low;
      m ^= low;
      --left;
    }
  }
  const uint64_t selw = (tid < NW ? gt_bits[wi] : 0ull) | take;
  int pos = block_incl_scan(__popcll(selw), sh.tmp, &total) - __popcll(selw);
  uint64_t m = selw;
  while (m) {
    const int bit = __ffsll((unsigned long long)m) - 1;
    m &= m - 1;
    out[pos++] = 64 * tid + bit;
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
  int total;
  int pos = block_incl_scan(cnt, scan, &total) - cnt;
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

hipError_t launch_page_meta(const LosaArgs& a, const void* k, void* kmin, void* kmax, int tail, hipStream_t st) {
  // pages holding the last `tail` tokens: at most ceil(tail / P) + 1 of them
  const int span = tail > 0 ? min(a.max_pages, (tail + a.page_size - 1) / a.page_size + 1) : a.max_pages;
  const int64_t n = (int64_t)(a.d / 8) * span;
  dim3 grid((unsigned)((n + 255) / 256), a.h_kv, a.batch);
  hipLaunchKernelGGL(page_meta_kernel, grid, dim3(256), 0, st, a, k, kmin, kmax, tail, span);
  return hipGetLastError();
}

hipError_t launch_locality(const LosaArgs& a, const void* qc, const void* qp, double* loc, int32_t* active,
                           hipStream_t st) {
  hipLaunchKernelGGL(locality_kernel, dim3(a.B, a.batch), dim3(64), 0, st, a, qc, qp, loc);
  if (hipError_t e = hipGetLastError()) return e;
  if (a.B <= kRankInQuest) return hipSuccess;   // ranked inside the QUEST launch
  hipLaunchKernelGGL(active_kernel, dim3(a.batch), dim3(256), 0, st, a, loc, active);
  return hipGetLastError();
}

hipError_t launch_quest_scores(const LosaArgs& a, const void* qc, const double* loc, int32_t* active,
                               const void* kmin, const void* kmax, double* scores, hipStream_t st) {
  dim3 grid((unsigned)((a.max_pages + 128 * kQpp - 1) / (128 * kQpp)), a.h_kv, a.batch);
  const double* rank_loc = a.B <= kRankInQuest ? loc : nullptr;
  if (a.bf16)
    hipLaunchKernelGGL(quest_score_kernel<true>, grid, dim3(256), 0, st, a, qc, rank_loc, active, kmin, kmax,
                       scores);
  else
    hipLaunchKernelGGL(quest_score_kernel<false>, grid, dim3(256), 0, st, a, qc, rank_loc, active, kmin, kmax,
                       scores);
  return hipGetLastError();
}

hipError_t launch_topk(const LosaArgs& a, const double* scores, int32_t* topk_pages, hipStream_t st) {
  const dim3 grid((unsigned)(a.batch * a.h_q * a.n_active));
  if (a.max_pages <= 256 * 32)
    hipLaunchKernelGGL(topk_kernel<32>, grid, dim3(256), 0, st, a, scores, topk_pages);
  else
    hipLaunchKernelGGL(topk_kernel<64>, grid, dim3(256), 0, st, a, scores, topk_pages);
  return hipGetLastError();
}

hipError_t launch_union(const LosaArgs& a, const int32_t* topk_pages, int32_t* union_pages, int32_t* union_count,
                        hipStream_t st) {
  hipLaunchKernelGGL(union_kernel, dim3((unsigned)(a.batch * a.h_kv)), dim3(256), 0, st, a, topk_pages,
                     union_pages, union_count);
  return hipGetLastError();
}

}  // namespace fb
