// One output row of the split reduction and log-space merge, in two phases (issue every
// load of the row, then finish it), so that a wave can keep several rows in flight.
//
// Merge ("Resumo Técnico: FlashBlock", §2 Mecanismo Central, merge equation):
//   m = max(L_out, L_in); A = (e^{L_out-m} A_out + e^{L_in-m} A_in) / (e^{L_out-m} + e^{L_in-m})
// Reuse ("Resumo Técnico: FlashBlock", §2 Estratégias de Reutilização Adaptativa): a row
// whose head reuses reads the cached (A_out, L_out) and leaves it untouched; a recomputed
// row reduces its prefix chunks, writes the cache and merges the very values it wrote, so
// reuse and recompute on unchanged inputs give bit-identical outputs.
// LoSA ("LoSA", §2 steps 2 and 4): active rows take the sparse prefix result into the
// cache; stable rows reuse their cached statistics; every row merges with the block part.
// Sparse residual ("Resumo Técnico: FlashBlock", §2, Estratégias de Reutilização
// Adaptativa, "Compatibilidade com Atenção Esparsa"): the selected pages are attended to at every step, the residual over the
// unselected pages is refreshed into the cache or reused from it, and the three parts are
// merged in log space.
#pragma once
#include "fb_device.hpp"
#include "fb_internal.hpp"

namespace fb {

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

// State of one output row between issuing its loads and finishing it.  A wave handles
// one row at a time; the row index is wave-uniform, so the reuse inputs (flag, sequence
// length, active list) are scalar loads, which do not wait behind vector loads.  By
// default every partial load of the row (prefix, block, cached row) is issued before the
// reuse decision is known; with DECIDE (large launches, bound by bytes) the decision comes
// first and only the loads the row uses are issued.  Issuing several rows before
// finishing any keeps their round trips in flight together.
template <int E, int UP, int UB>
struct RowState {
  RowPartials<E, UP> PP;
  RowPartials<E, UB> PB;
  float cached[E], cached_l;
  int64_t roff, pslot0, bslot0;
  int rowid, b, i, h, hk, jg, prow, nk;
  bool fresh, valid;
};

// UP / UB: prefix / block chunks whose loads are issued up front (further chunks, if
// any, are read during the reduction).  DECIDE: read the reuse decision first and load
// only what the row uses (the prefix chunks of a recomputed row, the cached row of a
// reused one): one more round trip, but a large combine moves a third fewer bytes.
template <int E, int UP, int UB, bool DECIDE = false>
__device__ __forceinline__ void row_issue(const CombineArgs& C, int rowid, int lane, RowState<E, UP, UB>& st) {
  const int h = rowid % C.h_q;
  const int i = (rowid / C.h_q) % C.B;
  const int b = rowid / (C.h_q * C.B);
  const int hk = h / C.G, jg = h % C.G;
  const int d = C.d;
  st.rowid = rowid;
  st.b = b;
  st.i = i;
  st.h = h;
  st.hk = hk;
  st.jg = jg;
  st.roff = (int64_t)rowid * d;
  st.valid = true;
  if (C.cu_q) {   // packed variable-length queries: the output row is the packed one
    const int q0 = C.cu_q[b];
    st.valid = i < C.cu_q[b + 1] - q0;
    st.rowid = (q0 + i) * C.h_q + h;
    st.roff = (int64_t)st.rowid * d;
    if (!st.valid) return;   // a padded row: nothing is loaded or written
  }
  const bool has_prefix = C.mode != kModeBlockOnly;

  // the LoSA active list decides which partial row to read
  st.prow = jg * C.B + i;
  st.fresh = true;
  if (C.mode == kModeLosa) {
    int pos = -1;
    for (int a = 0; a < C.n_active; ++a)
      if (C.active[b * C.n_active + a] == i) pos = a;
    st.fresh = pos >= 0;
    st.prow = jg * C.n_active + (pos < 0 ? 0 : pos);
  }

  // the reuse inputs: read first with DECIDE, else while the partials are in flight
  auto read_reuse = [&]() {
    if (C.mode != kModeLosa) {
      if (C.m_upd)
        st.fresh = C.m_upd[b] >= C.tau;
      else if (C.mask)
        st.fresh = C.mask[b * C.h_q + h] == 0;
    }
  };
  if constexpr (DECIDE) read_reuse();

  // the partial loads (all of them without DECIDE)
  st.pslot0 = (int64_t)(b * C.h_kv + hk) * C.p_splits;
  st.bslot0 = (int64_t)(b * C.h_kv + hk) * C.b_splits;
  st.cached_l = kNegInf;
  if (has_prefix && C.p_splits > 0 && (!DECIDE || st.fresh))
    issue_partials<E, UP>(C.po, C.pml, st.pslot0, C.p_rows, st.prow, C.p_splits, d, lane, st.PP);
  if (C.mode != kModePrefixOnly && C.b_splits > 0)
    issue_partials<E, UB>(C.bo, C.bml, st.bslot0, C.b_rows, jg * C.B + i, C.b_splits, d, lane, st.PB);
  if (has_prefix && C.mode != kModePrefixOnly && (!DECIDE || !st.fresh || C.sim_parts)) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      st.cached[e] = dd < d ? C.cache_a[st.roff + dd] : 0.f;
    }
    st.cached_l = C.cache_l[st.rowid];   // the same (packed) row index as every other cache access
  }
  if constexpr (!DECIDE) read_reuse();
  st.nk = C.n_uniform;
  if (C.page_count)
    st.nk = C.page_count[b * C.h_kv + hk] * C.page_size;
  else if (C.cu)
    st.nk = C.cu[b + 1] - C.cu[b];
}

template <int E, int UP, int UB>
__device__ __forceinline__ void row_finish(const CombineArgs& C, int lane, const RowState<E, UP, UB>& st) {
  const int d = C.d;
  const bool has_prefix = C.mode != kModeBlockOnly;
  float ao[E], ai[E], af[E];
  float lo = kNegInf, li = kNegInf, lf;

  // block-external part
  if (has_prefix) {
    if (st.fresh) {
      const int n = C.p_splits > 0 ? min(n_chunks(st.nk, C.p_chunk), C.p_splits) : 0;
      reduce_chunks<E, UP>(st.PP, C.po, C.pml, st.pslot0, C.p_rows, st.prow, n, d, lane, ao, lo);
      float* ca = C.cache_a + st.roff;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int dd = lane + 64 * e;
        if (dd < d) ca[dd] = ao[e];
      }
      if (lane == 0) C.cache_l[st.rowid] = lo;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) ao[e] = st.cached[e];
      lo = st.cached_l;
    }
    if (C.mode == kModePrefixOnly) return;
    if (C.mask_out && st.i == 0 && lane == 0) C.mask_out[st.b * C.h_q + st.h] = st.fresh ? 0 : 1;
    if (C.sim_parts) {   // the row's share of the head's cosine between the cache before and after
      double xy = 0.0, xx = 0.0, yy = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double x = st.cached[e], y = ao[e];   // lanes past d hold zeros
        xy += x * y;
        xx += x * x;
        yy += y * y;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        xy += __shfl_xor(xy, o);
        xx += __shfl_xor(xx, o);
        yy += __shfl_xor(yy, o);
      }
      if (lane == 0) {
        double* sp = C.sim_parts + (int64_t)st.rowid * 3;
        sp[0] = xy;
        sp[1] = xx;
        sp[2] = yy;
      }
    }
  }

  // block-internal part
  {
    const int n = C.b_splits > 0 ? min(n_chunks(C.B, C.b_chunk), C.b_splits) : 0;
    reduce_chunks<E, UB>(st.PB, C.bo, C.bml, st.bslot0, C.b_rows, st.jg * C.B + st.i, n, d, lane, ai, li);
  }
  if (C.mode == kModeBlockOnly) {
    float* pa = C.ain + st.roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) pa[dd] = ai[e];
    }
    if (lane == 0) C.lin[st.rowid] = li;
    return;
  }

  merge_row<E>(ao, lo, ai, li, af, lf);
  if (C.out_bf16) {
    uint16_t* out = (uint16_t*)C.a_full + st.roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) out[dd] = f32_to_bf16(af[e]);
    }
  } else {
    float* out = (float*)C.a_full + st.roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) out[dd] = af[e];
    }
  }
  if (C.l_full && lane == 0) C.l_full[st.rowid] = lf;
}

// Three-way log-space merge of one row (the two-way merge with a third term):
//   m = max_i L_i, A = sum_i e^{L_i - m} A_i / sum_i e^{L_i - m}, L = m + ln sum_i e^{L_i - m}.
// Parts with L = -inf weigh nothing; all three empty gives 0 / -inf.
template <int E>
__device__ __forceinline__ void merge3_row(const float (&a1)[E], float l1, const float (&a2)[E], float l2,
                                           const float (&a3)[E], float l3, float (&af)[E], float& lf) {
  const float m = fmaxf(fmaxf(l1, l2), l3);
  if (m == kNegInf) {
#pragma unroll
    for (int e = 0; e < E; ++e) af[e] = 0.f;
    lf = kNegInf;
    return;
  }
  const float w1 = l1 == kNegInf ? 0.f : fast_exp2((l1 - m) * kLog2e);
  const float w2 = l2 == kNegInf ? 0.f : fast_exp2((l2 - m) * kLog2e);
  const float w3 = l3 == kNegInf ? 0.f : fast_exp2((l3 - m) * kLog2e);
  const float den = w1 + w2 + w3;
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < E; ++e) af[e] = (w1 * a1[e] + w2 * a2[e] + w3 * a3[e]) * inv;
  lf = m + fast_log2(den) * kLn2;
}

// Loads of the first min(nmax, U) chunks of one row, each behind a uniform guard (no
// redundant loads when the plan has fewer chunks than U).
template <int E, int U>
__device__ __forceinline__ void issue_partials_guarded(const float* po, const float* pml, int64_t slot0, int rows,
                                                       int row, int nmax, int d, int lane, RowPartials<E, U>& P) {
  const int sl = lane < nmax ? lane : 0;
  const float* ml = pml + ((slot0 + sl) * rows + row) * 2;
  P.m = ml[0];
  P.l = ml[1];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < nmax) {
      const int64_t r = (slot0 + u) * rows + row;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int dd = lane + 64 * e;
        P.x[u][e] = dd < d ? po[r * d + dd] : 0.f;
      }
    }
  }
}

// One row of the sparse-residual step.  The selected-page and block partials and the
// cached residual row are loaded before the refresh flag is known; the complement
// partials, which only a refreshing row uses, after it.  A refreshing row reduces its
// complement chunks, writes them to the cache and merges the very values it wrote, so
// refresh and reuse on unchanged inputs give bit-identical outputs.
template <int E, int UP, int UR, int UB>
__device__ __forceinline__ void residual_row(const CombineArgs& C, int rowid, int lane) {
  const int h = rowid % C.h_q;
  const int i = (rowid / C.h_q) % C.B;
  const int b = rowid / (C.h_q * C.B);
  const int hk = h / C.G, jg = h % C.G;
  const int d = C.d;
  const int64_t roff = (int64_t)rowid * d;
  const int prow = jg * C.B + i;
  const int64_t grp = (int64_t)b * C.h_kv + hk;

  RowPartials<E, UP> PS;
  RowPartials<E, UR> PR;
  RowPartials<E, UB> PB;
  const int64_t sslot0 = grp * C.p_splits, rslot0 = grp * C.r_splits, bslot0 = grp * C.b_splits;
  if (C.p_splits > 0) issue_partials_guarded<E, UP>(C.po, C.pml, sslot0, C.p_rows, prow, C.p_splits, d, lane, PS);
  if (C.b_splits > 0) issue_partials_guarded<E, UB>(C.bo, C.bml, bslot0, C.b_rows, prow, C.b_splits, d, lane, PB);
  float cached[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int dd = lane + 64 * e;
    cached[e] = dd < d ? C.cache_a[roff + dd] : 0.f;
  }
  const float cached_l = C.cache_l[rowid];
  const bool fresh = C.mask ? C.mask[b * C.h_q + h] == 0 : true;
  const int ns = C.page_count[grp] * C.page_size;
  if (fresh && C.r_splits > 0)
    issue_partials_guarded<E, UR>(C.ro, C.rml, rslot0, C.p_rows, prow, C.r_splits, d, lane, PR);

  float as[E], ar[E], ai[E], af[E];
  float ls, lr, li, lf;
  {
    const int n = C.p_splits > 0 ? min(n_chunks(ns, C.p_chunk), C.p_splits) : 0;
    reduce_chunks<E, UP>(PS, C.po, C.pml, sslot0, C.p_rows, prow, n, d, lane, as, ls);
  }
  if (fresh) {
    const int nr = C.r_page_count[grp] * C.page_size;
    const int n = C.r_splits > 0 ? min(n_chunks(nr, C.r_chunk), C.r_splits) : 0;
    reduce_chunks<E, UR>(PR, C.ro, C.rml, rslot0, C.p_rows, prow, n, d, lane, ar, lr);
    float* ca = C.cache_a + roff;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int dd = lane + 64 * e;
      if (dd < d) ca[dd] = ar[e];
    }
    if (lane == 0) C.cache_l[rowid] = lr;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) ar[e] = cached[e];
    lr = cached_l;
  }
  {
    const int n = C.b_splits > 0 ? min(n_chunks(C.B, C.b_chunk), C.b_splits) : 0;
    reduce_chunks<E, UB>(PB, C.bo, C.bml, bslot0, C.b_rows, prow, n, d, lane, ai, li);
  }
  merge3_row<E>(as, ls, ar, lr, ai, li, af, lf);
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

}  // namespace fb
