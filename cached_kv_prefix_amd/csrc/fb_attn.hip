// Split-KV attention partials: the generic kernels behind the streaming and query-tiled
// ones (bf16 with d = 64, fp32 inputs, paged sources with pages of fewer than 16 tokens
// or groups of more than 128 rows) and the dispatch between the three.
//
// What is computed ("Resumo Técnico: FlashBlock", §2 Mecanismo Central; "LoSA", §2 step 3):
// for every query row of a (sequence, KV head) group and one contiguous chunk of that
// group's keys, the running softmax statistics of the chunk in base 2,
//     m = max_j s_j,  l = sum_j 2^(s_j - m),  O = sum_j 2^(s_j - m) v_j,
// with s_j = log2(e) * scale * <q, k_j>.  A second kernel (fb_combine.hip) reduces the
// chunks and applies the log-space merge.
//
// gfx950 design (bf16):
//   * one workgroup = 4 waves = one (sequence, KV head, query group, key chunk) item;
//   * keys stream through LDS in 128-key tiles (K and V rows padded to 2d+16 bytes); every
//     thread keeps the next tile's 16-byte chunks in registers while the waves compute on
//     the current tile, so HBM loads overlap the MFMA work;
//   * a wave owns 32 query rows; the waves that share a query tile (4 with 32 rows per
//     group, 2 with 64, 1 with >= 128) take the chunk's 32-key sub-tiles round-robin;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys x queries), so a lane holds one query
//     and 16 keys: the row max needs one cross-half exchange; P stays in registers and is
//     the B operand of O^T = V^T P^T, whose A operand reads V columns from LDS;
//   * the waves that share query rows are combined through LDS before one partial per
//     row is written.
#include "fb_attn_common.hpp"

namespace fb {

namespace {

// True when this item has work: the chunk is inside the key range and (with a reuse
// mask) at least one query head covered by the workgroup recomputes.
__device__ __forceinline__ bool item_live(const AttnArgs& A, const AttnSrc& S, int b, int hk,
                                          int wg_row0, int wg_rows) {
  if (S.m_upd) return S.m_upd[b] >= S.tau;
  if (!S.mask) return true;
  const int j0 = wg_row0 / S.rows_per_head;
  const int j1 = (wg_row0 + wg_rows - 1) / S.rows_per_head;
  for (int j = j0; j <= j1; ++j)
    if (S.mask[b * A.h_q + hk * A.G + j] == 0) return true;
  return false;
}

}  // namespace

#ifndef FB_ATTN_KT
#define FB_ATTN_KT 128                 // keys per LDS tile
#endif
#ifndef FB_ATTN_OCC
#define FB_ATTN_OCC 2                  // workgroups per CU the register budget targets
#endif
#ifndef FB_GRID_HEAD_MAJOR
#define FB_GRID_HEAD_MAJOR 1           // consecutive workgroups take consecutive heads
#endif

// Work item of a workgroup: (source split, KV head x query group, sequence).  With the
// head-major order, workgroups resident at the same time spread over all KV heads, whose
// rows interleave in memory, instead of walking one head's rows.
struct Item {
  int x, y;
};
__device__ __forceinline__ Item item_of(int heads_groups) {
#if FB_GRID_HEAD_MAJOR
  return Item{(int)blockIdx.y, (int)blockIdx.x};
#else
  (void)heads_groups;
  return Item{(int)blockIdx.x, (int)blockIdx.y};
#endif
}

template <int D>
__global__ void __launch_bounds__(256, FB_ATTN_OCC) attn_bf16_kernel(const AttnArgs A) {
  constexpr int KT = FB_ATTN_KT;       // keys per LDS tile
  constexpr int ROWB = 2 * D + 16;     // padded LDS row (bytes)
  constexpr int CPR = (2 * D) / 16;    // 16-byte chunks per key row
  constexpr int KPP = 256 / CPR;       // key rows covered by one pass of the workgroup
  constexpr int NCH = KT / KPP;        // chunks per thread per tile (K and V each)
  constexpr int NI = D / 16;           // MFMA steps along d for S
  constexpr int NT = D / 32;           // 32-wide output tiles along d
  constexpr int TILE_BYTES = 2 * KT * ROWB;
  constexpr int RED_BYTES = 4 * 32 * D * 4 + 2 * 4 * 32 * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES];
  __shared__ uint8_t kvalid[KT];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, ql = lane & 31;
  const Item it = item_of(0);
  const bool second = it.x >= A.src0.n_splits;
  const AttnSrc& S = second ? A.src1 : A.src0;
  const int split = second ? it.x - A.src0.n_splits : it.x;
  const int b = blockIdx.z;
  const int hk = it.y % A.h_kv;
  const int qg = it.y / A.h_kv;
  if (qg >= S.qgroups) return;
  const SeqInfo si = seq_info(S, b, hk, A.h_kv);
  const int kbeg = split * S.chunk;
  if (kbeg >= si.n_keys) return;
  const int kend = min(si.n_keys, kbeg + S.chunk);
  const int tq = S.tq, ks = 4 / tq;
  const int wg_row0 = qg * 32 * tq;
  const int wg_rows = min(S.rows - wg_row0, 32 * tq);
  if (!item_live(A, S, b, hk, wg_row0, wg_rows)) return;

  const int qt = w / ks, slice = w % ks;
  const bool wave_active = qt * 32 < wg_rows;
  const int row = wg_row0 + qt * 32 + ql;

  // Query fragment (B operand of S^T = K Q^T): lane holds d = 16*i + 8*g + 0..7.
  bf16x8 qf[NI];
  if (wave_active && row < S.rows) {
    const int j = row / S.rows_per_head, i = row % S.rows_per_head;
    const int tok = S.row_tok ? S.row_tok[b * S.rows_per_head + i] : i;
    const int h = hk * A.G + j;
    const uint16_t* qp = (const uint16_t*)A.q + ((int64_t)(b * A.B + tok) * A.h_q + h) * D + 8 * g;
#pragma unroll
    for (int i2 = 0; i2 < NI; ++i2) qf[i2] = *(const bf16x8*)(qp + 16 * i2);
  } else {
#pragma unroll
    for (int i2 = 0; i2 < NI; ++i2) qf[i2] = bf16x8{};
  }

  const int64_t tstride = (int64_t)A.h_kv * D;
  const uint16_t* kbase = (const uint16_t*)S.k + (int64_t)si.seq0 * tstride + hk * D;
  const uint16_t* vbase = (const uint16_t*)S.v + (int64_t)si.seq0 * tstride + hk * D;
  const int32_t* pg = S.pages ? S.pages + (int64_t)(b * A.h_kv + hk) * S.max_union : nullptr;
  const int col = tid % CPR, krow0 = tid / CPR;

  u32x4 rk[NCH], rv[NCH];
  uint32_t okm = 0;
#define FB_LOAD_TILE(T0)                                                              \
  do {                                                                                \
    okm = 0;                                                                          \
    _Pragma("unroll") for (int c = 0; c < NCH; ++c) {                                 \
      bool ok;                                                                        \
      const int tok = key_token(S, pg, (T0) + krow0 + c * KPP, kend, si.n_seq, ok);   \
      okm |= (uint32_t)ok << c;                                                       \
      rk[c] = *(const u32x4*)(kbase + tok * tstride + col * 8);                       \
      rv[c] = *(const u32x4*)(vbase + tok * tstride + col * 8);                       \
    }                                                                                 \
  } while (0)

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x16{};

  const int ntiles = (kend - kbeg + KT - 1) / KT;
  FB_LOAD_TILE(kbeg);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int kr = krow0 + c * KPP;
      *(u32x4*)(smem + kr * ROWB + col * 16) = rk[c];
      *(u32x4*)(smem + KT * ROWB + kr * ROWB + col * 16) = rv[c];
      if (col == 0) kvalid[kr] = (okm >> c) & 1u;
    }
    __syncthreads();
    if (t + 1 < ntiles) FB_LOAD_TILE(kbeg + (t + 1) * KT);
    if (!wave_active) continue;
    for (int st = 0; st < KT / 32; ++st) {
      // 32-key sub-tiles of the chunk are dealt round-robin to the ks waves of a query tile
      if ((t * (KT / 32) + st) % ks != slice) continue;
      const int kb = st * 32;
      if (kbeg + t * KT + kb >= kend) break;
      f32x16 acc = f32x16{};
      const unsigned char* kr = smem + (kb + ql) * ROWB + 16 * g;
#pragma unroll
      for (int i2 = 0; i2 < NI; ++i2) {
        const bf16x8 a = *(const bf16x8*)(kr + 32 * i2);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i2], acc, 0, 0, 0);
      }
      // acc[r] = S^T[key = kb + 8*(r/4) + 4*g + r%4][query = ql]
      float sv[16];
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
        const float x = kvalid[key] ? acc[r] * A.scale_log2 : kNegInf;
        sv[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = wave_max_xor32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] = fast_exp2(sv[r] - m_use);
        ps += sv[r];
      }
      ps = wave_add_xor32(ps);
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) o[tt] *= alpha;
      const unsigned char* vt = smem + KT * ROWB;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = (__bf16)sv[8 * c + j];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          bf16x8 va;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int key = kb + 16 * c + 8 * (j >> 2) + 4 * g + (j & 3);
            va[j] = *(const __bf16*)(vt + key * ROWB + (32 * tt + ql) * 2);
          }
          o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[tt], 0, 0, 0);
        }
      }
    }
  }

#undef FB_LOAD_TILE
  // Combine the waves that share query rows, then write one partial per row.
  __syncthreads();
  float* red = (float*)smem;
  float* red_m = red + 4 * 32 * D;
  float* red_l = red_m + 4 * 32;
  if (g == 0) {
    red_m[w * 32 + ql] = wave_active ? m_run : kNegInf;
    red_l[w * 32 + ql] = wave_active ? l_run : 0.f;
  }
  __syncthreads();
  {
    float M = kNegInf;
    for (int s = 0; s < ks; ++s) M = fmaxf(M, red_m[(qt * ks + s) * 32 + ql]);
    const float Mu = M == kNegInf ? 0.f : M;
    const float f = wave_active ? exp2_or_zero(m_run - Mu) : 0.f;
    float* dst = red + (w * 32 + ql) * D;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
        x[0] = o[tt][4 * r4 + 0] * f;
        x[1] = o[tt][4 * r4 + 1] * f;
        x[2] = o[tt][4 * r4 + 2] * f;
        x[3] = o[tt][4 * r4 + 3] * f;
        *(f32x4*)(dst + 32 * tt + 8 * r4 + 4 * g) = x;
      }
  }
  __syncthreads();
  const int64_t slot = (int64_t)(b * A.h_kv + hk) * S.n_splits + split;
  float* po = S.po + slot * S.rows * D;
  float* pml = S.pml + slot * S.rows * 2;
  for (int idx = tid; idx < wg_rows * (D / 4); idx += 256) {
    const int rl = idx / (D / 4), c4 = idx % (D / 4);
    const int qt2 = rl >> 5, q2 = rl & 31;
    f32x4 sum = f32x4{};
    for (int s = 0; s < ks; ++s) sum += *(const f32x4*)(red + ((qt2 * ks + s) * 32 + q2) * D + 4 * c4);
    *(f32x4*)(po + (int64_t)(wg_row0 + rl) * D + 4 * c4) = sum;
  }
  for (int rl = tid; rl < wg_rows; rl += 256) {
    const int qt2 = rl >> 5, q2 = rl & 31;
    float M = kNegInf;
    for (int s = 0; s < ks; ++s) M = fmaxf(M, red_m[(qt2 * ks + s) * 32 + q2]);
    const float Mu = M == kNegInf ? 0.f : M;
    float l = 0.f;
    for (int s = 0; s < ks; ++s) l += exp2_or_zero(red_m[(qt2 * ks + s) * 32 + q2] - Mu) * red_l[(qt2 * ks + s) * 32 + q2];
    pml[(wg_row0 + rl) * 2 + 0] = M;
    pml[(wg_row0 + rl) * 2 + 1] = l;
  }
}

// fp32 inputs: one wave per query row, lanes split the head dimension; the score of each
// key is a butterfly sum (identical on every lane), then the same online update.
__global__ void __launch_bounds__(256) attn_f32_kernel(const AttnArgs A) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const Item it = item_of(0);
  const bool second = it.x >= A.src0.n_splits;
  const AttnSrc& S = second ? A.src1 : A.src0;
  const int split = second ? it.x - A.src0.n_splits : it.x;
  const int b = blockIdx.z;
  const int hk = it.y % A.h_kv;
  const int qg = it.y / A.h_kv;
  if (qg >= S.qgroups) return;
  const SeqInfo si = seq_info(S, b, hk, A.h_kv);
  const int kbeg = split * S.chunk;
  if (kbeg >= si.n_keys) return;
  const int kend = min(si.n_keys, kbeg + S.chunk);
  const int wg_row0 = qg * 32;
  const int wg_rows = min(S.rows - wg_row0, 32);
  if (!item_live(A, S, b, hk, wg_row0, wg_rows)) return;
  const int D = A.d;
  const int64_t tstride = (int64_t)A.h_kv * D;
  const float* kbase = (const float*)S.k + (int64_t)si.seq0 * tstride + hk * D;
  const float* vbase = (const float*)S.v + (int64_t)si.seq0 * tstride + hk * D;
  const int32_t* pg = S.pages ? S.pages + (int64_t)(b * A.h_kv + hk) * S.max_union : nullptr;
  const int64_t slot = (int64_t)(b * A.h_kv + hk) * S.n_splits + split;

  for (int rl = w; rl < wg_rows; rl += 4) {
    const int row = wg_row0 + rl;
    const int j = row / S.rows_per_head, i = row % S.rows_per_head;
    const int tok = S.row_tok ? S.row_tok[b * S.rows_per_head + i] : i;
    const int h = hk * A.G + j;
    const float* qp = (const float*)A.q + ((int64_t)(b * A.B + tok) * A.h_q + h) * D;
    float qd[4], od[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dd = lane + 64 * e;
      qd[e] = dd < D ? qp[dd] : 0.f;
      od[e] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    for (int key = kbeg; key < kend; ++key) {
      bool ok;
      const int t = key_token(S, pg, key, kend, si.n_seq, ok);
      const float* kp = kbase + t * tstride;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = lane + 64 * e;
        if (dd < D) part = fmaf(qd[e], kp[dd], part);
      }
      float s = wave_sum(part) * A.scale_log2;
      if (!ok) s = kNegInf;
      const float m_new = fmaxf(m, s);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      const float p = fast_exp2(s - m_use);
      l = l * alpha + p;
      m = m_new;
      const float* vp = vbase + t * tstride;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = lane + 64 * e;
        if (dd < D) od[e] = od[e] * alpha + p * vp[dd];
      }
    }
    float* po = S.po + (slot * S.rows + row) * D;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dd = lane + 64 * e;
      if (dd < D) po[dd] = od[e];
    }
    if (lane == 0) {
      S.pml[(slot * S.rows + row) * 2 + 0] = m;
      S.pml[(slot * S.rows + row) * 2 + 1] = l;
    }
  }
}

namespace {
hipError_t launch_generic(const AttnArgs& a, bool bf16, hipStream_t st) {
  const int gx = a.src0.n_splits + a.src1.n_splits;
  const int qgroups = a.src0.qgroups > a.src1.qgroups ? a.src0.qgroups : a.src1.qgroups;
  if (gx == 0 || qgroups == 0) return hipSuccess;
#if FB_GRID_HEAD_MAJOR
  dim3 grid(a.h_kv * qgroups, gx, a.batch);
#else
  dim3 grid(gx, a.h_kv * qgroups, a.batch);
#endif
  if (bf16) {
    if (a.d == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}
}  // namespace

// bf16 groups of more than 32 rows go to the query-tiled kernel (fb_fa.hip), groups of at
// most 32 rows to the streaming kernel (fb_stream.hip), the rest to the LDS-tiled kernel
// above.  A launch whose sources differ in kind (paged / contiguous) is split into one
// launch per source.
hipError_t launch_attn(const AttnArgs& a, bool bf16, hipStream_t st) {
  const bool mixed = a.src0.n_splits > 0 && a.src1.n_splits > 0 &&
                     (a.src0.pages != nullptr) != (a.src1.pages != nullptr);
  if (mixed) {
    AttnArgs a0 = a, a1 = a;
    a0.src1.n_splits = 0;
    a0.src1.qgroups = 0;
    a1.src0.n_splits = 0;
    a1.src0.qgroups = 0;
    if (hipError_t e = launch_attn(a0, bf16, st)) return e;
    return launch_attn(a1, bf16, st);
  }
  if (bf16) {
    const int rows = a.src0.n_splits ? a.src0.rows : a.src1.rows;
    if (rows >= kFaMinRows && fa_ok(a, a.src0) && fa_ok(a, a.src1)) return launch_fa(a, st);
    if (stream_ok(a, a.src0, a.max_seqlen) && stream_ok(a, a.src1, a.max_seqlen)) return launch_stream(a, st);
  }
  return launch_generic(a, bf16, st);
}

}  // namespace fb
