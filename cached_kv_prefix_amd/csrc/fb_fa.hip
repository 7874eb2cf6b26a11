// Query-tiled attention for query groups of more than 32 rows: the video-sized block and
// its prefix pass (4680 rows per head, a dense contraction bound by the matrix cores),
// grouped-query prefixes (4 query heads x 32 block tokens share each K / V tile), 64-row
// blocks, the paged selected / complement passes of the sparse-residual step and the
// multi-branch pass.  Same split-KV partial-result format as the other attention
// kernels; fb_combine.hip reduces the chunks and merges.
//
// What is computed ("Resumo Técnico: FlashBlock", §2 Mecanismo Central): for the query
// rows of one (sequence, KV head) group and one key chunk, base-2 running statistics
//   m = max_j s_j,  l = sum_j 2^(s_j - m),  O = sum_j 2^(s_j - m) v_j,  s_j = log2(e) scale <q, k_j>.
//
// gfx950 design:
//   * a workgroup = W waves owns 32 * W * QT query rows (QT = 1); a wave owns 32 * QT rows;
//   * keys advance in 64-key tiles, double-buffered in LDS and shared by the W waves: the
//     next tiles are loaded into registers (16-byte row pieces, buffer loads) while the
//     current one is computed, then written to the other LDS buffer; one barrier per tile;
//   * groups of more than 128 rows (W = 8, matrix-bound): software pipeline, S of tile
//     t + 1 is issued before the softmax of tile t, so the matrix instructions and the
//     vector softmax of one wave are independent.  The two waves of a SIMD run the same
//     mix in step (one barrier per tile), so the softmax (about half the matrix time)
//     mostly adds to the matrix work: the kernel reaches about 0.4 of the bf16 peak;
//   * groups of 33-128 rows (W = 4, DEEP, memory-bound): no score pipelining, two tiles of
//     loads in flight (two register staging sets);
//   * a paged source (DEEP only, power-of-two pages): the chunk's page list is staged in
//     LDS once; each load piece computes its token offset without branches, and a key
//     past the chunk or a token outside the sequence gets an out-of-range offset (reads
//     zero) and is masked by the tile's validity ballot;
//   * packed queries (PACKED, DEEP only: the multi-branch pass, every branch padded to the
//     longest block): a wave whose rows are all padding of its branch loads its share of
//     each tile and meets every barrier but runs no matrix or softmax work and writes no
//     partial, so short branches cost memory time only;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K rows chunk-swizzled by key & 15 for
//     conflict-free ds_read_b128); softmax in registers, one query per lane; O^T = V^T P^T
//     with V^T from ds_read_b64_tr_b16 (V rows swizzled by key & 3);
//   * work items (source, split, group, query tile) are one flat grid, prefix items first:
//     they are the long ones, so the short block items fill in behind them.
#include "fb_attn_common.hpp"


namespace fb {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 fa_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

constexpr int kFaTile = 64;                 // keys per LDS tile
constexpr int kFaTileBytes = kFaTile * 256; // K (or V) bytes of one tile at d = 128

}  // namespace

// Items of one source: n_splits * batch * h_kv * qtiles, query tile fastest.
__device__ __forceinline__ int fa_qtiles(const AttnSrc& S, int rows_per_wg) {
  return (S.rows + rows_per_wg - 1) / rows_per_wg;
}

template <int QT, int W, bool DEEP, bool PAGED, bool PACKED>
__global__ void __launch_bounds__(64 * W, QT == 1 && W == 4 ? 2 : 1) attn_fa_kernel(const AttnArgs A) {
  constexpr int D = 128;
  constexpr int ROWS_WG = 32 * W * QT;
  constexpr int NP = 16 / W;                    // 16-byte pieces per thread per K (or V) tile
  static_assert(!PAGED || DEEP, "paged sources run on the deep-prefetch variant");
  static_assert(!PACKED || (DEEP && !PAGED), "packed queries run on the contiguous deep-prefetch variant");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2 * kFaTileBytes];   // [buf][K | V]
  __shared__ int32_t pl_lds[PAGED ? kFaMaxChunkPages : 1];                         // the chunk's pages

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ql = lane & 31;

  // ---- work item ----------------------------------------------------------------------
  int id = blockIdx.x;
  const int qt0 = fa_qtiles(A.src0, ROWS_WG);
  const int n0 = A.src0.n_splits * A.batch * A.h_kv * qt0;
  const bool second = id >= n0;
  const AttnSrc& S = second ? A.src1 : A.src0;
  if (second) id -= n0;
  const int qtn = second ? fa_qtiles(A.src1, ROWS_WG) : qt0;
  const int qt = id % qtn;
  id /= qtn;
  const int hk = id % A.h_kv;
  id /= A.h_kv;
  const int b = id % A.batch;
  const int split = id / A.batch;

  const SeqInfo si = seq_info(S, b, hk, A.h_kv);
  const int kbeg = split * S.chunk;
  if (kbeg >= si.n_keys) return;
  const int kend = min(si.n_keys, kbeg + S.chunk);
  const int rows = S.rows;
  const int r0 = qt * ROWS_WG;
  const int r1 = min(rows, r0 + ROWS_WG);
  if (S.m_upd) {
    if (S.m_upd[b] < S.tau) return;
  } else if (S.mask) {
    bool any = false;
    for (int j = r0 / S.rows_per_head; j <= (r1 - 1) / S.rows_per_head; ++j)
      any |= S.mask[b * A.h_q + hk * A.G + j] == 0;
    if (!any) return;
  }

  // ---- query fragments (B operand of S^T = K Q^T): lane holds d = 16 i2 + 8 g + 0..7 ----
  bf16x8 qf[QT][D / 16];
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    const int row = r0 + w * 32 * QT + 32 * qi + ql;
    if (row < rows) {
      const int j = row / S.rows_per_head, i = row % S.rows_per_head;
      const int tok = S.row_tok ? S.row_tok[b * S.rows_per_head + i] : i;
      const uint16_t* qp = (const uint16_t*)A.q + ((int64_t)(b * A.B + tok) * A.h_q + hk * A.G + j) * D + 8 * g;
#pragma unroll
      for (int i2 = 0; i2 < D / 16; ++i2) qf[qi][i2] = *(const bf16x8*)(qp + 16 * i2);
    } else {
#pragma unroll
      for (int i2 = 0; i2 < D / 16; ++i2) qf[qi][i2] = bf16x8{};
    }
  }

  // Packed queries: a wave whose rows are all padding (row i >= the branch's query count)
  // takes its share of the K / V tile loads and barriers but computes and writes nothing.
  bool wave_on = true;
  if constexpr (PACKED) {
    const int nb = S.cu_q[b + 1] - S.cu_q[b];
    bool lane_on = false;
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      const int row = r0 + w * 32 * QT + 32 * qi + ql;
      lane_on |= row < rows && row % S.rows_per_head < nb;
    }
    wave_on = __builtin_amdgcn_readfirstlane((int)(__ballot(lane_on) != 0)) != 0;
  }

  // ---- K / V tiles: thread piece u = row (tid >> 4) + 16 u, 16-byte chunk tid & 15 ------
  // Contiguous source: the buffer resources start at the chunk, and rows past the chunk
  // end read as zero.  Paged source (power-of-two page size 2^sh): they start at the
  // sequence, key `key` of the chunk is token pages[key >> sh] * 2^sh + (key & (2^sh - 1)),
  // and a key past the chunk end or a token past the sequence end is given the offset
  // nrec, which reads as zero; such keys are masked out of the softmax by the tile's
  // validity mask.
  const int64_t tstride = (int64_t)A.h_kv * D;
  const int tok0 = PAGED ? 0 : kbeg;
  const uint16_t* kbase = (const uint16_t*)S.k + ((int64_t)si.seq0 + tok0) * tstride + hk * D;
  const uint16_t* vbase = (const uint16_t*)S.v + ((int64_t)si.seq0 + tok0) * tstride + hk * D;
  const int nrec = ((PAGED ? si.n_seq : kend) - tok0) * (int)tstride * 2;
  int sh = 0, pbase = 0, npl = 1;
  if constexpr (PAGED) {
    sh = __builtin_ctz(S.page_size);
    pbase = kbeg >> sh;
    npl = ((kend - 1) >> sh) - pbase + 1;
    const int32_t* pg = S.pages + (int64_t)(b * A.h_kv + hk) * S.max_union + pbase;
    for (int i = tid; i < npl; i += 64 * W) pl_lds[i] = pg[i];
    __syncthreads();
  }
  const int pmask = (1 << sh) - 1;
  // Token of chunk key `key` >= kbeg, branch-free: keys past the chunk end read the last
  // staged page (the caller discards them).
  // A page index outside [0, n_seq >> sh] gives -1 (checked before the shift, which could
  // overflow), which every caller treats as outside the sequence.
  const int pg_lim = si.n_seq >> sh;
  auto paged_tok = [&](int key) -> int {
    const int pg = pl_lds[min((key >> sh) - pbase, npl - 1)];
    return (unsigned)pg <= (unsigned)pg_lim ? (pg << sh) + (key & pmask) : -1;
  };
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, nrec, 0x00020000);
  // A deep (memory-bound) item is the only reader of its K / V tiles: non-temporal loads.
  // The wide (matrix-bound) items of one group share each tile across their query tiles,
  // which the caches serve: plain loads (the non-temporal hint measured 4% slower there).
  constexpr int kPol = DEEP ? kKvLoadPolicy : 0;
  const int p_row = tid >> 4, p_chunk = tid & 15;
  const int g_off = (p_row * (int)tstride + p_chunk * 8) * 2;           // + 4 W u rows per piece
  const int g_step = 4 * W * (int)tstride * 2;
  // LDS: K row r chunk c at r*256 + ((c ^ (r & 15)) << 4); V row r at r*256 + ((c ^ 4 (r & 3)) << 4).
  int k_dst[NP], v_dst[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int r = p_row + 4 * W * u;
    k_dst[u] = r * 256 + ((p_chunk ^ (r & 15)) << 4);
    v_dst[u] = r * 256 + ((p_chunk ^ (4 * (r & 3))) << 4);
  }
  u32x4 kreg[2][NP], vreg[2][NP];   // two staging sets (the second one only when DEEP)
  int poff[NP];                      // paged: byte offsets of this thread's pieces of one tile
  const int ntile = (kend - kbeg + kFaTile - 1) / kFaTile;

  // Paged piece offsets of tile T (shared by its K and V loads).
#define FA_POFF(T)                                                                               \
  if constexpr (PAGED) {                                                                         \
    _Pragma("unroll") for (int u = 0; u < NP; ++u) {                                             \
      const int key_ = kbeg + (T) * kFaTile + p_row + 4 * W * u;                                 \
      const int tok_ = paged_tok(key_);                                                          \
      poff[u] = key_ < kend && (unsigned)tok_ < (unsigned)si.n_seq ? tok_ * (int)tstride * 2 + p_chunk * 16 : nrec; \
    }                                                                                            \
  }
#define FA_OFF(T, U) (PAGED ? poff[U] : (T) * kFaTile * (int)tstride * 2 + g_off + (U) * g_step)
  // Buffer loads: rows past the chunk end read as zero (and fetch nothing).
#define FA_LOAD_K(T, SET)                                                                        \
  _Pragma("unroll") for (int u = 0; u < NP; ++u) kreg[SET][u] = __builtin_bit_cast(u32x4,        \
      __builtin_amdgcn_raw_buffer_load_b128(krs, FA_OFF(T, u), 0, kPol));
#define FA_LOAD_V(T, SET)                                                                        \
  _Pragma("unroll") for (int u = 0; u < NP; ++u) vreg[SET][u] = __builtin_bit_cast(u32x4,        \
      __builtin_amdgcn_raw_buffer_load_b128(vrs, FA_OFF(T, u), 0, kPol));
#define FA_STORE_K(BUF, SET) _Pragma("unroll") for (int u = 0; u < NP; ++u) *(u32x4*)(lds[BUF] + k_dst[u]) = kreg[SET][u];
#define FA_STORE_V(BUF, SET) _Pragma("unroll") for (int u = 0; u < NP; ++u) *(u32x4*)(lds[BUF] + kFaTileBytes + v_dst[u]) = vreg[SET][u];

  // K operand read: key 32 s + ql, chunk 2 i2 + g -> stored chunk (2 i2) ^ (g ^ (ql & 15)).
  const int k_src = ql * 256;
  const int k_x = g ^ (ql & 15);
  // Transposed V read: 16-lane group (g, tr_h), position 4 tr_j + tr_q.
  const int tr_h = (lane >> 4) & 1, tr_j = (lane & 15) >> 2, tr_q = lane & 3;
  const int tr_base = (4 * g + tr_j) * 256 + (tr_q & 1) * 8;
  int tr_off[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) tr_off[t] = (4 * (t ^ tr_j) + 2 * tr_h + (tr_q >> 1)) * 16;

  float m_run[QT], l_run[QT];
  f32x16 o[QT][D / 32];
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    m_run[qi] = kNegInf;
    l_run[qi] = 0.f;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) o[qi][t] = f32x16{};
  }

  // S^T of one tile (two 32-key halves) from a K buffer.
#define FA_QK(ACC, KT)                                                                           \
  _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                                \
    _Pragma("unroll") for (int qi = 0; qi < QT; ++qi) ACC[qi][s] = f32x16{};                     \
    _Pragma("unroll") for (int i2 = 0; i2 < D / 16; ++i2) {                                      \
      const bf16x8 ka = *(const bf16x8*)((KT) + s * 32 * 256 + k_src + (((2 * i2) ^ k_x) << 4)); \
      _Pragma("unroll") for (int qi = 0; qi < QT; ++qi)                                          \
        ACC[qi][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qi][i2], ACC[qi][s], 0, 0, 0); \
    }                                                                                            \
  }
  // Online softmax of a tile's scores into bf16 P (B operand of O^T = V^T P^T), with the
  // lazy reference max: it is raised only when a score exceeds it by more than 2^8.
#define FA_SOFTMAX(ACC, PB)                                                                      \
  _Pragma("unroll") for (int qi = 0; qi < QT; ++qi) {                                            \
    float mx = kNegInf;                                                                          \
    _Pragma("unroll") for (int s = 0; s < 2; ++s)                                                \
      _Pragma("unroll") for (int r = 0; r < 16; ++r) mx = fmaxf(mx, ACC[qi][s][r]);              \
    mx = wave_max_xor32(mx) * A.scale_log2;                                                      \
    const bool need = mx > m_run[qi] + 8.0f;                                                     \
    if (__any(need)) {                                                                           \
      const float m_new = need ? mx : m_run[qi];                                                 \
      const float alpha = exp2_or_zero(m_run[qi] - m_new);                                       \
      l_run[qi] *= alpha;                                                                        \
      _Pragma("unroll") for (int d4 = 0; d4 < D / 32; ++d4) o[qi][d4] *= alpha;                  \
      m_run[qi] = m_new;                                                                         \
    }                                                                                            \
    const float m_use = m_run[qi] == kNegInf ? 0.f : m_run[qi];                                  \
    float ps = 0.f;                                                                              \
    _Pragma("unroll") for (int s = 0; s < 2; ++s)                                                \
      _Pragma("unroll") for (int c = 0; c < 2; ++c)                                              \
        _Pragma("unroll") for (int jj = 0; jj < 8; ++jj) {                                       \
          const float p_ = fast_exp2(fmaf(ACC[qi][s][8 * c + jj], A.scale_log2, -m_use));        \
          ps += p_;                                                                              \
          PB[qi][2 * s + c][jj] = (__bf16)p_;                                                    \
        }                                                                                        \
    ps = wave_add_xor32(ps);                                                                     \
    l_run[qi] += ps;                                                                             \
  }
  // O^T += V^T P^T: k-step (s, c) covers keys 32 s + 16 c + 8 (j >> 2) + 4 g + (j & 3).
#define FA_PV(PB, VT)                                                                            \
  _Pragma("unroll") for (int s = 0; s < 2; ++s)                                                  \
    _Pragma("unroll") for (int c = 0; c < 2; ++c) {                                              \
      const unsigned char* a_ = (VT) + s * 32 * 256 + c * 16 * 256 + tr_base;                    \
      _Pragma("unroll") for (int d4 = 0; d4 < D / 32; ++d4) {                                    \
        const s16x4 lo = fa_read_tr(a_ + tr_off[d4]);                                            \
        const s16x4 hi = fa_read_tr(a_ + 8 * 256 + tr_off[d4]);                                  \
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)); \
        _Pragma("unroll") for (int qi = 0; qi < QT; ++qi)                                        \
          o[qi][d4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, PB[qi][2 * s + c], o[qi][d4], 0, 0, 0); \
      }                                                                                          \
    }

  // Software pipeline: iteration t computes S of tile t + 1 while it runs the softmax and
  // P V of tile t (independent work the scheduler interleaves), so K is one tile ahead of V.
  // LDS buffer i holds a K tile and a V tile.  At the start of iteration t: K(t+1) in
  // buffer (t+1)&1, V(t) in buffer t&1; the iteration loads K(t+2) into buffer t&1 and
  // V(t+1) into buffer (t+1)&1, both last read in iteration t - 1.
  // Every tile but the last is full, so the loop body has no masking; the last tile is
  // finished after the loop.  The loop is unrolled by two so that the two score sets
  // swap roles without register copies.
  bf16x8 pb[QT][4];
  if constexpr (DEEP) {
    // Memory-bound groups (a few query tiles per K / V tile): no score pipelining, but two
    // tiles of loads in flight.  Iteration t loads tile t + 2 into staging set t&1,
    // computes tile t from LDS buffer t&1, then stores tile t + 1 (loaded an iteration
    // earlier) into buffer (t+1)&1, last read in iteration t - 1; one barrier per tile.
    f32x16 acc[QT][2];
#define FA_DEEP_ITER(T, CUR)                                                                     \
  {                                                                                              \
    FA_POFF((T) + 2);                                                                            \
    FA_LOAD_K((T) + 2, CUR);                                                                     \
    FA_LOAD_V((T) + 2, CUR);                                                                     \
    uint64_t vm_ = ~0ull;                                                                        \
    if constexpr (PAGED) {   /* validity of the tile's keys: lane = key */                       \
      const int key_ = kbeg + (T) * kFaTile + lane;                                              \
      vm_ = __ballot(key_ < kend && (unsigned)paged_tok(key_) < (unsigned)si.n_seq);             \
    }                                                                                            \
    if (!PACKED || wave_on) {                                                                    \
    FA_QK(acc, lds[CUR]);                                                                        \
    if (PAGED && vm_ != ~0ull) {   /* register r of half s holds key 32 s + 8 (r >> 2) + 4 g + (r & 3) */ \
      _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                            \
        const uint32_t wg_ = (uint32_t)(vm_ >> (32 * s)) >> (4 * g);                             \
        _Pragma("unroll") for (int r = 0; r < 16; ++r)                                           \
          if (!((wg_ >> (8 * (r >> 2) + (r & 3))) & 1u))                                         \
            _Pragma("unroll") for (int qi = 0; qi < QT; ++qi) acc[qi][s][r] = kNegInf;           \
      }                                                                                          \
    } else if (!PAGED && (T) == ntile - 1) {                                                     \
      const int kvalid = kend - kbeg - (T) * kFaTile;                                            \
      if (kvalid < kFaTile)                                                                      \
        _Pragma("unroll") for (int s = 0; s < 2; ++s)                                            \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                       \
            const int key = 32 * s + 8 * (r >> 2) + 4 * g + (r & 3);                             \
            if (key >= kvalid) _Pragma("unroll") for (int qi = 0; qi < QT; ++qi) acc[qi][s][r] = kNegInf; \
          }                                                                                      \
    }                                                                                            \
    FA_SOFTMAX(acc, pb);                                                                         \
    FA_PV(pb, lds[CUR] + kFaTileBytes);                                                          \
    }                                                                                            \
    FA_STORE_K((CUR) ^ 1, (CUR) ^ 1);                                                            \
    FA_STORE_V((CUR) ^ 1, (CUR) ^ 1);                                                            \
    __syncthreads();                                                                             \
  }
    FA_POFF(0);
    FA_LOAD_K(0, 0);
    FA_LOAD_V(0, 0);
    FA_POFF(1);
    FA_LOAD_K(1, 1);
    FA_LOAD_V(1, 1);
    FA_STORE_K(0, 0);
    FA_STORE_V(0, 0);
    __syncthreads();
    int t = 0;
    for (; t + 1 < ntile; t += 2) {
      FA_DEEP_ITER(t, 0);
      FA_DEEP_ITER(t + 1, 1);
    }
    if (t < ntile) FA_DEEP_ITER(t, 0);
#undef FA_DEEP_ITER
  } else {
  f32x16 acc[QT][2], acc_n[QT][2];
  FA_LOAD_K(0, 0);
  FA_LOAD_V(0, 0);
  FA_STORE_K(0, 0);
  FA_STORE_V(0, 0);
  FA_LOAD_K(1, 0);
  FA_STORE_K(1, 0);
  __syncthreads();
  FA_QK(acc, lds[0]);
  __syncthreads();   // K buffer 0 is rewritten in iteration 0
#define FA_ITER(T, CUR, ACC_C, ACC_N)                                                            \
  {                                                                                              \
    FA_LOAD_K((T) + 2, 0);                                                                       \
    FA_LOAD_V((T) + 1, 0);                                                                       \
    FA_QK(ACC_N, lds[(CUR) ^ 1]);                                                                \
    FA_SOFTMAX(ACC_C, pb);                                                                       \
    FA_PV(pb, lds[CUR] + kFaTileBytes);                                                          \
    FA_STORE_K(CUR, 0);                                                                          \
    FA_STORE_V((CUR) ^ 1, 0);                                                                    \
    __syncthreads();                                                                             \
  }
  int t = 0;
  for (; t + 2 < ntile; t += 2) {
    FA_ITER(t, 0, acc, acc_n);
    FA_ITER(t + 1, 1, acc_n, acc);
  }
  if (t + 1 < ntile) {
    FA_ITER(t, 0, acc, acc_n);
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
      acc[qi][0] = acc_n[qi][0];
      acc[qi][1] = acc_n[qi][1];
    }
  }
#undef FA_ITER
  {
    // last tile: keys past the chunk end are masked
    const int kvalid = kend - kbeg - (ntile - 1) * kFaTile;
    if (kvalid < kFaTile) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * s + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= kvalid)
#pragma unroll
            for (int qi = 0; qi < QT; ++qi) acc[qi][s][r] = kNegInf;
        }
    }
    FA_SOFTMAX(acc, pb);
    FA_PV(pb, lds[(ntile - 1) & 1] + kFaTileBytes);
  }
  }
#undef FA_POFF
#undef FA_OFF
#undef FA_LOAD_K
#undef FA_LOAD_V
#undef FA_STORE_K
#undef FA_STORE_V
#undef FA_QK
#undef FA_SOFTMAX
#undef FA_PV

  // ---- partial results: O^T tile d4, lane (g, ql) holds d = 32 d4 + 8 r4 + 4 g + 0..3 ----
  const int64_t slot = (int64_t)(b * A.h_kv + hk) * S.n_splits + split;
  float* po = S.po + slot * (int64_t)rows * D;
  float* pml = S.pml + slot * (int64_t)rows * 2;
#pragma unroll
  for (int qi = 0; qi < QT; ++qi) {
    const int row = r0 + w * 32 * QT + 32 * qi + ql;
    if (row >= rows || (PACKED && !wave_on)) continue;
#pragma unroll
    for (int d4 = 0; d4 < D / 32; ++d4)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
        x[0] = o[qi][d4][4 * r4 + 0];
        x[1] = o[qi][d4][4 * r4 + 1];
        x[2] = o[qi][d4][4 * r4 + 2];
        x[3] = o[qi][d4][4 * r4 + 3];
        *(f32x4*)(po + (int64_t)row * D + 32 * d4 + 8 * r4 + 4 * g) = x;
      }
    if (g == 0) {
      pml[row * 2 + 0] = m_run[qi];
      pml[row * 2 + 1] = l_run[qi];
    }
  }
}

// bf16, d = 128, chunks whole 64-key tiles apart; the K offsets of one chunk (contiguous)
// or one sequence (paged) are 32-bit.  A paged source needs a power-of-two page size, at
// most 128 rows (the deep-prefetch variant) and a chunk page list that fits in LDS.
bool fa_ok(const AttnArgs& a, const AttnSrc& s) {
  if (s.n_splits == 0) return true;
  if (a.d != 128) return false;
  if (s.pages) {
    const int P = s.page_size;
    if (P < 1 || (P & (P - 1)) || fa_waves(s.rows) != 4) return false;
    if (s.chunk / P + 2 > kFaMaxChunkPages) return false;
    return (int64_t)a.max_seqlen * a.h_kv * 128 * 2 < ((int64_t)1 << 31);
  }
  return (int64_t)s.chunk * a.h_kv * 128 * 2 < ((int64_t)1 << 31);
}

hipError_t launch_fa(const AttnArgs& a, hipStream_t st) {
  const int rows = a.src0.n_splits ? a.src0.rows : a.src1.rows;
  const int64_t rows_wg = fa_rows_per_item(rows);
  auto items = [&](const AttnSrc& s) -> int64_t {
    return s.n_splits ? (int64_t)s.n_splits * a.batch * a.h_kv * ((s.rows + rows_wg - 1) / rows_wg) : 0;
  };
  const int64_t n = items(a.src0) + items(a.src1);
  if (n == 0) return hipSuccess;
  if (n >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  // both sources of a launch are paged (selected / complement pages) or neither is
  const bool paged = (a.src0.n_splits ? a.src0.pages : a.src1.pages) != nullptr;
  if (a.src0.n_splits && a.src1.n_splits && (a.src0.pages != nullptr) != (a.src1.pages != nullptr))
    return hipErrorInvalidValue;
  if (paged && fa_waves(rows) != 4) return hipErrorInvalidValue;
  // up to 128 rows the pass streams K / V (deep prefetch); larger groups are matrix bound
  // packed queries (one source, no pages): waves of padding rows skip their compute
  const bool packed = a.src0.cu_q != nullptr && a.src1.n_splits == 0 && !paged;
  if (paged)
    hipLaunchKernelGGL((attn_fa_kernel<kFaQt, 4, true, true, false>), dim3((unsigned)n), dim3(256), 0, st, a);
  else if (fa_waves(rows) == 4 && packed)
    hipLaunchKernelGGL((attn_fa_kernel<kFaQt, 4, true, false, true>), dim3((unsigned)n), dim3(256), 0, st, a);
  else if (fa_waves(rows) == 4)
    hipLaunchKernelGGL((attn_fa_kernel<kFaQt, 4, true, false, false>), dim3((unsigned)n), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fa_kernel<kFaQt, 8, false, false, false>), dim3((unsigned)n), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace fb
