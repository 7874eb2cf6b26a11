// Streaming split-KV attention for query groups of at most 32 rows (the FlashBlock
// prefix pass of a dLLM block, the block pass at small B, the LoSA sparse pass over the
// union pages, and the selected / complement page passes of the sparse-residual step).
// Same partial-result format as fb_attn.hip.
//
// What is computed ("Resumo Técnico: FlashBlock", §2 Mecanismo Central; "LoSA", §2 step 3):
// for one (sequence, KV head) group and one key chunk, base-2 running statistics
//   m = max_j s_j,  l = sum_j 2^(s_j - m),  O = sum_j 2^(s_j - m) v_j,  s_j = log2(e) scale <q, k_j>.
//
// gfx950 design.  The pass reads every prefix key once and does ~32 flop per byte, so it
// is bound by HBM and the design goal is bytes in flight:
//   * the 4 waves of a workgroup are independent until the final combine; they walk the
//     chunk together in 32-key sub-tiles dealt round-robin (wave w takes sub-tiles w, w+4,
//     ...), so the workgroup reads one stream of consecutive rows (fewer, longer streams
//     keep HBM pages open longer than one stream per wave);
//   * each wave keeps NS sub-tiles in flight in registers (16 vector-memory operations
//     each; the per-wave counter holds 63).  K and V arrive the same way, as 16-byte row
//     pieces, four whole rows per instruction: loading K directly in the MFMA operand
//     layout (32 keys x 32 bytes per instruction) was measured to cost ~10% of the HBM
//     rate.  On reaching a sub-tile the wave writes both into its private LDS slots and
//     at once reuses the registers for the loads of sub-tile + NS.  Loads are buffer
//     loads: a plain load would let the optimiser fold the ring's loop-carried loads into
//     loads at their use, which drains the pipeline;
//   * the sub-tile sequence is straight-line code (TMAX steps, each entered only after
//     the previous one, with a uniform early exit) and every step issues the same loads
//     (past the end they fall outside the buffer resource and return zero without a
//     fetch), so the compiler's wait counts keep NS-1 sub-tiles outstanding; a loop
//     back-edge would make it drain all outstanding loads at the loop head;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the K operand is read from LDS with
//     ds_read_b128 (K rows stored with their 16-byte chunks XOR-swizzled by key & 15, so
//     16 keys of one chunk hit distinct banks); a lane holds one query and 16 keys, so
//     the row max/sum need one exchange between the two wave halves;
//   * O^T = V^T P^T: P stays in registers as the B operand; the V^T A operand comes from
//     ds_read_b64_tr_b16, which hands each lane 4 keys of its own V column.  V rows are
//     stored with their 16-byte chunks XOR-swizzled by (key & 3) so the four rows of one
//     transposed read fall in distinct LDS banks;
//   * a paged source (page size >= 16) reads the wave-uniform page indices of a sub-tile
//     with scalar loads, which do not queue behind the vector loads; a page index outside
//     the sequence is skipped.
#include "fb_attn_common.hpp"

#ifndef FB_STREAM_WG_PER_CU
#define FB_STREAM_WG_PER_CU 1
#endif

namespace fb {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i & 3 of the
// 4 x b16 addressed by lanes 4j + (i >> 2), j = 0..3 (a 4-key x 16-column transpose).
__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

}  // namespace

template <int NS, int TMAX, bool PAGED>
__global__ void __launch_bounds__(256, FB_STREAM_WG_PER_CU) attn_stream_kernel(const AttnArgs A) {
  constexpr int D = 128;
  constexpr int VB = 32 * D * 2;                    // K (or V) bytes of one 32-key sub-tile
  static_assert(NS >= 1 && NS <= 3, "pipeline depth (16 ops per sub-tile, counter max 63)");
  constexpr int RING = 4 * 2 * VB;                  // one K and one V slot per wave
  constexpr int RED = 4 * 32 * D * 4;               // final combine
  __shared__ __attribute__((aligned(16))) unsigned char vring[RING > RED ? RING : RED];
  __shared__ float red_m[4 * 32], red_l[4 * 32];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform (SGPR)
  const int g = lane >> 5, ql = lane & 31;
  const bool second = (int)blockIdx.y >= A.src0.n_splits;
  const AttnSrc& S = second ? A.src1 : A.src0;
  const int split = second ? (int)blockIdx.y - A.src0.n_splits : (int)blockIdx.y;
  const int b = blockIdx.z;
  const int hk = blockIdx.x;
  const SeqInfo si = seq_info(S, b, hk, A.h_kv);
  const int kbeg = split * S.chunk;
  if (kbeg >= si.n_keys) return;
  const int kend = min(si.n_keys, kbeg + S.chunk);
  const int rows = S.rows;                          // <= 32

  // This wave's keys: sub-tiles w, w + 4, ... of the chunk (chunk = 128 * TMAX at most);
  // sub-tile j of the wave starts at key kw0 + 128 j.
  const int kw0 = kbeg + 32 * w;
  const int kw1 = kend;
  const int nsub = __builtin_amdgcn_readfirstlane(kend > kw0 ? (kend - kw0 + 127) / 128 : 0);

  // Query fragment (B operand of S^T = K Q^T): lane holds d = 16*i + 8*g + 0..7.
  bf16x8 qf[D / 16];
  if (ql < rows) {
    const int j = ql / S.rows_per_head, i = ql % S.rows_per_head;
    const int tok = S.row_tok ? S.row_tok[b * S.rows_per_head + i] : i;
    const int h = hk * A.G + j;
    const uint16_t* qp = (const uint16_t*)A.q + ((int64_t)(b * A.B + tok) * A.h_q + h) * D + 8 * g;
#pragma unroll
    for (int i2 = 0; i2 < D / 16; ++i2) qf[i2] = *(const bf16x8*)(qp + 16 * i2);
  } else {
#pragma unroll
    for (int i2 = 0; i2 < D / 16; ++i2) qf[i2] = bf16x8{};
  }

  const int64_t tstride = (int64_t)A.h_kv * D;
  const uint16_t* kbase = (const uint16_t*)S.k + (int64_t)si.seq0 * tstride + hk * D;
  const uint16_t* vbase = (const uint16_t*)S.v + (int64_t)si.seq0 * tstride + hk * D;
  unsigned char* kslot = vring + w * 2 * VB;
  unsigned char* vslot = kslot + VB;
  // K / V buffer resources based at the chunk start (contiguous) or the sequence start
  // (paged); offsets are 32-bit byte offsets from there.
  // Rows past the chunk end (contiguous) or the sequence end (paged) are outside the
  // resource's range and read as zero; they are masked out of the softmax.
  const int tok_base = PAGED ? 0 : kbeg;
  const int tok_lim = PAGED ? si.n_seq : kend;
  const int nrec = (tok_lim - tok_base) * (int)tstride * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)tok_base * tstride), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)tok_base * tstride), 0, nrec, 0x00020000);
  const __attribute__((address_space(4))) int32_t* pgc =
      PAGED ? (const __attribute__((address_space(4))) int32_t*)(S.pages + (int64_t)(b * A.h_kv + hk) * S.max_union)
            : nullptr;
  const int last_pg = PAGED ? si.n_keys / S.page_size - 1 : 0;
  // Token of key `key` (ok = takes part in the softmax); p0 and pv[] are the first page of
  // the sub-tile and the indices of its (at most 3) pages.  Tokens past the resource range
  // read as zero.
  // A page index outside [0, n_seq / P] (checked before the multiply, which could
  // overflow) or a token past the sequence end is skipped.
  const int pg_lim = PAGED ? si.n_seq / S.page_size : 0;
  auto tok_of = [&](int key, int p0, const int (&pv)[3], bool& ok) -> int {
    ok = key < kw1;
    if (!PAGED) return key;
    const int rel = key / S.page_size - p0;
    const int pgi = rel == 0 ? pv[0] : (rel == 1 ? pv[1] : pv[2]);
    const int t = (unsigned)pgi <= (unsigned)pg_lim ? pgi * S.page_size + key % S.page_size : -1;
    ok = ok && (unsigned)t < (unsigned)si.n_seq;
    return t;
  };

  // Transposed V read: 16-lane group G = (g, h), position L = 4j + q.
  const int tr_h = (lane >> 4) & 1, tr_j = (lane & 15) >> 2, tr_q = lane & 3;
  const unsigned char* tr_base = vslot + (4 * g + tr_j) * 256 + (tr_q & 1) * 8;
  int tr_off[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) tr_off[t] = (4 * (t ^ tr_j) + 2 * tr_h + (tr_q >> 1)) * 16;
  // V staging: piece u of a lane is row 4u + (lane >> 4), 16-byte chunk lane & 15 of the
  // sub-tile; it is stored at chunk (lane & 15) ^ 4 * (lane >> 4) of that row.
  // K pieces go to the same rows, chunk (lane & 15) ^ (row & 15); row & 15 = 4 (u & 3) + v_row.
  const int v_row = lane >> 4;
  const int v_dst = v_row * 256 + (((lane & 15) ^ (4 * v_row)) << 4);
  int k_dst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) k_dst[u] = v_row * 256 + (((lane & 15) ^ (4 * u + v_row)) << 4);
  // K operand read: lane = key ql, chunk 2 i2 + g, stored at chunk (2 i2 + g) ^ (ql & 15).
  const int k_src_row = ql * 256;
  const int k_src_x = g ^ (ql & 15);

  u32x4 kreg[NS][8], vreg[NS][8];
  uint32_t vmask[NS];

#define FB_ISSUE(J, SLOT)                                                                     \
  do {                                                                                        \
    const int kb_ = kw0 + 128 * (J);                                                          \
    int p0_ = 0, pv_[3] = {0, 0, 0};                                                          \
    if (PAGED) {                                                                              \
      p0_ = kb_ / S.page_size;                                                                \
      pv_[0] = pgc[min(p0_, last_pg)];                                                        \
      pv_[1] = pgc[min(p0_ + 1, last_pg)];                                                    \
      pv_[2] = pgc[min(p0_ + 2, last_pg)];                                                    \
    }                                                                                         \
    bool ok_;                                                                                 \
    (void)tok_of(kb_ + ql, p0_, pv_, ok_);                                                    \
    vmask[SLOT] = (uint32_t)__ballot(ok_);                                                    \
    _Pragma("unroll") for (int u = 0; u < 8; ++u) {                                           \
      bool okv_;                                                                              \
      const int tv_ = tok_of(kb_ + 4 * u + v_row, p0_, pv_, okv_);                            \
      const int off_ = ((tv_ - tok_base) * (int)tstride + (lane & 15) * 8) * 2;               \
      kreg[SLOT][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off_, 0, kKvLoadPolicy)); \
      vreg[SLOT][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off_, 0, kKvLoadPolicy)); \
    }                                                                                         \
  } while (0)

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) o[t] = f32x16{};

  if (nsub > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) FB_ISSUE(s, s);
  }
  // The reuse decision is read once the first loads are in flight: an item whose heads all
  // reuse the cache leaves (its loads only fill registers), every other item has saved a
  // round trip.
  if (S.m_upd) {
    if (S.m_upd[b] < S.tau) return;
  } else if (S.mask) {
    bool any = false;
    for (int j = 0; j < A.G; ++j)
      if (j * S.rows_per_head < rows) any |= S.mask[b * A.h_q + hk * A.G + j] == 0;
    if (!any) return;
  }

#define FB_STEP(J)                                                                            \
  do {                                                                                      \
    constexpr int s = (J) % NS;                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                      \
_Pragma("unroll") for (int u = 0; u < 8; ++u) {                                           \
      *(u32x4*)(kslot + (u >> 2) * 4096 + (u & 3) * 1024 + k_dst[u & 3]) = kreg[s][u];      \
      *(u32x4*)(vslot + u * 1024 + v_dst) = vreg[s][u];                                      \
    }                                                                                       \
    const uint32_t vm = vmask[s];                                                           \
    FB_ISSUE((J) + NS, s);                                                                  \
                                                                                            \
    f32x16 acc = f32x16{};                                                                  \
_Pragma("unroll")                                                                           \
    for (int i2 = 0; i2 < D / 16; ++i2) {                                                   \
      const bf16x8 ka = *(const bf16x8*)(kslot + k_src_row + (((2 * i2) ^ k_src_x) << 4));  \
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[i2], acc, 0, 0, 0);             \
    }                                                                                       \
    float mx = kNegInf;                                                                     \
    if (vm == 0xffffffffu) {                                                                \
_Pragma("unroll")                                                                           \
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);                                  \
    } else {                                                                                \
_Pragma("unroll")                                                                           \
      for (int r = 0; r < 16; ++r) {                                                        \
        if (!((vm >> (8 * (r >> 2) + 4 * g + (r & 3))) & 1u)) acc[r] = kNegInf;             \
        mx = fmaxf(mx, acc[r]);                                                             \
      }                                                                                     \
    }                                                                                       \
    mx = wave_max_xor32(mx) * A.scale_log2;                                                 \
    /* lazy reference: raise m_run only when a score exceeds it by more than 2^8 */          \
    const bool need_ = mx > m_run + 8.0f;                                                   \
    if (__any(need_)) {                                                                     \
      const float m_new = need_ ? mx : m_run;                                               \
      const float alpha = exp2_or_zero(m_run - m_new);                                      \
      l_run *= alpha;                                                                       \
_Pragma("unroll")                                                                           \
      for (int t = 0; t < D / 32; ++t) o[t] *= alpha;                                       \
      m_run = m_new;                                                                        \
    }                                                                                       \
    const float m_use = m_run == kNegInf ? 0.f : m_run;                                     \
    float sv[16];                                                                           \
    float ps = 0.f;                                                                         \
_Pragma("unroll")                                                                           \
    for (int r = 0; r < 16; ++r) {                                                          \
      sv[r] = fast_exp2(fmaf(acc[r], A.scale_log2, -m_use));                                \
      ps += sv[r];                                                                          \
    }                                                                                       \
    ps = wave_add_xor32(ps);                                                                \
    l_run += ps;                                                                            \
_Pragma("unroll")                                                                           \
    for (int c = 0; c < 2; ++c) {                                                           \
      bf16x8 pb;                                                                            \
_Pragma("unroll")                                                                           \
      for (int jj = 0; jj < 8; ++jj) pb[jj] = (__bf16)sv[8 * c + jj];                       \
      const unsigned char* a = tr_base + c * 16 * 256;                                      \
_Pragma("unroll")                                                                           \
      for (int t = 0; t < D / 32; ++t) {                                                    \
        const s16x4 lo = lds_read_tr(a + tr_off[t]);                                        \
        const s16x4 hi = lds_read_tr(a + 8 * 256 + tr_off[t]);                              \
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)); \
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[t], 0, 0, 0);              \
      }                                                                                     \
    }                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                     \
  } while (0)

  static_assert(TMAX <= 48, "the step chain below is written out for 48 steps");
  // Straight-line steps: step j runs only if step j-1 ran, so every step has one
  // predecessor and the compiler's wait counts stay exact.
#define FB_LEVEL(J) if ((J) < TMAX && (J) < nsub) { FB_STEP(J);
  FB_LEVEL(0) FB_LEVEL(1) FB_LEVEL(2) FB_LEVEL(3) FB_LEVEL(4) FB_LEVEL(5) FB_LEVEL(6) FB_LEVEL(7)
  FB_LEVEL(8) FB_LEVEL(9) FB_LEVEL(10) FB_LEVEL(11) FB_LEVEL(12) FB_LEVEL(13) FB_LEVEL(14)
  FB_LEVEL(15) FB_LEVEL(16) FB_LEVEL(17) FB_LEVEL(18) FB_LEVEL(19) FB_LEVEL(20) FB_LEVEL(21)
  FB_LEVEL(22) FB_LEVEL(23) FB_LEVEL(24) FB_LEVEL(25) FB_LEVEL(26) FB_LEVEL(27) FB_LEVEL(28)
  FB_LEVEL(29) FB_LEVEL(30) FB_LEVEL(31) FB_LEVEL(32) FB_LEVEL(33) FB_LEVEL(34) FB_LEVEL(35)
  FB_LEVEL(36) FB_LEVEL(37) FB_LEVEL(38) FB_LEVEL(39) FB_LEVEL(40) FB_LEVEL(41) FB_LEVEL(42)
  FB_LEVEL(43) FB_LEVEL(44) FB_LEVEL(45) FB_LEVEL(46) FB_LEVEL(47)
  }}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}}
#undef FB_LEVEL
#undef FB_STEP
#undef FB_ISSUE

  // Combine the four waves (disjoint key ranges, same query rows), then write the partial.
  __syncthreads();
  float* red = (float*)vring;
  if (g == 0) {
    red_m[w * 32 + ql] = m_run;
    red_l[w * 32 + ql] = l_run;
  }
  __syncthreads();
  {
    float M = kNegInf;
    for (int s = 0; s < 4; ++s) M = fmaxf(M, red_m[s * 32 + ql]);
    const float Mu = M == kNegInf ? 0.f : M;
    const float f = exp2_or_zero(m_run - Mu);
    float* dst = red + (w * 32 + ql) * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
        x[0] = o[t][4 * r4 + 0] * f;
        x[1] = o[t][4 * r4 + 1] * f;
        x[2] = o[t][4 * r4 + 2] * f;
        x[3] = o[t][4 * r4 + 3] * f;
        *(f32x4*)(dst + 32 * t + 8 * r4 + 4 * g) = x;
      }
  }
  __syncthreads();
  const int64_t slot = (int64_t)(b * A.h_kv + hk) * S.n_splits + split;
  float* po = S.po + slot * rows * D;
  float* pml = S.pml + slot * rows * 2;
  for (int idx = tid; idx < rows * (D / 4); idx += 256) {
    const int r = idx / (D / 4), c4 = idx % (D / 4);
    f32x4 sum = f32x4{};
    for (int s = 0; s < 4; ++s) sum += *(const f32x4*)(red + (s * 32 + r) * D + 4 * c4);
    *(f32x4*)(po + (int64_t)r * D + 4 * c4) = sum;
  }
  for (int r = tid; r < rows; r += 256) {
    float M = kNegInf;
    for (int s = 0; s < 4; ++s) M = fmaxf(M, red_m[s * 32 + r]);
    const float Mu = M == kNegInf ? 0.f : M;
    float l = 0.f;
    for (int s = 0; s < 4; ++s) l += exp2_or_zero(red_m[s * 32 + r] - Mu) * red_l[s * 32 + r];
    pml[r * 2 + 0] = M;
    pml[r * 2 + 1] = l;
  }
}

// The streaming kernel covers bf16, d = 128, at most 32 rows per group, chunks of at most
// 128 * kStreamTmax keys; a paged source needs pages of at least 16 tokens.
bool stream_ok(const AttnArgs& a, const AttnSrc& s, int64_t max_tokens) {
  if (s.n_splits == 0) return true;
  if (a.d != 128 || s.rows > 32 || s.chunk > 128 * kStreamTmax) return false;
  // K offsets are 32-bit: a wave's keys (contiguous) or a whole sequence (paged)
  const int64_t span = s.pages ? max_tokens : s.chunk;
  if (span * a.h_kv * 128 * 2 >= ((int64_t)1 << 31)) return false;
  return !s.pages || s.page_size >= 16;
}

hipError_t launch_stream(const AttnArgs& a, hipStream_t st) {
  const int gy = a.src0.n_splits + a.src1.n_splits;
  if (gy == 0) return hipSuccess;
  dim3 grid(a.h_kv, gy, a.batch);
  // both sources of a launch are paged (selected / complement pages) or neither is
  const bool paged = (a.src0.n_splits ? a.src0.pages : a.src1.pages) != nullptr;
  if (a.src0.n_splits && a.src1.n_splits && (a.src0.pages != nullptr) != (a.src1.pages != nullptr))
    return hipErrorInvalidValue;
  if (paged) {
    hipLaunchKernelGGL((attn_stream_kernel<kStreamDepth, kStreamTmax, true>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_stream_kernel<kStreamDepth, kStreamTmax, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace fb
