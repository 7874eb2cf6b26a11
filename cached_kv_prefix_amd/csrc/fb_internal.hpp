// Internal job descriptors shared by the host launchers and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fb {

// One key source of the attention kernel.  Keys of sequence b are the tokens
//   contiguous:  seq0(b) + key,                          key < count(b)
//   paged:       seq0(b) + pages[b][hk][key / P] * P + key % P,
//                key < page_count[b][hk] * P, masked when the token is >= N_b
// with seq0(b) = cu ? cu[b] : b * n_uniform and count(b) = cu ? cu[b+1]-cu[b] : n_uniform.
// Rows of a (b, hk) group: r = j * rows_per_head + i for the group's j-th query head and
// row i, where i is the block token itself or row_tok[b][i] when row_tok is set.
struct AttnSrc {
  const void* k;
  const void* v;
  const int32_t* cu;
  int32_t n_uniform;
  const int32_t* pages;       // paged source (LoSA union), else null
  const int32_t* page_count;  // [batch][h_kv]
  int32_t page_size;
  int32_t max_union;
  int32_t chunk;              // keys per split (multiple of 128)
  int32_t n_splits;           // grid extent along x for this source
  int32_t rows_per_head;
  const int32_t* row_tok;     // [batch][rows_per_head] or null
  const int32_t* cu_q;        // packed queries: rows i >= cu_q[b+1] - cu_q[b] are padding, or null
  int32_t rows;               // G * rows_per_head
  int32_t tq;                 // 32-row query tiles per workgroup (1, 2 or 4)
  int32_t qgroups;            // ceil(rows / (32 * tq))
  const uint8_t* mask;        // [batch][h_q]: skip a workgroup whose heads all reuse
  const int32_t* m_upd;       // threshold rule instead of a mask: reuse where m_upd[b] < tau
  int32_t tau;
  float* po;                  // partial O   [batch][h_kv][n_splits][rows][d]
  float* pml;                 // partial m,l [batch][h_kv][n_splits][rows][2]
};

enum CombineMode { kModeStep = 0, kModePrefixOnly = 1, kModeBlockOnly = 2, kModeLosa = 3, kModeResidual = 4 };

struct CombineArgs {
  int32_t mode;
  int32_t batch, B, h_q, h_kv, G, d;
  // prefix partials (src0) and how many splits of each group are valid
  const float* po; const float* pml; int32_t p_rows; int32_t p_splits; int32_t p_chunk;
  const int32_t* cu; int32_t n_uniform;
  const int32_t* page_count; int32_t page_size;
  // block partials (src1)
  const float* bo; const float* bml; int32_t b_rows; int32_t b_splits; int32_t b_chunk;
  const uint8_t* mask;                 // step: [batch][h_q], null = recompute all
  const int32_t* m_upd; int32_t tau;   // step: threshold rule evaluated in place of mask
  const int32_t* active; int32_t n_active;   // LoSA
  // residual mode: the prefix partials are the selected pages (page_count); these are the
  // complement pages' partials (page counts r_page_count), which refresh the cache
  const float* ro; const float* rml; int32_t r_splits; int32_t r_chunk;
  const int32_t* r_page_count;
  // prefix-only mode over packed variable-length queries: row (b, i, h) is written to
  // packed row cu_q[b] + i (rows with i >= cu_q[b+1] - cu_q[b] are skipped)
  const int32_t* cu_q;
  // step mode: per row, the fp64 sums <old, new>, |old|^2, |new|^2 of the cached A_out
  // before and after the step ([batch][B][h_q][3]), or null
  double* sim_parts;
  // step mode: the reuse decision of every (b, h) is recorded here (1 = reused), or null
  uint8_t* mask_out;
  float* cache_a; float* cache_l;      // step/LoSA cache, or prefix-only outputs
  float* ain; float* lin;              // block-only outputs
  void* a_full; int32_t out_bf16; float* l_full;
};

struct AttnArgs {
  const void* q;              // [batch][B][h_q][d]
  int32_t batch, B, h_q, h_kv, G, d;
  int32_t max_seqlen;         // longest prefix (bounds 32-bit offsets of the stream kernel)
  float scale_log2;           // softmax_scale * log2(e)
  AttnSrc src0, src1;         // grid x: [0, src0.n_splits) then [.., + src1.n_splits)
};

// Streaming kernel (fb_stream.hip): sub-tiles in flight per wave, and the most 32-key
// sub-tiles a wave walks in one work item (its chunk is at most 4 * 32 * kStreamTmax keys).
#ifndef FB_STREAM_DEPTH
#define FB_STREAM_DEPTH 1
#endif
#ifndef FB_STREAM_TMAX
#define FB_STREAM_TMAX 40
#endif
constexpr int kStreamDepth = FB_STREAM_DEPTH;

// Cache policy of the K / V buffer loads of the attention kernels (the buffer
// instructions' aux operand: 2 = nt, the non-temporal hint).  Every K / V byte of a pass
// is read once, so the lines need not stay in the caches; a plain read of 537 MB ran at
// 6.7 TB/s with the hint against 6.0-6.1 TB/s without it on MI355X.
#ifndef FB_KV_LOAD_POLICY
#define FB_KV_LOAD_POLICY 2
#endif
constexpr int kKvLoadPolicy = FB_KV_LOAD_POLICY;
constexpr int kStreamTmax = FB_STREAM_TMAX;

// Query-tiled kernel (fb_fa.hip) for query groups of more than 32 rows: a wave owns
// 32 * kFaQt rows and a workgroup fa_waves(rows) waves (4 up to 128 rows, else 8).
#ifndef FB_FA_QT
#define FB_FA_QT 1
#endif
constexpr int kFaQt = FB_FA_QT;
constexpr int kFaMinRows = 33;
constexpr int kFaMaxChunkPages = 2048;   // page list of one paged chunk, staged in LDS
inline int fa_waves(int rows) { return rows <= 128 * kFaQt ? 4 : 8; }
inline int fa_rows_per_item(int rows) { return 32 * kFaQt * fa_waves(rows); }


hipError_t launch_attn(const AttnArgs& a, bool bf16, hipStream_t st);
bool stream_ok(const AttnArgs& a, const AttnSrc& s, int64_t max_tokens);
hipError_t launch_stream(const AttnArgs& a, hipStream_t st);
bool fa_ok(const AttnArgs& a, const AttnSrc& s);
hipError_t launch_fa(const AttnArgs& a, hipStream_t st);
hipError_t launch_combine(const CombineArgs& c, hipStream_t st);
hipError_t launch_lse_merge(int64_t rows, int32_t d, const float* ao, const float* lo,
                            const float* ai, const float* li, void* af, int out_bf16,
                            float* lf, hipStream_t st);
// *bad = whether a row to be reused (all rows, or by mask / m_upd < tau) holds NaN in cache_l
hipError_t launch_cache_check(const float* cache_l, int32_t batch, int32_t B, int32_t h_q, const uint8_t* mask,
                              const int32_t* m_upd, int32_t tau, bool all_rows, int32_t* bad, hipStream_t st);
hipError_t launch_mask_threshold(const int32_t* m, int32_t tau, int32_t batch, int32_t h_q,
                                 uint8_t* mask, hipStream_t st);
hipError_t launch_mask_similarity(const float* sim, float gamma, int64_t n, uint8_t* mask,
                                  hipStream_t st);
hipError_t launch_head_cosine(int32_t batch, int32_t B, int32_t h_q, int32_t d,
                              const float* a0, const float* a1, float* sim, hipStream_t st);
// sim[b][h] from the per-row sums the step's combine wrote (rows in order)
hipError_t launch_sim_reduce(int32_t batch, int32_t B, int32_t h_q, const double* parts, float* sim,
                             float gamma, uint8_t* next_mask, hipStream_t st);

// LoSA selection
struct LosaArgs {
  int32_t batch, B, h_q, h_kv, G, d;
  const int32_t* cu; int32_t n_uniform;
  int32_t page_size, topk, n_active, max_pages, max_union;
  int32_t bf16;
};
hipError_t launch_page_meta(const LosaArgs& a, const void* k, void* kmin, void* kmax, int tail,
                            hipStream_t st);
hipError_t launch_locality(const LosaArgs& a, const void* qc, const void* qp, double* loc,
                           int32_t* active, hipStream_t st);
// The active set is ranked by launch_locality (blocks of more than 256 tokens) or inside
// launch_quest_scores from the locality scores `loc` (which then writes `active`).
hipError_t launch_quest_scores(const LosaArgs& a, const void* qc, const double* loc, int32_t* active,
                               const void* kmin, const void* kmax, double* scores,
                               hipStream_t st);
hipError_t launch_topk(const LosaArgs& a, const double* scores, int32_t* topk_pages,
                       hipStream_t st);
hipError_t launch_union(const LosaArgs& a, const int32_t* topk_pages, int32_t* union_pages,
                        int32_t* union_count, hipStream_t st);


// FlashBlock with a cached sparse residual: the complement of each (sequence, KV head)
// page selection, for the groups where some query head refreshes the residual.
struct ResidualArgs {
  int32_t batch, h_q, h_kv, G;
  const int32_t* cu; int32_t n_uniform;
  int32_t page_size, max_pages, max_sel;
  const int32_t* sel_pages; const int32_t* sel_count;   // [batch][h_kv][max_sel], [batch][h_kv]
  const uint8_t* mask;                                  // [batch][h_q] or null (all refresh)
  int32_t* comp_pages; int32_t* comp_count;             // [batch][h_kv][max_pages], [batch][h_kv]
};
constexpr int kResidualMaxPages = 65536;
hipError_t launch_complement(const ResidualArgs& r, hipStream_t st);

// Block lifecycle: append a block to the packed prefix; small fills and copies.
struct AppendArgs {
  const void* k; const void* v;           // old prefix, [sum N][h_kv][d]
  const int32_t* cu; int32_t n_uniform;   // old offsets (or uniform length)
  const void* k_blk; const void* v_blk;   // [batch][B][h_kv][d]
  void* k_out; void* v_out;               // new prefix
  int32_t* cu_out;                        // new offsets or null
  int32_t batch, B, max_len;              // max_len: bound of every N_b
  int64_t row_bytes;                      // h_kv * d * element size
  int32_t tail_only;                      // in place (batch 1): write the block rows only
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
// row_tok[b][i] = the packed query row of token i of branch b (clamped into [0, total_q))
hipError_t launch_varlen_rows(const int32_t* cu_q, int32_t batch, int32_t b_max, int32_t total_q,
                              int32_t* row_tok, hipStream_t st);
hipError_t launch_fill_u8(uint8_t* p, int64_t n, uint8_t value, hipStream_t st);
hipError_t launch_fill_f32(float* p, int64_t n, float value, hipStream_t st);

}  // namespace fb
