// Host side of the C ABI declared in include/flashblock.h: argument validation (before
// anything is enqueued), the shape-only split plan, workspace carving and launches.
#include <algorithm>
#include <math.h>
#include <string.h>

#include "../../include/flashblock.h"
#include "fb_internal.hpp"

using namespace fb;

namespace {

#ifndef FB_TARGET_ITEMS
#define FB_TARGET_ITEMS 1024
#endif
#ifndef FB_STREAM_TARGET_ITEMS
#define FB_STREAM_TARGET_ITEMS 256   // the streaming kernel runs one workgroup per CU
#endif
#ifndef FB_MIN_CHUNK
#define FB_MIN_CHUNK 512
#endif
constexpr int kTileKeys = 128;                 // chunks are whole 128-key tiles
constexpr int kTargetItems = FB_TARGET_ITEMS;  // workgroups the split plan aims for
constexpr int kMinChunk = FB_MIN_CHUNK;        // smallest automatic chunk (keys)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

fb_status check_shape(const fb_shape* s) {
  if (!s) return FB_ERR_INVALID_ARG;
  if (s->batch < 1 || s->h_q < 1 || s->h_kv < 1 || s->head_dim < 1 || s->block < 1) return FB_ERR_INVALID_ARG;
  if (s->h_q % s->h_kv != 0) return FB_ERR_INVALID_ARG;
  if ((s->flags & ~FB_FLAG_CHECK_CACHE) != 0 || s->num_splits < 0) return FB_ERR_INVALID_ARG;
  if (!(s->softmax_scale >= 0.f) || !isfinite(s->softmax_scale)) return FB_ERR_INVALID_ARG;
  if (s->cu_seqlens_k ? s->max_seqlen_k < 0 : s->seqlen_k < 0) return FB_ERR_INVALID_ARG;
  if (s->dtype == FB_BF16) {
    if (s->head_dim != 64 && s->head_dim != 128) return FB_ERR_UNSUPPORTED;
  } else if (s->dtype == FB_F32) {
    if (s->head_dim > 256) return FB_ERR_UNSUPPORTED;
  } else {
    return FB_ERR_INVALID_ARG;
  }
  const int64_t rows = (int64_t)s->batch * s->block * s->h_q;
  if (rows * s->head_dim >= ((int64_t)1 << 40)) return FB_ERR_UNSUPPORTED;
  if (s->batch > 65535) return FB_ERR_UNSUPPORTED;                       // grid z
  // grid y = h_kv * query groups (at least 32 rows each)
  if ((int64_t)s->h_kv * cdiv((int64_t)(s->h_q / s->h_kv) * s->block, 32) > 65535) return FB_ERR_UNSUPPORTED;
  return FB_OK;
}

inline int max_prefix(const fb_shape* s) { return s->cu_seqlens_k ? s->max_seqlen_k : s->seqlen_k; }
inline float scale_of(const fb_shape* s) {
  return s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
}

// Rows of a (sequence, KV head) group and how the attention kernel tiles them.
struct RowPlan {
  int rows, rows_per_head, tq, qgroups;
};
RowPlan row_plan(const fb_shape* s, int rows_per_head) {
  RowPlan r;
  r.rows_per_head = rows_per_head;
  r.rows = (s->h_q / s->h_kv) * rows_per_head;
  if (s->dtype == FB_BF16)
    r.tq = r.rows <= 32 ? 1 : (r.rows <= 64 ? 2 : 4);
  else
    r.tq = 1;
  r.qgroups = (int)cdiv(r.rows, 32 * r.tq);
  return r;
}

// Key chunking of one source: depends on the shape only (deterministic results).
struct SplitPlan {
  int chunk, splits;
};
// `reserved` work items of the same launch (the block pass) come out of the streaming
// kernel's budget, so that the whole launch is resident at once: the block items are the
// last to be dispatched, and waiting for a free CU they would add their whole latency to
// the end of the launch.
bool stream_rows(const fb_shape* s, const RowPlan& rp) {
  return s->dtype == FB_BF16 && s->head_dim == 128 && rp.rows <= 32;
}
// Large query groups run on the query-tiled kernel: 128 * kFaQt rows per work item.
bool fa_rows(const fb_shape* s, const RowPlan& rp) {
  return s->dtype == FB_BF16 && s->head_dim == 128 && rp.rows >= kFaMinRows;
}
#ifndef FB_FA_TARGET_ITEMS
#define FB_FA_TARGET_ITEMS 512        // 8-wave items (one resident per CU): two rounds
#endif
#ifndef FB_FA_ITEM_OVERHEAD_KEYS
#define FB_FA_ITEM_OVERHEAD_KEYS 256  // set-up and tail of one 4-wave item, in keys streamed
#endif
SplitPlan split_plan(const fb_shape* s, const RowPlan& rp, int64_t max_keys, int forced, int64_t reserved = 0) {
  SplitPlan p;
  if (max_keys <= 0) {
    p.chunk = kTileKeys;
    p.splits = 0;
    return p;
  }
  int64_t want;
  if (forced > 0) {
    want = forced;
  } else {
    const int64_t items = (int64_t)s->batch * s->h_kv * rp.qgroups;
    if (stream_rows(s, rp)) {
      want = std::max<int64_t>(1, (FB_STREAM_TARGET_ITEMS - reserved) / items);
    } else if (fa_rows(s, rp)) {
      const int64_t fa_items = (int64_t)s->batch * s->h_kv * cdiv(rp.rows, fa_rows_per_item(rp.rows));
      if (fa_waves(rp.rows) == 4) {
        // 4-wave (memory-bound) items, 2 resident per CU: the split count that minimises
        // rounds of resident items x (keys per item + per-item set-up), so that the last
        // round is not a near-empty tail and items are not needlessly short.
        const int64_t slots = 2 * 256;
        int64_t best = 1, best_cost = INT64_MAX;
        for (int64_t sp = 1; sp <= 256; ++sp) {
          const int64_t ch = std::max<int64_t>(round_up(cdiv(max_keys, sp), kTileKeys), kMinChunk);
          if (cdiv(max_keys, ch) != sp) continue;   // rounding gives another split count: seen or to come
          const int64_t cost = cdiv(fa_items * sp, slots) * (ch + FB_FA_ITEM_OVERHEAD_KEYS);
          if (cost < best_cost) {
            best_cost = cost;
            best = sp;
          }
        }
        want = best;
      } else {
        // 8-wave (matrix-bound) items, 1 resident per CU: two rounds of them
        want = std::max<int64_t>(1, (FB_FA_TARGET_ITEMS + fa_items / 2) / fa_items);
      }
    } else {
      want = cdiv(kTargetItems, items);
    }
  }
  int64_t chunk = round_up(cdiv(max_keys, want), kTileKeys);
  if (forced <= 0 && chunk < kMinChunk) chunk = kMinChunk < round_up(max_keys, kTileKeys) ? kMinChunk : round_up(max_keys, kTileKeys);
  // a streaming work item walks at most 128 * kStreamTmax keys (longer prefixes take more items)
  if (forced <= 0 && stream_rows(s, rp)) chunk = std::min<int64_t>(chunk, 128 * kStreamTmax);
  p.chunk = (int)chunk;
  p.splits = (int)cdiv(max_keys, chunk);
  return p;
}

struct Region {
  size_t o_off, ml_off, bytes;
};
Region partial_region(const fb_shape* s, const RowPlan& rp, const SplitPlan& sp, size_t base) {
  Region r;
  const size_t slots = (size_t)s->batch * s->h_kv * sp.splits;
  r.o_off = base;
  r.ml_off = align256(base + slots * rp.rows * s->head_dim * sizeof(float));
  r.bytes = align256(r.ml_off + slots * rp.rows * 2 * sizeof(float)) - base;
  return r;
}

// Full plan of the dense step (prefix source 0, block source 1); the last 256 bytes hold
// the flag of the debug cache check.
struct StepPlan {
  RowPlan rp;
  SplitPlan pre, blk;
  Region rpre, rblk;
  size_t check_off, ws_bytes;
};
StepPlan step_plan(const fb_shape* s) {
  StepPlan p;
  p.rp = row_plan(s, s->block);
  p.blk = split_plan(s, p.rp, s->block, fa_rows(s, p.rp) ? 1 : 0);   // block items of the query-tiled kernel are long enough unsplit
  const int64_t blk_items = (int64_t)s->batch * s->h_kv * p.rp.qgroups * p.blk.splits;
  p.pre = split_plan(s, p.rp, max_prefix(s), s->num_splits, blk_items);
  p.rpre = partial_region(s, p.rp, p.pre, 0);
  p.rblk = partial_region(s, p.rp, p.blk, p.rpre.bytes);
  p.check_off = align256(p.rpre.bytes + p.rblk.bytes);
  p.ws_bytes = p.check_off + 256;
  return p;
}

AttnSrc make_src(const RowPlan& rp, const SplitPlan& sp, const void* k, const void* v, const int32_t* cu,
                 int n_uniform, float* ws, const Region& reg) {
  AttnSrc a;
  memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.cu = cu;
  a.n_uniform = n_uniform;
  a.chunk = sp.chunk;
  a.n_splits = sp.splits;
  a.rows_per_head = rp.rows_per_head;
  a.rows = rp.rows;
  a.tq = rp.tq;
  a.qgroups = rp.qgroups;
  a.po = (float*)((char*)ws + reg.o_off);
  a.pml = (float*)((char*)ws + reg.ml_off);
  return a;
}

AttnArgs base_args(const fb_shape* s, const void* q) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.batch = s->batch;
  a.B = s->block;
  a.h_q = s->h_q;
  a.h_kv = s->h_kv;
  a.G = s->h_q / s->h_kv;
  a.d = s->head_dim;
  a.max_seqlen = max_prefix(s);
  a.scale_log2 = scale_of(s) * 1.4426950408889634f;
  return a;
}

CombineArgs base_combine(const fb_shape* s, const StepPlan& p, float* ws) {
  CombineArgs c;
  memset(&c, 0, sizeof(c));
  c.batch = s->batch;
  c.B = s->block;
  c.h_q = s->h_q;
  c.h_kv = s->h_kv;
  c.G = s->h_q / s->h_kv;
  c.d = s->head_dim;
  c.po = (const float*)((char*)ws + p.rpre.o_off);
  c.pml = (const float*)((char*)ws + p.rpre.ml_off);
  c.p_rows = p.rp.rows;
  c.p_splits = p.pre.splits;
  c.p_chunk = p.pre.chunk;
  c.cu = s->cu_seqlens_k;
  c.n_uniform = s->seqlen_k;
  c.bo = (const float*)((char*)ws + p.rblk.o_off);
  c.bml = (const float*)((char*)ws + p.rblk.ml_off);
  c.b_rows = p.rp.rows;
  c.b_splits = p.blk.splits;
  c.b_chunk = p.blk.chunk;
  c.out_bf16 = s->dtype == FB_BF16;
  return c;
}

bool prefix_may_be_empty(const fb_shape* s) { return !s->cu_seqlens_k && s->seqlen_k == 0; }

fb_status check_inputs(const fb_shape* s, const void* q, const void* k, const void* v) {
  if (!q || !aligned16(q)) return FB_ERR_INVALID_ARG;
  if (!prefix_may_be_empty(s) && (!k || !v || !aligned16(k) || !aligned16(v))) return FB_ERR_INVALID_ARG;
  return FB_OK;
}

inline void rec(hipEvent_t e, hipStream_t st) {
  if (e) hipEventRecord(e, st);
}

fb_status hip_status(hipError_t e) { return e == hipSuccess ? FB_OK : FB_ERR_HIP; }

// FB_FLAG_CHECK_CACHE: whether every cache row the call would reuse has been written (a
// never-written row holds NaN in cache_l).  Runs before the call's own launches, writes
// only the flag in the workspace, and waits for it on the host.
fb_status check_cache(const fb_shape* s, const float* cache_l, const uint8_t* mask, const int32_t* m_upd,
                      int32_t tau, bool all_rows, void* flag, hipStream_t stream) {
  if (!(s->flags & FB_FLAG_CHECK_CACHE) || (!all_rows && !mask && !m_upd)) return FB_OK;
  int32_t* bad = (int32_t*)flag;
  hipError_t e = launch_cache_check(cache_l, s->batch, s->block, s->h_q, mask, m_upd, tau, all_rows, bad, stream);
  int32_t host = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&host, bad, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return FB_ERR_HIP;
  return host ? FB_ERR_CACHE_INVALID : FB_OK;
}

}  // namespace

extern "C" {

const char* fb_status_string(fb_status s) {
  switch (s) {
    case FB_OK: return "ok";
    case FB_ERR_INVALID_ARG: return "invalid argument";
    case FB_ERR_UNSUPPORTED: return "unsupported configuration";
    case FB_ERR_WORKSPACE: return "workspace too small";
    case FB_ERR_CACHE_INVALID: return "a reused cache row was never written";
    case FB_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t fb_workspace_size(const fb_shape* s) {
  if (check_shape(s) != FB_OK) return 0;
  return step_plan(s).ws_bytes;
}

fb_status fb_prefix_attn(const fb_shape* s, const void* q, const void* k, const void* v, float* a_out,
                         float* l_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  fb_status st = check_shape(s);
  if (st != FB_OK) return st;
  if ((st = check_inputs(s, q, k, v)) != FB_OK) return st;
  if (!a_out || !l_out) return FB_ERR_INVALID_ARG;
  const StepPlan p = step_plan(s);
  if (ws_bytes < p.ws_bytes || (p.ws_bytes && (!ws || !aligned16(ws)))) return FB_ERR_WORKSPACE;
  AttnArgs a = base_args(s, q);
  a.src0 = make_src(p.rp, p.pre, k, v, s->cu_seqlens_k, s->seqlen_k, (float*)ws, p.rpre);
  if (hipError_t e = launch_attn(a, s->dtype == FB_BF16, stream)) return hip_status(e);
  CombineArgs c = base_combine(s, p, (float*)ws);
  c.mode = kModePrefixOnly;
  c.cache_a = a_out;
  c.cache_l = l_out;
  return hip_status(launch_combine(c, stream));
}

fb_status fb_block_attn(const fb_shape* s, const void* q, const void* k_blk, const void* v_blk, float* a_in,
                        float* l_in, void* ws, size_t ws_bytes, hipStream_t stream) {
  fb_status st = check_shape(s);
  if (st != FB_OK) return st;
  if (!q || !k_blk || !v_blk || !aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk)) return FB_ERR_INVALID_ARG;
  if (!a_in || !l_in) return FB_ERR_INVALID_ARG;
  const StepPlan p = step_plan(s);
  if (ws_bytes < p.ws_bytes || (p.ws_bytes && (!ws || !aligned16(ws)))) return FB_ERR_WORKSPACE;
  AttnArgs a = base_args(s, q);
  a.src1 = make_src(p.rp, p.blk, k_blk, v_blk, nullptr, s->block, (float*)ws, p.rblk);
  if (hipError_t e = launch_attn(a, s->dtype == FB_BF16, stream)) return hip_status(e);
  CombineArgs c = base_combine(s, p, (float*)ws);
  c.mode = kModeBlockOnly;
  c.ain = a_in;
  c.lin = l_in;
  return hip_status(launch_combine(c, stream));
}

fb_status fb_lse_merge(int64_t rows, int32_t d, const float* a_out, const float* l_out, const float* a_in,
                       const float* l_in, void* a_full, fb_dtype out_dtype, float* l_full, hipStream_t stream) {
  if (rows < 0 || d < 1 || d > 256) return rows < 0 || d < 1 ? FB_ERR_INVALID_ARG : FB_ERR_UNSUPPORTED;
  if (out_dtype != FB_BF16 && out_dtype != FB_F32) return FB_ERR_INVALID_ARG;
  if (rows > 4 * (int64_t)INT32_MAX) return FB_ERR_UNSUPPORTED;   // four rows per workgroup
  if (rows == 0) return FB_OK;
  if (!a_out || !l_out || !a_in || !l_in || !a_full) return FB_ERR_INVALID_ARG;
  return hip_status(launch_lse_merge(rows, d, a_out, l_out, a_in, l_in, a_full, out_dtype == FB_BF16, l_full, stream));
}

namespace {
fb_status run_step(const fb_shape* s, const void* q, const void* k, const void* v, const void* k_blk,
                   const void* v_blk, const uint8_t* reuse_mask, const int32_t* m_upd, int32_t tau,
                   float* cache_a, float* cache_l, void* a_full, float* l_full, void* ws, size_t ws_bytes,
                   const fb_trace* trace, hipStream_t stream, double* sim_parts = nullptr,
                   uint8_t* mask_out = nullptr) {
  fb_status st = check_shape(s);
  if (st != FB_OK) return st;
  if ((st = check_inputs(s, q, k, v)) != FB_OK) return st;
  if (!k_blk || !v_blk || !aligned16(k_blk) || !aligned16(v_blk)) return FB_ERR_INVALID_ARG;
  if (!cache_a || !cache_l || !a_full) return FB_ERR_INVALID_ARG;
  const StepPlan p = step_plan(s);
  if (ws_bytes < p.ws_bytes || (p.ws_bytes && (!ws || !aligned16(ws)))) return FB_ERR_WORKSPACE;
  if ((st = check_cache(s, cache_l, reuse_mask, m_upd, tau, false, (char*)ws + p.check_off, stream)) != FB_OK)
    return st;
  AttnArgs a = base_args(s, q);
  a.src0 = make_src(p.rp, p.pre, k, v, s->cu_seqlens_k, s->seqlen_k, (float*)ws, p.rpre);
  a.src0.mask = reuse_mask;
  a.src0.m_upd = m_upd;
  a.src0.tau = tau;
  a.src1 = make_src(p.rp, p.blk, k_blk, v_blk, nullptr, s->block, (float*)ws, p.rblk);
  rec(trace ? trace->attn_begin : nullptr, stream);
  if (hipError_t e = launch_attn(a, s->dtype == FB_BF16, stream)) return hip_status(e);
  rec(trace ? trace->attn_end : nullptr, stream);
  CombineArgs c = base_combine(s, p, (float*)ws);
  c.mode = kModeStep;
  c.mask = reuse_mask;
  c.m_upd = m_upd;
  c.tau = tau;
  c.cache_a = cache_a;
  c.cache_l = cache_l;
  c.a_full = a_full;
  c.l_full = l_full;
  c.sim_parts = sim_parts;
  c.mask_out = mask_out;
  rec(trace ? trace->merge_begin : nullptr, stream);
  if (hipError_t e = launch_combine(c, stream)) return hip_status(e);
  rec(trace ? trace->merge_end : nullptr, stream);
  return FB_OK;
}
}  // namespace

fb_status fb_step(const fb_shape* s, const void* q, const void* k, const void* v, const void* k_blk,
                  const void* v_blk, const uint8_t* reuse_mask, float* cache_a, float* cache_l, void* a_full,
                  float* l_full, void* ws, size_t ws_bytes, const fb_trace* trace, hipStream_t stream) {
  return run_step(s, q, k, v, k_blk, v_blk, reuse_mask, nullptr, 0, cache_a, cache_l, a_full, l_full, ws,
                  ws_bytes, trace, stream);
}

fb_status fb_step_threshold(const fb_shape* s, const void* q, const void* k, const void* v, const void* k_blk,
                            const void* v_blk, const int32_t* m_updated, int32_t tau, float* cache_a,
                            float* cache_l, void* a_full, float* l_full, void* ws, size_t ws_bytes,
                            const fb_trace* trace, hipStream_t stream) {
  if (!m_updated) return FB_ERR_INVALID_ARG;
  return run_step(s, q, k, v, k_blk, v_blk, nullptr, m_updated, tau, cache_a, cache_l, a_full, l_full, ws,
                  ws_bytes, trace, stream);
}

fb_status fb_mask_threshold(const int32_t* m_updated, int32_t tau, int32_t batch, int32_t h_q, uint8_t* mask,
                            hipStream_t stream) {
  if (!m_updated || !mask || batch < 1 || h_q < 1) return FB_ERR_INVALID_ARG;
  if ((int64_t)batch * h_q > ((int64_t)INT32_MAX << 8)) return FB_ERR_UNSUPPORTED;
  return hip_status(launch_mask_threshold(m_updated, tau, batch, h_q, mask, stream));
}

fb_status fb_mask_similarity(const float* sim, float gamma, int64_t n, uint8_t* mask, hipStream_t stream) {
  if (n < 0 || (n > 0 && (!sim || !mask))) return FB_ERR_INVALID_ARG;
  if (n > ((int64_t)INT32_MAX << 8)) return FB_ERR_UNSUPPORTED;
  return hip_status(launch_mask_similarity(sim, gamma, n, mask, stream));
}

fb_status fb_head_cosine(int32_t batch, int32_t block, int32_t h_q, int32_t head_dim, const float* a_prev,
                         const float* a_cur, float* sim, hipStream_t stream) {
  if (batch < 1 || block < 1 || h_q < 1 || head_dim < 1 || !a_prev || !a_cur || !sim) return FB_ERR_INVALID_ARG;
  if ((int64_t)batch * h_q > INT32_MAX) return FB_ERR_UNSUPPORTED;   // one workgroup per (b, h)
  return hip_status(launch_head_cosine(batch, block, h_q, head_dim, a_prev, a_cur, sim, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// LoSA-style sparse path
// ---------------------------------------------------------------------------------------
namespace {

fb_status check_losa(const losa_shape* ls) {
  if (!ls) return FB_ERR_INVALID_ARG;
  fb_status st = check_shape(&ls->s);
  if (st != FB_OK) return st;
  const fb_shape& s = ls->s;
  if (ls->page_size < 1 || ls->topk < 1 || ls->n_active < 1 || ls->max_pages < 1) return FB_ERR_INVALID_ARG;
  if (ls->n_active > s.block) return FB_ERR_INVALID_ARG;
  if (s.block > 1024 || ls->max_pages > 16384 || s.head_dim % 8 != 0 || s.h_q > 1024) return FB_ERR_UNSUPPORTED;
  if ((int64_t)s.batch * s.h_q * ls->n_active > INT32_MAX) return FB_ERR_UNSUPPORTED;   // top-k grid
  if (cdiv(max_prefix(&s), ls->page_size) > ls->max_pages) return FB_ERR_INVALID_ARG;
  return FB_OK;
}

int union_cap(const losa_shape* ls) {
  const int64_t g = ls->s.h_q / ls->s.h_kv;
  const int64_t c = (int64_t)ls->n_active * g * ls->topk;
  return (int)(c < ls->max_pages ? c : ls->max_pages);
}

LosaArgs losa_args(const losa_shape* ls) {
  LosaArgs a;
  const fb_shape& s = ls->s;
  a.batch = s.batch;
  a.B = s.block;
  a.h_q = s.h_q;
  a.h_kv = s.h_kv;
  a.G = s.h_q / s.h_kv;
  a.d = s.head_dim;
  a.cu = s.cu_seqlens_k;
  a.n_uniform = s.seqlen_k;
  a.page_size = ls->page_size;
  a.topk = ls->topk;
  a.n_active = ls->n_active;
  a.max_pages = ls->max_pages;
  a.max_union = union_cap(ls);
  a.bf16 = s.dtype == FB_BF16;
  return a;
}

struct LosaPlan {
  StepPlan dense;        // block source and row plan of all B rows
  RowPlan rp_sparse;
  SplitPlan sp_sparse;
  Region r_sparse, r_block;
  size_t scores_off, active_off, loc_off, check_off, ws_bytes;
};
LosaPlan losa_plan(const losa_shape* ls) {
  LosaPlan p;
  const fb_shape* s = &ls->s;
  p.dense = step_plan(s);
  p.rp_sparse = row_plan(s, ls->n_active);
  p.sp_sparse = split_plan(s, p.rp_sparse, (int64_t)union_cap(ls) * ls->page_size, s->num_splits);
  p.r_sparse = partial_region(s, p.rp_sparse, p.sp_sparse, 0);
  p.r_block = partial_region(s, p.dense.rp, p.dense.blk, p.r_sparse.bytes);
  p.scores_off = p.r_sparse.bytes + p.r_block.bytes;
  const size_t scores = (size_t)s->batch * s->h_q * ls->n_active * ls->max_pages * sizeof(double);
  p.active_off = align256(p.scores_off + scores);
  p.loc_off = align256(p.active_off + (size_t)s->batch * ls->n_active * sizeof(int32_t));
  p.check_off = align256(p.loc_off + (size_t)s->batch * s->block * sizeof(double));
  p.ws_bytes = p.check_off + 256;
  return p;
}

fb_status run_selection(const losa_shape* ls, const LosaPlan& p, const void* q_cur, const void* q_prev,
                        const void* kmin, const void* kmax, int32_t* active, int32_t* topk_pages,
                        int32_t* union_pages, int32_t* union_count, void* ws, hipStream_t stream) {
  const LosaArgs la = losa_args(ls);
  double* scores = (double*)((char*)ws + p.scores_off);
  double* loc = (double*)((char*)ws + p.loc_off);
  if (hipError_t e = launch_locality(la, q_cur, q_prev, loc, active, stream)) return hip_status(e);
  if (hipError_t e = launch_quest_scores(la, q_cur, loc, active, kmin, kmax, scores, stream)) return hip_status(e);
  if (hipError_t e = launch_topk(la, scores, topk_pages, stream)) return hip_status(e);
  return hip_status(launch_union(la, topk_pages, union_pages, union_count, stream));
}

}  // namespace

extern "C" {

size_t losa_meta_bytes(const losa_shape* ls) {
  if (check_losa(ls) != FB_OK) return 0;
  const size_t el = ls->s.dtype == FB_BF16 ? 2 : 4;
  return (size_t)ls->s.batch * ls->s.h_kv * ls->s.head_dim * ls->max_pages * el;
}

size_t losa_workspace_size(const losa_shape* ls) {
  if (check_losa(ls) != FB_OK) return 0;
  return losa_plan(ls).ws_bytes;
}

int32_t losa_union_capacity(const losa_shape* ls) {
  if (check_losa(ls) != FB_OK) return 0;
  return union_cap(ls);
}

fb_status losa_page_meta(const losa_shape* ls, const void* k, void* kmin, void* kmax, hipStream_t stream) {
  fb_status st = check_losa(ls);
  if (st != FB_OK) return st;
  if (!kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)) return FB_ERR_INVALID_ARG;
  if (!k && !prefix_may_be_empty(&ls->s)) return FB_ERR_INVALID_ARG;
  return hip_status(launch_page_meta(losa_args(ls), k, kmin, kmax, 0, stream));
}

fb_status losa_select_union(const losa_shape* ls, const void* q_cur, const void* q_prev, const void* kmin,
                            const void* kmax, int32_t* active, int32_t* topk_pages, int32_t* union_pages,
                            int32_t* union_count, void* ws, size_t ws_bytes, hipStream_t stream) {
  fb_status st = check_losa(ls);
  if (st != FB_OK) return st;
  if (!q_cur || !q_prev || !kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)) return FB_ERR_INVALID_ARG;
  if (!active || !topk_pages || !union_pages || !union_count) return FB_ERR_INVALID_ARG;
  const LosaPlan p = losa_plan(ls);
  if (ws_bytes < p.ws_bytes || !ws || !aligned16(ws)) return FB_ERR_WORKSPACE;
  return run_selection(ls, p, q_cur, q_prev, kmin, kmax, active, topk_pages, union_pages, union_count, ws, stream);
}

fb_status losa_step(const losa_shape* ls, const void* q_cur, const void* q_prev, const void* k, const void* v,
                    const void* k_blk, const void* v_blk, const void* kmin, const void* kmax, float* cache_a,
                    float* cache_l, void* a_full, float* l_full, int32_t* active, int32_t* topk_pages,
                    int32_t* union_pages, int32_t* union_count, void* ws, size_t ws_bytes,
                    const fb_trace* trace, hipStream_t stream) {
  fb_status st = check_losa(ls);
  if (st != FB_OK) return st;
  const fb_shape* s = &ls->s;
  if ((st = check_inputs(s, q_cur, k, v)) != FB_OK) return st;
  if (!q_prev || !kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)) return FB_ERR_INVALID_ARG;
  if (!k_blk || !v_blk || !aligned16(k_blk) || !aligned16(v_blk)) return FB_ERR_INVALID_ARG;
  if (!cache_a || !cache_l || !a_full || !active || !topk_pages || !union_pages || !union_count)
    return FB_ERR_INVALID_ARG;
  const LosaPlan p = losa_plan(ls);
  if (ws_bytes < p.ws_bytes || !ws || !aligned16(ws)) return FB_ERR_WORKSPACE;
  // stable rows (every block with |A| < B has some) reuse their cached rows
  if ((st = check_cache(s, cache_l, nullptr, nullptr, 0, ls->n_active < s->block, (char*)ws + p.check_off,
                        stream)) != FB_OK)
    return st;

  rec(trace ? trace->select_begin : nullptr, stream);
  st = run_selection(ls, p, q_cur, q_prev, kmin, kmax, active, topk_pages, union_pages, union_count, ws, stream);
  if (st != FB_OK) return st;
  rec(trace ? trace->select_end : nullptr, stream);

  AttnArgs a = base_args(s, q_cur);
  a.src0 = make_src(p.rp_sparse, p.sp_sparse, k, v, s->cu_seqlens_k, s->seqlen_k, (float*)ws, p.r_sparse);
  a.src0.pages = union_pages;
  a.src0.page_count = union_count;
  a.src0.page_size = ls->page_size;
  a.src0.max_union = union_cap(ls);
  a.src0.row_tok = active;
  a.src1 = make_src(p.dense.rp, p.dense.blk, k_blk, v_blk, nullptr, s->block, (float*)ws, p.r_block);
  rec(trace ? trace->attn_begin : nullptr, stream);
  if (hipError_t e = launch_attn(a, s->dtype == FB_BF16, stream)) return hip_status(e);
  rec(trace ? trace->attn_end : nullptr, stream);

  CombineArgs c;
  memset(&c, 0, sizeof(c));
  c.mode = kModeLosa;
  c.batch = s->batch;
  c.B = s->block;
  c.h_q = s->h_q;
  c.h_kv = s->h_kv;
  c.G = s->h_q / s->h_kv;
  c.d = s->head_dim;
  c.po = (const float*)((char*)ws + p.r_sparse.o_off);
  c.pml = (const float*)((char*)ws + p.r_sparse.ml_off);
  c.p_rows = p.rp_sparse.rows;
  c.p_splits = p.sp_sparse.splits;
  c.p_chunk = p.sp_sparse.chunk;
  c.page_count = union_count;
  c.page_size = ls->page_size;
  c.bo = (const float*)((char*)ws + p.r_block.o_off);
  c.bml = (const float*)((char*)ws + p.r_block.ml_off);
  c.b_rows = p.dense.rp.rows;
  c.b_splits = p.dense.blk.splits;
  c.b_chunk = p.dense.blk.chunk;
  c.active = active;
  c.n_active = ls->n_active;
  c.cache_a = cache_a;
  c.cache_l = cache_l;
  c.a_full = a_full;
  c.l_full = l_full;
  c.out_bf16 = s->dtype == FB_BF16;
  rec(trace ? trace->merge_begin : nullptr, stream);
  if (hipError_t e = launch_combine(c, stream)) return hip_status(e);
  rec(trace ? trace->merge_end : nullptr, stream);
  return FB_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// FlashBlock with a cached sparse residual
// ---------------------------------------------------------------------------------------
namespace {

fb_status check_residual(const fb_residual_shape* rs) {
  if (!rs) return FB_ERR_INVALID_ARG;
  fb_status st = check_shape(&rs->s);
  if (st != FB_OK) return st;
  if (rs->page_size < 1 || rs->max_pages < 1 || rs->max_sel < 1 || rs->max_sel > rs->max_pages)
    return FB_ERR_INVALID_ARG;
  if (rs->max_pages > kResidualMaxPages) return FB_ERR_UNSUPPORTED;
  if (cdiv(max_prefix(&rs->s), rs->page_size) > rs->max_pages) return FB_ERR_INVALID_ARG;
  if ((int64_t)rs->max_pages * rs->page_size > INT32_MAX) return FB_ERR_UNSUPPORTED;   // 32-bit key indices
  return FB_OK;
}

// Sources of one step: the selected pages (0) and the complement pages (1) in one launch,
// the block in a second one.  Both page sources cover every row of the block.
struct ResidualPlan {
  RowPlan rp;
  SplitPlan sel, comp, blk;
  Region rsel, rcomp, rblk;
  size_t pages_off, count_off, check_off, ws_bytes;
};
ResidualPlan residual_plan(const fb_residual_shape* rs) {
  ResidualPlan p;
  const fb_shape* s = &rs->s;
  const int64_t prefix_pages = cdiv(max_prefix(s), rs->page_size);
  p.rp = row_plan(s, s->block);
  p.blk = split_plan(s, p.rp, s->block, fa_rows(s, p.rp) ? 1 : 0);
  p.sel = split_plan(s, p.rp, std::min<int64_t>(rs->max_sel, prefix_pages) * rs->page_size, s->num_splits);
  p.comp = split_plan(s, p.rp, prefix_pages * rs->page_size, s->num_splits);
  p.rsel = partial_region(s, p.rp, p.sel, 0);
  p.rcomp = partial_region(s, p.rp, p.comp, p.rsel.bytes);
  p.rblk = partial_region(s, p.rp, p.blk, p.rsel.bytes + p.rcomp.bytes);
  const size_t groups = (size_t)s->batch * s->h_kv;
  p.pages_off = p.rsel.bytes + p.rcomp.bytes + p.rblk.bytes;
  p.count_off = align256(p.pages_off + groups * rs->max_pages * sizeof(int32_t));
  p.check_off = align256(p.count_off + groups * sizeof(int32_t));
  p.ws_bytes = p.check_off + 256;
  return p;
}

}  // namespace

extern "C" {

size_t fb_residual_workspace_size(const fb_residual_shape* rs) {
  if (check_residual(rs) != FB_OK) return 0;
  return residual_plan(rs).ws_bytes;
}

fb_status fb_residual_step(const fb_residual_shape* rs, const void* q, const void* k, const void* v,
                           const void* k_blk, const void* v_blk, const int32_t* sel_pages,
                           const int32_t* sel_count, const uint8_t* reuse_mask, float* cache_a, float* cache_l,
                           void* a_full, float* l_full, void* ws, size_t ws_bytes, const fb_trace* trace,
                           hipStream_t stream) {
  fb_status st = check_residual(rs);
  if (st != FB_OK) return st;
  const fb_shape* s = &rs->s;
  if ((st = check_inputs(s, q, k, v)) != FB_OK) return st;
  if (!k_blk || !v_blk || !aligned16(k_blk) || !aligned16(v_blk)) return FB_ERR_INVALID_ARG;
  if (!sel_pages || !sel_count || !cache_a || !cache_l || !a_full) return FB_ERR_INVALID_ARG;
  const ResidualPlan p = residual_plan(rs);
  if (ws_bytes < p.ws_bytes || !ws || !aligned16(ws)) return FB_ERR_WORKSPACE;
  if ((st = check_cache(s, cache_l, reuse_mask, nullptr, 0, false, (char*)ws + p.check_off, stream)) != FB_OK)
    return st;
  int32_t* comp_pages = (int32_t*)((char*)ws + p.pages_off);
  int32_t* comp_count = (int32_t*)((char*)ws + p.count_off);

  ResidualArgs r;
  r.batch = s->batch;
  r.h_q = s->h_q;
  r.h_kv = s->h_kv;
  r.G = s->h_q / s->h_kv;
  r.cu = s->cu_seqlens_k;
  r.n_uniform = s->seqlen_k;
  r.page_size = rs->page_size;
  r.max_pages = rs->max_pages;
  r.max_sel = rs->max_sel;
  r.sel_pages = sel_pages;
  r.sel_count = sel_count;
  r.mask = reuse_mask;
  r.comp_pages = comp_pages;
  r.comp_count = comp_count;
  rec(trace ? trace->select_begin : nullptr, stream);
  if (hipError_t e = launch_complement(r, stream)) return hip_status(e);
  rec(trace ? trace->select_end : nullptr, stream);

  AttnArgs a = base_args(s, q);
  a.src0 = make_src(p.rp, p.sel, k, v, s->cu_seqlens_k, s->seqlen_k, (float*)ws, p.rsel);
  a.src0.pages = sel_pages;
  a.src0.page_count = sel_count;
  a.src0.page_size = rs->page_size;
  a.src0.max_union = rs->max_sel;
  a.src1 = make_src(p.rp, p.comp, k, v, s->cu_seqlens_k, s->seqlen_k, (float*)ws, p.rcomp);
  a.src1.pages = comp_pages;
  a.src1.page_count = comp_count;
  a.src1.page_size = rs->page_size;
  a.src1.max_union = rs->max_pages;
  a.src1.mask = reuse_mask;
  AttnArgs ab = base_args(s, q);
  ab.src1 = make_src(p.rp, p.blk, k_blk, v_blk, nullptr, s->block, (float*)ws, p.rblk);
  rec(trace ? trace->attn_begin : nullptr, stream);
  if (hipError_t e = launch_attn(a, s->dtype == FB_BF16, stream)) return hip_status(e);
  if (hipError_t e = launch_attn(ab, s->dtype == FB_BF16, stream)) return hip_status(e);
  rec(trace ? trace->attn_end : nullptr, stream);

  CombineArgs c;
  memset(&c, 0, sizeof(c));
  c.mode = kModeResidual;
  c.batch = s->batch;
  c.B = s->block;
  c.h_q = s->h_q;
  c.h_kv = s->h_kv;
  c.G = s->h_q / s->h_kv;
  c.d = s->head_dim;
  c.po = a.src0.po;
  c.pml = a.src0.pml;
  c.p_rows = p.rp.rows;
  c.p_splits = p.sel.splits;
  c.p_chunk = p.sel.chunk;
  c.page_count = sel_count;
  c.page_size = rs->page_size;
  c.ro = a.src1.po;
  c.rml = a.src1.pml;
  c.r_splits = p.comp.splits;
  c.r_chunk = p.comp.chunk;
  c.r_page_count = comp_count;
  c.bo = ab.src1.po;
  c.bml = ab.src1.pml;
  c.b_rows = p.rp.rows;
  c.b_splits = p.blk.splits;
  c.b_chunk = p.blk.chunk;
  c.mask = reuse_mask;
  c.cache_a = cache_a;
  c.cache_l = cache_l;
  c.a_full = a_full;
  c.l_full = l_full;
  c.out_bf16 = s->dtype == FB_BF16;
  rec(trace ? trace->merge_begin : nullptr, stream);
  if (hipError_t e = launch_combine(c, stream)) return hip_status(e);
  rec(trace ? trace->merge_end : nullptr, stream);
  return FB_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Block lifecycle: append, page metadata of the new pages, and the steps of one block
// ---------------------------------------------------------------------------------------
namespace {

inline size_t el_size(const fb_shape* s) { return s->dtype == FB_BF16 ? 2 : 4; }

struct BlockPlan {
  StepPlan step;
  size_t parts_off, sim_off, ws_bytes;
};
BlockPlan block_plan(const fb_shape* s) {
  BlockPlan p;
  p.step = step_plan(s);
  p.parts_off = align256(p.step.ws_bytes);   // per-row cosine sums, written by the step's combine
  p.sim_off = align256(p.parts_off + (size_t)s->batch * s->block * s->h_q * 3 * sizeof(double));
  p.ws_bytes = align256(p.sim_off + (size_t)s->batch * s->h_q * sizeof(float));
  return p;
}

}  // namespace

extern "C" {

fb_status fb_append_block(const fb_shape* s, const void* k, const void* v, const void* k_blk, const void* v_blk,
                          void* k_out, void* v_out, int32_t* cu_out, hipStream_t stream) {
  fb_status st = check_shape(s);
  if (st != FB_OK) return st;
  if (!k_blk || !v_blk || !k_out || !v_out) return FB_ERR_INVALID_ARG;
  if (!prefix_may_be_empty(s) && (!k || !v)) return FB_ERR_INVALID_ARG;
  const size_t row_bytes = (size_t)s->h_kv * s->head_dim * el_size(s);
  const uintptr_t need = row_bytes % 16 == 0 ? 15u : 3u;
  for (const void* p : {k, v, k_blk, v_blk, (const void*)k_out, (const void*)v_out})
    if (p && ((uintptr_t)p & need)) return FB_ERR_INVALID_ARG;
  const bool in_place = k_out == k && v_out == v && k != nullptr;
  if ((k_out == k) != (v_out == v) && k != nullptr) return FB_ERR_INVALID_ARG;
  if (in_place && s->batch != 1) return FB_ERR_INVALID_ARG;   // later sequences would move
  if (cu_out && (const int32_t*)cu_out == s->cu_seqlens_k) return FB_ERR_INVALID_ARG;
  if ((int64_t)s->batch * (max_prefix(s) + (int64_t)s->block) >= INT32_MAX) return FB_ERR_UNSUPPORTED;
  AppendArgs a;
  a.k = k;
  a.v = v;
  a.cu = s->cu_seqlens_k;
  a.n_uniform = s->seqlen_k;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k_out = k_out;
  a.v_out = v_out;
  a.cu_out = cu_out;
  a.batch = s->batch;
  a.B = s->block;
  a.max_len = max_prefix(s);
  a.row_bytes = (int64_t)row_bytes;
  a.tail_only = in_place ? 1 : 0;
  return hip_status(launch_append(a, stream));
}

fb_status losa_page_meta_append(const losa_shape* ls, int32_t n_appended, const void* k, void* kmin, void* kmax,
                                hipStream_t stream) {
  fb_status st = check_losa(ls);
  if (st != FB_OK) return st;
  if (n_appended < 1) return FB_ERR_INVALID_ARG;
  if (!k || !kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)) return FB_ERR_INVALID_ARG;
  return hip_status(launch_page_meta(losa_args(ls), k, kmin, kmax, n_appended, stream));
}

size_t fb_block_workspace_size(const fb_shape* s) {
  if (check_shape(s) != FB_OK) return 0;
  return block_plan(s).ws_bytes;
}

fb_status fb_block_run(const fb_shape* s, const fb_block_plan* plan, const void* q_steps, const void* k,
                       const void* v, const void* k_blk_steps, const void* v_blk_steps, const int32_t* m_steps,
                       float* cache_a, float* cache_l, void* a_full_steps, float* l_full_steps, uint8_t* masks,
                       float* sims, void* ws, size_t ws_bytes, hipStream_t stream) {
  fb_status st = check_shape(s);
  if (st != FB_OK) return st;
  if (!plan || plan->n_steps < 1) return FB_ERR_INVALID_ARG;
  if (plan->rule != FB_RULE_THRESHOLD && plan->rule != FB_RULE_SIMILARITY) return FB_ERR_INVALID_ARG;
  if (plan->rule == FB_RULE_THRESHOLD && !m_steps) return FB_ERR_INVALID_ARG;
  if (plan->rule == FB_RULE_SIMILARITY && !(plan->gamma == plan->gamma)) return FB_ERR_INVALID_ARG;
  if ((st = check_inputs(s, q_steps, k, v)) != FB_OK) return st;
  if (!k_blk_steps || !v_blk_steps || !aligned16(k_blk_steps) || !aligned16(v_blk_steps)) return FB_ERR_INVALID_ARG;
  if (!cache_a || !cache_l || !a_full_steps || !masks || !aligned16(cache_a)) return FB_ERR_INVALID_ARG;
  const BlockPlan p = block_plan(s);
  if (ws_bytes < p.ws_bytes || !ws || !aligned16(ws)) return FB_ERR_WORKSPACE;
  const int64_t bh = (int64_t)s->batch * s->h_q;
  const int64_t q_elems = bh * s->block * s->head_dim;
  const int64_t kb_elems = (int64_t)s->batch * s->block * s->h_kv * s->head_dim;
  const size_t el = el_size(s);
  // every step's operands stay 16-byte aligned
  if ((q_elems * el) % 16 != 0 || (kb_elems * el) % 16 != 0) return FB_ERR_UNSUPPORTED;
  double* parts = (double*)((char*)ws + p.parts_off);
  float* sim_ws = (float*)((char*)ws + p.sim_off);
  const bool cos_needed = plan->rule == FB_RULE_SIMILARITY || sims != nullptr;
  // Per step: the attention and combine launches of fb_step (the combine records the
  // decision it applied in masks[step]); with a similarity, the reduction of the per-row
  // cosine sums the combine wrote, which also writes the next step's per-head mask.
  for (int step = 0; step < plan->n_steps; ++step) {
    uint8_t* m = masks + step * bh;
    const uint8_t* mask_in = nullptr;   // null and no count: every head refreshes
    const int32_t* m_upd = nullptr;
    uint8_t* mask_out = m;
    if (plan->rule == FB_RULE_THRESHOLD && step >= 1) {
      m_upd = m_steps + (int64_t)step * s->batch;   // M < tau, evaluated in the step's kernels
    } else if (plan->rule == FB_RULE_SIMILARITY && step >= 2) {
      mask_in = m;                                  // written by the previous step's reduction
      mask_out = nullptr;
    }
    const char* qs = (const char*)q_steps + step * q_elems * el;
    const char* kbs = (const char*)k_blk_steps + step * kb_elems * el;
    const char* vbs = (const char*)v_blk_steps + step * kb_elems * el;
    char* af = (char*)a_full_steps + step * q_elems * el;
    float* lf = l_full_steps ? l_full_steps + step * bh * s->block : nullptr;
    st = run_step(s, qs, k, v, kbs, vbs, mask_in, m_upd, plan->tau, cache_a, cache_l, af, lf, ws, p.step.ws_bytes,
                  nullptr, stream, cos_needed && step >= 1 ? parts : nullptr, mask_out);
    if (st != FB_OK) return st;
    if (cos_needed) {
      float* sim_s = sims ? sims + step * bh : sim_ws;
      hipError_t e;
      if (step == 0) {
        if (sims && (e = launch_fill_f32(sim_s, bh, __builtin_nanf(""), stream)) != hipSuccess) return hip_status(e);
      } else {
        uint8_t* next = plan->rule == FB_RULE_SIMILARITY && step + 1 < plan->n_steps ? masks + (step + 1) * bh : nullptr;
        if ((e = launch_sim_reduce(s->batch, s->block, s->h_q, parts, sim_s, plan->gamma, next, stream)) != hipSuccess)
          return hip_status(e);
      }
    }
  }
  return FB_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Multi-branch prefix pass over packed variable-length queries
// ---------------------------------------------------------------------------------------
namespace {

fb_status check_varlen(const fb_varlen_shape* vs) {
  if (!vs) return FB_ERR_INVALID_ARG;
  fb_status st = check_shape(&vs->s);
  if (st != FB_OK) return st;
  if (!vs->cu_seqlens_q || vs->total_q < 0) return FB_ERR_INVALID_ARG;
  if ((int64_t)vs->total_q > (int64_t)vs->s.batch * vs->s.block) return FB_ERR_INVALID_ARG;
  if ((int64_t)vs->total_q * vs->s.h_q >= INT32_MAX) return FB_ERR_UNSUPPORTED;
  return FB_OK;
}

struct VarlenPlan {
  StepPlan step;
  size_t rows_off, ws_bytes;
};
VarlenPlan varlen_plan(const fb_varlen_shape* vs) {
  VarlenPlan p;
  p.step = step_plan(&vs->s);
  p.rows_off = align256(p.step.ws_bytes);
  p.ws_bytes = align256(p.rows_off + (size_t)vs->s.batch * vs->s.block * sizeof(int32_t));
  return p;
}

}  // namespace

extern "C" {

size_t fb_prefix_attn_varlen_workspace_size(const fb_varlen_shape* vs) {
  if (check_varlen(vs) != FB_OK) return 0;
  return varlen_plan(vs).ws_bytes;
}

fb_status fb_prefix_attn_varlen(const fb_varlen_shape* vs, const void* q, const void* k, const void* v,
                                float* a_out, float* l_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  fb_status st = check_varlen(vs);
  if (st != FB_OK) return st;
  const fb_shape* s = &vs->s;
  if (vs->total_q == 0) return FB_OK;
  if ((st = check_inputs(s, q, k, v)) != FB_OK) return st;
  if (!a_out || !l_out) return FB_ERR_INVALID_ARG;
  const VarlenPlan p = varlen_plan(vs);
  if (ws_bytes < p.ws_bytes || !ws || !aligned16(ws)) return FB_ERR_WORKSPACE;
  int32_t* row_tok = (int32_t*)((char*)ws + p.rows_off);
  if (hipError_t e = launch_varlen_rows(vs->cu_seqlens_q, s->batch, s->block, vs->total_q, row_tok, stream))
    return hip_status(e);
  AttnArgs a = base_args(s, q);
  a.B = 0;   // queries are addressed by the packed row map alone
  a.src0 = make_src(p.step.rp, p.step.pre, k, v, s->cu_seqlens_k, s->seqlen_k, (float*)ws, p.step.rpre);
  a.src0.row_tok = row_tok;
  a.src0.cu_q = vs->cu_seqlens_q;
  if (hipError_t e = launch_attn(a, s->dtype == FB_BF16, stream)) return hip_status(e);
  CombineArgs c = base_combine(s, p.step, (float*)ws);
  c.mode = kModePrefixOnly;
  c.cache_a = a_out;
  c.cache_l = l_out;
  c.cu_q = vs->cu_seqlens_q;
  return hip_status(launch_combine(c, stream));
}

}  // extern "C"
