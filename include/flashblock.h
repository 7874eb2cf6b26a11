/*
 * flashblock.h — C ABI of the MI355X (gfx950) FlashBlock / LoSA hot-path library.
 *
 * Method sources ("the pages"):
 *   [FB-pt]  "Resumo Técnico: FlashBlock" (gist.science, Portuguese), §2 Metodologia:
 *            "Mecanismo Central" (split into block-internal A_in over J_in and
 *            block-external A_out over J_out, cached A_out with L_out = log Z_out, and the
 *            log-space merge A_full = (e^{L_out-m} A_out + e^{L_in-m} A_in) /
 *            (e^{L_out-m} + e^{L_in-m}), m = max(L_out, L_in)); "Estratégias de
 *            Reutilização Adaptativa" (threshold rule M < tau; per-head rule sim > gamma).
 *            "Compatibilidade com Atenção Esparsa" (unselected keys as the block-external
 *            set, their residual contribution cached).
 *   [FB-abs] "FlashBlock: Attention Caching for Efficient Long-Context Block Diffusion",
 *            abstract: block-wise causal inference over a growing KV cache; FlashBlock as
 *            a complementary residual reuse strategy under sparse attention.
 *   [LoSA]   "LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion Language
 *            Models" (gist.science, Spanish), §1 (KV inflation: cost is the size of the
 *            union of the queries' selections) and §2 "El Algoritmo LoSA" steps 1-4.
 *   [BB]     "Resumen Técnico: BlockBatch" (gist.science, Spanish), "Optimización del
 *            Sistema": packed variable-length buffers (the cu_seqlens layout below).
 *
 * Conventions shared by every call
 *   - Ownership: the caller allocates every buffer (inputs, outputs, cache, workspace) in
 *     device memory; the library allocates no device memory, keeps no state between calls
 *     and may be called concurrently on different streams with disjoint buffers.
 *   - Execution: all work is enqueued on `stream`; no call synchronises the host (but for
 *     the debug check that FB_FLAG_CHECK_CACHE asks for).
 *   - Errors: arguments are checked on the host before anything is enqueued; on any
 *     error the call returns a non-zero fb_status and writes nothing.  A failed kernel
 *     launch returns FB_ERR_HIP.  No C++ exception crosses this interface.  Device-side
 *     values (cu_seqlens_k contents, masks, counts) are trusted: the caller keeps them
 *     within the documented ranges.
 *   - Layouts (row-major, innermost last):
 *       q, a_full, cache_a    [batch][B][h_q][d]
 *       cache_l, l_full       [batch][B][h_q]          (natural-log normalisers)
 *       k, v (prefix)         [sum_b N_b][h_kv][d]     packed by cu_seqlens_k
 *       k_blk, v_blk          [batch][B][h_kv][d]
 *       reuse mask            [batch][h_q] uint8, 1 = reuse the cache, 0 = recompute
 *     Query head h reads KV head h / (h_q / h_kv) (grouped-query attention).
 *   - Scores are softmax_scale * <q, k>; L values are natural logarithms of the softmax
 *     normaliser; an empty key set gives A = 0 and L = -inf.
 *   - Element types: FB_BF16 (bfloat16 in, fp32 accumulation) or FB_F32 (fp32 in and
 *     fp32 arithmetic).  The cache and every L buffer are always fp32.  a_full has the
 *     input element type.
 *   - Supported: head_dim 64 or 128 for FB_BF16, any head_dim in [1, 256] for FB_F32;
 *     h_q % h_kv == 0; B >= 1; batch >= 1.  Anything else returns FB_ERR_UNSUPPORTED.
 */
#ifndef FLASHBLOCK_H
#define FLASHBLOCK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fb_status {
  FB_OK = 0,
  FB_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, h_q % h_kv != 0, ...      */
  FB_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. bf16 with head_dim 96)     */
  FB_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the matching *_workspace_size()       */
  FB_ERR_CACHE_INVALID = 4,/* FB_FLAG_CHECK_CACHE: a cache row the call would reuse has
                              never been written (its cache_l entry is NaN)              */
  FB_ERR_HIP = 5           /* a HIP launch or runtime call failed                         */
} fb_status;

/* fb_shape.flags.
 * FB_FLAG_CHECK_CACHE (debug): a cache row that has never been written is marked by NaN in
 * cache_l (the caller fills a new cache's cache_l with NaN; every call that writes a row
 * stores a number or -inf there).  With the flag set, fb_step, fb_step_threshold,
 * fb_block_run, losa_step and fb_residual_step first check on the device every row the
 * call would reuse: rows of heads whose reuse bit is 1 or whose sequence has M < tau, and
 * for losa_step every row of a block that has stable rows (|A| < B).  If any of them holds
 * NaN, the call returns FB_ERR_CACHE_INVALID and writes nothing but its workspace.  The
 * check reads one flag back, so it synchronises `stream`: the one exception to the
 * no-synchronisation rule, for debug runs only.  The other calls ignore the flag. */
#define FB_FLAG_CHECK_CACHE 1u

typedef enum fb_dtype { FB_BF16 = 0, FB_F32 = 1 } fb_dtype;

typedef struct fb_shape {
  int32_t batch;               /* sequences in the batch                                  */
  int32_t h_q;                 /* query heads                                             */
  int32_t h_kv;                /* key/value heads; h_q % h_kv == 0                        */
  int32_t head_dim;            /* d                                                       */
  int32_t block;               /* B: block (query) tokens per sequence                    */
  const int32_t* cu_seqlens_k; /* device [batch + 1], prefix offsets, cu[0] = 0,
                                  non-decreasing; NULL: every prefix has seqlen_k tokens   */
  int32_t seqlen_k;            /* prefix length when cu_seqlens_k is NULL (may be 0)      */
  int32_t max_seqlen_k;        /* with cu_seqlens_k: an upper bound of every N_b (sizes
                                  the launch); ignored when cu_seqlens_k is NULL           */
  fb_dtype dtype;              /* element type of q, k, v, k_blk, v_blk and a_full        */
  float softmax_scale;         /* 0 selects 1/sqrt(head_dim)                              */
  int32_t num_splits;          /* prefix key chunks per sequence and KV head; 0 = chosen
                                  from the shape alone (deterministic for a given shape)   */
  uint32_t flags;              /* 0 or FB_FLAG_CHECK_CACHE; other bits are invalid        */
} fb_shape;

/* Optional timing hooks: each non-null event is recorded on the call's stream right
 * before / after the named kernel.  Recording changes no result. */
typedef struct fb_trace {
  hipEvent_t attn_begin, attn_end;    /* the attention kernel (prefix and block passes)  */
  hipEvent_t merge_begin, merge_end;  /* the split-reduction / merge / cache kernel      */
  hipEvent_t select_begin, select_end;/* LoSA selection (scores, top-k, union); residual: complement */
} fb_trace;

const char* fb_status_string(fb_status s);

/* Bytes of device workspace that fb_prefix_attn, fb_block_attn and fb_step need for
 * this shape (split-KV partial results).  0 on an invalid shape. */
size_t fb_workspace_size(const fb_shape* s);

/* Block-external pass [FB-pt §2 Mecanismo Central]: for every block query, attention over
 * its sequence's whole prefix.
 *   q [batch][B][h_q][d] (dtype); k, v [sum N_b][h_kv][d] (dtype)
 *   a_out [batch][B][h_q][d] fp32 (normalised within the prefix); l_out [batch][B][h_q]
 *   fp32 = log Z_out.  Empty prefix: a_out = 0, l_out = -inf. */
fb_status fb_prefix_attn(const fb_shape* s, const void* q, const void* k, const void* v,
                         float* a_out, float* l_out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* Block-internal pass [FB-pt §2 Mecanismo Central]: attention of every block query over
 * the B tokens of its own block, bidirectional (every block query sees every block key).
 *   k_blk, v_blk [batch][B][h_kv][d]; a_in fp32 [batch][B][h_q][d]; l_in [batch][B][h_q]. */
fb_status fb_block_attn(const fb_shape* s, const void* q, const void* k_blk,
                        const void* v_blk, float* a_in, float* l_in, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* Log-space merge [FB-pt §2, merge equation], row by row:
 *   m = max(l_out, l_in); A = (e^{l_out-m} a_out + e^{l_in-m} a_in) / (e^{l_out-m} + e^{l_in-m})
 *   l_full = m + log(e^{l_out-m} + e^{l_in-m})  (optional output; not printed on the pages)
 * a_out, a_in [rows][d] fp32; l_out, l_in [rows] fp32; a_full [rows][d] of out_dtype;
 * l_full [rows] fp32 or NULL.  Both sides empty (-inf) gives A = 0, l_full = -inf.
 * rows may be 0 (nothing is done). */
fb_status fb_lse_merge(int64_t rows, int32_t d, const float* a_out, const float* l_out,
                       const float* a_in, const float* l_in, void* a_full,
                       fb_dtype out_dtype, float* l_full, hipStream_t stream);

/* One FlashBlock denoising step [FB-pt §2]:
 *   for (b, h) with reuse_mask[b][h] == 0: (A_out, L_out) over the prefix is recomputed
 *     and written to cache_a / cache_l (rows of head h of sequence b);
 *   for (b, h) with reuse_mask[b][h] == 1: the prefix is not read and the cache rows are
 *     left untouched (they must hold a previous step's values);
 *   every row: (A_in, L_in) over the block, then a_full = merge(cache, in) and, if
 *   l_full is non-null, l_full = the merged log-normaliser.
 * reuse_mask may be NULL (recompute every head).  The first step of a block must use an
 * all-zero mask.  A KV head's prefix is read when any of its query heads recomputes.
 * With identical inputs and cache, reuse and recompute give bit-identical a_full. */
fb_status fb_step(const fb_shape* s, const void* q, const void* k, const void* v,
                  const void* k_blk, const void* v_blk, const uint8_t* reuse_mask,
                  float* cache_a, float* cache_l, void* a_full, float* l_full, void* ws,
                  size_t ws_bytes, const fb_trace* trace, hipStream_t stream);

/* fb_step with the threshold rule [FB-pt §2] evaluated inside the step's kernels:
 * identical results to fb_mask_threshold(m_updated, tau) followed by fb_step with that
 * mask, with one kernel launch fewer.  m_updated: device int32 [batch], the number of
 * tokens updated since the previous step (the first step of a block must pass a count
 * >= tau for every sequence). */
fb_status fb_step_threshold(const fb_shape* s, const void* q, const void* k, const void* v,
                            const void* k_blk, const void* v_blk, const int32_t* m_updated,
                            int32_t tau, float* cache_a, float* cache_l, void* a_full,
                            float* l_full, void* ws, size_t ws_bytes, const fb_trace* trace,
                            hipStream_t stream);

/* Bytes of the static device array that fb_step_noalloc uses on each GPU (64 MiB). */
#define FB_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* fb_step for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results and
 * errors as fb_step, without the workspace and the timing hooks: the split-KV partial
 * results go to a static device array of FB_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends.  A shape whose fb_workspace_size() is
 * larger returns FB_ERR_WORKSPACE and writes nothing (the dLLM step with a 32768-token
 * prefix and 32 heads needs about 4 MiB).  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.  On its first call on a device the library
 * looks up the array's address there (with that device current) and keeps it.  Every call
 * on one GPU shares that GPU's array, which keeps the last call's contents; nothing in it
 * needs to start at zero.  Calls that overlap on one GPU (other streams, other threads)
 * race on the array: the caller serialises them. */
fb_status fb_step_noalloc(const fb_shape* s, const void* q, const void* k, const void* v,
                          const void* k_blk, const void* v_blk, const uint8_t* reuse_mask,
                          float* cache_a, float* cache_l, void* a_full, float* l_full,
                          hipStream_t stream);

/* Threshold reuse rule [FB-pt §2]: mask[b][h] = (m_updated[b] < tau) for every h.
 * m_updated: device int32 [batch] (tokens updated since the previous step). */
fb_status fb_mask_threshold(const int32_t* m_updated, int32_t tau, int32_t batch,
                            int32_t h_q, uint8_t* mask, hipStream_t stream);

/* Per-head reuse rule [FB-pt §2]: mask[i] = (sim[i] > gamma), fp32 comparison, for
 * i < n.  sim: device fp32 [n]. */
fb_status fb_mask_similarity(const float* sim, float gamma, int64_t n, uint8_t* mask,
                             hipStream_t stream);

/* Per-head similarity estimate used with the per-head rule: cosine of the two heads'
 * B x d block-external outputs, sim[b][h] = <x, y> / (|x| |y|), accumulated in fp64 and
 * returned in fp32; a zero vector gives 0.  a_prev, a_cur fp32 [batch][B][h_q][d]. */
fb_status fb_head_cosine(int32_t batch, int32_t block, int32_t h_q, int32_t head_dim,
                         const float* a_prev, const float* a_cur, float* sim,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * LoSA-style sparse path [LoSA §2].
 * Page metadata layout (kmin and kmax, same element type as k):
 *   [batch][h_kv][head_dim / 8][max_pages][8]   (head_dim % 8 == 0)
 * page p of sequence b holds the element-wise min / max over its valid keys
 * (tokens 16p .. min(16p + 16, N_b) - 1 for page_size 16).
 * ------------------------------------------------------------------------------------ */
typedef struct losa_shape {
  fb_shape s;          /* B, heads, prefix lengths, dtype; s.block is the block size     */
  int32_t page_size;   /* tokens per page (>= 1)                                         */
  int32_t topk;        /* pages kept per (active query, head)                            */
  int32_t n_active;    /* |A|: active tokens per sequence, 1 <= n_active <= B <= 1024     */
  int32_t max_pages;   /* >= ceil(N_b / page_size) for every b; <= 16384                  */
} losa_shape;

/* Bytes of one metadata buffer (kmin or kmax). */
size_t losa_meta_bytes(const losa_shape* ls);
/* Workspace bytes for losa_select_union and losa_step. */
size_t losa_workspace_size(const losa_shape* ls);
/* Capacity of union_pages per (b, kv head): min(n_active * (h_q/h_kv) * topk, max_pages). */
int32_t losa_union_capacity(const losa_shape* ls);

/* Page min/max build (set-up for the selector, once per committed block). */
fb_status losa_page_meta(const losa_shape* ls, const void* k, void* kmin, void* kmax,
                         hipStream_t stream);

/* Selection half of the sparse step [LoSA §2 steps 1 and 3]:
 *   1. score[b][i] = mean over (head, dim) of (q_cur - q_prev)^2 (fp64, summed per head
 *      over dims, then over heads, each left to right);  active[b] = the n_active tokens
 *      with the largest score, ties to the lower index, ascending.
 *   3. for every active token a and query head h: page score
 *      S = sum_d max(q_d kmin_d, q_d kmax_d) over the KV head's page metadata (fp64,
 *      left to right over d); topk_pages[b][h][a] = the topk best pages (score desc,
 *      index asc), ascending, padded with -1 when the sequence has fewer pages;
 *      union_pages[b][g] = the ascending union over the active tokens and the query heads
 *      of KV head g, union_count[b][g] its length.
 * Shapes: active int32 [batch][n_active]; topk_pages int32 [batch][h_q][n_active][topk];
 * union_pages int32 [batch][h_kv][losa_union_capacity]; union_count int32 [batch][h_kv]. */
fb_status losa_select_union(const losa_shape* ls, const void* q_cur, const void* q_prev,
                            const void* kmin, const void* kmax, int32_t* active,
                            int32_t* topk_pages, int32_t* union_pages,
                            int32_t* union_count, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* One sparse step t >= 1 [LoSA §2 steps 1-4]: losa_select_union, then
 *   - active rows (token in active, every query head): attention over every token of the
 *     union pages of their KV head (tokens >= N_b excluded); the result replaces their
 *     cache rows (o_p, L_p);
 *   - stable rows: cache rows untouched, prefix not read;
 *   - every row: block pass and a_full = merge(cache, in) (l_full optional).
 * The cache must hold every row's prefix statistics from an earlier step (for example a
 * fb_step with an all-zero mask). */
fb_status losa_step(const losa_shape* ls, const void* q_cur, const void* q_prev,
                    const void* k, const void* v, const void* k_blk, const void* v_blk,
                    const void* kmin, const void* kmax, float* cache_a, float* cache_l,
                    void* a_full, float* l_full, int32_t* active, int32_t* topk_pages,
                    int32_t* union_pages, int32_t* union_count, void* ws, size_t ws_bytes,
                    const fb_trace* trace, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * FlashBlock with a cached sparse residual [FB-pt §2, Estratégias de Reutilização
 * Adaptativa, "Compatibilidade com Atenção Esparsa"; FB-abs: a complementary residual
 * reuse strategy for sparse attention]: the prefix keys that a sparse selection leaves
 * out are treated as the block-external set, and their attention (the residual) is cached.
 * ------------------------------------------------------------------------------------ */
typedef struct fb_residual_shape {
  fb_shape s;          /* B, heads, prefix lengths, dtype                                 */
  int32_t page_size;   /* tokens per page (>= 1); page p holds tokens p*P .. p*P + P - 1  */
  int32_t max_pages;   /* >= ceil(N_b / page_size) for every b; <= 65536                  */
  int32_t max_sel;     /* capacity of sel_pages per (b, kv head), 1 <= max_sel <= max_pages */
} fb_residual_shape;

/* Workspace bytes for fb_residual_step (partials of the three passes and the complement
 * page lists).  0 on an invalid shape. */
size_t fb_residual_workspace_size(const fb_residual_shape* rs);

/* One step with a cached residual.  Selection S[b][g] = sel_pages[b][g][0 .. sel_count[b][g]),
 * distinct page indices below ceil(N_b / page_size), any order (for example the
 * losa_select_union output, with max_sel = losa_union_capacity); sel_count in [0, max_sel].
 * Indices outside [0, ceil(N_b / page_size)) are skipped, and a count above max_sel reads
 * max_sel entries (no access leaves the list or the sequence).
 *   every row, every step: (A_s, L_s) = attention over the tokens of S of its KV head;
 *   rows of heads with reuse_mask[b][h] == 0 (refresh): (A_r, L_r) = attention over the
 *     prefix tokens outside S, written to cache_a / cache_l;
 *   rows of heads with reuse_mask[b][h] == 1 (reuse): the pages outside S are not read;
 *     (A_r, L_r) = the cache rows, left untouched;
 *   every row: (A_in, L_in) over the block, then the three-way log-space merge
 *     m = max(L_s, L_r, L_in), a_full = sum_i e^{L_i-m} A_i / sum_i e^{L_i-m},
 *     l_full = m + log sum_i e^{L_i-m} (optional output).
 * Tokens >= N_b do not exist (the tail page is partial).  A refresh step attends to every
 * prefix token exactly once, so it equals full attention over prefix and block.  The first
 * step must refresh every head.  reuse_mask may be NULL (refresh every head).  With
 * identical inputs and cache, reuse and refresh give bit-identical a_full. */
fb_status fb_residual_step(const fb_residual_shape* rs, const void* q, const void* k, const void* v,
                           const void* k_blk, const void* v_blk, const int32_t* sel_pages,
                           const int32_t* sel_count, const uint8_t* reuse_mask, float* cache_a,
                           float* cache_l, void* a_full, float* l_full, void* ws, size_t ws_bytes,
                           const fb_trace* trace, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Block lifecycle [FB-abs: block-wise causal inference over a KV cache that grows block by
 * block; FB-pt §2 "Estratégias de Reutilização Adaptativa" for the two reuse rules].
 * ------------------------------------------------------------------------------------ */

/* Append a finished block to the prefix: for every sequence b the new prefix is the old
 * one (N_b tokens of k, v as s describes them) followed by the block's B tokens
 * k_blk[b], v_blk[b].
 *   k_out, v_out [sum_b (N_b + B)][h_kv][d] (dtype); cu_out: device int32 [batch + 1]
 *   receives the new offsets (cu[b] + b*B, or b*(seqlen_k + B) for a uniform prefix); it
 *   may be NULL and must not be s->cu_seqlens_k.
 *   In place (k_out == k and v_out == v) is allowed for batch == 1 only: then only the B
 *   block rows are written, after the prefix (the buffers must hold N + B tokens).  Any
 *   other overlap of outputs and inputs is not allowed.  k, v may be NULL for an empty
 *   uniform prefix. */
fb_status fb_append_block(const fb_shape* s, const void* k, const void* v, const void* k_blk,
                          const void* v_blk, void* k_out, void* v_out, int32_t* cu_out,
                          hipStream_t stream);

/* Page metadata after an append: ls describes the grown prefix; the pages that hold one of
 * the last n_appended tokens of each sequence are rebuilt from k, the others are left as
 * they are.  When kmin/kmax held the metadata of the old prefix the result equals
 * losa_page_meta over the grown prefix, bit for bit. */
fb_status losa_page_meta_append(const losa_shape* ls, int32_t n_appended, const void* k,
                                void* kmin, void* kmax, hipStream_t stream);

typedef enum fb_reuse_rule { FB_RULE_THRESHOLD = 0, FB_RULE_SIMILARITY = 1 } fb_reuse_rule;

typedef struct fb_block_plan {
  int32_t n_steps;   /* S >= 1 denoising steps of the block                                 */
  int32_t rule;      /* fb_reuse_rule                                                        */
  int32_t tau;       /* threshold rule: sequence b reuses at step s >= 1 when M_s[b] < tau   */
  float gamma;       /* similarity rule: head h reuses at step s >= 2 when sim_{s-1} > gamma  */
} fb_block_plan;

/* Workspace bytes for fb_block_run (a step's workspace, per-row cosine sums, similarities). */
size_t fb_block_workspace_size(const fb_shape* s);

/* The S steps of one block, each an fb_step, with the reuse mask of every step chosen by
 * the plan's rule and recorded in masks (the reuse statistics):
 *   threshold: step 0 refreshes every head; step s >= 1 uses fb_mask_threshold(M_s, tau);
 *   similarity: after step s >= 1, sim_s[b][h] = fb_head_cosine(cache_a before step s,
 *     cache_a after it) (two consecutive computed A_out of the head; a head that reused
 *     keeps its cache, so its similarity is 1); steps 0 and 1 refresh every head, step
 *     s >= 2 uses fb_mask_similarity(sim_{s-1}, gamma).
 * Per-step operands are consecutive in memory:
 *   q_steps [S][batch][B][h_q][d]; k_blk_steps, v_blk_steps [S][batch][B][h_kv][d];
 *   m_steps [S][batch] int32 (threshold rule; step 0's entry is not read);
 *   a_full_steps [S][batch][B][h_q][d] (dtype); l_full_steps [S][batch][B][h_q] or NULL;
 *   masks [S][batch][h_q] uint8 (output); sims [S][batch][h_q] fp32 or NULL (output; step
 *   0 holds NaN; with the threshold rule the similarities are reported, not used).
 * cache_a / cache_l: the cache, left holding the last step's values; its contents on entry
 * are not read (step 0 refreshes).  One step's q and block K/V must be a multiple of 16 bytes
 * (FB_ERR_UNSUPPORTED otherwise). */
fb_status fb_block_run(const fb_shape* s, const fb_block_plan* plan, const void* q_steps,
                       const void* k, const void* v, const void* k_blk_steps,
                       const void* v_blk_steps, const int32_t* m_steps, float* cache_a,
                       float* cache_l, void* a_full_steps, float* l_full_steps, uint8_t* masks,
                       float* sims, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Several branches in one prefix pass [BB, "Optimización del Sistema": the query positions
 * of all active branches, each with its own block size and its own KV cache, packed into
 * one variable-length buffer and processed in one pass].
 * ------------------------------------------------------------------------------------ */
typedef struct fb_varlen_shape {
  fb_shape s;                  /* s.batch = branches; s.block = B_max, a bound of every
                                  branch's block; prefixes as in fb_shape (branch b's own)  */
  const int32_t* cu_seqlens_q; /* device [batch + 1]: branch b owns packed query rows
                                  cu_q[b] .. cu_q[b+1]-1, cu_q[0] = 0, B_b <= B_max        */
  int32_t total_q;             /* cu_seqlens_q[batch] (host copy; sizes the launch)        */
} fb_varlen_shape;

/* Workspace bytes for fb_prefix_attn_varlen; 0 on an invalid shape. */
size_t fb_prefix_attn_varlen_workspace_size(const fb_varlen_shape* vs);

/* Block-external pass of every branch [FB-pt §2 Mecanismo Central], one launch for all:
 * each packed query attends to its own branch's prefix.
 *   q [total_q][h_q][d] (dtype); a_out [total_q][h_q][d] fp32; l_out [total_q][h_q] fp32.
 * A branch with an empty prefix gives a_out = 0, l_out = -inf; an empty branch (B_b = 0)
 * has no rows.  total_q == 0 does nothing. */
fb_status fb_prefix_attn_varlen(const fb_varlen_shape* vs, const void* q, const void* k,
                                const void* v, float* a_out, float* l_out, void* ws,
                                size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FLASHBLOCK_H */
