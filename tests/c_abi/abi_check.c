/* The C ABI used from plain C (C99, gcc): sizes from shapes alone, and argument errors
 * returned before anything is enqueued.  Needs no GPU: no call here reaches a launch.
 * Prints one line per check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "flashblock.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  void* p = (void*)(uintptr_t)0x10000; /* never dereferenced: every call below fails first */
  fb_shape s;
  memset(&s, 0, sizeof(s));
  s.batch = 1; s.h_q = 32; s.h_kv = 32; s.head_dim = 128; s.block = 32; s.seqlen_k = 32768;
  s.dtype = FB_BF16;

  check(strcmp(fb_status_string(FB_OK), "ok") == 0, "status string");
  size_t ws = fb_workspace_size(&s);
  check(ws > 0 && ws == fb_workspace_size(&s), "step workspace from the shape alone");
  check(fb_block_workspace_size(&s) > ws, "block driver workspace adds its own buffers");

  fb_shape bad = s;
  bad.h_kv = 5;
  check(fb_workspace_size(&bad) == 0, "h_q % h_kv != 0 gives size 0");
  check(fb_step(&bad, p, p, p, p, p, NULL, p, p, p, NULL, p, ws, NULL, NULL) == FB_ERR_INVALID_ARG,
        "fb_step rejects the shape");
  check(fb_step(&s, NULL, p, p, p, p, NULL, p, p, p, NULL, p, ws, NULL, NULL) == FB_ERR_INVALID_ARG,
        "fb_step rejects a null query");
  check(fb_step(&s, p, p, p, p, p, NULL, p, p, p, NULL, p, ws - 1, NULL, NULL) == FB_ERR_WORKSPACE,
        "fb_step rejects a short workspace");
  check(fb_lse_merge(-1, 128, NULL, NULL, NULL, NULL, NULL, FB_F32, NULL, NULL) == FB_ERR_INVALID_ARG,
        "fb_lse_merge rejects negative rows");

  losa_shape ls;
  memset(&ls, 0, sizeof(ls));
  ls.s = s; ls.s.block = 64; ls.s.seqlen_k = 131072; ls.page_size = 16; ls.topk = 64; ls.n_active = 8;
  ls.max_pages = 8192;
  check(losa_union_capacity(&ls) == 512, "union capacity |A| * G * topk");
  check(losa_meta_bytes(&ls) == (size_t)32 * 128 * 8192 * 2, "page metadata bytes");
  check(losa_workspace_size(&ls) > 0, "sparse workspace");

  fb_residual_shape rs;
  memset(&rs, 0, sizeof(rs));
  rs.s = ls.s; rs.page_size = 16; rs.max_pages = 8192; rs.max_sel = 512;
  size_t rws = fb_residual_workspace_size(&rs);
  check(rws > 0, "residual workspace");
  check(fb_residual_step(&rs, p, p, p, p, p, NULL, p, NULL, p, p, p, NULL, p, rws, NULL, NULL) ==
            FB_ERR_INVALID_ARG, "residual step rejects a null selection");

  fb_varlen_shape vs;
  memset(&vs, 0, sizeof(vs));
  vs.s = s; vs.s.batch = 6; vs.s.block = 128; vs.cu_seqlens_q = (const int32_t*)p; vs.total_q = 252;
  check(fb_prefix_attn_varlen_workspace_size(&vs) > 0, "multi-branch workspace");
  vs.total_q = 6 * 128 + 1;
  check(fb_prefix_attn_varlen_workspace_size(&vs) == 0, "more rows than branches x B_max");

  fb_block_plan plan = {8, FB_RULE_SIMILARITY, 0, 0.95f};
  check(fb_block_run(&s, &plan, p, p, p, p, p, NULL, p, p, p, NULL, NULL, NULL, p,
                     fb_block_workspace_size(&s), NULL) == FB_ERR_INVALID_ARG,
        "block driver rejects a missing mask output");

  printf("%d failure(s)\n", failures);
  return failures ? 1 : 0;
}
