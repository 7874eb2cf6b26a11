/* The C ABI used from plain C on the GPU, with no other runtime than HIP: device buffers
 * from hipMalloc, one FlashBlock step ("Resumo Técnico: FlashBlock", §2 Mecanismo Central)
 * and the checks that hold between the library's own calls:
 *   - the step's cache equals the block-external pass fb_prefix_attn (A_out, L_out);
 *   - the step's A_full equals fb_lse_merge of fb_prefix_attn and fb_block_attn
 *     (up to the bf16 rounding of A_full);
 *   - a reuse step on unchanged inputs gives the fresh step's outputs bit for bit and
 *     leaves the cache untouched;
 *   - the threshold rule with a count at or above tau recomputes, bit for bit as fb_step;
 *   - a short workspace is refused before anything is written;
 *   - with FB_FLAG_CHECK_CACHE, reusing a never-written cache (cache_l all NaN) is refused
 *     with FB_ERR_CACHE_INVALID and nothing is written; recomputing everything runs.
 * Parity against the fp64 oracle is the Python suite's job; this program shows the
 * boundary on its own.  Prints one line per check and exits non-zero on a failure. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flashblock.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("FAIL %s: %s\n", what, hipGetErrorString(e));
    ++failures;
    return 0;
  }
  return 1;
}

/* xorshift32 -> uniform [-1, 1) */
static uint32_t rng_state = 12345u;
static float uniform(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (float)(rng_state >> 8) / 8388608.0f - 1.0f;
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

static void* dev_upload(const void* host, size_t bytes) {
  void* d = NULL;
  if (!hip_ok(hipMalloc(&d, bytes), "hipMalloc")) return NULL;
  if (host && !hip_ok(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice), "upload")) return NULL;
  return d;
}

static int download(void* host, const void* dev, size_t bytes) {
  return hip_ok(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost), "download");
}

static uint16_t* bf16_array(size_t n, float scale) {
  uint16_t* a = (uint16_t*)malloc(n * 2);
  for (size_t i = 0; i < n; ++i) a[i] = to_bf16(scale * uniform());
  return a;
}

int main(void) {
  const int batch = 2, h_q = 8, h_kv = 2, d = 128, B = 8;   /* 4 heads x 8 tokens = 32 rows per group */
  const int32_t cu[3] = {0, 700, 1000};
  const int n_tok = 1000;
  const size_t rows = (size_t)batch * B * h_q;
  const float scale = 1.0f / sqrtf((float)d) * 3.0f;

  uint16_t* hq = bf16_array(rows * d, scale);
  uint16_t* hk = bf16_array((size_t)n_tok * h_kv * d, scale);
  uint16_t* hv = bf16_array((size_t)n_tok * h_kv * d, 1.0f);
  uint16_t* hkb = bf16_array((size_t)batch * B * h_kv * d, scale);
  uint16_t* hvb = bf16_array((size_t)batch * B * h_kv * d, 1.0f);

  void* q = dev_upload(hq, rows * d * 2);
  void* k = dev_upload(hk, (size_t)n_tok * h_kv * d * 2);
  void* v = dev_upload(hv, (size_t)n_tok * h_kv * d * 2);
  void* kb = dev_upload(hkb, (size_t)batch * B * h_kv * d * 2);
  void* vb = dev_upload(hvb, (size_t)batch * B * h_kv * d * 2);
  int32_t* dcu = (int32_t*)dev_upload(cu, sizeof(cu));
  if (failures) return 1;

  fb_shape s;
  memset(&s, 0, sizeof(s));
  s.batch = batch; s.h_q = h_q; s.h_kv = h_kv; s.head_dim = d; s.block = B;
  s.cu_seqlens_k = dcu; s.max_seqlen_k = 700; s.dtype = FB_BF16;
  const size_t ws_bytes = fb_workspace_size(&s);
  check(ws_bytes > 0, "workspace size");

  float* cache_a = (float*)dev_upload(NULL, rows * d * 4);
  float* cache_l = (float*)dev_upload(NULL, rows * 4);
  void* a_full = dev_upload(NULL, rows * d * 2);
  float* l_full = (float*)dev_upload(NULL, rows * 4);
  float* a_out = (float*)dev_upload(NULL, rows * d * 4);
  float* l_out = (float*)dev_upload(NULL, rows * 4);
  float* a_in = (float*)dev_upload(NULL, rows * d * 4);
  float* l_in = (float*)dev_upload(NULL, rows * 4);
  float* a_m = (float*)dev_upload(NULL, rows * d * 4);
  float* l_m = (float*)dev_upload(NULL, rows * 4);
  void* ws = dev_upload(NULL, ws_bytes);
  uint8_t zeros[16], ones[16];
  memset(zeros, 0, sizeof(zeros));
  memset(ones, 1, sizeof(ones));
  uint8_t* mask0 = (uint8_t*)dev_upload(zeros, (size_t)batch * h_q);
  uint8_t* mask1 = (uint8_t*)dev_upload(ones, (size_t)batch * h_q);
  const int32_t m_hi[2] = {9, 4};
  int32_t* dm = (int32_t*)dev_upload(m_hi, sizeof(m_hi));
  if (failures) return 1;

  float* c_a = (float*)malloc(rows * d * 4);
  float* c_l = (float*)malloc(rows * 4);
  uint16_t* f_a = (uint16_t*)malloc(rows * d * 2);
  float* f_l = (float*)malloc(rows * 4);
  float* x_a = (float*)malloc(rows * d * 4);
  float* x_l = (float*)malloc(rows * 4);
  uint16_t* g_a = (uint16_t*)malloc(rows * d * 2);
  float* g_l = (float*)malloc(rows * 4);

  /* fresh step */
  check(fb_step(&s, q, k, v, kb, vb, mask0, cache_a, cache_l, a_full, l_full, ws, ws_bytes, NULL, NULL) == FB_OK,
        "fb_step (every head recomputes)");
  hip_ok(hipDeviceSynchronize(), "fresh step");
  download(c_a, cache_a, rows * d * 4);
  download(c_l, cache_l, rows * 4);
  download(f_a, a_full, rows * d * 2);
  download(f_l, l_full, rows * 4);

  /* the three passes separately */
  check(fb_prefix_attn(&s, q, k, v, a_out, l_out, ws, ws_bytes, NULL) == FB_OK, "fb_prefix_attn");
  check(fb_block_attn(&s, q, kb, vb, a_in, l_in, ws, ws_bytes, NULL) == FB_OK, "fb_block_attn");
  check(fb_lse_merge((int64_t)rows, d, a_out, l_out, a_in, l_in, a_m, FB_F32, l_m, NULL) == FB_OK, "fb_lse_merge");
  hip_ok(hipDeviceSynchronize(), "separate passes");
  download(x_a, a_out, rows * d * 4);
  download(x_l, l_out, rows * 4);
  {
    double ea = 0.0, el = 0.0;
    for (size_t i = 0; i < rows * d; ++i) ea = fmax(ea, fabs((double)x_a[i] - c_a[i]) / (1.0 + fabs(c_a[i])));
    for (size_t i = 0; i < rows; ++i) el = fmax(el, fabs((double)x_l[i] - c_l[i]) / (1.0 + fabs(c_l[i])));
    printf("     cache vs fb_prefix_attn: max rel err A %.2e, L %.2e\n", ea, el);
    check(ea <= 1e-5 && el <= 1e-5, "the step's cache is the block-external pass");
  }
  download(x_a, a_m, rows * d * 4);
  download(x_l, l_m, rows * 4);
  {
    double ea = 0.0, el = 0.0;
    for (size_t i = 0; i < rows * d; ++i) {
      const double ref = x_a[i];
      const double e = fabs((double)from_bf16(f_a[i]) - ref) - fabs(ref) * (1.0 / 256.0);
      ea = fmax(ea, e);
    }
    for (size_t i = 0; i < rows; ++i) el = fmax(el, fabs((double)x_l[i] - f_l[i]) / (1.0 + fabs(f_l[i])));
    printf("     A_full vs merge of the passes: excess over bf16 rounding %.2e, L rel err %.2e\n", ea, el);
    check(ea <= 1e-5 && el <= 1e-5, "A_full is the merge of the two passes");
  }

  /* reuse on unchanged inputs: bit for bit, cache untouched */
  check(fb_step(&s, q, k, v, kb, vb, mask1, cache_a, cache_l, a_full, l_full, ws, ws_bytes, NULL, NULL) == FB_OK,
        "fb_step (every head reuses)");
  hip_ok(hipDeviceSynchronize(), "reuse step");
  download(g_a, a_full, rows * d * 2);
  download(g_l, l_full, rows * 4);
  download(x_a, cache_a, rows * d * 4);
  download(x_l, cache_l, rows * 4);
  check(memcmp(g_a, f_a, rows * d * 2) == 0 && memcmp(g_l, f_l, rows * 4) == 0,
        "reuse gives the fresh step's A_full and L_full bit for bit");
  check(memcmp(x_a, c_a, rows * d * 4) == 0 && memcmp(x_l, c_l, rows * 4) == 0, "reuse leaves the cache untouched");

  /* threshold rule: counts 9 and 4 with tau 4 -> both sequences recompute */
  check(fb_step_threshold(&s, q, k, v, kb, vb, dm, 4, cache_a, cache_l, a_full, l_full, ws, ws_bytes, NULL, NULL) ==
            FB_OK, "fb_step_threshold (M >= tau everywhere)");
  hip_ok(hipDeviceSynchronize(), "threshold step");
  download(g_a, a_full, rows * d * 2);
  download(x_a, cache_a, rows * d * 4);
  check(memcmp(g_a, f_a, rows * d * 2) == 0 && memcmp(x_a, c_a, rows * d * 4) == 0,
        "the threshold rule recomputes as fb_step with a zero mask");

  /* short workspace: refused, nothing written */
  check(hip_ok(hipMemset(a_full, 0x5a, rows * d * 2), "sentinel"), "sentinel written");
  check(fb_step(&s, q, k, v, kb, vb, mask0, cache_a, cache_l, a_full, l_full, ws, ws_bytes - 1, NULL, NULL) ==
            FB_ERR_WORKSPACE, "a short workspace is refused");
  hip_ok(hipDeviceSynchronize(), "refused step");
  download(g_a, a_full, rows * d * 2);
  {
    int untouched = 1;
    for (size_t i = 0; i < rows * d; ++i) untouched &= g_a[i] == 0x5a5a;
    check(untouched, "nothing was written");
  }

  /* debug cache check: a fresh cache (cache_l all NaN) may not be reused */
  {
    fb_shape sd = s;
    sd.flags = FB_FLAG_CHECK_CACHE;
    hip_ok(hipMemset(cache_l, 0xff, rows * 4), "NaN cache_l");   /* 0xffffffff is a NaN */
    hip_ok(hipMemset(a_full, 0x5a, rows * d * 2), "sentinel");
    check(fb_step(&sd, q, k, v, kb, vb, mask1, cache_a, cache_l, a_full, l_full, ws, ws_bytes, NULL, NULL) ==
              FB_ERR_CACHE_INVALID, "reusing a never-written cache is refused (FB_FLAG_CHECK_CACHE)");
    download(g_a, a_full, rows * d * 2);
    int untouched = 1;
    for (size_t i = 0; i < rows * d; ++i) untouched &= g_a[i] == 0x5a5a;
    check(untouched, "nothing was written");
    check(fb_step(&sd, q, k, v, kb, vb, mask0, cache_a, cache_l, a_full, l_full, ws, ws_bytes, NULL, NULL) == FB_OK,
          "recomputing every head runs with the check on");
    hip_ok(hipDeviceSynchronize(), "checked step");
    download(g_a, a_full, rows * d * 2);
    check(memcmp(g_a, f_a, rows * d * 2) == 0, "the checked step gives the fresh step's A_full bit for bit");
  }

  void* bufs[] = {q, k, v, kb, vb, dcu, cache_a, cache_l, a_full, l_full, a_out, l_out, a_in, l_in, a_m, l_m, ws,
                  mask0, mask1, dm};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) hip_ok(hipFree(bufs[i]), "hipFree");
  free(hq); free(hk); free(hv); free(hkb); free(hvb);
  free(c_a); free(c_l); free(f_a); free(f_l); free(x_a); free(x_l); free(g_a); free(g_l);
  printf("%d failure(s)\n", failures);
  return failures ? 1 : 0;
}
