// Device helpers shared by the attention kernels: where a work item's keys live.
#pragma once
#include "fb_device.hpp"
#include "fb_internal.hpp"

namespace fb {

struct SeqInfo {
  int seq0, n_seq, n_keys;
};

// Prefix / block / union-page extent of sequence b for KV head hk.
__device__ __forceinline__ SeqInfo seq_info(const AttnSrc& S, int b, int hk, int h_kv) {
  SeqInfo r;
  if (S.cu) {
    r.seq0 = S.cu[b];
    r.n_seq = S.cu[b + 1] - r.seq0;
  } else {
    r.seq0 = b * S.n_uniform;
    r.n_seq = S.n_uniform;
  }
  // a page count is clamped to the list's capacity, so no key reads past the list
  r.n_keys = S.pages ? min(S.page_count[b * h_kv + hk], S.max_union) * S.page_size : r.n_seq;
  return r;
}

// Token (within the sequence) of source key `key`; clamps to a readable token and
// reports whether the key takes part in the softmax.
__device__ __forceinline__ int key_token(const AttnSrc& S, const int32_t* pg, int key, int kend, int n_seq,
                                         bool& ok) {
  ok = key < kend;
  if (!ok) key = kend - 1;
  if (pg) {
    // 64-bit: a page index outside the sequence must not wrap into it
    const int64_t t64 = (int64_t)pg[key / S.page_size] * S.page_size + key % S.page_size;
    int t = (int)t64;
    if (t64 < 0 || t64 >= n_seq) {   // a page outside the sequence: skipped
      ok = false;
      t = n_seq > 0 ? n_seq - 1 : 0;
    }
    return t;
  }
  return key;
}

}  // namespace fb
