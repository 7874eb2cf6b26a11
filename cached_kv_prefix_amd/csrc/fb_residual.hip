// Complement page lists for FlashBlock with a cached sparse residual.
//
// "Resumo Técnico: FlashBlock", §2, Estratégias de Reutilização Adaptativa,
// "Compatibilidade com Atenção Esparsa": the prefix keys that a sparse selection leaves out play the
// part of the block-external set, and their attention is cached and reused.  A step that
// refreshes the residual attends to exactly those keys, so it needs, per (sequence, KV
// head), the ascending list of the prefix pages outside the selection.
//
// One workgroup per (KV head, sequence): the selection is scattered into an LDS bitmap of
// the sequence's pages, every thread counts the unselected pages of its run of bitmap
// words, a block scan turns the counts into output positions, and each thread writes its
// pages in ascending order.  A group whose query heads all reuse the cached residual gets
// an empty list: nothing of the complement is read in that step.
#include "fb_device.hpp"
#include "fb_internal.hpp"

namespace fb {

__global__ void __launch_bounds__(256) complement_kernel(const ResidualArgs r) {
  __shared__ uint32_t bits[kResidualMaxPages / 32];
  __shared__ int tmp[4];
  const int hk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t grp = (int64_t)b * r.h_kv + hk;
  if (r.mask) {   // uniform over the workgroup
    bool any = false;
    for (int j = 0; j < r.G; ++j) any |= r.mask[b * r.h_q + hk * r.G + j] == 0;
    if (!any) {   // an empty list: the complement pass of this group reads nothing
      if (tid == 0) r.comp_count[grp] = 0;
      return;
    }
  }
  const int n = r.cu ? r.cu[b + 1] - r.cu[b] : r.n_uniform;
  const int np = min((n + r.page_size - 1) / r.page_size, r.max_pages);
  const int nw = (np + 31) / 32;
  for (int i = tid; i < nw; i += 256) bits[i] = 0u;
  __syncthreads();

  const int cnt = max(0, min(r.sel_count[grp], r.max_sel));
  const int32_t* sel = r.sel_pages + grp * r.max_sel;
  for (int i = tid; i < cnt; i += 256) {
    const int p = sel[i];
    if (p >= 0 && p < np) atomicOr(&bits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();

  // thread t owns bitmap words [t * wpt, t * wpt + wpt)
  const int wpt = (nw + 255) / 256;
  auto free_bits = [&](int wi) -> uint32_t {
    const int lo = wi * 32;
    const uint32_t valid = np - lo >= 32 ? 0xffffffffu : ((1u << (np - lo)) - 1u);
    return ~bits[wi] & valid;
  };
  int c = 0;
  for (int k = 0; k < wpt; ++k) {
    const int wi = tid * wpt + k;
    if (wi < nw) c += __popc(free_bits(wi));
  }
  int total;
  int pos = block_incl_scan(c, tmp, &total) - c;
  int32_t* out = r.comp_pages + grp * r.max_pages;
  for (int k = 0; k < wpt; ++k) {
    const int wi = tid * wpt + k;
    if (wi >= nw) break;
    uint32_t m = free_bits(wi);
    while (m) {
      out[pos++] = wi * 32 + __ffs(m) - 1;
      m &= m - 1u;
    }
  }
  if (tid == 0) r.comp_count[grp] = total;
}

hipError_t launch_complement(const ResidualArgs& r, hipStream_t st) {
  if (r.batch == 0 || r.h_kv == 0) return hipSuccess;
  if (r.max_pages > kResidualMaxPages) return hipErrorInvalidValue;
  hipLaunchKernelGGL(complement_kernel, dim3(r.h_kv, r.batch), dim3(256), 0, st, r);
  return hipGetLastError();
}

}  // namespace fb
