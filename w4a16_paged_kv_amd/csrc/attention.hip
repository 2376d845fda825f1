// Paged-attention decode kernel for gfx950: one workgroup of eight
// wavefronts per (split of pages, KV head, sequence); the work itself is
// attn_item in attn_item.h.
#include <hip/hip_runtime.h>

#include "attn_item.h"

namespace w4 {

// At most 128 VGPRs, so two workgroups share a CU (four wavefronts per
// SIMD): the many-sequence workloads need that memory parallelism (32
// sequences, contexts up to 8192: 120 -> 85 us with the bound).
// The grid is (sequence, KV head, split) with the split slowest, so the
// dispatcher sends every sequence's first splits before any later ones and
// the items past a short sequence's last split (which exit at once) come at
// the end (32 sequences, contexts 128-8192: 78 -> 75 us).
template <int D, int GQ>
__global__ __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void paged_attn_kernel(AttnArgs a) {
  attn_item<D, GQ, kAttnWaves * 64>(a, blockIdx.z, blockIdx.y, blockIdx.x);
}

bool attention_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 ||
                                                 group == 7 || group == 8);
}

// Pages per split: one page per wavefront until the launch would exceed
// about 512 workgroups, then up to eight (several pages per wavefront overlap
// one page's K/V latency with the previous page's work, and longer items
// spend less of their time in the combine and merge tail; measured at 16
// sequences of 1024-4096 tokens: 2048 workgroups 45.6 us, 512 28.2 us; at
// 32 sequences of 128-8192 tokens: four pages per wavefront 75 us, eight
// 69 us, sixteen 70.5 us); at most 128 splits per sequence (the merge keeps
// two floats per (head, split) in LDS).
int attention_pages_per_split(int batch, int n_kv_heads, int max_pages) {
  const long units = (long)batch * n_kv_heads * max_pages;
  int per_wave = 1;
  while (per_wave < 8 && units / ((long)kAttnWaves * per_wave) > 512) per_wave *= 2;
  int pps = kAttnWaves * per_wave;
  while ((max_pages + pps - 1) / pps > 128) pps *= 2;
  return pps;
}

template <int D, int GQ>
static hipError_t launch_dg(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((paged_attn_kernel<D, GQ>), dim3(a.batch, a.n_kv_heads, a.max_splits),
                     dim3(kAttnWaves * 64), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_dg<D, 1>(a, s);
    case 2: return launch_dg<D, 2>(a, s);
    case 4: return launch_dg<D, 4>(a, s);
    case 7: return launch_dg<D, 7>(a, s);
    case 8: return launch_dg<D, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, int group, hipStream_t s) {
  if (head_dim == 64) return launch_d<64>(a, group, s);
  if (head_dim == 128) return launch_d<128>(a, group, s);
  return hipErrorInvalidValue;
}

}  // namespace w4
