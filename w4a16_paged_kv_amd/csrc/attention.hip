// Paged-attention decode kernel for gfx950: one workgroup of eight
// wavefronts per (split of pages, KV head, sequence); the work itself is
// attn_item in attn_item.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_item.h"

namespace w4 {

// At most 128 VGPRs, so two workgroups share a CU (four wavefronts per
// SIMD): the many-sequence workloads need that memory parallelism (32
// sequences, contexts up to 8192: 120 -> 85 us with the bound).
// The grid is (sequence, KV head, split) with the split slowest, so the
// dispatcher sends every sequence's first splits before any later ones and
// the items past a short sequence's last split (which exit at once) come at
// the end (32 sequences, contexts 128-8192: 78 -> 75 us).
template <int D, int GQ, bool EARLY, bool NTL>
__global__ __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void paged_attn_kernel(AttnArgs a) {
  attn_item<D, GQ, kAttnWaves * 64, EARLY, NTL>(a, blockIdx.z, blockIdx.y, blockIdx.x);
}

bool attention_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 ||
                                                 group == 7 || group == 8);
}

// Pages per split: one page per wavefront until the launch would exceed
// about 256 workgroups, then up to 32 (several pages per wavefront overlap
// one page's K/V latency with the previous page's work, and longer items
// spend less of their time in the combine and merge tail; measured at 16
// sequences of 1024-4096 tokens: 2048 workgroups 45.6 us, 512 28.2 us, and
// with page ids read by scalar loads 512 workgroups 24.5 us, 256 (eight pages
// per wavefront) 2.407 against 2.463 ms per step; at 32 sequences of
// 128-8192 tokens, with K slices in score operand order and the first page
// issued early: eight pages per wavefront 54.5 us, sixteen 53.1 us,
// thirty-two 51.0 us); at most 128 splits per sequence (the merge keeps two
// floats per (head, split) in LDS).
int attention_pages_per_split(int batch, int n_kv_heads, int max_pages) {
  const long units = (long)batch * n_kv_heads * max_pages;
  int per_wave = 1;
  while (per_wave < 32 && units / ((long)kAttnWaves * per_wave) > 256) per_wave *= 2;
  int pps = kAttnWaves * per_wave;
  while ((max_pages + pps - 1) / pps > 128) pps *= 2;
  return pps;
}

template <int D, int GQ>
static hipError_t launch_dg(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.batch, a.n_kv_heads, a.max_splits), block(kAttnWaves * 64);
  // several pages per wavefront: the first page's loads go out before the
  // queries are staged. With two to eight pages per wavefront K/V are read
  // non-temporally (batch-16 step, 16 sequences of 1024-4096 tokens: 2.177
  // -> 2.124 ms). Non-temporal loads were slower with one page per
  // wavefront (batch-1 step 1.2368 -> 1.2438 ms) and with 32 (32 sequences
  // of 128-8192 tokens: 52.6 -> 55.7 us), so those keep the default policy.
  if (a.pages_per_split > kAttnWaves && a.pages_per_split <= 8 * kAttnWaves)
    hipLaunchKernelGGL((paged_attn_kernel<D, GQ, true, true>), grid, block, 0, s, a);
  else if (a.pages_per_split > kAttnWaves)
    hipLaunchKernelGGL((paged_attn_kernel<D, GQ, true, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((paged_attn_kernel<D, GQ, false, false>), grid, block, 0, s, a);
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

// ------------------------------------------- allocation-free standalone call
// paged_attention_decode_noalloc keeps the split partials, arrival counters
// and error count in this file-scope device array instead of a caller's
// workspace. Each GPU holds its own copy for the life of the process; its
// address on a device comes from hipGetSymbolAddress once, with that device
// current (the array's name in host code is only a host-side stand-in).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

static std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device.
static int scratch_address(void** out) {
  int dev = 0;
  W4_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(W4_EINVAL, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    W4_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W4_OK;
}

}  // namespace w4

using namespace w4;

W4_EXPORT size_t paged_attention_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

W4_EXPORT int paged_attention_decode_noalloc(const uint16_t* q, const void* k_pool, const void* v_pool,
                                             const int32_t* page_tables, const int32_t* ctx_lens,
                                             int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t num_pages, int32_t max_pages,
                                             uint16_t* out, void* stream) {
  clear_error();
  const size_t need = paged_attention_workspace_bytes(batch, n_heads, n_kv_heads, head_dim, max_pages);
  if (need == 0 || num_pages < 1)
    return fail(W4_EINVAL, "paged_attention_decode_noalloc: unsupported shape batch=%d heads=%d/%d "
                "head_dim=%d max_pages=%d num_pages=%d", batch, n_heads, n_kv_heads, head_dim, max_pages,
                num_pages);
  if (need > kNoallocScratchBytes)
    return fail(W4_EINVAL, "paged_attention_decode_noalloc: this call needs %zu bytes of scratch, more than the "
                "%zu the library holds per device; use paged_attention_decode with a workspace", need,
                kNoallocScratchBytes);
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return attention_standalone("paged_attention_decode_noalloc", q, k_pool, v_pool, page_tables, ctx_lens,
                              batch, n_heads, n_kv_heads, head_dim, num_pages, max_pages, ws,
                              kNoallocScratchBytes, out, stream);
}

