// Persistent decoder-layer kernel for gfx950: the five operations of a
// decoder layer (qkv + RoPE + K/V write, paged attention, o-projection +
// residual, gate/up + SiLU-mul, down + residual) in one cooperative launch of
// one 1024-thread workgroup per CU.
//
// Between operations all workgroups meet at a grid barrier. Before waiting
// there, every wavefront already issues the first weight loads of the next
// operation (weights depend on nothing the previous operation writes), so
// HBM keeps streaming through the barrier, and the gap between separate
// kernel launches disappears. Each operation runs the same device code with
// the same work split as its own kernel (gemv_b1.h, attn_item.h), so the
// results are identical bit for bit. Activations cross workgroups and XCDs
// through device-coherent loads and stores; the barrier's flags likewise.
// Every wait is bounded: a workgroup that waits too long marks the launch
// aborted, every other workgroup sees the mark and leaves, and the launch
// counts one device error.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_item.h"

namespace w4 {

__device__ __forceinline__ void st32_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld32_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a has reached b (wrap-safe epoch comparison)
__device__ __forceinline__ bool reached(uint32_t a, uint32_t b) { return (int32_t)(a - b) >= 0; }

constexpr long kSpinLimit = 1L << 17;  // polls (each >= one memory round trip, ~0.1 s in all) before giving up

// Barrier words: [0] launch sequence, [16] release epoch, [32] abort epoch,
// [64 + 16 w] arrival epoch of workgroup w (one 64-byte line each).
constexpr int kBarSeq = 0, kBarRelease = 16, kBarAbort = 32, kBarArrive = 64;

// Grid barrier `epoch` (base + 1, base + 2, ...) of the launch numbered
// base / kPersistEpochs. Workgroup 0 gathers every arrival (one thread per
// workgroup, all polling at once), then releases;
// each wait also polls the abort word, which holds the epoch a timed-out wait
// gave up at (so an abort of an earlier launch is ignored). Returns false in
// every thread if this launch aborted. Each wavefront has waited for its own
// stores before calling.
__device__ __forceinline__ bool grid_sync(uint32_t* bar, uint32_t base, uint32_t epoch) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) s_ok = 1;
  __syncthreads();
  if (threadIdx.x == 0) st32_agent(bar + kBarArrive + 16 * blockIdx.x, epoch);
  if (blockIdx.x == 0) {
    // thread w watches workgroup w's arrival (all in parallel)
    for (unsigned w = threadIdx.x; w < gridDim.x; w += blockDim.x) {
      long n = 0;
      while (!reached(ld32_agent(bar + kBarArrive + 16 * w), epoch)) {
        if (reached(ld32_agent(bar + kBarAbort), base + 1)) {
          s_ok = 0;
          break;
        }
        if (++n > kSpinLimit) {
          st32_agent(bar + kBarAbort, epoch);
          s_ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && s_ok) st32_agent(bar + kBarRelease, epoch);
  } else if (threadIdx.x == 0) {
    long n = 0;
    while (!reached(ld32_agent(bar + kBarRelease), epoch)) {
      if (reached(ld32_agent(bar + kBarAbort), base + 1)) {
        s_ok = 0;
        break;
      }
      if (++n > kSpinLimit) {
        st32_agent(bar + kBarAbort, epoch);
        s_ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return s_ok != 0;
}

// One projection as a phase: prefetch this wavefront's first weight batch,
// wait at the barrier for the previous operation (unless it is the first of
// the launch), then stage the activation row and finish exactly as the
// projection's own kernel does.
template <int EPI, int S, int IT>
__device__ __forceinline__ bool gemv_phase(const GemvArgs& a, int tw, uint32_t* bar, uint32_t base, uint32_t epoch,
                           uint8_t* smem) {
  using Part = GemvB1Sel<EPI, S, IT>;
  constexpr bool NORM = Part::NORM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Part g;
  g.assign(a, blockIdx.x, tw, wave);
  g.prefetch();
  if (epoch != base && !grid_sync(bar, base, epoch)) return false;
  StageRegs<IT, NORM> st;
  stage_load(st, a.x, a.gamma, a.k, kB1Threads);
  const QkvPre pre = qkv_pre<EPI>(a, blockIdx.x, tw);
  const int kpad = a.groups * kGroup;
  g.clear(smem, kpad, tw);
  float* nred = reinterpret_cast<float*>(smem + (size_t)kpad * 2) + gemv_b1_red_floats(S, kB1Threads / 64, tw);
  stage_row_mfma(st, a.eps, a.k, kpad, reinterpret_cast<uint16_t*>(smem), nred, nullptr, kB1Threads);
  g.finish(a, blockIdx.x, tw, wave, smem, pre);
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores are complete before the next barrier
  return true;
}

// Attention as a phase: work items (split, KV head, sequence) round-robin
// over the workgroups, eight page wavefronts each (no next-page register
// prefetch, so the phase fits a 1024-thread workgroup).
template <int D, int GQ>
__device__ __forceinline__ bool attn_phase(const AttnArgs& at, uint32_t* bar, uint32_t base, uint32_t epoch) {
  if (!grid_sync(bar, base, epoch)) return false;
  const int items = at.max_splits * at.n_kv_heads * at.batch;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int split = it % at.max_splits, rest = it / at.max_splits;
    attn_item<D, GQ, kB1Threads, true>(at, split, rest % at.n_kv_heads, rest / at.n_kv_heads);
    __syncthreads();  // the item's LDS is reused by the next one
  }
  __builtin_amdgcn_s_waitcnt(0);
  return true;
}

// One instantiation per supported configuration: head size and group, and
// the (S, IT) split of each projection (qkv, o, gate/up, down).
template <int D, int GQ, int SQ, int IQ, int SO, int IO, int SG, int IG, int SD, int ID>
__global__ __launch_bounds__(kB1Threads) void decode_layer_kernel(LayerPhases t) {
  extern __shared__ __align__(16) uint8_t smem[];
  const uint32_t seq = ld32_agent(t.bar + kBarSeq);
  const uint32_t base = seq * kPersistEpochs;  // this launch's barriers: base + 1 .. base + 4
  bool ok = gemv_phase<EPI_QKV, SQ, IQ>(t.qkv, t.tw_q, t.bar, base, base, smem) &&
            attn_phase<D, GQ>(t.attn, t.bar, base, base + 1) &&
            gemv_phase<EPI_RESID, SO, IO>(t.o, t.tw_o, t.bar, base, base + 2, smem) &&
            gemv_phase<EPI_SILU, SG, IG>(t.gate_up, t.tw_g, t.bar, base, base + 3, smem) &&
            gemv_phase<EPI_RESID, SD, ID>(t.down, t.tw_d, t.bar, base, base + 4, smem);
  (void)ok;
  // every workgroup read the sequence word before the launch's first barrier,
  // which all of them have passed: the next launch may start from seq + 1
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (reached(ld32_agent(t.bar + kBarAbort), base + 1)) atomicAdd(t.attn.err, 1u);
    st32_agent(t.bar + kBarSeq, seq + 1);
  }
}

// The instantiated configurations: Qwen2.5-7B (head 128, group 7) and the
// miniature test shape (hidden 448, head 64, group 7, FFN 1536).
struct PersistCfg {
  int d, gq;
  B1Split q, o, g, dn;
  const void* fn;
};

#define W4_CFG(D, GQ, SQ, TQ, IQ, SO, TO, IO, SG, TG, IG, SD, TD, ID)                           \
  PersistCfg {                                                                                 \
    D, GQ, {SQ, TQ, IQ}, {SO, TO, IO}, {SG, TG, IG}, {SD, TD, ID},                              \
        reinterpret_cast<const void*>(&decode_layer_kernel<D, GQ, SQ, IQ, SO, IO, SG, IG, SD, ID>) \
  }

static const PersistCfg* persistent_cfg(const w4_config& c) {
  static const PersistCfg cfgs[] = {
      W4_CFG(128, 7, 4, 2, 1, 8, 1, 1, 1, 10, 1, 8, 1, 3),
      W4_CFG(64, 7, 2, 1, 1, 2, 1, 1, 2, 1, 1, 4, 1, 1),
  };
  const int gq = c.n_heads / c.n_kv_heads;
  const B1Split q = w4_b1_split(w4_tiles((c.n_heads + 2 * c.n_kv_heads) * c.head_dim), w4_groups(c.hidden));
  const B1Split o = w4_b1_split(w4_tiles(c.hidden), w4_groups(c.n_heads * c.head_dim));
  const B1Split g = w4_b1_split(w4_tiles(2 * c.ffn), w4_groups(c.hidden));
  const B1Split dn = w4_b1_split(w4_tiles(c.hidden), w4_groups(c.ffn));
  auto same = [](const B1Split& a, const B1Split& b) { return a.s == b.s && a.tw == b.tw && a.it == b.it; };
  for (const PersistCfg& k : cfgs)
    if (k.d == c.head_dim && k.gq == gq && same(k.q, q) && same(k.o, o) && same(k.g, g) && same(k.dn, dn))
      return &k;
  return nullptr;
}
#undef W4_CFG

size_t persistent_bar_words(int grid) { return (size_t)kBarArrive + 16 * (size_t)grid; }

size_t persistent_lds_bytes(const w4_config& c) {
  size_t m = 0;
  for (int k : {c.hidden, c.n_heads * c.head_dim, c.ffn})
    for (int sp : {1, 2})  // runs or K split, 16 tiles at most
      m = std::max(m, gemv_b1_lds_bytes(w4_groups(k), sp, kB1Threads / 64, 16));
  return m;
}

// Co-resident workgroups (one per CU) the persistent kernel can run this
// configuration on, or 0 if it has no instantiation for it or the device
// cannot keep one 1024-thread workgroup on every CU.
int persistent_grid(const w4_config& c) {
  const PersistCfg* k = persistent_cfg(c);
  if (!k) return 0;
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k->fn, kB1Threads, persistent_lds_bytes(c)) !=
          hipSuccess ||
      per_cu < 1)
    return 0;
  // every projection's workgroups must fit the grid
  const int tiles[4] = {w4_tiles((c.n_heads + 2 * c.n_kv_heads) * c.head_dim), w4_tiles(c.hidden),
                        w4_tiles(2 * c.ffn), w4_tiles(c.hidden)};
  const B1Split* sps[4] = {&k->q, &k->o, &k->g, &k->dn};
  for (int i = 0; i < 4; ++i)
    if (ceil_div(tiles[i], sps[i]->tw) > cus) return 0;
  return cus;
}

hipError_t launch_persistent(const LayerPhases& t, const w4_config& c, int grid, hipStream_t s) {
  const PersistCfg* k = persistent_cfg(c);
  if (!k) return hipErrorInvalidValue;
  void* args[] = {const_cast<LayerPhases*>(&t)};
  return hipLaunchCooperativeKernel(k->fn, dim3(grid), dim3(kB1Threads), args, (unsigned)persistent_lds_bytes(c),
                                    s);
}

}  // namespace w4
