// W4A16 projections and the fp16 lm_head for gfx950.
//
// Weights: symmetric group-wise INT4, group 128 along the input dimension,
// dequantised value q * s ("How to build your own LLM runtime from
// scratch", Architectural decisions and optimizations). lm_head and RMSNorm
// stay in FP16 (same section).
//
// Batch 1 is a bandwidth-bound GEMV. It still runs on the matrix cores: the
// packed block is laid out as the B operand of v_mfma_f32_16x16x32_f16, the
// dequantisation is exact with one AND-OR and one packed subtract per weight
// pair, and the MFMA does the multiply-accumulate (gemv_b1.h). Batches 2..16
// turn each projection into a skinny dense contraction on the same
// instruction.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gemv_b1.h"

namespace w4 {

// Copies x[0..k) (fp16, k % 8 == 0) into LDS xs[0..kpad), zero padded, and if
// gamma is given replaces it by fp16(x * rsqrt(mean(x^2) + eps) * gamma)
// (RMSNorm, kept in FP16). NT threads take part; red needs NT/64 floats.
// Ends with a barrier.
__device__ void stage_x(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                        float eps, int k, int kpad, uint16_t* xs, float* red, const int NT) {
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int i = tid * 8; i < kpad; i += NT * 8) {
    u4_t v = {0u, 0u, 0u, 0u};
    if (i < k) v = *reinterpret_cast<const u4_t*>(x + i);
    *reinterpret_cast<u4_t*>(xs + i) = v;
    if (gamma) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h2_t h = as_h2(v[c]);
        const float a = (float)h[0], b = (float)h[1];
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
    }
  }
  if (gamma) {
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < NT / 64; ++w) tot += red[w];
    const float rs = 1.0f / sqrtf(tot / (float)k + eps);
    for (int i = tid * 8; i < k; i += NT * 8) {
      u4_t v = *reinterpret_cast<const u4_t*>(xs + i);
      const u4_t g = *reinterpret_cast<const u4_t*>(gamma + i);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h2_t hv = as_h2(v[c]), hg = as_h2(g[c]);
        h2_t r;
        r[0] = (_Float16)((float)hv[0] * rs * (float)hg[0]);
        r[1] = (_Float16)((float)hv[1] * rs * (float)hg[1]);
        v[c] = __builtin_bit_cast(uint32_t, r);
      }
      *reinterpret_cast<u4_t*>(xs + i) = v;
    }
  }
  __syncthreads();
}

// Copies the staged (normalised) activations back to global memory.
__device__ __forceinline__ void store_xs(const uint16_t* xs, int k, uint16_t* dst, const int NT) {
  for (int i = threadIdx.x * 8; i < k; i += NT * 8)
    *reinterpret_cast<u4_t*>(dst + i) = *reinterpret_cast<const u4_t*>(xs + i);
}

// ------------------------------------------------------------ batch 1
// One launch per projection: S wavefronts per tile on TW tiles (S TW <= 16;
// any further wavefronts only help stage the activations), IT activation
// words per thread: the same decomposition and arithmetic as the projection
// phases of the persistent layer kernel. The
// activation loads go out first, then the first weight batch, so the
// prologue waits for the activations only (the vector-memory counter is in
// order).
template <int EPI, int S, int IT>
__global__ __launch_bounds__(1024) void w4_gemv_b1_kernel(GemvArgs a, int TW) {
  constexpr bool NORM = GemvB1<EPI, S, IT>::NORM;
  const int NT = blockDim.x;
  extern __shared__ __align__(16) uint8_t smem[];
  const int kpad = a.groups * kGroup;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  StageRegs<IT, NORM> st;
  stage_load(st, a.x, a.gamma, a.k, NT);
  const QkvPre pre = qkv_pre<EPI>(a, blockIdx.x, TW);
  GemvB1<EPI, S, IT> g;
  g.assign(a, blockIdx.x, TW, wave);
  g.prefetch();
  __builtin_amdgcn_sched_barrier(0);  // keep the prologue's arithmetic behind the first weight loads
  float* nred = reinterpret_cast<float*>(smem + (size_t)kpad * 2) + (NT / 64) * 16 + TW * 16;
  stage_row_mfma(st, a.eps, a.k, kpad, reinterpret_cast<uint16_t*>(smem), nred,
                 (a.xn_out && blockIdx.x == 0) ? a.xn_out : nullptr, NT);
  g.finish(a, blockIdx.x, TW, wave, smem, pre);
}

// ------------------------------------------------------- batch 2..16, MFMA
// D[m][n] = sum_k x[m][k] W[n][k] over one 128-column group with four
// v_mfma_f32_16x16x32_f16; lane l supplies A row m = l & 15 (batch row,
// clamped to batch-1) and B column n = l & 15 (weight row), both for the
// k-slots 8 (l >> 4) .. +8 of each step, which the packed layout provides.
// The fp32 group result is scaled per weight row and accumulated.
// Activations come pre-normalised; columns >= k read as zero.

template <int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void w4_gemm_mfma_kernel(GemvArgs a) {
  constexpr int NT = WAVES * 64;
  __shared__ float red[WAVES][16][17];
  __shared__ float tot[16][17];
  const int G = a.groups;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + (size_t)t * G * 64 + lane;
  const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.w + (size_t)a.tiles * G * 1024) +
                       (size_t)t * G * 16 + (lane & 15);
  const int mrow = min(lane & 15, a.batch - 1);
  const uint16_t* xr = a.x + (size_t)mrow * a.x_stride + 32 * (lane >> 4);

  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int base = wave; base < G; base += U * WAVES) {
    u4_t wv[U];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = base + u * WAVES;
      wv[u] = g < G ? __builtin_nontemporal_load(wb + (size_t)g * 64) : (u4_t){0u, 0u, 0u, 0u};
      sc[u] = g < G ? h2f(sb[(size_t)g * 16]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = base + u * WAVES;
      if (g < G) {
        f4_t d = {0.f, 0.f, 0.f, 0.f};
        const u4_t* xp = reinterpret_cast<const u4_t*>(xr + (size_t)g * kGroup);
        const int col0 = g * kGroup + 32 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u4_t xv = col0 + 8 * j < a.k ? xp[j] : (u4_t){0u, 0u, 0u, 0u};
          const h8_t av = __builtin_bit_cast(h8_t, xv);
          u4_t braw;
#pragma unroll
          for (int i = 0; i < 4; ++i) braw[i] = __builtin_bit_cast(uint32_t, nib_pair(wv[u][j], i));
          const h8_t bv = __builtin_bit_cast(h8_t, braw);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, d, 0, 0, 0);
        }
        acc += d * sc[u];
      }
    }
  }
  // acc[j] = D[m = 4 (lane >> 4) + j][n = lane & 15]
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][4 * (lane >> 4) + j][lane & 15] = acc[j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 256; idx += NT) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][idx >> 4][idx & 15];
    tot[idx >> 4][idx & 15] = v;
  }
  __syncthreads();
  constexpr int per = epi_items<EPI>();
  for (int item = threadIdx.x; item < a.batch * per; item += NT)
    epilogue<EPI>(a, item / per, t, item % per, &tot[item / per][0]);
}

// ------------------------------------------------------------ fp16 lm_head

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void f16_gemv_b1_kernel(F16GemvArgs a) {
  constexpr int NT = WAVES * 64;
  extern __shared__ __align__(16) uint8_t smem[];
  const int C = a.cblocks;
  const int kpad = (C * 32 + kGroup - 1) / kGroup * kGroup;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)kpad * 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * WAVES + wave;  // one 16-row tile per wavefront
  const bool live = t < a.tiles;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + (size_t)(live ? t : 0) * C * 64 + lane;

  u4_t cur[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    cur[u] = (live && u < C) ? __builtin_nontemporal_load(wb + (size_t)u * 64) : (u4_t){0u, 0u, 0u, 0u};
  stage_x(a.x, a.gamma, a.eps, a.k, kpad, xs, red, NT);
  if (a.xn_out && blockIdx.x == 0) store_xs(xs, a.k, a.xn_out, NT);
  if (!live) return;
  const uint16_t* xl = xs + 8 * (lane >> 4);
  float acc = 0.f;
  for (int base = 0; base < C; base += kUnroll) {
    u4_t nxt[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = base + kUnroll + u;
      nxt[u] = c < C ? __builtin_nontemporal_load(wb + (size_t)c * 64) : (u4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = base + u;
      if (c < C) {
        const u4_t xv = *reinterpret_cast<const u4_t*>(xl + 32 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(as_h2(cur[u][i]), as_h2(xv[i]), acc, false);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) cur[u] = nxt[u];
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  const int row = 16 * t + lane;
  if (lane < 16 && row < a.n) a.y[row] = f2h(acc);
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void f16_gemm_mfma_kernel(F16GemvArgs a) {
  const int C = a.cblocks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * WAVES + wave;
  if (t >= a.tiles) return;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + (size_t)t * C * 64 + lane;
  const int mrow = min(lane & 15, a.batch - 1);
  const uint16_t* xr = a.x + (size_t)mrow * a.x_stride + 8 * (lane >> 4);
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;
  for (int base = 0; base < C; base += U) {
    u4_t wv[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u;
      wv[u] = c < C ? __builtin_nontemporal_load(wb + (size_t)c * 64) : (u4_t){0u, 0u, 0u, 0u};
      xv[u] = (c < C && 32 * c + 8 * (lane >> 4) < a.k) ? *reinterpret_cast<const u4_t*>(xr + 32 * c)
                                                           : (u4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xv[u]),
                                                  __builtin_bit_cast(h8_t, wv[u]), acc, 0, 0, 0);
  }
  const int row = 16 * t + (lane & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = 4 * (lane >> 4) + j;
    if (m < a.batch && row < a.n) a.y[(size_t)m * a.y_stride + row] = f2h(acc[j]);
  }
}

// ------------------------------------------------------------ small kernels

// y[b] = fp16(x[b] * rsqrt(mean(x[b]^2) + eps) * gamma), zero padded to the
// next multiple of 128 columns (batched path: the MFMA kernels read it).
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t* x, int x_stride,
                                                           const uint16_t* gamma, float eps, int k,
                                                           uint16_t* y, int y_stride) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const uint16_t* xr = x + (size_t)b * x_stride;
  uint16_t* yr = y + (size_t)b * y_stride;
  float ss = 0.f;
  for (int i = threadIdx.x; i < k; i += 256) {
    const float v = h2f(xr[i]);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rs = 1.0f / sqrtf(tot / (float)k + eps);
  const int kpad = (k + kGroup - 1) / kGroup * kGroup;
  for (int i = threadIdx.x; i < kpad; i += 256)
    yr[i] = i < k ? f2h(h2f(xr[i]) * rs * h2f(gamma[i])) : (uint16_t)0;
}

__global__ __launch_bounds__(256) void embed_plan_kernel(TokenPlanArgs a) {
  const int b = blockIdx.x;
  if (a.tokens) {
    int tok = a.tokens[b];
    if (tok < 0 || tok >= a.vocab) {
      if (threadIdx.x == 0) atomicAdd(a.err, 1u);
      tok = tok < 0 ? 0 : a.vocab - 1;
    }
    const uint16_t* src = a.table + (size_t)tok * a.hidden;
    uint16_t* dst = a.x + (size_t)b * a.hidden;
    for (int i = threadIdx.x * 8; i < a.hidden; i += 256 * 8)
      *reinterpret_cast<u4_t*>(dst + i) = *reinterpret_cast<const u4_t*>(src + i);
  }
  if (threadIdx.x >= 64) return;
  const int pos = a.positions[b];
  if (threadIdx.x == 0) {
    const bool pos_ok = pos >= 0 && pos < a.max_pages * kPage;
    const int page = pos_ok ? a.page_tables[(size_t)b * a.max_pages + (pos >> 4)] : -1;
    const bool ok = pos_ok && page >= 0 && page < a.num_pages;
    a.slot[b] = ok ? page * kPage + (pos & 15) : -1;
    if (!ok) atomicAdd(a.err, 1u);
  }
  const int half = a.head_dim / 2;
  for (int i = threadIdx.x; i < half; i += 64) {
    const double th = (double)pos * pow((double)a.rope_base, -2.0 * (double)i / (double)a.head_dim);
    float* r = a.rope + ((size_t)b * half + i) * 2;
    r[0] = (float)cos(th);
    r[1] = (float)sin(th);
  }
}

__global__ void fill_u32_kernel(uint32_t* p, size_t count, uint32_t value) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// ---------------------------------------------------------------- launchers

// (the batch-1 split policy is described with B1Split in gemv_b1.h)
B1Split w4_b1_split(int tiles, int groups) {
  const int tw = std::min(16, ceil_div(tiles, 256));
  int s = 1;
  for (int c : {8, 4, 2})
    if (groups >= 2 * c && c * tw <= 8) {
      s = c;
      break;
    }
  const int it = ceil_div(groups * kGroup, 8 * kB1Threads);  // per thread, at kB1Threads
  return {s, tw, it};
}

template <int EPI, int S, int IT>
static void launch_b1(const GemvArgs& a, int tw, int nt, hipStream_t s) {
  const size_t lds = gemv_b1_lds_bytes(a.groups, nt / 64, tw);
  hipLaunchKernelGGL((w4_gemv_b1_kernel<EPI, S, IT>), dim3(ceil_div(a.tiles, tw)), dim3(nt), lds, s, a, tw);
}

// The workgroup is its S * TW working wavefronts (at least four), unless
// the activation row then needs more than kMaxIt words per thread; then it
// has kB1Threads threads like the persistent kernel's phases. The staged
// row and every product are the same either way, and so is the RMSNorm sum
// when the row fits one pass of the threads (8 * nt >= k: each thread then
// holds one word, the words past k are zero).
constexpr int kMaxIt = 5;
template <int EPI, int S>
static hipError_t launch_b1_it(const GemvArgs& a, const B1Split& sp, hipStream_t s) {
  int nt = std::max(256, 64 * S * sp.tw);
  int it = ceil_div(a.groups * kGroup, 8 * nt);
  if (it > kMaxIt) {
    nt = kB1Threads;
    it = sp.it;
  }
  switch (it) {
    case 1: launch_b1<EPI, S, 1>(a, sp.tw, nt, s); return hipSuccess;
    case 2: launch_b1<EPI, S, 2>(a, sp.tw, nt, s); return hipSuccess;
    case 3: launch_b1<EPI, S, 3>(a, sp.tw, nt, s); return hipSuccess;
    case 4: launch_b1<EPI, S, 4>(a, sp.tw, nt, s); return hipSuccess;
    case 5: launch_b1<EPI, S, 5>(a, sp.tw, nt, s); return hipSuccess;
  }
  return hipErrorInvalidValue;  // activation row longer than one workgroup can stage
}

template <int EPI>
static hipError_t launch_w4_epi(const GemvArgs& a, hipStream_t s) {
  if (a.batch == 1) {
    // the batch-1 kernel applies RMSNorm exactly for the QKV and gate/up epilogues
    if ((a.gamma != nullptr) != (EPI == EPI_QKV || EPI == EPI_SILU)) return hipErrorInvalidValue;
    const B1Split sp = w4_b1_split(a.tiles, a.groups);
    hipError_t e = hipErrorInvalidValue;
    switch (sp.s) {
      case 8: e = launch_b1_it<EPI, 8>(a, sp, s); break;
      case 4: e = launch_b1_it<EPI, 4>(a, sp, s); break;
      case 2: e = launch_b1_it<EPI, 2>(a, sp, s); break;
      case 1: e = launch_b1_it<EPI, 1>(a, sp, s); break;
    }
    if (e != hipSuccess) return e;
  } else {
    constexpr int WAVES = 4;
    hipLaunchKernelGGL((w4_gemm_mfma_kernel<EPI, WAVES>), dim3(a.tiles), dim3(WAVES * 64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_w4_gemv(int epi, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_w4_epi<EPI_STORE>(a, s);
    case EPI_RESID: return launch_w4_epi<EPI_RESID>(a, s);
    case EPI_SILU: return launch_w4_epi<EPI_SILU>(a, s);
    case EPI_QKV: return launch_w4_epi<EPI_QKV>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_f16_gemv(const F16GemvArgs& a, hipStream_t s) {
  constexpr int WAVES = 4;
  const int grid = ceil_div(a.tiles, WAVES);
  if (a.batch == 1) {
    const size_t kpad = round_up((size_t)a.cblocks * 32, kGroup);
    const size_t lds = kpad * 2 + WAVES * sizeof(float);
    hipLaunchKernelGGL((f16_gemv_b1_kernel<WAVES>), dim3(grid), dim3(WAVES * 64), lds, s, a);
  } else {
    hipLaunchKernelGGL((f16_gemm_mfma_kernel<WAVES>), dim3(grid), dim3(WAVES * 64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const uint16_t* x, int32_t x_stride, const uint16_t* gamma, float eps,
                               int32_t k, uint16_t* y, int32_t y_stride, int32_t batch,
                               hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(batch), dim3(256), 0, s, x, x_stride, gamma, eps, k,
                     y, y_stride);
  return hipGetLastError();
}

hipError_t launch_embed_plan(const TokenPlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(embed_plan_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const int grid = (int)std::min<size_t>(1024, (count + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid), dim3(256), 0, s, p, count, value);
  return hipGetLastError();
}

}  // namespace w4
