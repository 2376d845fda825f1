// W4A16 projections and the fp16 lm_head for gfx950.
//
// Weights: symmetric group-wise INT4, group 128 along the input dimension,
// dequantised value q * s ("How to build your own LLM runtime from
// scratch", Architectural decisions and optimizations). lm_head and RMSNorm
// stay in FP16 (same section).
//
// Batch 1 is a bandwidth-bound GEMV. It still runs on the matrix cores: the
// packed block is laid out as the B operand of v_mfma_f32_16x16x32_f16, the
// codes dequantise exactly with one AND-OR and one packed subtract per weight
// pair (half of them as 16q, met by activations staged divided by 16), and
// the MFMA does the multiply-accumulate (gemv_b1.h). Batches 2..16
// turn each projection into a skinny dense contraction on the same
// instruction.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

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
// One launch per projection: S wavefronts per tile on TW tiles (S TW <= 8),
// or kRangeWaves contiguous runs when S == 1; any further wavefronts only
// help stage the activations. IT activation words per thread. The
// activation loads go out first, then the first weight
// batch, so the prologue waits for the activations only (the vector-memory
// counter is in order).
template <int EPI, int S, int IT>
__global__ __launch_bounds__(1024) void w4_gemv_b1_kernel(GemvArgs a, int TW) {
  using Part = GemvB1Sel<EPI, S, IT>;
  constexpr bool NORM = Part::NORM;
  const int NT = blockDim.x;
  extern __shared__ __align__(16) uint8_t smem[];
  const int kpad = a.groups * kGroup;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  StageRegs<IT, NORM> st;
  stage_load(st, a.x, a.gamma, a.k, NT);
  // every wavefront's activation loads reach the CU's memory pipeline before
  // any weight prefetch (down projection 9.2 -> 8.6 us): the barrier waits
  // for no load
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const QkvPre pre = qkv_pre<EPI>(a, blockIdx.x, TW);
  Part g;
  g.assign(a, blockIdx.x, TW, wave);
  g.prefetch();
  __builtin_amdgcn_sched_barrier(0);  // keep the prologue's arithmetic behind the first weight loads
  g.clear(smem, kpad, TW);
  float* nred = reinterpret_cast<float*>(smem + (size_t)kpad * 2) + gemv_b1_red_floats(S, NT / 64, TW);
  stage_row_mfma(st, a.eps, a.k, kpad, reinterpret_cast<uint16_t*>(smem), nred,
                 (a.xn_out && blockIdx.x == 0) ? a.xn_out : nullptr, NT);
  g.finish(a, blockIdx.x, TW, wave, smem, pre);
}

// ------------------------------------------------------- batch 2..16, MFMA
// The batch-1 decomposition with all 16 A rows real: the activation rows
// (RMSNorm applied while staging when gamma is given; rows >= batch zero)
// are staged in LDS in the MFMA k-slot order, a window of GW groups at a
// time (one window up to K = 4096, 128 KiB of LDS at most; rows padded by 16
// bytes so the 16 lanes of a lane group, one row each, read distinct banks),
// and the same packed blocks, exact dequantisation and
// v_mfma_f32_16x16x32_f16 give D[batch row][weight row] in every lane. TW
// tiles per workgroup, S wavefronts per tile; each wavefront streams its
// window's blocks two batches of two ahead.
//
// Staging: each half of the threads (a whole number of wavefronts, NT >= 2
// round_up(8 GW, 64)) takes 8 of the 16 rows, thread t of a half the
// window's 16-column segment t: two natural 8-column words per row, whose
// 32-bit pairs are the segment's two slot words as they stand, so a thread
// issues its 16 activation loads and two RMSNorm-weight loads at once,
// before the window's first weight batch. When the whole row is one window
// the RMSNorm sums come from those same registers (per-thread partial sums
// of each row, reduced on the VALU per wavefront and in wavefront order
// through LDS); longer rows with RMSNorm take a pre-pass over the rows
// instead. (Reading the rows twice, sums then staging, and the RMSNorm
// weights once per row took gate/up from 12.4 us of prologue to ~3 us; the
// segment staging replaced one word of all 16 rows per thread with DPP quad
// permutes: batch-16 step 2.394 -> 2.213 ms.)
constexpr int kRowsThreads = 768;  // launch bound: 16 activation words per thread stay in registers
constexpr int kMaxChunks = 8;      // K split: at most 8 workgroups per tile group (rows up to 32768 columns)
template <int EPI, int S>
__global__ __launch_bounds__(kRowsThreads) void w4_gemm_rows_kernel(GemvArgs a, int TW, int GW, int CH) {
  constexpr int kUnroll = 2;  // blocks per batch (batch-16 step: 2.568 ms with three, 2.561 with two)
  extern __shared__ __align__(16) uint8_t smem[];
  const int NT = blockDim.x, NW = NT >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.groups;
  const int KW = GW * kGroup + 8;  // row stride: 16 bytes of padding spread the 16 rows over the LDS banks
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);                        // [16][KW]
  float* red = reinterpret_cast<float*>(smem + (size_t)16 * KW * 2);       // [NW][16][16]
  float* vals = red + NW * 256;                                            // [TW][16][16]
  const int tg = blockIdx.x / CH, kc = blockIdx.x % CH;  // tile group, K chunk (chunks of a group adjacent)
  const int t = tg * TW + wave / S, ks = wave % S;
  const int k1 = CH > 1 ? min(G, (kc + 1) * GW) : G;       // groups [kc GW, k1)
  const bool live = wave < S * TW && t < a.tiles;
  const size_t base = (size_t)(live ? t : 0) * G;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + base * 64 + lane;
  const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.w + (size_t)a.tiles * G * 1024) + base * 16 + (lane & 15);
  const uint16_t* xl = xs + (size_t)(lane & 15) * KW + 32 * (lane >> 4);
  const uint32_t mlo = vgpr_const(kMaskLo), mhi = vgpr_const(kMaskHi);
  const bool one_window = G <= GW;
  __shared__ __align__(16) float s_rs[16];
  __shared__ __align__(16) float s_ss[kRowsThreads / 64][8];
  // RMSNorm over rows longer than one window: wavefront w sums the squares
  // of rows w, w + NW, .. in a pre-pass
  if (a.gamma && !one_window) {
    const int kw = a.k / 8;
    for (int m = wave; m < 16; m += NW) {
      float ss = 0.f;
      if (m < a.batch)
        for (int w0 = 0; w0 < kw; w0 += 8 * 64) {
          u4_t v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            v[j] = *reinterpret_cast<const u4_t*>(a.x + (size_t)m * a.x_stride + 8 * min(w0 + lane + 64 * j, kw - 1));
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (w0 + lane + 64 * j < kw)
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const h2_t h = as_h2(v[j][c]);
                ss = fmaf((float)h[0], (float)h[0], ss);
                ss = fmaf((float)h[1], (float)h[1], ss);
              }
        }
      ss = wave_sum(ss);
      if (lane == 0) s_rs[m] = 1.0f / sqrtf(ss / (float)a.k + a.eps);
    }
    __syncthreads();
  }
  f4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = kc * GW; g0 < k1; g0 += GW) {
    const int gn = min(GW, k1 - g0);
    const int ng = (live && ks < gn) ? (gn - ks + S - 1) / S : 0;  // groups g0 + ks + S i, i < ng
    const int last = ng > 0 ? ng - 1 : 0;
    u4_t bufA[kUnroll], bufB[kUnroll];
    uint32_t scA[kUnroll], scB[kUnroll];
    auto load = [&](u4_t* buf, uint32_t* sc, int i0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int g = min(g0 + ks + S * min(i0 + u, last), G - 1);
        sc[u] = sb[(size_t)g * 16];
        buf[u] = __builtin_nontemporal_load(wb + (size_t)g * 64);
      }
    };
    auto compute = [&](const u4_t* buf, const uint32_t* sc, int i0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (i0 + u < ng) {
          const f4_t d = mfma_block(buf[u], xl + (size_t)(ks + S * (i0 + u)) * kGroup, mlo, mhi);
          acc += d * h2f((uint16_t)sc[u]);
        }
    };
    // Staging: thread t takes rows 8 h .. 8 h + 8 (h = t / JW, uniform per
    // wavefront) of the window's 16-column segment sj = t % JW, as two natural
    // 8-column words per row. The slot groups 2 p and 2 p + 1 of a 32-column
    // chunk hold the 32-bit pairs (0, 2) and (1, 3) of the chunk's words 2 p
    // and 2 p + 1, so a segment's two slot words come from its own two words
    // (no exchange between lanes). Loads past k and of rows >= batch read zero.
    const int JW = (8 * GW + 63) & ~63;
    const int hh = __builtin_amdgcn_readfirstlane((int)threadIdx.x / JW);
    const int sj = (int)threadIdx.x % JW;
    const int col = 128 * g0 + 16 * sj;
    const bool stager = hh < 2;
    u4_t xa[8], xb[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = 8 * hh + r;
      const __amdgpu_buffer_rsrc_t rx =
          range_rsrc(a.x + (size_t)min(m, 15) * a.x_stride, stager && m < a.batch ? 2 * a.k : 0);
      xa[r] = ld128(rx, 2 * col);
      xb[r] = ld128(rx, 2 * col + 16);
    }
    const __amdgpu_buffer_rsrc_t rg = range_rsrc(a.gamma ? a.gamma : a.x, a.gamma ? 2 * a.k : 0);
    const u4_t ga = ld128(rg, 2 * col), gb = ld128(rg, 2 * col + 16);
    __builtin_amdgcn_sched_barrier(0);
    load(bufA, scA, 0);  // the window's first weight batch, behind the activation loads
    __builtin_amdgcn_sched_barrier(0);
    if (a.gamma && one_window) {  // each row's sum of squares: per thread, per wavefront, then in wavefront order
      float ss[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        ss[r] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {  // two squares per fp16 dot product, accumulated in fp32
          const h2_t h = as_h2(c < 4 ? xa[r][c] : xb[r][c - 4]);
          ss[r] = __builtin_amdgcn_fdot2(h, h, ss[r], false);
        }
      }
      // the rows' reductions without a branch between them, so their
      // dependent DPP chains interleave
#pragma unroll
      for (int r = 0; r < 8; ++r) ss[r] = wave_sum(ss[r]);
      if (lane == 0 && stager) {
        *reinterpret_cast<f4_t*>(&s_ss[wave][0]) = (f4_t){ss[0], ss[1], ss[2], ss[3]};
        *reinterpret_cast<f4_t*>(&s_ss[wave][4]) = (f4_t){ss[4], ss[5], ss[6], ss[7]};
      }
      __syncthreads();
      if (threadIdx.x < 16) {  // row 8 h + r: the wavefronts of half h
        const int h = threadIdx.x >> 3, r = threadIdx.x & 7;
        float tot = 0.f;
        for (int w = h * (JW / 64); w < (h + 1) * (JW / 64); ++w) tot += s_ss[w][r];
        s_rs[threadIdx.x] = 1.0f / sqrtf(tot / (float)a.k + a.eps);
      }
    }
    __syncthreads();  // s_rs ready; the previous window's reads of xs are done
    {
      // per row: fp16(x * rs * gamma) with RMSNorm (the batch-1 staging's
      // rounding), the normalised row to xn_out from workgroup 0, the two slot
      // words to LDS
      float rsv[8];
      if (a.gamma) {
        const int hs = stager ? hh : 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f4_t r4 = *reinterpret_cast<const f4_t*>(&s_rs[8 * hs + 4 * q]);
#pragma unroll
          for (int j = 0; j < 4; ++j) rsv[4 * q + j] = r4[j];
        }
      }
      // (x rs) gamma as two fused multiply-adds with a zero addend, each
      // taking its fp16 operand without a separate conversion: x rs rounded
      // to fp32, its product with gamma rounded to fp16 (the compiler may
      // round that product once, straight to fp16, where the plain products
      // round it to fp32 first: at most one fp16 unit apart, on ties)
      auto scale = [&](u4_t& w, const u4_t g, float rs) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const h2_t hv = as_h2(w[c]), hg = as_h2(g[c]);
          h2_t r;
          r[0] = (_Float16)fmaf(fmaf((float)hv[0], rs, 0.f), (float)hg[0], 0.f);
          r[1] = (_Float16)fmaf(fmaf((float)hv[1], rs, 0.f), (float)hg[1], 0.f);
          w[c] = __builtin_bit_cast(uint32_t, r);
        }
      };
      const bool xn = a.gamma && a.xn_out && blockIdx.x == 0 && stager;
      const bool store = stager && sj < 8 * GW;
      const h2_t q16 = {(_Float16)0.0625f, (_Float16)0.0625f};  // odd slot groups: x / 16 (see slot_word)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int m = 8 * hh + r;
        if (a.gamma) {
          scale(xa[r], ga, rsv[r]);
          scale(xb[r], gb, rsv[r]);
        }
        if (xn && m < a.batch) {
          uint16_t* xo = a.xn_out + (size_t)m * a.xn_stride + col;
          if (col < a.k) *reinterpret_cast<u4_t*>(xo) = xa[r];
          if (col + 8 < a.k) *reinterpret_cast<u4_t*>(xo + 8) = xb[r];
        }
        if (store) {
          const u4_t ev = {xa[r][0], xa[r][2], xb[r][0], xb[r][2]};
          const u4_t od = {__builtin_bit_cast(uint32_t, as_h2(xa[r][1]) * q16),
                           __builtin_bit_cast(uint32_t, as_h2(xa[r][3]) * q16),
                           __builtin_bit_cast(uint32_t, as_h2(xb[r][1]) * q16),
                           __builtin_bit_cast(uint32_t, as_h2(xb[r][3]) * q16)};
          uint16_t* dst = xs + (size_t)m * KW + 16 * sj;
          *reinterpret_cast<u4_t*>(dst) = ev;
          *reinterpret_cast<u4_t*>(dst + 8) = od;
        }
      }
    }
    __syncthreads();
    for (int i = 0; i < ng; i += 2 * kUnroll) {
      load(bufB, scB, i + kUnroll);
      compute(bufA, scA, i);
      if (i + kUnroll >= ng) break;
      load(bufA, scA, i + 2 * kUnroll);
      compute(bufB, scB, i + kUnroll);
    }
  }
  // lane l: acc[j] = D[batch row 4 (l >> 4) + j][weight row l & 15]
  if (wave < S * TW)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(wave * 16 + 4 * (lane >> 4) + j) * 16 + (lane & 15)] = acc[j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < TW * 256; idx += NT) {
    const int tl = idx >> 8, mn = idx & 255;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < S; ++k) v += red[(tl * S + k) * 256 + mn];
    vals[idx] = v;
  }
  __syncthreads();
  if (CH > 1) {
    // K split: store this chunk's sums, count the tile group's arrivals; the
    // last workgroup adds the CH chunks in order and runs the epilogue.
    // Partial sums move between workgroups (and XCDs) through device-coherent
    // 16-byte stores and loads; each workgroup's stores complete before it
    // counts itself.
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(a.kpart + (size_t)tg * CH * TW * 256);
    for (int q = threadIdx.x; q < TW * 64; q += NT)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, *reinterpret_cast<const f4_t*>(vals + 4 * q)),
                                             rp, 16 * (kc * TW * 64 + q), 0, kPolicySc1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last_k;
    if (threadIdx.x == 0)
      s_last_k = __hip_atomic_fetch_add(a.kcount + tg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(CH - 1);
    __syncthreads();
    if (!s_last_k) return;
    for (int q = threadIdx.x; q < TW * 64; q += NT) {
      f4_t part[kMaxChunks];  // every chunk's load in flight at once, then the sum in chunk order
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        part[c] = __builtin_bit_cast(f4_t, ld128_agent(rp, 16 * (min(c, CH - 1) * TW * 64 + q)));
      f4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < CH) v += part[c];
      *reinterpret_cast<f4_t*>(vals + 4 * q) = v;
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.kcount + tg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  constexpr int per = epi_items<EPI>();
  for (int item = threadIdx.x; item < TW * a.batch * per; item += NT) {
    const int tl = item / (a.batch * per), r = item % (a.batch * per);
    const int m = r / per, i = r % per;
    const int tt = tg * TW + tl;
    if (tt < a.tiles) epilogue<EPI>(a, m, tt, i, vals + (tl * 16 + m) * 16);
  }
}

// ------------------------------------------------------------ fp16 lm_head

// Batch 1: one round of workgroups (two per CU), each with TPW consecutive
// 16-row tiles; their 1 KiB blocks (16 rows x 32 columns, consecutive in
// memory) are cut into WAVES contiguous runs weighted by SIMD slot like the
// W4 runs, U blocks per batch with the next batch in flight. A run leaves
// one partial sum per tile it touched in LDS ([TPW][WAVES][16], cleared
// before the row is staged); each tile adds them in wavefront order. With
// one four-wavefront workgroup per four tiles (2376 workgroups, more than
// one round) the 7B lm_head took 166 us per launch; this takes 161 us.
template <int WAVES, int U>
__global__ __launch_bounds__(WAVES * 64) void f16_gemv_b1_kernel(F16GemvArgs a, int TPW) {
  constexpr int NT = WAVES * 64;
  extern __shared__ __align__(16) uint8_t smem[];
  const int C = a.cblocks;
  const int kpad = (C * 32 + kGroup - 1) / kGroup * kGroup;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)kpad * 2);  // [TPW][WAVES][16]
  float* nred = red + TPW * WAVES * 16;                            // RMSNorm scratch
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * TPW;
  const int th = min(TPW, a.tiles - t0);
  int b0, n;
  weighted_run<WAVES>(th * C, w, b0, n);
  const int last = n > 0 ? n - 1 : 0;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + ((size_t)t0 * C + min(b0, th * C - 1)) * 64 + lane;
  u4_t cur[U];
#pragma unroll
  for (int u = 0; u < U; ++u) cur[u] = __builtin_nontemporal_load(wb + (size_t)min(u, last) * 64);
  for (int i = threadIdx.x; i < TPW * WAVES * 16; i += NT) red[i] = 0.f;
  stage_x(a.x, a.gamma, a.eps, a.k, kpad, xs, nred, NT);
  if (a.xn_out && blockIdx.x == 0) store_xs(xs, a.k, a.xn_out, NT);
  const uint16_t* xl = xs + 8 * (lane >> 4);
  int c = n > 0 ? b0 % C : 0, tl = n > 0 ? b0 / C : 0;  // block column and tile of the next block
  float acc = 0.f;
  auto flush = [&]() {  // lanes l, l + 16, l + 32, l + 48 hold row l's column quarters
    float r = acc + __shfl_xor(acc, 16);
    r += __shfl_xor(r, 32);
    if (lane < 16) red[(tl * WAVES + w) * 16 + lane] = r;
  };
  for (int base = 0; base < n; base += U) {
    u4_t nxt[U];
#pragma unroll
    for (int u = 0; u < U; ++u) nxt[u] = __builtin_nontemporal_load(wb + (size_t)min(base + U + u, last) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u < n) {
        const u4_t xv = *reinterpret_cast<const u4_t*>(xl + 32 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(as_h2(cur[u][i]), as_h2(xv[i]), acc, false);
        if (++c == C) {  // the run leaves tile tl
          flush();
          acc = 0.f;
          c = 0;
          ++tl;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
  if (c != 0) flush();  // the run ends inside tile tl
  __syncthreads();
  for (int i = threadIdx.x; i < th * 16; i += NT) {
    const int t = i / 16, r = i % 16;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < WAVES; ++k) v += red[(t * WAVES + k) * 16 + r];
    const int row = 16 * (t0 + t) + r;
    if (row < a.n) a.y[row] = f2h(v);
  }
}

// Batch 2..16: each wavefront computes TT tiles, so one load of the
// activation operand (16 rows x 32 columns, from L2) serves TT weight blocks
// (batch-16 7B lm_head: one tile per wavefront 200 us, two 186 us, four
// 193 us). Weight blocks past the last tile re-read it; their rows are not
// stored. OP: the activations come in the A-operand order (a.xop, written
// by the RMSNorm kernel: chunk c's 64 lanes as 1 KiB of contiguous memory)
// instead of as rows (16 rows x 64 bytes per load): 184-185 -> 178-179 us.
template <int WAVES, bool OP>
__global__ __launch_bounds__(WAVES * 64) void f16_gemm_mfma_kernel(F16GemvArgs a) {
  constexpr int TT = 2, U = 8;
  const int C = a.cblocks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * WAVES + wave) * TT;
  if (t0 >= a.tiles) return;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + lane;
  const int mrow = min(lane & 15, a.batch - 1);
  const uint16_t* xr = a.x + (size_t)mrow * a.x_stride + 8 * (lane >> 4);
  f4_t acc[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) acc[q] = (f4_t){0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < C; base += U) {
    u4_t wv[TT][U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u;
      if (OP)
        xv[u] = c < C ? *reinterpret_cast<const u4_t*>(a.xop + ((size_t)c * 64 + lane) * 8) : (u4_t){0u, 0u, 0u, 0u};
      else
        xv[u] = (c < C && 32 * c + 8 * (lane >> 4) < a.k) ? *reinterpret_cast<const u4_t*>(xr + 32 * c)
                                                           : (u4_t){0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < TT; ++q) {
        const int t = min(t0 + q, a.tiles - 1);
        wv[q][u] = c < C ? __builtin_nontemporal_load(wb + ((size_t)t * C + c) * 64) : (u4_t){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < TT; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xv[u]),
                                                       __builtin_bit_cast(h8_t, wv[q][u]), acc[q], 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int row = 16 * (t0 + q) + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = 4 * (lane >> 4) + j;
      if (m < a.batch && row < a.n) a.y[(size_t)m * a.y_stride + row] = f2h(acc[q][j]);
    }
  }
}

// ------------------------------------------------------------ small kernels

// y[b] = fp16(x[b] * rsqrt(mean(x[b]^2) + eps) * gamma), zero padded to the
// next multiple of 128 columns (batched path: the MFMA kernels read it).
// With yop (rows b < 16, vectorised path only), the same values also go to
// yop in the A-operand order of v_mfma_f32_16x16x32_f16: 8-column word w of
// row b at lane b + 16 (w % 4) of 32-column chunk w / 4, 16 bytes per lane.
// Rows up to kRmsWords 16-byte words per thread are read once into registers
// (16-byte loads and stores); others take the element loop. Either way
// y = (x * rs) * gamma in fp32, rounded once, zeros up to the 128-column pad.
template <bool VEC>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t* x, int x_stride,
                                                           const uint16_t* gamma, float eps, int k,
                                                           uint16_t* y, int y_stride, uint16_t* yop) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const uint16_t* xr = x + (size_t)b * x_stride;
  uint16_t* yr = y + (size_t)b * y_stride;
  const int kpad = (k + kGroup - 1) / kGroup * kGroup;
  float ss = 0.f;
  u4_t xv[VEC ? kRmsWords : 1];
  if (VEC) {
#pragma unroll
    for (int w = 0; w < kRmsWords; ++w) {
      const int c = 8 * (threadIdx.x + 256 * w);
      xv[w] = c < k ? *reinterpret_cast<const u4_t*>(xr + c) : (u4_t){0u, 0u, 0u, 0u};
      const h8_t h = __builtin_bit_cast(h8_t, xv[w]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf((float)h[e], (float)h[e], ss);
    }
  } else {
    for (int i = threadIdx.x; i < k; i += 256) {
      const float v = h2f(xr[i]);
      ss = fmaf(v, v, ss);
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rs = 1.0f / sqrtf(tot / (float)k + eps);
  if (VEC) {
#pragma unroll
    for (int w = 0; w < kRmsWords; ++w) {
      const int c = 8 * (threadIdx.x + 256 * w);
      if (c >= kpad) break;
      u4_t o = {0u, 0u, 0u, 0u};
      if (c < k) {
        const h8_t h = __builtin_bit_cast(h8_t, xv[w]);
        const h8_t g = __builtin_bit_cast(h8_t, *reinterpret_cast<const u4_t*>(gamma + c));
        h8_t r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)((float)h[e] * rs * (float)g[e]);
        o = __builtin_bit_cast(u4_t, r);
      }
      *reinterpret_cast<u4_t*>(yr + c) = o;
      if (yop) {
        const int w = c / 8;
        *reinterpret_cast<u4_t*>(yop + ((size_t)(w >> 2) * 64 + b + 16 * (w & 3)) * 8) = o;
      }
    }
  } else {
    for (int i = threadIdx.x; i < kpad; i += 256)
      yr[i] = i < k ? f2h(h2f(xr[i]) * rs * h2f(gamma[i])) : (uint16_t)0;
  }
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
    const int page = pos_ok ? a.page_tables[(size_t)b * a.pt_stride + (pos >> 4)] : -1;
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
  const size_t lds = gemv_b1_lds_bytes(a.groups, S, nt / 64, tw);
  hipLaunchKernelGGL((w4_gemv_b1_kernel<EPI, S, IT>), dim3(ceil_div(a.tiles, tw)), dim3(nt), lds, s, a, tw);
}

// The workgroup is its working wavefronts (S * TW, or kRangeWaves when
// S == 1; at least four), unless the activation row then needs more than
// kMaxIt words per thread; then it has kB1Threads threads. The staged
// row and every product are the same either way, and so is the RMSNorm sum
// when the row fits one pass of the threads (8 * nt >= k: each thread then
// holds one word, the words past k are zero).
constexpr int kMaxIt = 5;
template <int EPI, int S>
static hipError_t launch_b1_it(const GemvArgs& a, const B1Split& sp, hipStream_t s) {
  int nt = std::max(256, 64 * (S == 1 ? kRangeWaves : S * sp.tw));
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

// Kernels above 64 KiB of dynamic LDS need the per-function opt-in once (the
// limit covers the kernel's static LDS too: 160 KiB per workgroup in all).
constexpr int kRowsMaxDynLds = 160 * 1024 - 1024;
template <int EPI, int S>
static hipError_t launch_rows(const GemvArgs& a, const RowsPlan& p, int nt, size_t lds, hipStream_t s) {
  if (lds > (size_t)kRowsMaxDynLds) return hipErrorInvalidValue;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&w4_gemm_rows_kernel<EPI, S>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kRowsMaxDynLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((w4_gemm_rows_kernel<EPI, S>), dim3(ceil_div(a.tiles, p.tw) * p.ch), dim3(nt), lds, s, a, p.tw,
                     p.gw, p.ch);
  return hipGetLastError();
}

// Rows longer than one window (more than 32 groups) with split-K buffers:
// CH = ceil(groups / 32) workgroups per tile group, each one window of
// consecutive groups, and TW tiles per workgroup so that about one round of
// workgroups covers the chip; every workgroup then stages a CH-th of the
// activation rows instead of all of them (down projection, batch 16: 606 KiB
// of activations per workgroup for 148 KiB of weights before the split).
RowsPlan w4_rows_plan(int tiles, int groups, bool split_k) {
  if (!split_k || groups <= 32 || groups > 32 * kMaxChunks) {
    const B1Split sp = w4_b1_split(tiles, groups);
    // many tiles: more than one workgroup per CU
    return {sp.s, std::min(sp.tw, kRowsThreads / (64 * sp.s)), std::min(groups, 32), 1};
  }
  const int ch = ceil_div(groups, 32);
  const int gw = ceil_div(groups, ch);
  const int tw = std::max(1, std::min(kRowsThreads / 64, ceil_div(tiles * ch, 256)));
  int s = 1;
  for (int c : {8, 4, 2})
    if (gw >= 2 * c && 64 * c * tw <= kRowsThreads) {
      s = c;
      break;
    }
  return {s, tw, gw, ch};
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
    if (a.batch > 16) return hipErrorInvalidValue;
    // the split-K path needs its buffers, and RMSNorm needs whole rows
    if ((a.kpart == nullptr) != (a.kcount == nullptr)) return hipErrorInvalidValue;
    const RowsPlan p = w4_rows_plan(a.tiles, a.groups, a.kpart != nullptr && a.gamma == nullptr);
    // activation window: at most 4096 columns (128 KiB of LDS); two threads
    // per 16-column segment, each half of the threads a whole number of wavefronts
    const int nt = std::max({256, 64 * p.s * p.tw, 2 * (int)round_up(8 * p.gw, 64)});
    const size_t lds = (size_t)16 * (p.gw * kGroup + 8) * 2 + ((size_t)(nt / 64) * 256 + (size_t)p.tw * 256) * 4;
    hipError_t e = hipSuccess;
    switch (p.s) {
      case 8: e = launch_rows<EPI, 8>(a, p, nt, lds, s); break;
      case 4: e = launch_rows<EPI, 4>(a, p, nt, lds, s); break;
      case 2: e = launch_rows<EPI, 2>(a, p, nt, lds, s); break;
      case 1: e = launch_rows<EPI, 1>(a, p, nt, lds, s); break;
      default: e = hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
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

// Compute units of the current device (workgroups of one round), cached.
static int device_cus() {
  static std::atomic<int> cached[64];  // zero-initialised; racing callers store the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

hipError_t launch_f16_gemv(const F16GemvArgs& a, hipStream_t s) {
  if (a.batch == 1) {
    constexpr int WAVES = 8, U = 8;
    const int tpw = ceil_div(a.tiles, 2 * device_cus());
    const size_t kpad = round_up((size_t)a.cblocks * 32, kGroup);
    const size_t lds = kpad * 2 + (size_t)(tpw * WAVES * 16 + 16) * 4;
    if (lds > 64 * 1024) return hipErrorInvalidValue;  // a very large vocabulary or hidden size
    hipLaunchKernelGGL((f16_gemv_b1_kernel<WAVES, U>), dim3(ceil_div(a.tiles, tpw)), dim3(WAVES * 64), lds, s, a,
                       tpw);
  } else {
    constexpr int WAVES = 4;
    if (a.xop)
      hipLaunchKernelGGL((f16_gemm_mfma_kernel<WAVES, true>), dim3(ceil_div(a.tiles, WAVES * 2)), dim3(WAVES * 64), 0,
                         s, a);
    else
      hipLaunchKernelGGL((f16_gemm_mfma_kernel<WAVES, false>), dim3(ceil_div(a.tiles, WAVES * 2)), dim3(WAVES * 64), 0,
                         s, a);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const uint16_t* x, int32_t x_stride, const uint16_t* gamma, float eps,
                               int32_t k, uint16_t* y, int32_t y_stride, int32_t batch,
                               hipStream_t s, uint16_t* yop) {
  const bool vec = rmsnorm_rows_vectorised(k, x_stride, y_stride) &&
                   ((uintptr_t)x | (uintptr_t)y | (uintptr_t)gamma | (uintptr_t)yop) % 16 == 0;
  if (yop && (!vec || batch > 16)) return hipErrorInvalidValue;
  if (vec)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<true>, dim3(batch), dim3(256), 0, s, x, x_stride, gamma, eps, k, y,
                       y_stride, yop);
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<false>, dim3(batch), dim3(256), 0, s, x, x_stride, gamma, eps, k, y,
                       y_stride, yop);
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
