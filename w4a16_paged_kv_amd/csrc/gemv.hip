// W4A16 projections and the fp16 lm_head for gfx950.
//
// Weights: symmetric group-wise INT4, group 128 along the input dimension,
// dequantised value q * s ("How to build your own LLM runtime from
// scratch", Architectural decisions and optimizations). lm_head and RMSNorm
// stay in FP16 (same section).
//
// Batch 1 is a bandwidth-bound GEMV. It still runs on the matrix cores: the
// packed block is laid out as the B operand of v_mfma_f32_16x16x32_f16, a
// nibble turns into an exact fp16 (a subnormal) with one AND, and the MFMA
// does the multiply-accumulate that would otherwise cost as many vector
// instructions as the dequantisation. Batches 2..16 turn each projection
// into a skinny dense contraction on the same instruction.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "w4_internal.h"

namespace w4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// Nibbles at bits 4i and 16+4i of a packed word -> the exact fp16 pair
// (q_{2i}, q_{2i+1}). 0x6400 is 1024.0; its ulp is 1, so 0x6400|u == 1024+u.
__device__ __forceinline__ h2_t nib_pair(uint32_t word, int i) {
  const uint32_t v = ((word >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
  return __builtin_bit_cast(h2_t, v) - (h2_t){(_Float16)1032.0f, (_Float16)1032.0f};
}

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// Sum over one lane's 32 columns of a block: 4 words x 4 nibble pairs.
__device__ __forceinline__ float dot_block(const u4_t w, const uint16_t* __restrict__ xl) {
  const u4_t* xp = reinterpret_cast<const u4_t*>(xl);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u4_t xv = xp[j];
    s = __builtin_amdgcn_fdot2(nib_pair(w[j], 0), as_h2(xv[0]), s, false);
    s = __builtin_amdgcn_fdot2(nib_pair(w[j], 1), as_h2(xv[1]), s, false);
    s = __builtin_amdgcn_fdot2(nib_pair(w[j], 2), as_h2(xv[2]), s, false);
    s = __builtin_amdgcn_fdot2(nib_pair(w[j], 3), as_h2(xv[3]), s, false);
  }
  return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

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

// ------------------------------------------------------------- epilogues

__device__ __forceinline__ void kv_store(const QkvEpilogue& e, uint16_t* pool, int slot, int kvh, int dim0,
                                         int dim1, float v0, float v1) {
  if (slot < 0) return;  // invalid position or page: counted by the token plan
  uint16_t* dst = pool + (((size_t)(slot >> 4) * e.n_kv_heads + kvh) * kPage + (slot & 15)) * e.head_dim;
  dst[dim0] = f2h(v0);
  dst[dim1] = f2h(v1);
}

// Rows i and i+8 of tile t hold the rotate-half RoPE pair (dim0, dim0 + D/2)
// of one head (QKV packing role).
__device__ __forceinline__ int qkv_head(const QkvEpilogue& e, int t) { return (kTileRows * t) / e.head_dim; }
__device__ __forceinline__ int qkv_dim0(const QkvEpilogue& e, int t, int i) {
  return 8 * (((kTileRows * t) % e.head_dim) / kTileRows) + i;
}

// q/k heads are rotated by (c, sn), the token plan's rotation of the pair
// (angle pos * base^(-2 dim0 / D)), and rounded once to fp16; v heads are
// rounded unrotated. k/v go to the token's page slot.
__device__ void epi_qkv(const GemvArgs& a, int m, int t, int i, float y0, float y1, float c, float sn,
                        int slot) {
  const QkvEpilogue& e = a.qkv;
  const int D = e.head_dim;
  const int head = qkv_head(e, t);
  const int dim0 = qkv_dim0(e, t, i), dim1 = D / 2 + dim0;
  if (e.bias) {
    y0 += h2f(e.bias[head * D + dim0]);
    y1 += h2f(e.bias[head * D + dim1]);
  }
  if (head < e.n_heads + e.n_kv_heads) {
    const float r0 = y0 * c - y1 * sn;
    const float r1 = y1 * c + y0 * sn;
    if (head < e.n_heads) {
      uint16_t* q = e.q_out + (size_t)m * e.q_stride + head * D;
      q[dim0] = f2h(r0);
      q[dim1] = f2h(r1);
    } else {
      kv_store(e, e.k_pool, slot, head - e.n_heads, dim0, dim1, r0, r1);
    }
  } else {
    kv_store(e, e.v_pool, slot, head - e.n_heads - e.n_kv_heads, dim0, dim1, y0, y1);
  }
}

template <int EPI>
__device__ __forceinline__ constexpr int epi_items() {
  return (EPI == EPI_SILU || EPI == EPI_QKV) ? 8 : 16;
}

// Applies the epilogue to item i of tile t for batch row m; vals[16] are the
// fp32 results of the tile's 16 physical rows.
template <int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, int m, int t, int i, const float* vals) {
  if (EPI == EPI_QKV) {
    const int pair = qkv_dim0(a.qkv, t, i);
    const float* cs = a.qkv.rope + ((size_t)m * (a.qkv.head_dim / 2) + pair) * 2;
    epi_qkv(a, m, t, i, vals[i], vals[i + 8], cs[0], cs[1], a.qkv.slot[m]);
  } else if (EPI == EPI_SILU) {
    const int o = 8 * t + i;
    if (o < a.n / 2) {
      const float g = vals[i], u = vals[i + 8];
      a.y[(size_t)m * a.y_stride + o] = f2h(g / (1.0f + expf(-g)) * u);
    }
  } else {
    const int row = kTileRows * t + i;
    if (row < a.n) {
      float v = vals[i];
      if (EPI == EPI_RESID) v += h2f(a.resid[(size_t)m * a.y_stride + row]);
      a.y[(size_t)m * a.y_stride + row] = f2h(v);
    }
  }
}

// ------------------------------------------------------------ batch 1, MFMA
// The 16 bytes a lane holds of a packed block are already the B operand of
// v_mfma_f32_16x16x32_f16 (weight row l & 15, eight k-slots per lane group
// l >> 4), so batch 1 runs on the matrix cores too: A carries the activation
// row (A rows 1..15 are don't-care) and D row 0 comes out in lanes 0..15.
//
// Dequantisation stays exact: 0x6400 | u is 1024 + u in fp16 (ulp 1), so
// OR-ing a nibble pair masked with 0x000F000F into 0x64006400 and
// subtracting 1032 gives (q, q'); the pair four bits higher (mask 0x00F000F0)
// gives 16q after subtracting 1152, and the activations paired with those
// slots are staged divided by 16. One AND-OR and one packed subtract per
// weight pair; the multiply-accumulate runs on the matrix cores.
//
// A workgroup of WAVES wavefronts covers WAVES/S tiles; the S wavefronts of a
// tile take its 128-column groups round-robin (K split inside the workgroup),
// so small matrices still put thousands of wavefronts on the chip and large
// ones keep the activation prologue amortised over several tiles. Each
// wavefront streams its blocks U at a time with the next U loads in flight.

constexpr int kUnroll = 4;  // blocks per batch; two batches in flight

constexpr uint32_t kMaskLo = 0x000F000Fu;  // nibble offsets (0,1) / (4,5) of a word
constexpr uint32_t kMaskHi = 0x00F000F0u;  // nibble offsets (2,3) / (6,7), as 16u

// Activation staging for the MFMA path works in slot groups: slot group sg
// is the 8 k-slots of MFMA r = sg % 4 in 32-column chunk c = sg / 4, i.e.
// xs[8 sg .. 8 sg + 8). Its columns sit in the two 8-column words
// j0 = 2 (r / 2) and j0 + 1 of the chunk, at offsets 2 (r % 2) + {0, 1, 4, 5}:
// 32-bit pairs e = r % 2 and e + 2 of each word. A thread loads natural
// 8-column word wd = tid + it * NT (it < IT) of x (and of the RMSNorm
// weights) ahead of the weight stream, normalises it and builds slot group
// sg = wd from the words of its own 4-lane quad (the quad of lanes 4c..4c+3
// holds chunk c) with DPP quad permutes.

template <int IT, bool NORM>
struct StageRegs {
  u4_t x[IT], g[NORM ? IT : 1];
};

template <int IT, bool NORM>
__device__ __forceinline__ void stage_load(StageRegs<IT, NORM>& r, const uint16_t* __restrict__ x,
                                           const uint16_t* __restrict__ gamma, int k, int NT) {
  // unconditional loads from clamped addresses (a branch around a load makes
  // the compiler wait for it on the spot); words past k are zeroed after the
  // wait, in stage_row_mfma
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = min(8 * (threadIdx.x + it * NT), k - 8);
    r.x[it] = *reinterpret_cast<const u4_t*>(x + c);
    if (NORM) r.g[it] = *reinterpret_cast<const u4_t*>(gamma + c);
  }
}

__device__ __forceinline__ uint32_t quad_perm(uint32_t v, int ctrl_is_odd) {
  // quad_perm [0,0,2,2] (0xA0) or [1,1,3,3] (0xF5)
  return ctrl_is_odd ? (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xF5, 0xF, 0xF, false)
                     : (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xA0, 0xF, 0xF, false);
}

// Stages the row: with NORM it becomes fp16(x * rsqrt(mean(x^2) + eps) *
// gamma) (RMSNorm in FP16); the slots of odd r are divided by 16 (exact
// fp16 scaling). The natural-order (normalised) row also goes to xn_out if
// given. Ends with a barrier. Requires kpad <= 8 * IT * NT.
template <int IT, bool NORM>
__device__ void stage_row_mfma(const StageRegs<IT, NORM>& r, float eps, int k, int kpad, uint16_t* xs,
                               float* red, uint16_t* xn_out, const int NT) {
  // every use of the loaded words comes first, in straight-line code: a
  // branch here would make the compiler wait for all loads in flight,
  // weights included
  const int tid = threadIdx.x;
  const int e = tid & 1;                      // r % 2 of this lane's slot groups (NT % 4 == 0)
  u4_t xv[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const bool in = 8 * (tid + it * NT) < k;
#pragma unroll
    for (int d = 0; d < 4; ++d) xv[it][d] = in ? r.x[it][d] : 0u;
  }
  float rs = 1.f;
  if (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const h2_t v = as_h2(xv[it][d]);
        ss = fmaf((float)v[0], (float)v[0], ss);
        ss = fmaf((float)v[1], (float)v[1], ss);
      }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < NT / 64; ++w) tot += red[w];
    rs = 1.0f / sqrtf(tot / (float)k + eps);
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const h2_t hv = as_h2(xv[it][d]), hg = as_h2(r.g[it][d]);
        h2_t v;
        v[0] = (_Float16)((float)hv[0] * rs * (float)hg[0]);
        v[1] = (_Float16)((float)hv[1] * rs * (float)hg[1]);
        xv[it][d] = __builtin_bit_cast(uint32_t, v);
      }
  }
  const h2_t sc = e ? (h2_t){(_Float16)0.0625f, (_Float16)0.0625f} : (h2_t){(_Float16)1.0f, (_Float16)1.0f};
  u4_t o[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    // words j0 (lanes {0,0,2,2} of the quad) and j0 + 1 (lanes {1,1,3,3})
    const uint32_t a0 = quad_perm(xv[it][0], 0), a1 = quad_perm(xv[it][1], 0);
    const uint32_t a2 = quad_perm(xv[it][2], 0), a3 = quad_perm(xv[it][3], 0);
    const uint32_t b0 = quad_perm(xv[it][0], 1), b1 = quad_perm(xv[it][1], 1);
    const uint32_t b2 = quad_perm(xv[it][2], 1), b3 = quad_perm(xv[it][3], 1);
    o[it][0] = __builtin_bit_cast(uint32_t, as_h2(e ? a1 : a0) * sc);
    o[it][1] = __builtin_bit_cast(uint32_t, as_h2(e ? a3 : a2) * sc);
    o[it][2] = __builtin_bit_cast(uint32_t, as_h2(e ? b1 : b0) * sc);
    o[it][3] = __builtin_bit_cast(uint32_t, as_h2(e ? b3 : b2) * sc);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int wd = tid + it * NT;
    if (8 * wd < kpad) *reinterpret_cast<u4_t*>(xs + 8 * wd) = o[it];
    if (xn_out && 8 * wd < k) *reinterpret_cast<u4_t*>(xn_out + 8 * wd) = xv[it];
  }
  __syncthreads();
}

// A constant held in a VGPR, so v_and_or_b32 can pair it with an SGPR operand.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// Sum over one block of q * x for weight row lane & 15: d[0] of lanes 0..15
// after four chained MFMAs over the lane group's staged chunk xl.
__device__ __forceinline__ float mfma_block_b1(const u4_t w, const uint16_t* __restrict__ xl, uint32_t mlo,
                                               uint32_t mhi) {
  const u4_t* xp = reinterpret_cast<const u4_t*>(xl);
  f4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t m = (r & 1) ? mhi : mlo;
    const h2_t bias = (r & 1) ? (h2_t){(_Float16)1152.0f, (_Float16)1152.0f}
                              : (h2_t){(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t w0 = w[2 * (r >> 1)], w1 = w[2 * (r >> 1) + 1];
    auto q2 = [&](uint32_t v) {
      return __builtin_bit_cast(uint32_t, as_h2((v & m) | 0x64006400u) - bias);
    };
    const u4_t b = {q2(w0), q2(w0 >> 8), q2(w1), q2(w1 >> 8)};
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xp[r]), __builtin_bit_cast(h8_t, b),
                                               d, 0, 0, 0);
  }
  return d[0];
}

template <int EPI, int S, int IT>
__global__ __launch_bounds__(1024) void w4_gemv_b1_kernel(GemvArgs a) {
  // S wavefronts per tile, TW tiles per workgroup (blockDim.x = 64 S TW);
  // IT activation words per thread
  const int NT = blockDim.x;
  const int WAVES = NT / 64;
  const int TW = WAVES / S;
  extern __shared__ __align__(16) uint8_t smem[];
  const int G = a.groups;
  const int kpad = G * kGroup;
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)kpad * 2);  // [WAVES][16]
  float* vals = red + WAVES * 16;                                  // [TW][16]
  float* nred = vals + TW * 16;                                    // [WAVES]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * TW + wave / S;  // this wavefront's tile
  const int ks = wave % S;                   // first group; then every S-th
  const bool live = t < a.tiles;
  const int ng = live ? (G - ks + S - 1) / S : 0;  // groups of this wavefront
  const int last = ng > 0 ? ng - 1 : 0;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + ((size_t)(live ? t : 0) * G + ks) * 64 + lane;
  const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.w + (size_t)a.tiles * G * 1024) +
                       ((size_t)(live ? t : 0) * G + ks) * 16 + (lane & 15);

  // 1. this thread's activation slot groups (and RMSNorm weights) first
  constexpr bool NORM = EPI == EPI_QKV || EPI == EPI_SILU;  // batch 1: RMSNorm prologue
  StageRegs<IT, NORM> st;
  stage_load(st, a.x, a.gamma, a.k, NT);
  // QKV: the epilogue threads' RoPE rotations and the token's K/V slot, also
  // ahead of the weights
  float rc = 1.f, rsn = 0.f;
  int slot = -1;
  if (EPI == EPI_QKV && threadIdx.x < TW * 8) {
    const int tt = blockIdx.x * TW + threadIdx.x / 8;
    if (tt < a.tiles) {
      const int pair = qkv_dim0(a.qkv, tt, threadIdx.x % 8);
      const float2 cs = *reinterpret_cast<const float2*>(a.qkv.rope + 2 * pair);
      rc = cs.x;
      rsn = cs.y;
      slot = a.qkv.slot[0];
    }
  }
  // 2. weight blocks, two batches of kUnroll in flight. Loads are issued
  // unconditionally (past the wavefront's last group they re-read that block)
  // so the compiler's wait counts stay exact; scales stay fp16 until used.
  u4_t bufA[kUnroll], bufB[kUnroll];
  uint32_t scA[kUnroll], scB[kUnroll];  // one scale per register: no packing waits
  auto load = [&](u4_t* buf, uint32_t* sc, int i0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = min(i0 + u, last);
      buf[u] = __builtin_nontemporal_load(wb + (size_t)i * S * 64);
      sc[u] = sb[(size_t)i * S * 16];
    }
  };
  const uint16_t* xl = xs + 32 * (lane >> 4) + ks * kGroup;
  const uint32_t mlo = vgpr_const(kMaskLo), mhi = vgpr_const(kMaskHi);
  float acc = 0.f;
  auto compute = [&](const u4_t* buf, const uint32_t* sc, int i0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i0 + u < ng) {
        const float d = mfma_block_b1(buf[u], xl + (size_t)(i0 + u) * S * kGroup, mlo, mhi);
        acc = fmaf(d, h2f((uint16_t)sc[u]), acc);
      }
  };
  load(bufA, scA, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep the prologue's arithmetic behind the first weight loads
  // 3. activation prologue (waits for the activation loads only)
  stage_row_mfma(st, a.eps, a.k, kpad, xs, nred, (a.xn_out && blockIdx.x == 0) ? a.xn_out : nullptr, NT);
  // 4. stream
  for (int i = 0; i < ng; i += 2 * kUnroll) {
    load(bufB, scB, i + kUnroll);
    compute(bufA, scA, i);
    if (i + kUnroll >= ng) break;
    load(bufA, scA, i + 2 * kUnroll);
    compute(bufB, scB, i + kUnroll);
  }
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (threadIdx.x < TW * 16) {
    const int tl = threadIdx.x / 16, r = threadIdx.x % 16;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < S; ++k) v += red[(tl * S + k) * 16 + r];
    vals[tl * 16 + r] = v;
  }
  __syncthreads();
  constexpr int per = epi_items<EPI>();
  if (threadIdx.x < TW * per) {
    const int tl = threadIdx.x / per;
    const int tt = blockIdx.x * TW + tl;
    if (tt < a.tiles) {
      const int i = threadIdx.x % per;
      if (EPI == EPI_QKV)
        epi_qkv(a, 0, tt, i, vals[tl * 16 + i], vals[tl * 16 + i + 8], rc, rsn, slot);
      else
        epilogue<EPI>(a, 0, tt, i, vals + tl * 16);
    }
  }
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

// Batch-1 work split. TW = ceil(tiles / 256) tiles per workgroup, so a
// matrix of up to 256 x 16 tiles runs as at most one workgroup per CU: each
// CU then stages the activation row once, and no second workgroup on a CU
// waits for its activations behind the first one's weight stream. The S
// wavefronts of a tile split its groups (S <= groups / 2, S * TW <= 16), so
// small matrices still put thousands of wavefronts in flight.
struct B1Split {
  int s, tw, it;
};

static B1Split w4_b1_split(int tiles, int groups) {
  const int tw = std::min(16, ceil_div(tiles, 256));
  int s = 1;
  for (int c : {16, 8, 4, 2})
    if (groups >= 2 * c && c * tw <= 16) {
      s = c;
      break;
    }
  const int nt = 64 * s * tw;
  const int it = ceil_div(groups * kGroup, 8 * nt);  // activation words per thread
  return {s, tw, it};
}

template <int EPI, int S, int IT>
static void launch_b1(const GemvArgs& a, int tw, hipStream_t s) {
  const int waves = S * tw;
  const size_t lds = (size_t)a.groups * kGroup * 2 + (waves * 16 + tw * 16 + waves) * sizeof(float);
  hipLaunchKernelGGL((w4_gemv_b1_kernel<EPI, S, IT>), dim3(ceil_div(a.tiles, tw)), dim3(waves * 64), lds, s,
                     a);
}

template <int EPI, int S>
static hipError_t launch_b1_it(const GemvArgs& a, const B1Split& sp, hipStream_t s) {
  switch (sp.it) {
    case 1: launch_b1<EPI, S, 1>(a, sp.tw, s); return hipSuccess;
    case 2: launch_b1<EPI, S, 2>(a, sp.tw, s); return hipSuccess;
    case 3: launch_b1<EPI, S, 3>(a, sp.tw, s); return hipSuccess;
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
      case 16: e = launch_b1_it<EPI, 16>(a, sp, s); break;
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
