// Batch-1 W4A16 GEMV as device code: activation staging, the MFMA block
// product, fused epilogues and the per-wavefront streaming worker.
//
// Weights: symmetric group-wise INT4, group 128 along the input dimension,
// dequantised value q * s ("How to build your own LLM runtime from
// scratch", Architectural decisions and optimizations). RMSNorm stays in
// FP16 (same section).
//
// Activations and outputs cross workgroups (and XCDs, whose L2 caches are
// not coherent with each other): every activation load and every output
// store here is device-coherent (sc1), which costs nothing measurable for
// these few kilobytes.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "w4_internal.h"

namespace w4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

__device__ __forceinline__ int f_bits(float v) { return __builtin_bit_cast(int, v); }
__device__ __forceinline__ float bits_f(int v) { return __builtin_bit_cast(float, v); }

// Cross-lane reductions on the VALU rather than through LDS permutes:
// DPP row rotates and quad permutes inside a 16-lane row, v_permlane16_swap
// / v_permlane32_swap across rows. ror4 + ror8 combine lanes i, i+4, i+8,
// i+12 of a row; xor1 + xor2 the four lanes of a quad; rows_* lanes i, i^16,
// i^32, i^48 (every lane receives the result).
__device__ __forceinline__ float ror4(float v) {
  return bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ float ror8(float v) {
  return bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor1(float v) {
  return bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return bits_f(__builtin_amdgcn_update_dpp(0, f_bits(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(f_bits(v), f_bits(v), false, false);
  v = fmaxf(bits_f(a[0]), bits_f(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(f_bits(v), f_bits(v), false, false);
  return fmaxf(bits_f(b[0]), bits_f(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(f_bits(v), f_bits(v), false, false);
  v = bits_f(a[0]) + bits_f(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(f_bits(v), f_bits(v), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}
// Sum over the 64 lanes, in the same order in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += ror4(v);
  v += ror8(v);
  v += dpp_xor1(v);
  v += dpp_xor2(v);
  return rows_sum(v);
}

// Device-coherent accesses, for data that workgroups of one launch exchange:
// 16-bit stores through the atomic builtins, buffer loads and stores with the
// sc1 policy bit. Data passed from one launch to a later one needs neither,
// but the decode epilogues still store this way (residual rows, SiLU rows,
// q and the new token's K/V): written through, they leave no dirty lines for
// the launch's end (batch-1 o-proj and down 0.2 us faster per launch than
// plain stores; with the SiLU and qkv stores written through too, the
// batch-1 step 1.2380-1.2395 -> 1.2343-1.2349 ms, batch 16 unchanged).
__device__ __forceinline__ void st16_agent(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A 16-bit store, written through (device scope) or plain.
__device__ __forceinline__ void st16(uint16_t* p, uint16_t v, bool through) {
  if (through)
    st16_agent(p, v);
  else
    *p = v;
}

// a raw buffer of 2^31 - 1 bytes at base
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
// A raw buffer of `bytes` bytes at base: loads at or past the end read zero
// without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u4_t ld128(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
constexpr int kPolicySc1 = 16;  // buffer instruction cache-policy operand: sc1
__device__ __forceinline__ u4_t ld128_agent(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kPolicySc1));
}
__device__ __forceinline__ u2_t ld64_agent(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kPolicySc1));
}

// ------------------------------------------------------------- epilogues

// Element (token t, dim d) of a (page, head) V slice sits in the operand
// order of the attention's P V product (v_mfma_f32_16x16x16_f16, A = a
// 16-dim slice of V^T): lane L = d % 16 + 16 (t / 4) holds tokens t / 4 * 4
// .. +4 of dim d for two consecutive 16-dim slices, 16 contiguous bytes per
// lane and slice pair, so one 16-byte load per lane fetches two operands:
// offset ((d / 32) * 64 + L) * 8 + ((d / 16) % 2) * 4 + t % 4.
__host__ __device__ __forceinline__ int v_slice_offset(int t, int d) {
  return ((d >> 5) * 64 + (d & 15) + 16 * (t >> 2)) * 8 + ((d >> 4) & 1) * 4 + (t & 3);
}

// Element (token t, dim d) of a (page, head) K slice sits in the operand
// order of the attention's scores (v_mfma_f32_16x16x32_f16, A = the page's
// K): for the 32-dim step i = d / 32, lane L = t + 16 ((d / 8) % 4) holds
// dims 32 i + 8 ((d / 8) % 4) .. +8 of token t, so the 64 lanes' operands of
// one step are 1 KiB of contiguous memory (one coalesced 16-byte load per
// lane; rows of the natural [16][D] slice read 64 bytes of each of 16 rows
// per instruction, at a third of the rate from L2): offset (64 i + L) * 8 +
// d % 8.
__host__ __device__ __forceinline__ int k_slice_offset(int t, int d) {
  return ((d >> 5) * 64 + 16 * ((d >> 3) & 3) + t) * 8 + (d & 7);
}

// One token's K or V values (dims dim0, dim1 of KV head kvh) into its page
// slot, in the slice orders above (written through, or plain).
__device__ __forceinline__ void kv_store(const QkvEpilogue& e, uint16_t* pool, bool v_layout, int slot, int kvh,
                                         int dim0, int dim1, float v0, float v1, bool through) {
  if (slot < 0) return;  // invalid position or page: counted by the token plan
  uint16_t* sl = pool + ((size_t)(slot >> 4) * e.n_kv_heads + kvh) * kPage * e.head_dim;
  const int t = slot & 15;
  st16(&sl[v_layout ? v_slice_offset(t, dim0) : k_slice_offset(t, dim0)], f2h(v0), through);
  st16(&sl[v_layout ? v_slice_offset(t, dim1) : k_slice_offset(t, dim1)], f2h(v1), through);
}

// Rows i and i+8 of tile t hold the rotate-half RoPE pair (dim0, dim0 + D/2)
// of one head (QKV packing role).
__device__ __forceinline__ int qkv_head(const QkvEpilogue& e, int t) { return (kTileRows * t) / e.head_dim; }
__device__ __forceinline__ int qkv_dim0(const QkvEpilogue& e, int t, int i) {
  return 8 * (((kTileRows * t) % e.head_dim) / kTileRows) + i;
}

// q/k heads are rotated by (c, sn), the token plan's rotation of the pair
// (angle pos * base^(-2 dim0 / D)), and rounded once to fp16; v heads are
// rounded unrotated. k/v go to the token's page slot. through: q and k/v
// written through (decode) or plain (prefill, whose attention re-reads the
// pages from L2).
__device__ void epi_qkv(const GemvArgs& a, int m, int t, int i, float y0, float y1, float c, float sn,
                        int slot, bool through) {
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
      st16(&q[dim0], f2h(r0), through);
      st16(&q[dim1], f2h(r1), through);
    } else {
      kv_store(e, e.k_pool, false, slot, head - e.n_heads, dim0, dim1, r0, r1, through);
    }
  } else {
    kv_store(e, e.v_pool, true, slot, head - e.n_heads - e.n_kv_heads, dim0, dim1, y0, y1, through);
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
    epi_qkv(a, m, t, i, vals[i], vals[i + 8], cs[0], cs[1], a.qkv.slot[m], true);
  } else if (EPI == EPI_SILU) {
    const int o = 8 * t + i;
    if (o < a.n / 2) {
      const float g = vals[i], u = vals[i + 8];
      st16_agent(&a.y[(size_t)m * a.y_stride + o], f2h(g / (1.0f + expf(-g)) * u));
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
// The dequantised codes are exact: 0x6400 | u is 1024 + u in fp16 (ulp 1),
// so OR-ing a nibble pair masked with 0x000F000F into 0x64006400 and
// subtracting 1032 gives (q, q'); the pair four bits higher (mask 0x00F000F0)
// gives 16q after subtracting 1152, and the activations paired with those
// slots are staged divided by 16. That quotient is exact for |x| >= 2^-10;
// below, x / 16 is an fp16 subnormal rounded to a multiple of 2^-24 (an
// error of at most 2^-25 per activation, before the 16q weight and the
// scale). One AND-OR and one packed subtract per weight pair; the
// multiply-accumulate runs on the matrix cores.
//
// A workgroup of WAVES wavefronts covers WAVES/S tiles; the S wavefronts of a
// tile take its 128-column groups round-robin (K split inside the workgroup),
// so small matrices still put thousands of wavefronts on the chip and large
// ones keep the activation prologue amortised over several tiles. Each
// wavefront streams its blocks U at a time with the next U loads in flight.

// Blocks per batch, two batches in flight. Batch-1 step on the 7B shape:
// batches of 2, 3, 4, 6, 8 blocks gave 1.297, 1.265, 1.275, 1.384, 1.451 ms
// (three: gate/up 14.8 -> 14.6 us, down 8.7 -> 8.35 us, o-proj 4.23 -> 4.09 us;
// the batch-16 step 2.584 -> 2.557 ms).
constexpr int kUnroll = 3;

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
  // wait, in stage_row_mfma. x was written by an earlier launch: plain loads.
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int c = min(8 * (threadIdx.x + it * NT), k - 8);
    r.x[it] = ld128(rx, 2 * c);
    if (NORM) r.g[it] = *reinterpret_cast<const u4_t*>(gamma + c);
  }
}

__device__ __forceinline__ uint32_t quad_perm(uint32_t v, int ctrl_is_odd) {
  // quad_perm [0,0,2,2] (0xA0) or [1,1,3,3] (0xF5)
  return ctrl_is_odd ? (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xF5, 0xF, 0xF, false)
                     : (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xA0, 0xF, 0xF, false);
}

// Slot group sg = wd of the natural word xv held by this lane (e = wd % 2),
// built from the words of its 4-lane quad; the slots of odd r are divided
// by 16 (exact for |x| >= 2^-10, rounded to the fp16 subnormal grid below).
// All four lanes of the quad must take part.
__device__ __forceinline__ u4_t slot_word(const u4_t xv, int e) {
  const h2_t sc = e ? (h2_t){(_Float16)0.0625f, (_Float16)0.0625f} : (h2_t){(_Float16)1.0f, (_Float16)1.0f};
  // words j0 (lanes {0,0,2,2} of the quad) and j0 + 1 (lanes {1,1,3,3})
  const uint32_t a0 = quad_perm(xv[0], 0), a1 = quad_perm(xv[1], 0);
  const uint32_t a2 = quad_perm(xv[2], 0), a3 = quad_perm(xv[3], 0);
  const uint32_t b0 = quad_perm(xv[0], 1), b1 = quad_perm(xv[1], 1);
  const uint32_t b2 = quad_perm(xv[2], 1), b3 = quad_perm(xv[3], 1);
  u4_t o;
  o[0] = __builtin_bit_cast(uint32_t, as_h2(e ? a1 : a0) * sc);
  o[1] = __builtin_bit_cast(uint32_t, as_h2(e ? a3 : a2) * sc);
  o[2] = __builtin_bit_cast(uint32_t, as_h2(e ? b1 : b0) * sc);
  o[3] = __builtin_bit_cast(uint32_t, as_h2(e ? b3 : b2) * sc);
  return o;
}

// Stages the row: with NORM it becomes fp16(x * rsqrt(mean(x^2) + eps) *
// gamma) (RMSNorm in FP16); the slots of odd r are divided by 16 (see
// slot_word). The natural-order (normalised) row also goes to xn_out if
// given. Ends with a barrier. Requires kpad <= 8 * IT * NT, NT <= 1024 and
// red[16] 16-byte aligned.
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
    // the per-wavefront sums in order (slots past NT / 64 read as zero)
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f4_t r4 = *reinterpret_cast<const f4_t*>(red + 4 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) tot += 4 * q + j < NT / 64 ? r4[j] : 0.f;
    }
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
  u4_t o[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) o[it] = slot_word(xv[it], e);
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

// One block's product on the matrix cores: four chained MFMAs over the lane
// group's staged chunk xl (A row l & 15); lane l ends with
// D[activation row 4 (l >> 4) + j][weight row l & 15].
__device__ __forceinline__ f4_t mfma_block(const u4_t w, const uint16_t* __restrict__ xl, uint32_t mlo,
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
  return d;
}
// Batch 1: every lane group reads the same activation row; D row 0 (d[0] of
// lanes 0..15) is the row sum for weight row lane & 15.
__device__ __forceinline__ float mfma_block_b1(const u4_t w, const uint16_t* __restrict__ xl, uint32_t mlo,
                                               uint32_t mhi) {
  return mfma_block(w, xl, mlo, mhi)[0];
}

// What a batch-1 epilogue thread reads besides the products, loaded at the
// start of the launch so the epilogue does not wait on memory: the QKV
// epilogue's RoPE rotation and the token's K/V slot (token plan, written by
// an earlier launch; thread i < tw * 8 of virtual workgroup vb rotates pair
// i % 8 of tile vb * tw + i / 8), and the residual element of a residual
// epilogue (thread i < tw * 16 adds row 16 (vb * tw + i / 16) + i % 16; the
// residual is written only by that same thread, after this read).
struct QkvPre {
  float c, s;
  int slot;
  float resid;
};

template <int EPI>
__device__ __forceinline__ QkvPre qkv_pre(const GemvArgs& a, int vb, int tw) {
  QkvPre p{1.f, 0.f, -1, 0.f};
  if (EPI == EPI_RESID) {
    // every thread loads, from a clamped address (no branch around the load,
    // which would make the compiler wait for it here); only the epilogue's
    // threads use the value
    const int tt = min(vb * tw + (int)threadIdx.x / 16, a.tiles - 1);
    const int row = min(kTileRows * tt + (int)threadIdx.x % 16, a.n - 1);
    p.resid = h2f(a.resid[row]);
  }
  if (EPI == EPI_QKV && (int)threadIdx.x < tw * 8) {
    const int tt = vb * tw + threadIdx.x / 8;
    if (tt < a.tiles) {
      const int pair = qkv_dim0(a.qkv, tt, threadIdx.x % 8);
      const float2 cs = *reinterpret_cast<const float2*>(a.qkv.rope + 2 * pair);
      p.c = cs.x;
      p.s = cs.y;
      p.slot = a.qkv.slot[0];
    }
  }
  return p;
}

// Threads of a batch-1 GEMV workgroup whose activation row needs more than
// kMaxIt words per thread at S * TW wavefronts (same decomposition, same
// results).
constexpr int kB1Threads = 1024;

// Batch-1 work split. TW = ceil(tiles / 256) tiles per workgroup, so a
// matrix of up to 256 x 16 tiles runs as at most one workgroup per CU: each
// CU then stages the activation row once, and no second workgroup on a CU
// waits for its activations behind the first one's weight stream. The S
// wavefronts of a tile split its groups (S <= groups / 2, S * TW <= 8).
// Measured on the 7B shapes: eight wavefronts per CU stream faster than
// sixteen (qkv 6.0 -> 5.0 us, down 10.0 -> 9.1 us), because the CU issues
// the oldest wavefront's loads first and the youngest ones fall behind.
// IT activation words per thread. (B1Split, w4_b1_split: w4_internal.h.)
// With S == 1 (a workgroup holds more tiles than it has wavefronts) the
// workgroup's blocks are instead cut into kRangeWaves contiguous runs
// (GemvB1Range below).
constexpr int kRangeWaves = 8;

// Floats of per-wavefront partial sums a batch-1 GEMV keeps in LDS after the
// staged row: [waves][16] (K split) or [tw][kRangeWaves][16] (runs), then
// the reduced [tw][16].
__host__ __device__ constexpr int gemv_b1_red_floats(int s, int waves, int tw) {
  return (s == 1 ? tw * kRangeWaves * 16 : waves * 16) + tw * 16;
}
// LDS of one batch-1 GEMV: the staged activation row, then reductions.
__host__ __device__ constexpr size_t gemv_b1_lds_bytes(int groups, int s, int waves, int tw) {
  return (size_t)groups * kGroup * 2 + (size_t)(gemv_b1_red_floats(s, waves, tw) + 16) * 4;  // + 16 RMSNorm slots
}

// One wavefront's share of a batch-1 GEMV. Virtual workgroup vb covers tiles
// vb * tw .. vb * tw + tw - 1; its working wavefront w takes tile
// vb * tw + w / S and the 128-column groups w % S, w % S + S, ... (waves at or
// past S * tw, and tiles past the end, take none). Weight blocks stream two
// batches of kUnroll ahead; loads are issued unconditionally (past the
// wavefront's last group they re-read that block) so the compiler's wait
// counts stay exact, and scales stay fp16 in their own registers until used.
template <int EPI, int S, int IT>
struct GemvB1 {
  // a one-word-per-thread row with an eight-way K split (the 7B o-projection)
  // streams batches of two blocks: 4.08 -> 3.99 us per launch
  static constexpr int kUnroll = (S == 8 && IT == 1) ? 2 : w4::kUnroll;
  static constexpr bool NORM = EPI == EPI_QKV || EPI == EPI_SILU;  // batch 1: RMSNorm prologue
  int t, ks, ng, last;
  const u4_t* wb;
  const uint16_t* sb;
  u4_t bufA[kUnroll], bufB[kUnroll];
  uint32_t scA[kUnroll], scB[kUnroll];

  __device__ __forceinline__ void assign(const GemvArgs& a, int vb, int tw, int w) {
    const int lane = threadIdx.x & 63;
    t = vb * tw + w / S;
    ks = w % S;
    const bool live = w >= 0 && w < S * tw && t < a.tiles;
    ng = live ? (a.groups - ks + S - 1) / S : 0;
    last = ng > 0 ? ng - 1 : 0;
    const size_t base = (size_t)(live ? t : 0) * a.groups + ks;
    wb = reinterpret_cast<const u4_t*>(a.w) + base * 64 + lane;
    sb = reinterpret_cast<const uint16_t*>(a.w + (size_t)a.tiles * a.groups * 1024) + base * 16 + (lane & 15);
  }
  __device__ __forceinline__ void load(u4_t* buf, uint32_t* sc, int i0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = min(i0 + u, last);
      buf[u] = __builtin_nontemporal_load(wb + (size_t)i * S * 64);
      sc[u] = sb[(size_t)i * S * 16];
    }
  }
  // the first batch of weight blocks: needs nothing the previous operation writes
  __device__ __forceinline__ void prefetch() { load(bufA, scA, 0); }
  // LDS the partial sums need cleared before the row is staged: none
  __device__ __forceinline__ void clear(uint8_t*, int, int) {}

  // After the activation row is staged in LDS (xs): stream the remaining
  // blocks, reduce the S wavefronts of each tile in LDS, apply the epilogue.
  // All nt threads of the workgroup take part (the barriers are uniform).
  __device__ void finish(const GemvArgs& a, int vb, int tw, int w, uint8_t* smem, const QkvPre& pre) {
    const int lane = threadIdx.x & 63;
    const int kpad = a.groups * kGroup;
    const int waves = blockDim.x / 64;
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(smem);
    float* red = reinterpret_cast<float*>(smem + (size_t)kpad * 2);  // [waves][16]
    float* vals = red + waves * 16;                                  // [tw][16]
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
    for (int i = 0; i < ng; i += 2 * kUnroll) {
      load(bufB, scB, i + kUnroll);
      compute(bufA, scA, i);
      if (i + kUnroll >= ng) break;
      load(bufA, scA, i + 2 * kUnroll);
      compute(bufB, scB, i + kUnroll);
    }
    if (w >= 0 && w < S * tw && lane < 16) red[w * 16 + lane] = acc;
    __syncthreads();
    if ((int)threadIdx.x < tw * 16) {
      const int tl = threadIdx.x / 16, r = threadIdx.x % 16;
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < S; ++k) v += red[(tl * S + k) * 16 + r];
      vals[tl * 16 + r] = v;
    }
    __syncthreads();
    constexpr int per = epi_items<EPI>();
    if ((int)threadIdx.x < tw * per) {
      const int tl = threadIdx.x / per;
      const int tt = vb * tw + tl;
      if (tt < a.tiles) {
        const int i = threadIdx.x % per;
        if (EPI == EPI_QKV)
          epi_qkv(a, 0, tt, i, vals[tl * 16 + i], vals[tl * 16 + i + 8], pre.c, pre.s, pre.slot, true);
        else if (EPI == EPI_RESID) {
          const int row = kTileRows * tt + i;
          if (row < a.n) st16_agent(a.y + row, f2h(vals[tl * 16 + i] + pre.resid));  // write-through: measured faster here
        } else
          epilogue<EPI>(a, 0, tt, i, vals + tl * 16);
      }
    }
  }
};

// One wavefront's share of a batch-1 GEMV whose workgroup holds more tiles
// than wavefronts (S == 1; the gate/up projection of the 7B shape: ten
// tiles of 28 groups). The workgroup's blocks, tile after tile (consecutive
// in memory), are cut into kRangeWaves contiguous runs; a run may end inside
// a tile, so each wavefront leaves one partial sum per tile it touched in
// LDS ([tile][wavefront][16], cleared before the row is staged) and the
// tile's sum adds them in wavefront order. The CU serves the oldest
// wavefront of each SIMD first, so the first SIMD slot (wavefronts 0..3)
// takes 5/4 of the blocks of the second and both slots finish together
// (7B gate/up per launch: ten one-tile wavefronts 15.3-16.1 us, eight equal
// runs 15.8 us, eight 5:4 runs 14.4-15.0 us).
// Run [b0, b0 + n) of wavefront w < W when B blocks are cut into W
// contiguous runs weighted 5 for the first SIMD slot (w < 4), 4 after it.
template <int W>
__device__ __forceinline__ void weighted_run(int B, int w, int& b0, int& n) {
  int tot = 0, pre = 0;
#pragma unroll
  for (int v = 0; v < W; ++v) {
    const int wt = v < 4 ? 5 : 4;
    pre += v < w ? wt : 0;
    tot += wt;
  }
  b0 = (int)((long)B * pre / tot);
  n = (int)((long)B * (pre + (w < 4 ? 5 : 4)) / tot) - b0;
}

template <int EPI, int IT>
struct GemvB1Range {
  static constexpr bool NORM = EPI == EPI_QKV || EPI == EPI_SILU;
  static constexpr int W = kRangeWaves;
  int b0, n, last, g0, tl0;
  const u4_t* wb;
  const uint16_t* sb;
  u4_t bufA[kUnroll], bufB[kUnroll];
  uint32_t scA[kUnroll], scB[kUnroll];

  __device__ __forceinline__ void assign(const GemvArgs& a, int vb, int tw, int w) {
    const int lane = threadIdx.x & 63;
    const int t0 = vb * tw;
    const int B = min(tw, a.tiles - t0) * a.groups;  // this workgroup's blocks (>= 1)
    b0 = 0;
    n = 0;
    if (w >= 0 && w < W) weighted_run<W>(B, w, b0, n);
    last = n > 0 ? n - 1 : 0;
    g0 = n > 0 ? b0 % a.groups : 0;
    tl0 = n > 0 ? b0 / a.groups : 0;
    const size_t base = (size_t)t0 * a.groups + min(b0, B - 1);  // an empty run re-reads a block of its workgroup
    wb = reinterpret_cast<const u4_t*>(a.w) + base * 64 + lane;
    sb = reinterpret_cast<const uint16_t*>(a.w + (size_t)a.tiles * a.groups * 1024) + base * 16 + (lane & 15);
  }
  __device__ __forceinline__ void load(u4_t* buf, uint32_t* sc, int i0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = min(i0 + u, last);
      buf[u] = __builtin_nontemporal_load(wb + (size_t)i * 64);
      sc[u] = sb[(size_t)i * 16];
    }
  }
  __device__ __forceinline__ void prefetch() { load(bufA, scA, 0); }
  // zeroes the [tw][W][16] partial sums (a wavefront writes only the tiles its run touches)
  __device__ __forceinline__ void clear(uint8_t* smem, int kpad, int tw) {
    float* red = reinterpret_cast<float*>(smem + (size_t)kpad * 2);
    for (int i = threadIdx.x; i < tw * W * 16; i += blockDim.x) red[i] = 0.f;
  }

  __device__ void finish(const GemvArgs& a, int vb, int tw, int w, uint8_t* smem, const QkvPre& pre) {
    const int lane = threadIdx.x & 63;
    const int kpad = a.groups * kGroup;
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(smem);
    float* red = reinterpret_cast<float*>(smem + (size_t)kpad * 2);  // [tw][W][16]
    float* vals = red + tw * W * 16;                                 // [tw][16]
    const uint16_t* xl = xs + 32 * (lane >> 4);
    const uint32_t mlo = vgpr_const(kMaskLo), mhi = vgpr_const(kMaskHi);
    float acc = 0.f;
    int g = g0, tl = tl0;
    auto compute = [&](const u4_t* buf, const uint32_t* sc, int i0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (i0 + u < n) {
          const float d = mfma_block_b1(buf[u], xl + (size_t)g * kGroup, mlo, mhi);
          acc = fmaf(d, h2f((uint16_t)sc[u]), acc);
          if (++g == a.groups) {  // the run leaves tile tl
            if (lane < 16) red[(tl * W + w) * 16 + lane] = acc;
            acc = 0.f;
            g = 0;
            ++tl;
          }
        }
    };
    for (int i = 0; i < n; i += 2 * kUnroll) {
      load(bufB, scB, i + kUnroll);
      compute(bufA, scA, i);
      if (i + kUnroll >= n) break;
      load(bufA, scA, i + 2 * kUnroll);
      compute(bufB, scB, i + kUnroll);
    }
    if (g != 0 && lane < 16) red[(tl * W + w) * 16 + lane] = acc;  // the run ends inside tile tl
    __syncthreads();
    if ((int)threadIdx.x < tw * 16) {
      const int tl = threadIdx.x / 16, r = threadIdx.x % 16;
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < W; ++k) v += red[(tl * W + k) * 16 + r];
      vals[tl * 16 + r] = v;
    }
    __syncthreads();
    constexpr int per = epi_items<EPI>();
    if ((int)threadIdx.x < tw * per) {
      const int tl = threadIdx.x / per;
      const int tt = vb * tw + tl;
      if (tt < a.tiles) {
        const int i = threadIdx.x % per;
        if (EPI == EPI_QKV)
          epi_qkv(a, 0, tt, i, vals[tl * 16 + i], vals[tl * 16 + i + 8], pre.c, pre.s, pre.slot, true);
        else if (EPI == EPI_RESID) {
          const int row = kTileRows * tt + i;
          if (row < a.n) st16_agent(a.y + row, f2h(vals[tl * 16 + i] + pre.resid));  // write-through: measured faster here
        } else
          epilogue<EPI>(a, 0, tt, i, vals + tl * 16);
      }
    }
  }
};

// The batch-1 decomposition for a split: contiguous runs when S == 1, else
// the K split.
template <int EPI, int S, int IT>
using GemvB1Sel = typename std::conditional<S == 1, GemvB1Range<EPI, IT>, GemvB1<EPI, S, IT>>::type;

}  // namespace w4
