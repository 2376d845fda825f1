// W4A8 variant of the INT4 projections for gfx950, measured against the
// W4A16 arithmetic in the same decomposition.
//
// The pages found, on Hopper, that multiplying INT8 activations (__dp4a) lost
// to unpacking the INT4 weights for 16-bit math (prmt.b32) in the gate/up/
// down GEMVs ("How to build your own LLM runtime from scratch", Architectural
// decisions and optimizations). gfx950 has both paths on its matrix cores:
// v_mfma_i32_16x16x64_i8 for INT8 x INT8 -> INT32, and the fp16 MFMA the
// W4A16 path uses. This kernel runs either, with everything else equal: one
// wavefront per 16-row weight tile streaming all its 128-column groups, the
// activation rows (batch <= 16) staged once per workgroup in LDS.
//
// INT8 path: each activation row is quantised symmetrically, s_x = max|x| /
// 127 and x_q = round-half-even(x / s_x) in float32, clamped to +-127. A
// packed word's nibbles u = q + 8 split into two 4-byte words of u values
// with one AND and one shift-AND; the MFMA sums u * x_q over 64 k-slots in
// INT32 and the offset is removed exactly per group: sum q x_q = sum u x_q -
// 8 sum x_q (the group sums of x_q are staged with the rows). The group's
// fp16 scale multiplies that integer in fp32, and s_x multiplies the row at
// the end. fp16 path: the decode GEMV's exact nibble-to-fp16 dequantisation
// and v_mfma_f32_16x16x32_f16 (gemv_b1.h).
#include <hip/hip_runtime.h>

#include "gemv_b1.h"

namespace w4 {

typedef int i4_t __attribute__((ext_vector_type(4)));

constexpr int kAxWaves = 8;    // wavefronts (tiles) per workgroup
constexpr int kAxUnroll = 3;   // blocks per batch, two batches in flight

// INT8 staging order inside a 32-column chunk: byte t of staged word j holds
// natural column 8 j + kI8Perm[t] -- the order in which the low and high
// nibbles of packed word j come out of (w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F).
__device__ __constant__ int kI8Perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};

template <bool I8>
__global__ __launch_bounds__(kAxWaves * 64) void w4ax_gemv_kernel(W4AxArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int NT = blockDim.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.groups, kpad = G * kGroup, B = a.batch;
  const int words = kpad / 8;                       // 8-column words per row
  constexpr int EB = I8 ? 1 : 2;                    // bytes per staged activation
  uint8_t* xs = smem;                               // [B + 1][kpad] staged rows, row B all zero
  int32_t* gsum = reinterpret_cast<int32_t*>(smem + (size_t)(B + 1) * kpad * EB);  // [B][G] (INT8)
  float* sx = reinterpret_cast<float*>(gsum + (size_t)B * G);                       // [16]
  float* red = sx + 16;                                                            // [16][kAxWaves]

  // ---- stage the rows (and, for INT8, their scales and group sums)
  if (I8) {
    for (int r = 0; r < B; ++r) {
      float m = 0.f;
      for (int wd = tid; wd < words; wd += NT) {
        const int c = 8 * wd;
        if (c < a.k) {
          const u4_t v = *reinterpret_cast<const u4_t*>(a.x + (size_t)r * a.x_stride + c);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const h2_t h = as_h2(v[d]);
            m = fmaxf(m, fmaxf(fabsf((float)h[0]), fabsf((float)h[1])));
          }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) red[r * kAxWaves + wave] = m;
    }
    __syncthreads();
    if (tid < B) {
      float m = 0.f;
      for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, red[tid * kAxWaves + w]);
      sx[tid] = m / 127.0f;
    }
    __syncthreads();
    // words of a 128-column group are 16 consecutive wd: with NT a multiple of
    // 64 they are the 16 lanes of one DPP row, whose sum is the group sum
    for (int r = 0; r <= B; ++r) {
      const float s = r < B ? sx[r] : 0.f;
      for (int wd0 = 0; wd0 < words; wd0 += NT) {
        const int wd = wd0 + tid;
        const int c = 8 * wd;
        uint8_t q8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        float part = 0.f;
        if (r < B && c < a.k && s > 0.f) {
          const u4_t v = *reinterpret_cast<const u4_t*>(a.x + (size_t)r * a.x_stride + c);
          int qn[8];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const h2_t h = as_h2(v[d]);
            qn[2 * d] = (int)fminf(127.f, fmaxf(-127.f, rintf(__fdiv_rn((float)h[0], s))));
            qn[2 * d + 1] = (int)fminf(127.f, fmaxf(-127.f, rintf(__fdiv_rn((float)h[1], s))));
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            q8[t] = (uint8_t)(int8_t)qn[kI8Perm[t]];
            part += (float)qn[t];
          }
        }
        if (wd < words) {
          u2_t packed;
          packed[0] = q8[0] | (q8[1] << 8) | (q8[2] << 16) | ((uint32_t)q8[3] << 24);
          packed[1] = q8[4] | (q8[5] << 8) | (q8[6] << 16) | ((uint32_t)q8[7] << 24);
          *reinterpret_cast<u2_t*>(xs + (size_t)r * kpad + c) = packed;
        }
        // the 16 lanes of this DPP row hold group (wd0 + tid) / 16's words
        part += ror4(part);
        part += ror8(part);
        part += dpp_xor1(part);
        part += dpp_xor2(part);
        if (r < B && (tid & 15) == 0 && wd < words) gsum[r * G + wd / 16] = (int32_t)part;
      }
    }
  } else {
    for (int r = 0; r <= B; ++r)
      for (int wd0 = 0; wd0 < words; wd0 += NT) {
        const int wd = wd0 + tid;
        const int c = 8 * wd;
        u4_t v = {0u, 0u, 0u, 0u};
        if (r < B && c < a.k) v = *reinterpret_cast<const u4_t*>(a.x + (size_t)r * a.x_stride + c);
        const u4_t o = slot_word(v, wd & 1);   // the decode GEMV's k-slot order (every quad lane)
        if (wd < words) *reinterpret_cast<u4_t*>(xs + ((size_t)r * kpad + c) * 2) = o;
      }
  }
  __syncthreads();

  // ---- one wavefront per tile: stream its G blocks
  const int t = blockIdx.x * kAxWaves + wave;
  const bool live = t < a.tiles;
  const int tt = live ? t : 0;
  const u4_t* wb = reinterpret_cast<const u4_t*>(a.w) + (size_t)tt * G * 64 + lane;
  const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.w + (size_t)a.tiles * G * 1024) + (size_t)tt * G * 16 + (lane & 15);
  const int arow = min(lane & 15, B);     // rows past the batch read the zero row
  const int c32 = 32 * (lane >> 4);
  u4_t bufA[kAxUnroll], bufB[kAxUnroll];
  uint32_t scA[kAxUnroll], scB[kAxUnroll];
  auto load = [&](u4_t* buf, uint32_t* sc, int i0) {
#pragma unroll
    for (int u = 0; u < kAxUnroll; ++u) {
      const int i = min(i0 + u, G - 1);
      buf[u] = __builtin_nontemporal_load(wb + (size_t)i * 64);
      sc[u] = sb[(size_t)i * 16];
    }
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const uint32_t mlo = vgpr_const(kMaskLo), mhi = vgpr_const(kMaskHi);
  auto compute = [&](const u4_t* buf, const uint32_t* sc, int i0) {
#pragma unroll
    for (int u = 0; u < kAxUnroll; ++u) {
      const int g = i0 + u;
      if (g < G) {
        const float s = h2f((uint16_t)sc[u]);
        if (I8) {
          const u4_t w = buf[u];
          const uint8_t* xr = xs + (size_t)arow * kpad + g * kGroup + c32;
          const i4_t a0 = __builtin_bit_cast(i4_t, *reinterpret_cast<const u4_t*>(xr));
          const i4_t a1 = __builtin_bit_cast(i4_t, *reinterpret_cast<const u4_t*>(xr + 16));
          const i4_t b0 = {(int)(w[0] & 0x0F0F0F0Fu), (int)((w[0] >> 4) & 0x0F0F0F0Fu),
                           (int)(w[1] & 0x0F0F0F0Fu), (int)((w[1] >> 4) & 0x0F0F0F0Fu)};
          const i4_t b1 = {(int)(w[2] & 0x0F0F0F0Fu), (int)((w[2] >> 4) & 0x0F0F0F0Fu),
                           (int)(w[3] & 0x0F0F0F0Fu), (int)((w[3] >> 4) & 0x0F0F0F0Fu)};
          i4_t d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, (i4_t){0, 0, 0, 0}, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, d, 0, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int br = 4 * (lane >> 4) + j;
            const int gs = br < B ? gsum[br * G + g] : 0;
            acc[j] = fmaf(s, (float)(d[j] - 8 * gs), acc[j]);
          }
        } else {
          const uint16_t* xl = reinterpret_cast<const uint16_t*>(xs) + (size_t)arow * kpad + g * kGroup + c32;
          const f4_t d = mfma_block(buf[u], xl, mlo, mhi);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] = fmaf(s, d[j], acc[j]);
        }
      }
    }
  };
  load(bufA, scA, 0);
  for (int i = 0; i < G; i += 2 * kAxUnroll) {
    load(bufB, scB, i + kAxUnroll);
    compute(bufA, scA, i);
    if (i + kAxUnroll >= G) break;
    load(bufA, scA, i + 2 * kAxUnroll);
    compute(bufB, scB, i + kAxUnroll);
  }
  // lane l: D[batch row 4 (l >> 4) + j][weight row l & 15]
  const int row = kTileRows * tt + (lane & 15);
  if (live && row < a.n)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int br = 4 * (lane >> 4) + j;
      if (br < B) a.y[(size_t)br * a.y_stride + row] = f2h(I8 ? acc[j] * sx[br] : acc[j]);
    }
}

size_t w4ax_lds_bytes(int groups, int batch, bool int8) {
  const size_t kpad = (size_t)groups * kGroup;
  return (size_t)(batch + 1) * kpad * (int8 ? 1 : 2) + (size_t)batch * groups * 4 + (16 + 16 * kAxWaves) * 4;
}

template <bool I8>
static hipError_t launch_ax(const W4AxArgs& a, hipStream_t s) {
  const size_t lds = w4ax_lds_bytes(a.groups, a.batch, I8);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&w4ax_gemv_kernel<I8>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((w4ax_gemv_kernel<I8>), dim3(ceil_div(a.tiles, kAxWaves)), dim3(kAxWaves * 64), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_w4ax_gemv(const W4AxArgs& a, bool int8, hipStream_t s) {
  return int8 ? launch_ax<true>(a, s) : launch_ax<false>(a, s);
}

}  // namespace w4
