// Prefill of a prompt for gfx950: the W4A16 projections as M-row GEMMs on
// the matrix cores, and causal attention of the prompt rows over the pages.
//
// Before decoding, a prompt runs through the model once: every token's K/V
// goes into the sequence's pages and the last token's logits give the first
// generated token ("How to build your own LLM runtime from scratch", Key
// performance metrics: time to first token of a 512-token prompt). Each
// prompt row gets exactly the decode step's arithmetic at its own position;
// the rows meet only through the pages (causal attention).
//
// Weights are the packed w4g128 blocks the decode step reads (symmetric INT4,
// group 128 along the input dimension; "How to build your own LLM runtime from
// scratch", Architectural decisions and optimizations): at M = 512 rows a
// projection is a dense contraction (gate/up: 139 GFLOP against 70 MB of
// weights), so the kernel reuses each dequantised block for many rows.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_item.h"
#include "gemv_b1.h"

namespace w4 {

// ---------------------------------------------------------------- W4A16 GEMM
// Workgroup = WM x WN wavefronts; wavefront (wm, wn) computes rows
// [m0 + 16 MR wm, +16 MR) x weight tiles [t0 + NTW wn, +NTW) as MR x NTW
// 16x16 blocks of v_mfma_f32_16x16x32_f16 (A = activation rows from LDS,
// B = the lane's 16 bytes of a packed block, exactly dequantised as in the
// decode GEMV). Per 128-column group the four MFMAs of a block start from
// zero and the group's fp32 scale is applied to the sum (acc += s * D), so
// the result is the fp32 sum over groups of exact per-group products, as at
// batch 1.
//
// The operands move by the 16-byte buffer-to-LDS loads of gfx950
// (buffer_load_dwordx4 ... lds: lane L's 16 bytes land at the LDS base + 16 L)
// into a ring of two or three stages, each holding one 128-column group: the
// activation rows in natural order (row r's 16-byte word w at physical slot
// w ^ swz(r & 15), swz swapping the two 2-bit halves of its argument: measured
// on gfx950, the 64 reads of one MFMA operand then take 4 LDS cycles per
// ds_read_b128, against 8 with w ^ (r & 15) or a rotation), the workgroup's
// packed weight blocks, and each wavefront's scales.
// One or two groups are in flight while one is multiplied, with no registers
// spent on staging. MFMA r takes word r of the lane's 16 weight bytes,
// dequantised in natural column order (the nibbles of columns 2i and 2i + 1
// sit at bits 4i and 16 + 4i: a mask of the word, or of the word shifted by
// 8, gives each pair as one fp16x2), so its activation operand is the row's
// natural 16-byte word 4 (lane / 16) + r, read from LDS as is.

// The prefill epilogue of one accumulator value: lane l holds weight row
// l & 15 of tile t for activation row m; its partner (weight row (l & 15) ^ 8)
// comes from ror8, taken by every lane before any branch. Every output here
// (and the residual) passes between kernels, so plain loads and stores do.
template <int EPI>
__device__ __forceinline__ void pf_epilogue(const GemvArgs& a, int m, int t, int i, float v, float partner) {
  if (m >= a.batch || t >= a.tiles) return;
  if (EPI == EPI_QKV) {
    if (i < 8) {
      const int pair = qkv_dim0(a.qkv, t, i);
      const float* cs = a.qkv.rope + ((size_t)m * (a.qkv.head_dim / 2) + pair) * 2;
      epi_qkv(a, m, t, i, v, partner, cs[0], cs[1], a.qkv.slot[m], false);
    }
  } else if (EPI == EPI_SILU) {
    const int o = 8 * t + i;
    if (i < 8 && o < a.n / 2) a.y[(size_t)m * a.y_stride + o] = f2h(v / (1.0f + expf(-v)) * partner);
  } else {
    const int row = kTileRows * t + i;
    if (row < a.n) {
      if (EPI == EPI_RESID) v += h2f(a.resid[(size_t)m * a.y_stride + row]);
      a.y[(size_t)m * a.y_stride + row] = f2h(v);
    }
  }
}

template <int WM, int WN, int MR, int NTW, int NS>
struct PfRing {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kRows = 16 * MR * WM;
  static constexpr int kTiles = NTW * WN;
  static constexpr int kABytes = kRows * kGroup * 2;
  static constexpr int kWBytes = kTiles * 1024;
  static constexpr int kSBytes = WM * WN * 256;        // one 4-byte load per lane of each wavefront
  static constexpr int kStage = kABytes + kWBytes + kSBytes;
  static constexpr int kAInst = kABytes / (kThreads * 16);
  static constexpr int kWInst = kWBytes / (kThreads * 16);
  static constexpr int kInst = kAInst + kWInst + 1;    // vector-memory instructions per stage per thread
  static_assert(kABytes % (kThreads * 16) == 0 && kWBytes % (kThreads * 16) == 0, "whole DMA rounds");
  static_assert(NTW * 32 <= 256, "a wavefront's scales fit one 4-byte load");
  static_assert(kInst < 64, "vmcnt range");
  static_assert(NS == 2 || NS == 3, "two or three stages");
};

typedef __attribute__((address_space(3))) void* lptr_t;


// LDS slot key of an activation row (mod 16): its 2-bit halves swapped
__device__ __forceinline__ int swz(int x) { return ((x & 3) << 2) | (x >> 2); }

// buffer-to-LDS copies: lane L's 16 (4) bytes at voffset + soffset land at the
// LDS base + 16 L (4 L)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)lds_base, 4, voff, soff, 0, 0);
}

// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// WPE: wavefronts per SIMD the register allocation must allow. KS > 1: the
// 128-column groups are split over KS workgroups (blockIdx.z), whose fp32
// sums meet in a.kpart; the last of a tile block's workgroups to arrive (a
// counter in a.kcount, zero between launches) adds them in split order and
// runs the epilogue.
template <int EPI, int WM, int WN, int MR, int NTW, int NS, int WPE, int KS>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void w4_gemm_prefill_dma_kernel(GemvArgs a) {
  using T = PfRing<WM, WN, MR, NTW, NS>;
  // separate arrays, so the compiler's wait analysis tells the slot being
  // filled from the slot being read
  __shared__ __align__(16) uint8_t ring0[T::kStage];
  __shared__ __align__(16) uint8_t ring1[T::kStage];
  __shared__ __align__(16) uint8_t ring2[NS == 3 ? T::kStage : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int m0 = blockIdx.x * T::kRows;                // row blocks fastest: neighbours share weights
  const int tg0 = blockIdx.y * T::kTiles;              // the workgroup's first weight tile
  const int G = a.groups;
  const int kz = KS > 1 ? (int)blockIdx.z : 0;
  const int gb = kz * G / KS, ng = (kz + 1) * G / KS - gb;   // this workgroup's groups [gb, gb + ng)
  // Buffer resources rebased at the workgroup's first row and first tile:
  // every offset fits 32 bits at any batch, a group advances through the
  // scalar offset alone (no per-load address arithmetic), and the hardware's
  // range check drops reads past the last row's end (the columns of a partial
  // last group are zeroed in LDS anyway).
  const int rows = min(T::kRows, a.batch - m0);      // real rows of this workgroup
  const int ntl = min(T::kTiles, a.tiles - tg0);      // real tiles of this workgroup
  const __amdgpu_buffer_rsrc_t rx =
      range_rsrc(reinterpret_cast<const uint8_t*>(a.x) + 2 * (size_t)m0 * a.x_stride,
                 2 * ((rows - 1) * a.x_stride + a.k));
  const __amdgpu_buffer_rsrc_t rw = range_rsrc(a.w + (size_t)tg0 * G * 1024, ntl * G * 1024);
  const __amdgpu_buffer_rsrc_t rs = range_rsrc(a.w + (size_t)a.tiles * G * 1024 + (size_t)tg0 * G * 32, ntl * G * 32);

  // per-thread load offsets, fixed across groups: A (row r, physical word p
  // <- logical word p ^ swz(r & 15); rows past the last repeat it), W (the
  // workgroup's blocks in tile order), S (word l % 8 of tile (l / 8) % NTW of
  // the wavefront's tiles: every lane loads, so every wavefront issues the same
  // count of loads on every path; lanes past 8 NTW repeat words nobody reads)
  uint32_t voa[T::kAInst], vow[T::kWInst];
#pragma unroll
  for (int i = 0; i < T::kAInst; ++i) {
    const int ci = tid + i * T::kThreads;              // 16-byte chunk of the A region
    const int r = ci >> 4, p = ci & 15;
    voa[i] = 2 * (min(r, rows - 1) * a.x_stride + 8 * (p ^ swz(r & 15)));
  }
#pragma unroll
  for (int i = 0; i < T::kWInst; ++i) {
    const int ci = tid + i * T::kThreads;
    vow[i] = min(ci >> 6, ntl - 1) * G * 1024 + 16 * (ci & 63);
  }
  const uint32_t vos = min(wn * NTW + ((lane >> 3) & (NTW - 1)), ntl - 1) * G * 32 + 4 * (lane & 7);

  auto issue = [&](int g, uint8_t* st) {
#pragma unroll
    for (int i = 0; i < T::kAInst; ++i)
      dma16(rx, voa[i], g * kGroup * 2, st + 16 * (wave * 64 + i * T::kThreads));
#pragma unroll
    for (int i = 0; i < T::kWInst; ++i)
      dma16(rw, vow[i], g * 1024, st + T::kABytes + 16 * (wave * 64 + i * T::kThreads));
    dma4(rs, vos, g * 32, st + T::kABytes + T::kWBytes + wave * 256);
  };

  f4_t acc[MR][NTW];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = (f4_t){0.f, 0.f, 0.f, 0.f};
  const uint32_t mlo = vgpr_const(kMaskLo), mhi = vgpr_const(kMaskHi);
  const h2_t bias = (h2_t){(_Float16)1032.0f, (_Float16)1032.0f};
  const h2_t sixteenth = (h2_t){(_Float16)0.0625f, (_Float16)0.0625f};
  const h2_t bias16 = (h2_t){(_Float16)72.0f, (_Float16)72.0f};
  // nibble pair at bits (0, 16) of v: 1024 + u - 1032 = q; at bits (4, 20):
  // (1024 + 16 u) / 16 - 72 = q (both exact in fp16)
  auto qlo = [&](uint32_t v) { return __builtin_bit_cast(uint32_t, as_h2((v & mlo) | 0x64006400u) - bias); };
  auto qhi = [&](uint32_t v) {
    return __builtin_bit_cast(uint32_t, as_h2((v & mhi) | 0x64006400u) * sixteenth - bias16);
  };
  const int x15 = lane & 15, c4 = 4 * (lane >> 4);   // row within a block, first word of the lane's chunk
  const int key = swz(x15);

  auto compute = [&](const uint8_t* st) {
    const uint8_t* A = st + (size_t)(16 * MR * wm + x15) * (kGroup * 2);
    const uint8_t* W = st + T::kABytes + (size_t)(wn * NTW) * 1024 + 16 * lane;
    const uint16_t* S = reinterpret_cast<const uint16_t*>(st + T::kABytes + T::kWBytes + wave * 256);
    u4_t wv[NTW];
    float sc[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      wv[j] = *reinterpret_cast<const u4_t*>(W + j * 1024);
      sc[j] = h2f(S[j * 16 + x15]);
    }
    f4_t d[MR][NTW];
#pragma unroll
    for (int r = 0; r < 4; ++r) {                  // MFMA r: word r of the lane's 16-byte chunk
      h8_t bw[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const uint32_t p = wv[j][r];
        bw[j] = __builtin_bit_cast(h8_t, (u4_t){qlo(p), qhi(p), qlo(p >> 8), qhi(p >> 8)});
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        const h8_t av = *reinterpret_cast<const h8_t*>(A + (size_t)16 * i * (kGroup * 2) + 16 * ((c4 + r) ^ key));
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          d[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bw[j], r == 0 ? (f4_t){0.f, 0.f, 0.f, 0.f} : d[i][j],
                                                           0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(sc[j], d[i][j][q], acc[i][j][q]);
  };

  // Ring of NS stages: the workgroup's l-th group in ring l % NS, NS - 1
  // groups in flight. With three stages every stage issues exactly kInst
  // loads per thread (past the last group they reload it into the slot no
  // later stage reads), so one wait form holds everywhere: at stage l the
  // loads of l + 1 are the only ones newer than those of l. With two, a stage
  // waits for all its loads. Columns at or past k (a partial last group) are
  // zeroed in LDS before that group is multiplied, as the decode GEMV zeroes
  // them.
  const bool ragged = (a.k & (kGroup - 1)) != 0;
  auto stage = [&](int l, uint8_t* cur, uint8_t* nxt) {
    const int g = gb + l;
    // this thread's loads of stage g are done; after the barrier every
    // thread's are, and every wavefront has consumed its reads of stage
    // g - 1 (whose ring slot the next loads overwrite). A bare s_barrier:
    // __syncthreads() would also wait for the loads still in flight.
    if constexpr (NS == 3) wait_vm<T::kInst>(); else wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (ragged && g == G - 1) {                     // uniform across the workgroup
#pragma unroll
      for (int i = 0; i < T::kAInst; ++i) {
        const int ci = tid + i * T::kThreads;
        const int r = ci >> 4, p = ci & 15;
        if (g * kGroup + 8 * (p ^ swz(r & 15)) >= a.k) *reinterpret_cast<u4_t*>(cur + 16 * ci) = (u4_t){0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if constexpr (NS == 3) issue(gb + min(l + 2, ng - 1), nxt);
    else if (l + 1 < ng) issue(g + 1, nxt);
    compute(cur);
  };
  issue(gb, ring0);
  int l = 0;
  if constexpr (NS == 3) {
    issue(gb + min(1, ng - 1), ring1);
    for (; l + 3 <= ng; l += 3) {
      stage(l, ring0, ring2);
      stage(l + 1, ring1, ring0);
      stage(l + 2, ring2, ring1);
    }
    if (l < ng) {                                    // nested, so no path reads a slot still being filled
      stage(l, ring0, ring2);
      if (l + 1 < ng) stage(l + 1, ring1, ring0);
    }
  } else {
    for (; l + 2 <= ng; l += 2) {
      stage(l, ring0, ring1);
      stage(l + 1, ring1, ring0);
    }
    if (l < ng) stage(l, ring0, ring1);
  }
  wait_vm<0>();                                      // no load may land in LDS after the workgroup ends

  if constexpr (KS > 1) {
    // Partial sums move between workgroups (and XCDs) through device-scope
    // 16-byte stores and loads; each workgroup's stores complete before it
    // counts itself. Lane l's block (i, j) of wavefront w sits at f4 index
    // ((w MR + i) NTW + j) 64 + l of the workgroup's split slice.
    constexpr int PB = T::kThreads / 64 * MR * NTW * 64;          // f4 per split slice
    const int blk = blockIdx.y * gridDim.x + blockIdx.x;
    const __amdgpu_buffer_rsrc_t rp = buf_rsrc(a.kpart + (size_t)blk * KS * PB * 4);
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, acc[i][j]), rp,
                                               16 * (kz * PB + ((wave * MR + i) * NTW + j) * 64 + lane), 0,
                                               kPolicySc1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(a.kcount + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(KS - 1);
    __syncthreads();
    if (!s_last) return;                             // uniform across the workgroup
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        f4_t part[KS];                               // every split's load in flight, then the sum in split order
#pragma unroll
        for (int c = 0; c < KS; ++c)
          part[c] = c == kz ? acc[i][j]
                            : __builtin_bit_cast(f4_t, ld128_agent(rp, 16 * (c * PB + ((wave * MR + i) * NTW + j) * 64 + lane)));
        f4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KS; ++c) v += part[c];
        acc[i][j] = v;
      }
    if (tid == 0) __hip_atomic_store(a.kcount + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const int i16 = lane & 15;
  const int t0 = tg0 + wn * NTW;
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v = acc[i][j][q];
        const float partner = ror8(v);
        const int m = m0 + 16 * MR * wm + 16 * i + 4 * (lane >> 4) + q;
        pf_epilogue<EPI>(a, m, t0 + j, i16, v, partner);
      }
}

template <int EPI, int WM, int WN, int MR, int NTW, int NS, int WPE, int KS = 1>
static hipError_t launch_pf_tile(const GemvArgs& a, hipStream_t s) {
  using T = PfRing<WM, WN, MR, NTW, NS>;
  hipLaunchKernelGGL((w4_gemm_prefill_dma_kernel<EPI, WM, WN, MR, NTW, NS, WPE, KS>),
                     dim3(ceil_div(a.batch, T::kRows), ceil_div(a.tiles, T::kTiles), KS), dim3(T::kThreads), 0, s, a);
  return hipGetLastError();
}

// Groups split over four workgroups when split storage is given, for long
// rows (64 groups and more) with fewer 64-row workgroups than three per CU:
// 64-row tiles then, instead of 32-row tiles. Measured at 512 rows: down
// (148 groups) 99-109 us unsplit with 32-row tiles, 83.3 us split; o-proj and
// qkv (28 groups) split in two took 30.1 and 39.8 us against 24 and 35 us
// unsplit, the split's stores, counter and reloads outweighing its gain.
static int pf_splits(int rows, int tiles, int groups) {
  const long wg64 = (long)ceil_div(rows, 64) * ceil_div(tiles, 8);
  return wg64 < 768 && groups >= 64 ? 4 : 1;
}

// Split storage of one prefill GEMM, enough for any row count up to `rows`:
// KS slices of every 64-row x 8-tile block's fp32 sums and one arrival
// counter per block. A GEMM splits only below 768 blocks, so the most blocks
// a split launch has is min(ceil(rows / 64), 767 / tile blocks) row blocks.
static long pf_split_blocks(int rows, int n) {
  const long tb = ceil_div(w4_tiles(n), 8);
  return std::min<long>(ceil_div(rows, 64), 767 / tb) * tb;
}
size_t pf_split_floats(int rows, int n, int k) {
  if (pf_splits(1, w4_tiles(n), w4_groups(k)) == 1) return 0;          // never splits
  return (size_t)pf_splits(1, w4_tiles(n), w4_groups(k)) * pf_split_blocks(rows, n) * 64 * 128;
}
size_t pf_split_counters(int rows, int n, int k) {
  if (pf_splits(1, w4_tiles(n), w4_groups(k)) == 1) return 0;
  return (size_t)pf_split_blocks(rows, n);
}

template <int EPI>
static hipError_t launch_pf_epi(const GemvArgs& a, hipStream_t s) {
  // a workgroup's activation rows and weight blocks are addressed by 32-bit
  // buffer offsets
  if (2 * (128 * (long)a.x_stride + a.k) > INT32_MAX || 8L * a.groups * 1024 > INT32_MAX) return hipErrorInvalidValue;
  // One row of four wavefronts, each on its own two weight tiles (no
  // dequantisation done twice), three workgroups per CU: measured at 512
  // rows, the gate/up shape (over 1000 workgroups) runs fastest with 64-row
  // tiles and a two-stage ring (153.7 us against 174.8 with 32-row tiles),
  // the narrower shapes with 32-row tiles and three stages (qkv 31.1 us,
  // o-proj 23.5, down 108.3, against 35.8 / 29.2 / 139.7).
  if ((long)ceil_div(a.batch, 64) * ceil_div(a.tiles, 8) >= 1024) return launch_pf_tile<EPI, 1, 4, 4, 2, 2, 3>(a, s);
  if (a.kpart && a.kcount) {                         // split storage given (w4_prefill)
    const int ks = pf_splits(a.batch, a.tiles, a.groups);
    if (ks == 4) return launch_pf_tile<EPI, 1, 4, 4, 2, 2, 3, 4>(a, s);
  }
  return launch_pf_tile<EPI, 1, 4, 2, 2, 3, 3>(a, s);
}

hipError_t launch_w4_gemm_prefill(int epi, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_pf_epi<EPI_STORE>(a, s);
    case EPI_RESID: return launch_pf_epi<EPI_RESID>(a, s);
    case EPI_SILU: return launch_pf_epi<EPI_SILU>(a, s);
    case EPI_QKV: return launch_pf_epi<EPI_QKV>(a, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------- causal attention
// Work item = (16 prompt rows, query head): one workgroup of kPfaWaves
// wavefronts. Prompt row m sits at position start + m and attends positions
// [0, start + m] of its sequence, read through the page table (token t of the
// sequence in page page_table[t / 16], slot t % 16: "Building a Custom LLM
// Inference Runtime on H100", The Three Critical Bugs, Bug 1). The products
// run on the matrix cores as in the decode kernel, with the 16 query columns
// being the item's 16 rows: S^T = K Q^T (v_mfma_f32_16x16x32_f16, the K
// slice in its operand order, lane l ends with S[token 4 (l >> 4) + j][row
// l & 15]), base-2 online softmax per
// row in fp32, O^T = V^T P^T (v_mfma_f32_16x16x16_f16, P entering as two
// fp16 terms). A token past a row's position scores -inf.
//
// The pages go in steps of two (32 tokens, one softmax update per step);
// wavefront w takes steps w, w + W, w + 2W, ... so the long items of the
// causal triangle spread over W wavefronts, whose (m, l, O) states merge by
// log-sum-exp through LDS at the end (as the decode attention merges its
// splits). Each wavefront keeps a ring of four page buffers in registers:
// one step is multiplied while its next is in flight.
// Measured at 512 rows (one full-shape layer): 1, 2, 3, 4 or 8 wavefronts per
// item, 26.1, 24.8, 27.0, 27.6, 45.5 us.
constexpr int kPfaWaves = 2;

template <int D, int GQ>
__global__ __launch_bounds__(kPfaWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int NK = D / 32, NS = D / 16, W = kPfaWaves;
  __shared__ float sm_m[W][16], sm_l[W][16];
  __shared__ f4_t sm_o[W][NS][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // longest items first (the last row blocks attend the most pages), every
  // head of an item together: the short items fill the end of the launch
  const int blk = gridDim.y - 1 - blockIdx.y, h = blockIdx.x, kvh = h / GQ;
  const int r0 = 16 * blk;                       // first prompt row of the item
  const int last_row = min(r0 + 15, a.n - 1);
  const int p_last = a.start + last_row;         // the item's last position
  const int pe = p_last / kPage + 1;             // pages of the item
  const int qi = lane & 15, kc = 8 * (lane >> 4), tk = 4 * (lane >> 4);
  const int my_pos = a.start + r0 + qi;          // this lane's query row position (for the mask)

  // q and the pages were written by earlier kernels: plain loads, which the
  // XCD's L2 serves to the item's wavefronts and to the later row blocks.
  // The 16 rows' queries are the B operand (row qi, dims 32 kk + kc .. + 8).
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(a.q);
  const int qrow = min(r0 + qi, a.n - 1);
  u4_t qb[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) qb[kk] = ld128(rq, 2 * (qrow * a.q_stride + h * D + 32 * kk + kc));

  const float scale = kLog2e / sqrtf((float)D);
  float m_h = -INFINITY, l_h = 0.f;              // softmax state of row qi
  f4_t acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = (f4_t){0.f, 0.f, 0.f, 0.f};
  const size_t slice = (size_t)kPage * D;
  u4_t kb[4][NK], vb[4][NS / 2];
  bool bad = false;                              // a page id outside the pool (reported once)
  // the page table is read-only here: read through the constant address space
  // it becomes a scalar load, which does not wait behind the K/V loads in flight
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)a.page_table;
  // every step issues its loads (past the item's last page they reread it),
  // so no branch sits between a load and its use
  auto load_kv = [&](int p, u4_t* kk, u4_t* vv) {
    int id = ptab[min(min(p, pe - 1), a.max_pages - 1)];
    const bool out = id < 0 || id >= a.num_pages;
    bad |= out;
    id = __builtin_amdgcn_readfirstlane(out ? 0 : id);
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(a.k_pool + ((size_t)id * a.n_kv_heads + kvh) * slice);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(a.v_pool + ((size_t)id * a.n_kv_heads + kvh) * slice);
#pragma unroll
    for (int i = 0; i < NK; ++i) kk[i] = ld128(rk, 16 * (64 * i + lane));  // K slice in score operand order
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) vv[i] = ld128(rv, 16 * (64 * i + lane));
  };
  // Only the prompt's last page can hold slots no prompt row wrote (every
  // other slot of these pages holds a written token, whose weight is exactly
  // 0 for rows before it): its V values past the last prompt position are
  // zeroed, so such slots add nothing even if they hold NaN.
  const int tail_page = (a.start + a.n - 1) / kPage, tail_valid = (a.start + a.n - 1) % kPage + 1;
  auto zero_tail = [&](u4_t* vf) {
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) {
      h8_t v8 = __builtin_bit_cast(h8_t, vf[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tk + (j & 3) >= tail_valid) v8[j] = (_Float16)0.f;
      vf[i] = __builtin_bit_cast(u4_t, v8);
    }
  };
  auto step = [&](int p, const u4_t* k0, u4_t* v0, const u4_t* k1, u4_t* v1) {
    // uniform: which of the step's pages belong to the item (a page past it
    // scores -inf, so its weights are exactly 0 and the rescale exactly 1)
    const bool one = p < pe, two = p + 1 < pe;
    f4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, k0[kk]), __builtin_bit_cast(h8_t, qb[kk]),
                                                  s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, k1[kk]), __builtin_bit_cast(h8_t, qb[kk]),
                                                  s1, 0, 0, 0);
    }
    float sv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = one && kPage * p + tk + j <= my_pos ? s0[j] * scale : -INFINITY;
      sv[4 + j] = two && kPage * (p + 1) + tk + j <= my_pos ? s1[j] * scale : -INFINITY;
    }
    float lm = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) lm = fmaxf(lm, sv[j]);
    const float n_h = fmaxf(m_h, rows_max(lm));
    const bool none = n_h == -INFINITY;          // no token of this row seen yet
    // raw v_exp_f32: weights below 2^-126 of the row maximum reach no fp16 output
    const float al = none ? 1.f : __builtin_amdgcn_exp2f(m_h - n_h);
    float pj[8];
    h4_t ph0, pl0, ph1, pl1;
#pragma unroll
    for (int j = 0; j < 8; ++j) pj[j] = none ? 0.f : __builtin_amdgcn_exp2f(sv[j] - n_h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ph0[j] = (_Float16)pj[j];
      pl0[j] = (_Float16)(pj[j] - (float)ph0[j]);
      ph1[j] = (_Float16)pj[4 + j];
      pl1[j] = (_Float16)(pj[4 + j] - (float)ph1[j]);
    }
    l_h = l_h * al + rows_sum(((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7])));
    m_h = n_h;
    if (p == tail_page) zero_tail(v0);
    if (p + 1 == tail_page) zero_tail(v1);
    if (one) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const u4_t vp = v0[i >> 1];
        const h4_t v4 = __builtin_bit_cast(h4_t, (i & 1) ? (u2_t){vp[2], vp[3]} : (u2_t){vp[0], vp[1]});
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v4, ph0, acc[i] * al, 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v4, pl0, acc[i], 0, 0, 0);
      }
    }
    if (two) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const u4_t vp = v1[i >> 1];
        const h4_t v4 = __builtin_bit_cast(h4_t, (i & 1) ? (u2_t){vp[2], vp[3]} : (u2_t){vp[0], vp[1]});
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v4, ph1, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v4, pl1, acc[i], 0, 0, 0);
      }
    }
  };
  // this wavefront's steps start at pages 2 wave, 2 (wave + W), ...
  const int pw = 2 * wave, ps = 2 * W;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    load_kv(pw + ps * j, kb[2 * j], vb[2 * j]);
    load_kv(pw + ps * j + 1, kb[2 * j + 1], vb[2 * j + 1]);
    __builtin_amdgcn_sched_barrier(0);           // issued in step order
  }
  // at each step exactly the next step's 2 (NK + NS / 2) loads are newer than its own
  constexpr int kNewer = 2 * (NK + NS / 2);
  for (int p0 = pw; p0 < pe; p0 += 2 * ps) {
    wait_vm<kNewer>();
    __builtin_amdgcn_sched_barrier(0);
    step(p0, kb[0], vb[0], kb[1], vb[1]);
    load_kv(p0 + 2 * ps, kb[0], vb[0]);
    load_kv(p0 + 2 * ps + 1, kb[1], vb[1]);
    wait_vm<kNewer>();
    __builtin_amdgcn_sched_barrier(0);
    step(p0 + ps, kb[2], vb[2], kb[3], vb[3]);
    load_kv(p0 + 3 * ps, kb[2], vb[2]);
    load_kv(p0 + 3 * ps + 1, kb[3], vb[3]);
  }
  wait_vm<0>();                                  // the rereads past the item land before the merge
  if (bad && lane == 0) atomicAdd(a.err, 1u);

  // merge the W states: o = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w
  // (a wavefront that saw no token of a row has m_w = -inf and weight 0)
  if (lane < 16) {
    sm_m[wave][qi] = m_h;
    sm_l[wave][qi] = l_h;
  }
#pragma unroll
  for (int i = 0; i < NS; ++i) sm_o[wave][i][lane] = acc[i];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][qi]);
  float wt[W], L = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float mw = sm_m[w][qi];
    wt[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    L += wt[w] * sm_l[w][qi];
  }
  // lane l: O[row l & 15][dim 16 i + 4 (l >> 4) + j]; wavefront w writes dim blocks i = w, w + W, ...
  const int row = r0 + qi;
  if (row < a.n) {
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    uint16_t* out = a.out + (size_t)row * a.out_stride + h * D;
    const __amdgpu_buffer_rsrc_t ro = buf_rsrc(out);
#pragma unroll
    for (int i = wave; i < NS; i += W) {
      f4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < W; ++w) o += wt[w] * sm_o[w][i][lane];
      h4_t r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = (_Float16)(o[j] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, r), ro, 2 * (16 * i + tk), 0, 0);
    }
  }
}

template <int D>
static hipError_t launch_pfa_d(const PrefillAttnArgs& a, int group, hipStream_t s) {
  const dim3 grid(a.n_heads, ceil_div(a.n, 16)), block(kPfaWaves * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_attn_kernel<D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_attn_kernel<D, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_attn_kernel<D, 4>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((prefill_attn_kernel<D, 7>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((prefill_attn_kernel<D, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PrefillAttnArgs& a, int head_dim, int group, hipStream_t s) {
  if (head_dim == 64) return launch_pfa_d<64>(a, group, s);
  if (head_dim == 128) return launch_pfa_d<128>(a, group, s);
  return hipErrorInvalidValue;
}

}  // namespace w4

namespace w4 {

// ------------------------------------------------------------ KV page copies
// Natural-layout K/V rows (token, KV head, D values) to and from the cache's
// page slices: K slices in the score operand order of k_slice_offset, V
// slices in the P V operand order of v_slice_offset. One thread per (token, KV head, 8 dims); token i of the
// call sits at position start + i, in page page_table[pos / 16], slot
// pos % 16. A page id outside [0, num_pages) skips the token (nothing is
// read or written for it; the host validates ids it can see).
__global__ __launch_bounds__(256) void kv_pages_kernel(KvCopyArgs a) {
  const int per_tok = a.n_kv_heads * (a.head_dim / 8);
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)a.n * per_tok) return;
  const int tok = (int)(i / per_tok), rem = (int)(i % per_tok);
  const int kvh = rem / (a.head_dim / 8), d0 = 8 * (rem % (a.head_dim / 8));
  const int pos = a.start + tok;
  const int page = a.page_table[pos >> 4];
  if (page < 0 || page >= a.num_pages) return;
  const size_t slice = ((size_t)page * a.n_kv_heads + kvh) * kPage * a.head_dim;
  const int t = pos & 15;
  const size_t nat = ((size_t)tok * a.n_kv_heads + kvh) * a.head_dim + d0;
  // the 8 dims d0 .. d0 + 8 of token t are one 16-byte word of the K slice
  uint16_t* kp = a.k_pool + slice + k_slice_offset(t, d0);
  uint16_t* vp = a.v_pool + slice;
  if (a.to_pages) {
    *reinterpret_cast<u4_t*>(kp) = *reinterpret_cast<const u4_t*>(a.k + nat);
    const u4_t v8 = *reinterpret_cast<const u4_t*>(a.v + nat);
    const uint16_t* vv = reinterpret_cast<const uint16_t*>(&v8);
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[v_slice_offset(t, d0 + j)] = vv[j];
  } else {
    *reinterpret_cast<u4_t*>(a.k + nat) = *reinterpret_cast<const u4_t*>(kp);
    u4_t v8;
    uint16_t* vv = reinterpret_cast<uint16_t*>(&v8);
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = vp[v_slice_offset(t, d0 + j)];
    *reinterpret_cast<u4_t*>(a.v + nat) = v8;
  }
}

hipError_t launch_kv_pages(const KvCopyArgs& a, hipStream_t s) {
  const long threads = (long)a.n * a.n_kv_heads * (a.head_dim / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_pages_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace w4
