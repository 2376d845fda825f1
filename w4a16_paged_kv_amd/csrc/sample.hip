// Greedy token choice over fp16 logits: out[b] = the index of the largest
// logit of row b, the lowest such index when several are equal.
//
// This closes the token loop that the orchestrator of "Building a Custom LLM
// Inference Runtime on H100" (Architecture Overview) runs around the decode
// step: the chosen token is the next step's input.
//
// Each row is cut into at most 64 chunks of at least 2048 logits, one
// 256-thread workgroup per (chunk, row), so a single row is read by many
// CUs at once: a workgroup reads its chunk with 16-byte loads when the row
// start is 16-byte aligned (chunks start at multiples of 8 elements), else
// with 2-byte loads, keeps each thread's best (value, index) over ascending
// indices, reduces with cross-lane shuffles and LDS, and stores one
// (value, index) partial. A one-wavefront workgroup per row then reduces
// the row's partials. Comparisons are made on the fp16 values widened to
// fp32 (exact); the index breaks ties, so the reduction order does not
// matter. NaN never compares larger or equal, so it is never chosen; a row
// with no non-NaN value yields -1.
#include <algorithm>
#include <climits>

#include "sample.h"

namespace w4 {

namespace {

constexpr int kChunkThreads = 256;
constexpr int kMinChunk = 2048;

struct ArgmaxPartial {
  float v;
  int32_t i;
};

struct ChunkPlan {
  int chunk, nchunks;
};

ChunkPlan chunk_plan(int vocab) {
  const int target = std::min(kArgmaxMaxChunks, ceil_div(vocab, kMinChunk));
  const int chunk = (int)round_up((size_t)ceil_div(vocab, target), 8);
  return {chunk, ceil_div(vocab, chunk)};
}

__device__ inline bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ inline void take(float v, int i, float& bv, int& bi) {
  if (better(v, i, bv, bi)) {
    bv = v;
    bi = i;
  }
}

__device__ inline float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ inline void wave_best(float& bv, int& bi) {
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oi = __shfl_xor(bi, m);
    take(ov, oi, bv, bi);
  }
}

// grid (nchunks, batch): chunk c of row b covers [c * chunk, min(vocab, (c + 1) * chunk)).
__global__ __launch_bounds__(kChunkThreads) void argmax_chunks_kernel(const uint16_t* logits,
                                                                       int vocab, int chunk,
                                                                       ArgmaxPartial* partials) {
  const int c = blockIdx.x, b = blockIdx.y;
  const uint16_t* row = logits + (size_t)b * vocab;
  const int lo = c * chunk;
  const int hi = min(vocab, lo + chunk);
  float bv = -INFINITY;
  int bi = INT_MAX;
  int scalar_from = lo;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    const uint4* rv = reinterpret_cast<const uint4*>(row);
    for (int v = lo / 8 + (int)threadIdx.x; v < hi / 8; v += kChunkThreads) {
      const uint4 w = rv[v];
      const uint32_t parts[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        take(half_bits_to_float(parts[j] & 0xffffu), 8 * v + 2 * j, bv, bi);
        take(half_bits_to_float(parts[j] >> 16), 8 * v + 2 * j + 1, bv, bi);
      }
    }
    scalar_from = max(lo, hi / 8 * 8);
  }
  for (int i = scalar_from + (int)threadIdx.x; i < hi; i += kChunkThreads)
    take(half_bits_to_float(row[i]), i, bv, bi);
  wave_best(bv, bi);
  __shared__ float sv[kChunkThreads / 64];
  __shared__ int si[kChunkThreads / 64];
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = bv;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kChunkThreads / 64; ++w) take(sv[w], si[w], bv, bi);
    partials[(size_t)b * gridDim.x + c] = {bv, bi};
  }
}

// grid (batch), one wavefront: the row's nchunks partials -> out[b].
__global__ __launch_bounds__(64) void argmax_final_kernel(const ArgmaxPartial* partials,
                                                          int nchunks, int32_t* out) {
  const int b = blockIdx.x;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int c = threadIdx.x; c < nchunks; c += 64) {
    const ArgmaxPartial p = partials[(size_t)b * nchunks + c];
    take(p.v, p.i, bv, bi);
  }
  wave_best(bv, bi);
  if (threadIdx.x == 0) out[b] = bi == INT_MAX ? -1 : bi;
}

}  // namespace

size_t argmax_workspace_bytes(int batch, int vocab) {
  return (size_t)batch * chunk_plan(vocab).nchunks * sizeof(ArgmaxPartial);
}

hipError_t launch_argmax_f16(const uint16_t* logits, int batch, int vocab, void* partials,
                             int32_t* out, hipStream_t s) {
  const ChunkPlan p = chunk_plan(vocab);
  auto* part = static_cast<ArgmaxPartial*>(partials);
  hipLaunchKernelGGL(argmax_chunks_kernel, dim3(p.nchunks, batch), dim3(kChunkThreads), 0, s,
                     logits, vocab, p.chunk, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_final_kernel, dim3(batch), dim3(64), 0, s, part, p.nchunks, out);
  return hipGetLastError();
}

}  // namespace w4

W4_EXPORT size_t w4_argmax_workspace_bytes(int32_t batch, int32_t vocab) {
  if (batch < 1 || batch > 65535 || vocab < 1) return 0;
  return w4::argmax_workspace_bytes(batch, vocab);
}

W4_EXPORT int w4_argmax_f16(const uint16_t* logits, int32_t batch, int32_t vocab, void* workspace,
                            size_t ws_bytes, int32_t* out, void* stream) {
  w4::clear_error();
  if (!logits || !out || !workspace) return w4::fail(W4_EINVAL, "w4_argmax_f16: null pointer");
  if (batch < 1 || batch > 65535 || vocab < 1)
    return w4::fail(W4_EINVAL, "w4_argmax_f16: batch %d (1..65535) or vocab %d (>= 1)", batch, vocab);
  if (!w4::aligned256(logits) || !w4::aligned256(workspace) || !w4::aligned256(out))
    return w4::fail(W4_EALIGN, "w4_argmax_f16: logits, workspace or out not 256-byte aligned");
  const size_t need = w4::argmax_workspace_bytes(batch, vocab);
  if (ws_bytes < need)
    return w4::fail(W4_EINVAL, "w4_argmax_f16: workspace %zu bytes < %zu", ws_bytes, need);
  W4_HIP(w4::launch_argmax_f16(logits, batch, vocab, workspace, out, static_cast<hipStream_t>(stream)));
  return W4_OK;
}
