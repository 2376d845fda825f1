// Greedy token choice over fp16 logits: out[b] = the index of the largest
// logit of row b, the lowest such index when several are equal.
//
// This closes the token loop that the orchestrator of "Building a Custom LLM
// Inference Runtime on H100" (Architecture Overview) runs around the decode
// step: the chosen token is the next step's input.
//
// One workgroup of 1024 threads per row: the row (vocab * 2 bytes, 297 KiB
// at vocab 152064) is read once with 16-byte loads when the row start is
// 16-byte aligned, else with 2-byte loads. Each thread keeps its best
// (value, index) over ascending indices, then the 16 wavefronts reduce with
// cross-lane shuffles and LDS. Comparisons are made on the fp16 values
// widened to fp32 (exact). NaN never compares larger or equal, so it is
// never chosen; a row with no non-NaN value yields -1.
#include <climits>

#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int kArgmaxThreads = 1024;

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

__global__ __launch_bounds__(kArgmaxThreads) void argmax_rows_kernel(const uint16_t* logits,
                                                                      int vocab, int32_t* out) {
  const int b = blockIdx.x;
  const uint16_t* row = logits + (size_t)b * vocab;
  float bv = -INFINITY;
  int bi = INT_MAX;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  int scalar_from = 0;
  if (vec) {
    const int nvec = vocab / 8;
    const uint4* rv = reinterpret_cast<const uint4*>(row);
    for (int c = threadIdx.x; c < nvec; c += kArgmaxThreads) {
      const uint4 w = rv[c];
      const uint32_t parts[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        take(half_bits_to_float(parts[j] & 0xffffu), 8 * c + 2 * j, bv, bi);
        take(half_bits_to_float(parts[j] >> 16), 8 * c + 2 * j + 1, bv, bi);
      }
    }
    scalar_from = nvec * 8;
  }
  for (int i = scalar_from + threadIdx.x; i < vocab; i += kArgmaxThreads)
    take(half_bits_to_float(row[i]), i, bv, bi);

  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m);
    const int oi = __shfl_xor(bi, m);
    take(ov, oi, bv, bi);
  }
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgmaxThreads / 64; ++w) take(sv[w], si[w], bv, bi);
    out[b] = bi == INT_MAX ? -1 : bi;
  }
}

}  // namespace

hipError_t launch_argmax_f16(const uint16_t* logits, int batch, int vocab, int32_t* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(batch), dim3(kArgmaxThreads), 0, s, logits, vocab,
                     out);
  return hipGetLastError();
}

}  // namespace w4

W4_EXPORT int w4_argmax_f16(const uint16_t* logits, int32_t batch, int32_t vocab, int32_t* out,
                            void* stream) {
  w4::clear_error();
  if (!logits || !out) return w4::fail(W4_EINVAL, "w4_argmax_f16: null pointer");
  if (batch < 1 || batch > 65535 || vocab < 1)
    return w4::fail(W4_EINVAL, "w4_argmax_f16: batch %d (1..65535) or vocab %d (>= 1)", batch, vocab);
  W4_HIP(w4::launch_argmax_f16(logits, batch, vocab, out, static_cast<hipStream_t>(stream)));
  return W4_OK;
}
