// Internal declarations of the greedy token choice (sample.hip), shared with
// the generation loop of the model runtime. Not part of the C ABI.
#pragma once

#include "w4_internal.h"

namespace w4 {

constexpr int kArgmaxMaxChunks = 64;   // workgroups per logits row, at most

// Bytes of (value, index) partials for `batch` rows of `vocab` logits.
size_t argmax_workspace_bytes(int batch, int vocab);
// out[b] = argmax of logits row b; partials: device, argmax_workspace_bytes.
hipError_t launch_argmax_f16(const uint16_t* logits, int batch, int vocab, void* partials,
                             int32_t* out, hipStream_t s);

}  // namespace w4
