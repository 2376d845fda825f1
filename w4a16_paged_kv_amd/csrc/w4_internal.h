// Internal declarations shared by the host runtime and the HIP kernels of
// libw4a16. Nothing here is part of the C ABI (include/w4a16.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "w4a16.h"

#define W4_EXPORT extern "C" __attribute__((visibility("default")))

namespace w4 {

// ----------------------------------------------------------------- errors
// Sets the thread-local message returned by w4_last_error and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Registry of live handles (KV pools, models): a handle is registered when
// created and removed when destroyed, so a call with a destroyed handle is
// refused (W4_ESTATE) instead of touching freed memory, and a second
// destroy does nothing. An address handed out again to a new handle counts
// as that new handle.
void handle_register(const void* h);
bool handle_release(const void* h);   // true if h was live (and is now removed)
bool handle_live(const void* h);

#define W4_HIP(call)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess)                                                                \
      return ::w4::fail(W4_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));         \
  } while (0)

inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kPage = 16;       // tokens per KV page
constexpr int kGroup = 128;     // input columns per INT4 scale group
constexpr int kTileRows = 16;   // rows per packed tile

// ----------------------------------------------------------- packed sizes
__host__ __device__ inline int w4_tiles(int n) { return ceil_div(n, kTileRows); }
__host__ __device__ inline int w4_groups(int k) { return ceil_div(k, kGroup); }

// --------------------------------------------------------- kernel arguments
enum Epi : int {
  EPI_STORE = 0,  // y[row] = fp16(acc)
  EPI_RESID = 1,  // y[row] = fp16(resid[row] + acc)           (residual add)
  EPI_SILU = 2,   // y[8t+i] = fp16(silu(acc_gate) * acc_up)    (GATE_UP role)
  EPI_QKV = 3     // RoPE on q/k, q -> q_out, k/v -> KV pages    (QKV role)
};

// Everything the QKV epilogue needs: RoPE at the token's position and the
// store of its K/V into the layer's pages. The per-token parts (slot and
// rotation) are the same in every layer and come from the token plan.
struct QkvEpilogue {
  uint16_t* q_out;            // [B][q_stride] fp16, q heads in logical order
  int32_t q_stride;
  uint16_t* k_pool;           // [P][Hkv][16 * D], slices in score operand order (k_slice_offset)
  uint16_t* v_pool;           // [P][Hkv][16 * D], slices in P V operand order (v_slice_offset)
  const uint16_t* bias;       // fp16 [(Hq+2Hkv)D] logical order, or nullptr
  const int32_t* slot;        // token plan: [B] page * 16 + position % 16, or -1 (no K/V store)
  const float* rope;          // token plan: [B][D/2][2] cos, sin of pair i's angle
  int32_t n_heads, n_kv_heads, head_dim;
};

// Embedding lookup and the token plan of one step, one workgroup per
// sequence: x[b] = E[tokens[b]] (skipped without tokens); slot[b] = the K/V
// slot of the token at positions[b] (page from the page table), -1 and one
// error count if the position or its page is invalid; rope[b][i] = cos, sin
// of positions[b] * rope_base^(-2i/D), computed in double.
struct TokenPlanArgs {
  const int32_t* tokens;      // [B] or nullptr
  const uint16_t* table;      // [vocab][hidden]
  int32_t vocab, hidden;
  uint16_t* x;                // [B][hidden]
  const int32_t* positions;   // [B]
  const int32_t* page_tables; // [B][pt_stride]: row b at page_tables + b * pt_stride
  int32_t pt_stride;          // max_pages, or 0 when every row is one sequence (prefill)
  int32_t max_pages, num_pages;
  int32_t head_dim;
  float rope_base;
  int32_t* slot;              // [B]
  float* rope;                // [B][head_dim / 2][2]
  int32_t batch;
  uint32_t* err;
};

struct GemvArgs {
  const uint8_t* w;       // packed weights (nibble section, then scales)
  int32_t n, k;           // logical rows / columns
  int32_t tiles, groups;  // ceil(n/16), ceil(k/128)
  const uint16_t* x;      // input fp16 [B][x_stride]
  int32_t x_stride;
  const uint16_t* gamma;  // RMSNorm weight applied to each row of x first, or nullptr
  float eps;
  uint16_t* y;            // output fp16 [B][y_stride]
  int32_t y_stride;
  const uint16_t* resid;  // EPI_RESID: residual input [B][y_stride] (may alias y)
  uint16_t* xn_out;       // with gamma: workgroup 0 also stores the normalised rows here, or nullptr
  int32_t xn_stride;      // row stride of xn_out (batch > 1)
  int32_t batch;
  QkvEpilogue qkv;
  // batch > 1, rows longer than one activation window: K split over the
  // workgroups of a tile group (w4_rows_plan), partial sums
  // [workgroups][TW][16][16] and arrival counters [tile groups] (zero between
  // launches); nullptr: one workgroup per tile group, windows in turn
  float* kpart;
  uint32_t* kcount;
};

struct F16GemvArgs {
  const uint8_t* w;       // pack_weights_f16 layout
  int32_t n, k;
  int32_t tiles, cblocks; // ceil(n/16), ceil(k/32)
  const uint16_t* x;
  int32_t x_stride;
  const uint16_t* gamma;  // optional RMSNorm (batch-1 kernel)
  float eps;
  uint16_t* y;
  int32_t y_stride;
  uint16_t* xn_out;       // with gamma: workgroup 0 also stores the normalised rows here, or nullptr
  int32_t xn_stride;      // row stride of xn_out (batch > 1)
  int32_t batch;
  const uint16_t* xop;    // batch 2..16: x in the A-operand order (launch_rmsnorm_rows' yop), or nullptr
};

struct AttnArgs {
  const uint16_t* q;          // [B][q_stride], heads of D values
  int32_t q_stride;
  const uint16_t* k_pool;     // [P][Hkv][16 * D], slices in score operand order (k_slice_offset)
  const uint16_t* v_pool;     // [P][Hkv][16 * D], slices in P V operand order (v_slice_offset)
  const int32_t* page_tables; // [B][max_pages]
  const int32_t* ctx_lens;    // [B]
  int32_t batch;
  int32_t max_pages, num_pages;
  int32_t n_heads, n_kv_heads;
  int32_t pages_per_split, max_splits;
  float* partials;            // [B][Hkv][max_splits][GQ][D + 4]: o[D], m, l, 2 unused
  uint32_t* counters;         // [B][Hkv], zero between launches
  uint16_t* out;              // [B][out_stride]
  int32_t out_stride;
  uint32_t* err;
};

// Causal attention of n prompt rows of one sequence (prefill.hip): row m at
// position start + m attends positions [0, start + m] through page_table.
struct PrefillAttnArgs {
  const uint16_t* q;          // [n][q_stride], heads of D values (after RoPE)
  int32_t q_stride;
  const uint16_t* k_pool;     // [P][Hkv][16 * D], slices in score operand order (k_slice_offset)
  const uint16_t* v_pool;     // [P][Hkv][16 * D], slices in P V operand order
  const int32_t* page_table;  // [max_pages] of the sequence
  int32_t max_pages, num_pages;
  int32_t start, n;
  int32_t n_heads, n_kv_heads;
  uint16_t* out;              // [n][out_stride]
  int32_t out_stride;
  uint32_t* err;
};

// The W4A8 / same-split W4A16 variant GEMV (w4a8.hip): one wavefront per tile.
struct W4AxArgs {
  const uint8_t* w;       // packed w4g128 weights
  int32_t n, k, tiles, groups;
  const uint16_t* x;      // fp16 [batch][x_stride]
  int32_t x_stride;
  uint16_t* y;            // fp16 [batch][y_stride]
  int32_t y_stride;
  int32_t batch;          // 1..16
};
size_t w4ax_lds_bytes(int groups, int batch, bool int8);
hipError_t launch_w4ax_gemv(const W4AxArgs& a, bool int8, hipStream_t s);

// Copies between natural-layout K/V rows [n][Hkv][D] and one layer's pages.
struct KvCopyArgs {
  uint16_t* k_pool;           // [P][Hkv][16 * D], slices in score operand order (k_slice_offset)
  uint16_t* v_pool;           // [P][Hkv][16 * D], P V operand order
  const int32_t* page_table;  // device [>= ceil((start + n) / 16)]
  int32_t num_pages, n_kv_heads, head_dim;
  int32_t start, n;
  uint16_t* k;                // [n][Hkv][D]
  uint16_t* v;
  int32_t to_pages;           // 1: rows -> pages, 0: pages -> rows
};

// Batch-1 GEMV work split (policy in gemv_b1.h): S wavefronts per tile, TW
// tiles per 1024-thread workgroup, IT activation words per thread.
struct B1Split {
  int s, tw, it;
};
B1Split w4_b1_split(int tiles, int groups);

// Batch 2..16 work split: S wavefronts per tile, TW tiles per workgroup, an
// activation window of GW groups, CH workgroups per tile group, each taking
// GW consecutive groups (CH = 1: one workgroup takes all groups, a window at
// a time).
struct RowsPlan {
  int s, tw, gw, ch;
};
RowsPlan w4_rows_plan(int tiles, int groups, bool split_k);
inline size_t w4_rows_kpart_floats(const RowsPlan& p, int tiles) {
  return p.ch > 1 ? (size_t)ceil_div(tiles, p.tw) * p.ch * p.tw * 256 : 0;
}
inline size_t w4_rows_kcount_words(const RowsPlan& p, int tiles) {
  return p.ch > 1 ? (size_t)ceil_div(tiles, p.tw) : 0;
}

// Launchers (return hipGetLastError of the launch).
hipError_t launch_w4_gemv(int epi, const GemvArgs& a, hipStream_t s);
hipError_t launch_f16_gemv(const F16GemvArgs& a, hipStream_t s);
hipError_t launch_rmsnorm_rows(const uint16_t* x, int32_t x_stride, const uint16_t* gamma,
                               float eps, int32_t k, uint16_t* y, int32_t y_stride,
                               int32_t batch, hipStream_t s, uint16_t* yop = nullptr);
// Whether launch_rmsnorm_rows takes its vectorised path (16-byte accesses,
// the only one that can also write yop), given 16-byte aligned pointers.
constexpr int kRmsWords = 4;  // 16-byte words per thread: 256 x 4 x 8 = 8192 columns
inline bool rmsnorm_rows_vectorised(int k, int x_stride, int y_stride) {
  return k % 8 == 0 && x_stride % 8 == 0 && y_stride % 8 == 0 && k <= 256 * 8 * kRmsWords;
}
hipError_t launch_embed_plan(const TokenPlanArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int head_dim, int group, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t s);
// Prefill (prefill.hip): a.batch = prompt rows (any count); epilogues as the
// decode projections, with row m's token plan entries for EPI_QKV.
// Split storage a prefill GEMM of `rows` rows, n outputs and k inputs uses
// (fp32 sums and arrival counters; 0 if it does not split). Counters start
// at zero and every split GEMM leaves them at zero.
size_t pf_split_floats(int rows, int n, int k);
size_t pf_split_counters(int rows, int n, int k);
hipError_t launch_w4_gemm_prefill(int epi, const GemvArgs& a, hipStream_t s);
hipError_t launch_prefill_attention(const PrefillAttnArgs& a, int head_dim, int group, hipStream_t s);
hipError_t launch_kv_pages(const KvCopyArgs& a, hipStream_t s);
bool attention_supported(int head_dim, int group);
// paged_attention_decode on a given scratch region (see model.cpp).
int attention_standalone(const char* who, const uint16_t* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t num_pages,
                         int32_t max_pages, void* workspace, size_t ws_bytes, uint16_t* out,
                         void* stream);

// Pages per attention split for a batch / context size: enough workgroups to
// cover the chip, each split at least one page per wavefront (eight pages).
int attention_pages_per_split(int batch, int n_kv_heads, int max_pages);
inline size_t attention_partial_floats(int batch, int n_kv_heads, int max_splits, int group,
                                       int head_dim) {
  return (size_t)batch * n_kv_heads * max_splits * group * (head_dim + 4);  // o[D], m, l, 2 unused
}

}  // namespace w4
