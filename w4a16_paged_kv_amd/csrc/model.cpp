// Decode runtime of libw4a16: workspace carving, host validation, staging,
// the per-layer kernel sequence, and hipGraph capture/replay of the step.
//
// Static preallocation: KV cache and activation buffers come from the caller
// up front, nothing is allocated per step ("Building a Custom LLM Inference
// Runtime on H100", Implementation Guide: Step-by-Step). Step inputs are
// copied into fixed staging before a captured graph is launched, never inside
// the capture (same page, The Three Critical Bugs, Bug 3), and every
// sub-buffer is 256-byte aligned (Bug 2 there asks for aligned intermediate
// buffers).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <tuple>
#include <vector>

#include "sample.h"
#include "w4_internal.h"

namespace w4 {

struct WsLayout {
  size_t err, counters, tokens, positions, ctx, pt, slot, rope, x, xn, xop, q, o, h, partials, kpart, kcount,
      amax, total;
  int xn_stride, o_stride, h_stride, max_splits;
};

static WsLayout ws_layout(const w4_config& c, int max_batch, int max_pages) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  const int group = c.n_heads / c.n_kv_heads;
  L.xn_stride = (int)round_up(c.hidden, kGroup);
  L.o_stride = (int)round_up((size_t)c.n_heads * c.head_dim, kGroup);
  L.h_stride = (int)round_up(c.ffn, kGroup);
  L.max_splits = ceil_div(max_pages, 4);
  L.err = take(256);
  L.counters = take((size_t)max_batch * c.n_kv_heads * 4);
  L.tokens = take((size_t)max_batch * 4);
  L.positions = take((size_t)max_batch * 4);
  L.ctx = take((size_t)max_batch * 4);
  L.pt = take((size_t)max_batch * max_pages * 4);
  L.slot = take((size_t)max_batch * 4);
  L.rope = take((size_t)max_batch * (c.head_dim / 2) * 2 * 4);
  L.x = take((size_t)max_batch * c.hidden * 2);
  L.xn = take((size_t)max_batch * L.xn_stride * 2);
  // batch > 1: the final RMSNorm's rows again in the lm_head's A-operand
  // order (16 rows x 32 columns per KiB)
  L.xop = max_batch > 1 ? take((size_t)L.xn_stride * 32) : 0;
  L.q = take((size_t)max_batch * c.n_heads * c.head_dim * 2);
  L.o = take((size_t)max_batch * L.o_stride * 2);
  L.h = take((size_t)max_batch * L.h_stride * 2);
  L.partials = take(attention_partial_floats(max_batch, c.n_kv_heads, L.max_splits, group,
                                             c.head_dim) * 4);
  // batch > 1: K split of the o and down projections when their rows are
  // longer than one activation window (partial sums and arrival counters)
  size_t kp = 0, kw = 0;
  if (max_batch > 1)
    for (int k : {c.n_heads * c.head_dim, c.ffn}) {
      const RowsPlan p = w4_rows_plan(w4_tiles(c.hidden), w4_groups(k), true);
      kp = std::max(kp, w4_rows_kpart_floats(p, w4_tiles(c.hidden)));
      kw = std::max(kw, w4_rows_kcount_words(p, w4_tiles(c.hidden)));
    }
  L.kpart = kp ? take(kp * 4) : 0;
  L.kcount = kw ? take(kw * 4) : 0;
  L.amax = take(argmax_workspace_bytes(max_batch, c.vocab));   // greedy token choice partials
  L.total = off;
  return L;
}

static int check_config(const w4_config* c) {
  if (!c) return fail(W4_EINVAL, "null config");
  if (c->hidden <= 0 || c->hidden % 8 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
      c->n_heads % c->n_kv_heads || c->ffn <= 0 || c->ffn % 8 || c->vocab <= 0 || c->n_layers <= 0)
    return fail(W4_EINVAL, "unsupported config: hidden=%d (mult. of 8) heads=%d/%d ffn=%d (mult. of 8) "
                "vocab=%d layers=%d", c->hidden, c->n_heads, c->n_kv_heads, c->ffn, c->vocab, c->n_layers);
  if (!attention_supported(c->head_dim, c->n_heads / c->n_kv_heads))
    return fail(W4_EINVAL, "unsupported head_dim %d / GQA group %d (head_dim 64 or 128, group 1, 2, 4, 7 or 8)",
                c->head_dim, c->n_heads / c->n_kv_heads);
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f))
    return fail(W4_EINVAL, "bad rms_eps %g or rope_base %g", c->rms_eps, c->rope_base);
  return W4_OK;
}

}  // namespace w4

using namespace w4;

struct w4_model {
  w4_config cfg;
  std::vector<w4_layer_weights> layers;
  w4_weights weights;
  uint16_t* kv = nullptr;
  int32_t num_pages = 0, max_batch = 0, max_pages = 0;
  uint8_t* ws = nullptr;
  WsLayout L;
  bool use_graph = true;
  hipStream_t cap_stream = nullptr;
  // key: batch, logits, device-input pointers (null for host inputs)
  typedef std::tuple<int, const void*, const void*, const void*, const void*, const void*> Key;
  std::map<Key, hipGraphExec_t> graphs;
  // Host inputs reach the staged tokens / positions / ctx / page-table slots
  // (consecutive workspace regions) as one copy from a pinned host image of
  // that region. Two images are used in turn; the event recorded after an
  // image's copy is waited on before the image is rewritten.
  uint8_t* stage_img = nullptr;  // 2 x stage_bytes, pinned
  size_t stage_bytes = 0;
  hipEvent_t stage_ev[2] = {nullptr, nullptr};
  int stage_next = 0;
  int32_t* gen_tokens = nullptr;  // pinned [max_batch]: the greedy loop's chosen tokens

  template <class T>
  T* at(size_t off) { return reinterpret_cast<T*>(ws + off); }
  uint16_t* k_pool(int l) {
    return kv + (size_t)(2 * l) * num_pages * cfg.n_kv_heads * kPage * cfg.head_dim;
  }
  uint16_t* v_pool(int l) {
    return kv + (size_t)(2 * l + 1) * num_pages * cfg.n_kv_heads * kPage * cfg.head_dim;
  }
};

// The model's own stream, events and pinned buffers (any may be null). A
// staging copy may still be queued behind the caller's work: each image is
// freed only after its event.
static void release_model_resources(w4_model* m) {
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  for (hipEvent_t ev : m->stage_ev)
    if (ev) {
      (void)hipEventSynchronize(ev);
      (void)hipEventDestroy(ev);
    }
  if (m->stage_img) (void)hipHostFree(m->stage_img);
  if (m->gen_tokens) (void)hipHostFree(m->gen_tokens);
}

namespace w4 {

// Device-resident per-step inputs (staging or caller-provided).
struct StepInputs {
  const int32_t* tokens;
  const int32_t* positions;
  const int32_t* page_tables;
  const int32_t* ctx_lens;
};

#define W4_LAUNCH(call)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (call);                                                              \
    if (e_ != hipSuccess)                                                                \
      return ::w4::fail(W4_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));         \
  } while (0)

static GemvArgs gemv_args(const void* w, int n, int k, const uint16_t* x, int x_stride,
                          const uint16_t* gamma, float eps, uint16_t* y, int y_stride,
                          const uint16_t* resid, int batch) {
  GemvArgs a{};
  a.w = static_cast<const uint8_t*>(w);
  a.n = n;
  a.k = k;
  a.tiles = w4_tiles(n);
  a.groups = w4_groups(k);
  a.x = x;
  a.x_stride = x_stride;
  a.gamma = gamma;
  a.eps = eps;
  a.y = y;
  a.y_stride = y_stride;
  a.resid = resid;
  a.batch = batch;
  return a;
}

// Arguments of the operations of decoder layer l for `batch` sequences. The
// residual stream goes x_in -> (o projection) x_out -> (down projection)
// x_out; q, o and h live in the workspace. The RMSNorms run while the qkv and
// gate/up projections stage their activation rows (the normalised rows also
// go to xn, from workgroup 0).
static GemvArgs qkv_args(w4_model* m, int l, const uint16_t* x_in, int batch) {
  const w4_config& c = m->cfg;
  const w4_layer_weights& W = m->layers[l];
  const WsLayout& L = m->L;
  uint16_t* xn = m->at<uint16_t>(L.xn);
  const int qkv_rows = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  GemvArgs a = gemv_args(W.qkv, qkv_rows, c.hidden, x_in, c.hidden, W.attn_norm, c.rms_eps, nullptr, 0, nullptr,
                         batch);
  a.xn_out = xn;
  a.xn_stride = L.xn_stride;
  a.qkv.q_out = m->at<uint16_t>(L.q);
  a.qkv.q_stride = c.n_heads * c.head_dim;
  a.qkv.k_pool = m->k_pool(l);
  a.qkv.v_pool = m->v_pool(l);
  a.qkv.bias = W.qkv_bias;
  a.qkv.slot = m->at<int32_t>(L.slot);
  a.qkv.rope = m->at<float>(L.rope);
  a.qkv.n_heads = c.n_heads;
  a.qkv.n_kv_heads = c.n_kv_heads;
  a.qkv.head_dim = c.head_dim;
  return a;
}

static AttnArgs attn_args(w4_model* m, int l, const StepInputs& in, int batch) {
  const w4_config& c = m->cfg;
  const WsLayout& L = m->L;
  AttnArgs at{};
  at.q = m->at<uint16_t>(L.q);
  at.q_stride = c.n_heads * c.head_dim;
  at.k_pool = m->k_pool(l);
  at.v_pool = m->v_pool(l);
  at.page_tables = in.page_tables;
  at.ctx_lens = in.ctx_lens;
  at.batch = batch;
  at.max_pages = m->max_pages;
  at.num_pages = m->num_pages;
  at.n_heads = c.n_heads;
  at.n_kv_heads = c.n_kv_heads;
  at.pages_per_split = attention_pages_per_split(batch, c.n_kv_heads, m->max_pages);
  at.max_splits = ceil_div(m->max_pages, at.pages_per_split);
  at.partials = m->at<float>(L.partials);
  at.counters = m->at<uint32_t>(L.counters);
  at.out = m->at<uint16_t>(L.o);
  at.out_stride = L.o_stride;
  at.err = m->at<uint32_t>(L.err);
  return at;
}

// batch > 1: the K-split buffers, if the workspace has them
static void with_ksplit(w4_model* m, GemvArgs& a) {
  if (a.batch > 1 && m->L.kcount) {
    a.kpart = m->at<float>(m->L.kpart);
    a.kcount = m->at<uint32_t>(m->L.kcount);
  }
}

static GemvArgs oproj_args(w4_model* m, int l, const uint16_t* x_in, uint16_t* x_out, int batch) {
  const w4_config& c = m->cfg;
  GemvArgs a = gemv_args(m->layers[l].o, c.hidden, c.n_heads * c.head_dim, m->at<uint16_t>(m->L.o),
                         m->L.o_stride, nullptr, 0.f, x_out, c.hidden, x_in, batch);
  with_ksplit(m, a);
  return a;
}

static GemvArgs gate_up_args(w4_model* m, int l, const uint16_t* x, int batch) {
  const w4_config& c = m->cfg;
  const w4_layer_weights& W = m->layers[l];
  const WsLayout& L = m->L;
  uint16_t* xn = m->at<uint16_t>(L.xn);
  uint16_t* h = m->at<uint16_t>(L.h);
  GemvArgs a = gemv_args(W.gate_up, 2 * c.ffn, c.hidden, x, c.hidden, W.mlp_norm, c.rms_eps, h, L.h_stride,
                         nullptr, batch);
  a.xn_out = xn;
  a.xn_stride = L.xn_stride;
  return a;
}

static GemvArgs down_args(w4_model* m, int l, uint16_t* x, int batch) {
  const w4_config& c = m->cfg;
  GemvArgs a = gemv_args(m->layers[l].down, c.hidden, c.ffn, m->at<uint16_t>(m->L.h), m->L.h_stride, nullptr,
                         0.f, x, c.hidden, x, batch);
  with_ksplit(m, a);
  return a;
}

// Enqueues one operation of decoder layer l for `batch` sequences.
static int enqueue_op(w4_model* m, int op, int l, const uint16_t* x_in, uint16_t* x_out,
                      const StepInputs& in, int batch, hipStream_t s) {
  const w4_config& c = m->cfg;
  switch (op) {
    case W4_OP_QKV:  // RMSNorm while staging, qkv projection, RoPE, K/V page write
      W4_LAUNCH(launch_w4_gemv(EPI_QKV, qkv_args(m, l, x_in, batch), s));
      return W4_OK;
    case W4_OP_ATTN: {  // paged attention, split over pages, LSE merge by the last split
      const AttnArgs at = attn_args(m, l, in, batch);
      // the partials buffer holds max_pages / 4 splits per (sequence, KV head)
      if (at.max_splits > m->L.max_splits)
        return fail(W4_EINVAL, "attention split of %d pages needs %d splits > %d", at.pages_per_split,
                    at.max_splits, m->L.max_splits);
      W4_LAUNCH(launch_attention(at, c.head_dim, c.n_heads / c.n_kv_heads, s));
      return W4_OK;
    }
    case W4_OP_OPROJ:  // o projection + residual
      W4_LAUNCH(launch_w4_gemv(EPI_RESID, oproj_args(m, l, x_in, x_out, batch), s));
      return W4_OK;
    case W4_OP_GATE_UP:  // RMSNorm while staging, gate/up with SiLU-mul
      W4_LAUNCH(launch_w4_gemv(EPI_SILU, gate_up_args(m, l, x_out, batch), s));
      return W4_OK;
    case W4_OP_DOWN:  // down projection + residual
      W4_LAUNCH(launch_w4_gemv(EPI_RESID, down_args(m, l, x_out, batch), s));
      return W4_OK;
  }
  return fail(W4_EINVAL, "unknown layer op %d", op);
}

// Enqueues one decoder layer: x_out = layer(x_in) for `batch` sequences.
static int enqueue_layer(w4_model* m, int l, const uint16_t* x_in, uint16_t* x_out,
                         const StepInputs& in, int batch, hipStream_t s) {
  for (int op = W4_OP_QKV; op <= W4_OP_DOWN; ++op) {
    int rc = enqueue_op(m, op, l, x_in, x_out, in, batch, s);
    if (rc) return rc;
  }
  return W4_OK;
}

static int enqueue_lm_head(w4_model* m, const uint16_t* x, int batch, uint16_t* logits,
                           hipStream_t s) {
  const w4_config& c = m->cfg;
  F16GemvArgs f{};
  f.w = static_cast<const uint8_t*>(m->weights.lm_head);
  f.n = c.vocab;
  f.k = c.hidden;
  f.tiles = w4_tiles(c.vocab);
  f.cblocks = ceil_div(c.hidden, 32);
  f.y = logits;
  f.y_stride = c.vocab;
  f.batch = batch;
  f.eps = c.rms_eps;
  if (batch == 1) {
    f.x = x;
    f.x_stride = c.hidden;
    f.gamma = m->weights.final_norm;
    f.xn_out = m->at<uint16_t>(m->L.xn);
  } else {
    uint16_t* xn = m->at<uint16_t>(m->L.xn);
    uint16_t* xop = rmsnorm_rows_vectorised(c.hidden, c.hidden, m->L.xn_stride) ? m->at<uint16_t>(m->L.xop) : nullptr;
    W4_LAUNCH(launch_rmsnorm_rows(x, c.hidden, m->weights.final_norm, c.rms_eps, c.hidden, xn,
                                  m->L.xn_stride, batch, s, xop));
    f.x = xn;
    f.x_stride = m->L.xn_stride;
    f.xop = xop;
  }
  W4_LAUNCH(launch_f16_gemv(f, s));
  return W4_OK;
}

// Embedding lookup (if tokens is given) and the step's token plan: every
// layer's QKV epilogue reads the token's K/V slot and RoPE rotations from it.
static int enqueue_plan(w4_model* m, const int32_t* tokens, const StepInputs& in, int batch,
                        hipStream_t s) {
  const w4_config& c = m->cfg;
  TokenPlanArgs p{};
  p.tokens = tokens;
  p.table = m->weights.embed;
  p.vocab = c.vocab;
  p.hidden = c.hidden;
  p.x = m->at<uint16_t>(m->L.x);
  p.positions = in.positions;
  p.page_tables = in.page_tables;
  p.pt_stride = m->max_pages;
  p.max_pages = m->max_pages;
  p.num_pages = m->num_pages;
  p.head_dim = c.head_dim;
  p.rope_base = c.rope_base;
  p.slot = m->at<int32_t>(m->L.slot);
  p.rope = m->at<float>(m->L.rope);
  p.batch = batch;
  p.err = m->at<uint32_t>(m->L.err);
  W4_LAUNCH(launch_embed_plan(p, s));
  return W4_OK;
}

static int enqueue_step(w4_model* m, const StepInputs& in, int batch, uint16_t* logits,
                        hipStream_t s) {
  const w4_config& c = m->cfg;
  uint16_t* x = m->at<uint16_t>(m->L.x);
  int rc0 = enqueue_plan(m, in.tokens, in, batch, s);
  if (rc0) return rc0;
  for (int l = 0; l < c.n_layers; ++l) {
    int rc = enqueue_layer(m, l, x, x, in, batch, s);
    if (rc) return rc;
  }
  return enqueue_lm_head(m, x, batch, logits, s);
}

// Host validation of one step's inputs; nothing is enqueued on failure.
static int validate_step(int vocab, int num_pages, int max_pages, const int32_t* tokens,
                         const int32_t* positions, const int32_t* page_tables,
                         const int32_t* ctx_lens, int batch) {
  for (int b = 0; b < batch; ++b) {
    if (tokens && (tokens[b] < 0 || tokens[b] >= vocab))
      return fail(W4_ERANGE, "tokens[%d] = %d outside [0, %d)", b, tokens[b], vocab);
    const int ctx = ctx_lens[b];
    if (ctx < 1 || ctx > max_pages * kPage)
      return fail(W4_ERANGE, "ctx_lens[%d] = %d outside [1, %d]", b, ctx, max_pages * kPage);
    if (positions[b] != ctx - 1)
      return fail(W4_ERANGE, "positions[%d] = %d but ctx_lens[%d] - 1 = %d", b, positions[b], b,
                  ctx - 1);
    const int32_t* row = page_tables + (size_t)b * max_pages;
    for (int p = 0; p < ceil_div(ctx, kPage); ++p)
      if (row[p] < 0 || row[p] >= num_pages)
        return fail(W4_ERANGE, "page_tables[%d][%d] = %d outside [0, %d)", b, p, row[p], num_pages);
  }
  // two sequences must not write the same (page, slot)
  for (int b = 0; b < batch; ++b)
    for (int b2 = b + 1; b2 < batch; ++b2) {
      const int pb = page_tables[(size_t)b * max_pages + positions[b] / kPage];
      const int pb2 = page_tables[(size_t)b2 * max_pages + positions[b2] / kPage];
      if (pb == pb2 && positions[b] % kPage == positions[b2] % kPage)
        return fail(W4_ERANGE, "sequences %d and %d write the same KV slot (page %d, slot %d)", b,
                    b2, pb, positions[b] % kPage);
    }
  return W4_OK;
}

static int validate_inputs(const w4_model* m, const int32_t* tokens, const int32_t* positions,
                           const int32_t* page_tables, const int32_t* ctx_lens, int batch) {
  return validate_step(m->cfg.vocab, m->num_pages, m->max_pages, tokens, positions, page_tables,
                       ctx_lens, batch);
}

// The pinned image of the staged-input region that the next copy uses,
// viewed as its four slots; waits until the image's previous copy has run,
// so the caller may overwrite it.
struct StageImage {
  int idx;
  uint8_t* base;
  int32_t *tokens, *positions, *ctx, *pt;
};
static int stage_image(w4_model* m, StageImage& im) {
  const WsLayout& L = m->L;
  im.idx = m->stage_next;
  W4_HIP(hipEventSynchronize(m->stage_ev[im.idx]));
  im.base = m->stage_img + (size_t)im.idx * m->stage_bytes;
  im.tokens = reinterpret_cast<int32_t*>(im.base);
  im.positions = reinterpret_cast<int32_t*>(im.base + (L.positions - L.tokens));
  im.ctx = reinterpret_cast<int32_t*>(im.base + (L.ctx - L.tokens));
  im.pt = reinterpret_cast<int32_t*>(im.base + (L.pt - L.tokens));
  return W4_OK;
}
// One copy of the image to the staged slots (from the tokens slot, or from
// the positions slot when the tokens are not staged), then the image's event.
static int stage_commit(w4_model* m, const StageImage& im, bool with_tokens, int batch, hipStream_t s) {
  const WsLayout& L = m->L;
  const size_t from = with_tokens ? 0 : L.positions - L.tokens;
  const size_t bytes = L.pt - L.tokens + (size_t)batch * m->max_pages * 4 - from;
  W4_HIP(hipMemcpyAsync(m->ws + L.tokens + from, im.base + from, bytes, hipMemcpyHostToDevice, s));
  W4_HIP(hipEventRecord(m->stage_ev[im.idx], s));
  m->stage_next = im.idx ^ 1;
  return W4_OK;
}

// Host arrays to the staged slots: one pinned copy, or, while the stream is
// being captured (a pinned copy would become a graph node that reads the
// image at every replay), the arrays copied one by one.
static int stage_inputs(w4_model* m, const int32_t* tokens, const int32_t* positions,
                        const int32_t* page_tables, const int32_t* ctx_lens, int batch,
                        hipStream_t s) {
  const WsLayout& L = m->L;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  W4_HIP(hipStreamIsCapturing(s, &cs));
  if (cs != hipStreamCaptureStatusNone) {
    if (tokens) W4_HIP(hipMemcpyAsync(m->ws + L.tokens, tokens, batch * 4, hipMemcpyHostToDevice, s));
    W4_HIP(hipMemcpyAsync(m->ws + L.positions, positions, batch * 4, hipMemcpyHostToDevice, s));
    W4_HIP(hipMemcpyAsync(m->ws + L.ctx, ctx_lens, batch * 4, hipMemcpyHostToDevice, s));
    W4_HIP(hipMemcpyAsync(m->ws + L.pt, page_tables, (size_t)batch * m->max_pages * 4,
                          hipMemcpyHostToDevice, s));
    return W4_OK;
  }
  StageImage im;
  int rc = stage_image(m, im);
  if (rc) return rc;
  if (tokens) std::memcpy(im.tokens, tokens, batch * 4);
  std::memcpy(im.positions, positions, batch * 4);
  std::memcpy(im.ctx, ctx_lens, batch * 4);
  std::memcpy(im.pt, page_tables, (size_t)batch * m->max_pages * 4);
  return stage_commit(m, im, tokens != nullptr, batch, s);
}

static StepInputs staged(w4_model* m) {
  return {m->at<int32_t>(m->L.tokens), m->at<int32_t>(m->L.positions), m->at<int32_t>(m->L.pt),
          m->at<int32_t>(m->L.ctx)};
}

// Runs the step eagerly or through a graph captured once per key.
static int run_step(w4_model* m, const StepInputs& in, int batch, uint16_t* logits,
                    hipStream_t s, const void* key_inputs) {
  if (!m->use_graph) return enqueue_step(m, in, batch, logits, s);
  w4_model::Key key(batch, logits, key_inputs ? in.tokens : nullptr,
                    key_inputs ? in.positions : nullptr, key_inputs ? in.page_tables : nullptr,
                    key_inputs ? in.ctx_lens : nullptr);
  auto it = m->graphs.find(key);
  if (it == m->graphs.end()) {
    hipGraph_t graph = nullptr;
    W4_HIP(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
    int rc = enqueue_step(m, in, batch, logits, m->cap_stream);
    hipError_t e = hipStreamEndCapture(m->cap_stream, &graph);
    if (rc) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return fail(W4_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(W4_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
    it = m->graphs.emplace(key, exec).first;
  }
  W4_HIP(hipGraphLaunch(it->second, s));
  return W4_OK;
}

static int check_model(const w4_model* m, int batch) {
  if (!handle_live(m)) return fail(W4_ESTATE, "null or destroyed model");
  if (batch < 1 || batch > m->max_batch)
    return fail(W4_EINVAL, "batch %d outside [1, %d]", batch, m->max_batch);
  return W4_OK;
}

}  // namespace w4

W4_EXPORT int w4_validate_step(const w4_config* cfg, int32_t num_pages, int32_t max_batch,
                               int32_t max_pages, const int32_t* tokens, const int32_t* positions,
                               const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch) {
  clear_error();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || batch > max_batch || max_pages < 1 || num_pages < 1)
    return fail(W4_EINVAL, "batch %d outside [1, %d] or max_pages=%d num_pages=%d", batch,
                max_batch, max_pages, num_pages);
  if (!positions || !page_tables || !ctx_lens) return fail(W4_EINVAL, "null input array");
  return validate_step(cfg->vocab, num_pages, max_pages, tokens, positions, page_tables, ctx_lens,
                       batch);
}

W4_EXPORT size_t w4_workspace_bytes(const w4_config* cfg, int32_t max_batch, int32_t max_pages) {
  if (check_config(cfg) || max_batch < 1 || max_batch > 16 || max_pages < 1) return 0;
  return ws_layout(*cfg, max_batch, max_pages).total;
}

W4_EXPORT int w4_model_create(const w4_config* cfg, const w4_weights* weights, void* kv_cache,
                              int32_t num_pages, void* workspace, size_t ws_bytes,
                              int32_t max_batch, int32_t max_pages, w4_model** out) {
  clear_error();
  if (!out || !weights || !weights->layers || !kv_cache || !workspace)
    return fail(W4_EINVAL, "w4_model_create: null pointer");
  int rc = check_config(cfg);
  if (rc) return rc;
  if (max_batch < 1 || max_batch > 16 || max_pages < 1 || num_pages < 1 || num_pages > (1 << 26) ||
      max_pages > (1 << 26))
    return fail(W4_EINVAL, "w4_model_create: max_batch=%d (1..16) max_pages=%d num_pages=%d (pages at most 2^26)",
                max_batch, max_pages, num_pages);
  const WsLayout L = ws_layout(*cfg, max_batch, max_pages);
  if (ws_bytes < L.total)
    return fail(W4_EINVAL, "w4_model_create: workspace %zu bytes < %zu", ws_bytes, L.total);
  if (!aligned256(kv_cache) || !aligned256(workspace))
    return fail(W4_EALIGN, "w4_model_create: kv_cache/workspace not 256-byte aligned");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const w4_layer_weights& W = weights->layers[l];
    const void* ptrs[] = {W.qkv, W.o, W.gate_up, W.down, W.attn_norm, W.mlp_norm};
    for (const void* p : ptrs) {
      if (!p) return fail(W4_EINVAL, "w4_model_create: layer %d has a null weight", l);
      if (!aligned256(p)) return fail(W4_EALIGN, "w4_model_create: layer %d weight not 256-byte aligned", l);
    }
    if (W.qkv_bias && !aligned256(W.qkv_bias))
      return fail(W4_EALIGN, "w4_model_create: layer %d qkv_bias not 256-byte aligned", l);
  }
  const void* top[] = {weights->embed, weights->final_norm, weights->lm_head};
  for (const void* p : top)
    if (p && !aligned256(p)) return fail(W4_EALIGN, "w4_model_create: embed/final_norm/lm_head not 256-byte aligned");

  auto* m = new w4_model;
  m->cfg = *cfg;
  m->layers.assign(weights->layers, weights->layers + cfg->n_layers);
  m->weights = *weights;
  m->weights.layers = nullptr;
  m->kv = static_cast<uint16_t*>(kv_cache);
  m->num_pages = num_pages;
  m->max_batch = max_batch;
  m->max_pages = max_pages;
  m->ws = static_cast<uint8_t*>(workspace);
  m->L = L;
  m->stage_bytes = round_up(L.pt - L.tokens + (size_t)max_batch * max_pages * 4, 256);
  hipError_t e = hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(m->ws), L.total / 4, 0u, m->cap_stream);
  if (e == hipSuccess) e = hipStreamSynchronize(m->cap_stream);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&m->stage_img), 2 * m->stage_bytes, 0);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&m->gen_tokens), (size_t)max_batch * 4, 0);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&m->stage_ev[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    release_model_resources(m);
    delete m;
    return fail(W4_EHIP, "w4_model_create: %s", hipGetErrorString(e));
  }
  handle_register(m);
  *out = m;
  return W4_OK;
}

W4_EXPORT void w4_model_destroy(w4_model* m) {
  if (!handle_release(m)) return;  // null, already destroyed or never created
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second);
  release_model_resources(m);
  delete m;
}

W4_EXPORT int w4_set_graph(w4_model* m, int enabled) {
  clear_error();
  if (!handle_live(m)) return fail(W4_ESTATE, "null or destroyed model");
  m->use_graph = enabled != 0;
  return W4_OK;
}

W4_EXPORT int decode_step(w4_model* m, const int32_t* tokens, const int32_t* positions,
                          const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                          uint16_t* logits, void* stream) {
  clear_error();
  int rc = check_model(m, batch);
  if (rc) return rc;
  if (!tokens || !positions || !page_tables || !ctx_lens || !logits)
    return fail(W4_EINVAL, "decode_step: null pointer");
  if (!m->weights.embed || !m->weights.lm_head || !m->weights.final_norm)
    return fail(W4_EINVAL, "decode_step: model has no embedding / final norm / lm_head");
  if (!aligned256(logits)) return fail(W4_EALIGN, "decode_step: logits not 256-byte aligned");
  rc = validate_inputs(m, tokens, positions, page_tables, ctx_lens, batch);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = stage_inputs(m, tokens, positions, page_tables, ctx_lens, batch, s);
  if (rc) return rc;
  return run_step(m, staged(m), batch, logits, s, nullptr);
}

W4_EXPORT int decode_step_device(w4_model* m, const int32_t* tokens, const int32_t* positions,
                                 const int32_t* page_tables, const int32_t* ctx_lens,
                                 int32_t batch, uint16_t* logits, void* stream) {
  clear_error();
  int rc = check_model(m, batch);
  if (rc) return rc;
  if (!tokens || !positions || !page_tables || !ctx_lens || !logits)
    return fail(W4_EINVAL, "decode_step_device: null pointer");
  if (!m->weights.embed || !m->weights.lm_head || !m->weights.final_norm)
    return fail(W4_EINVAL, "decode_step_device: model has no embedding / final norm / lm_head");
  const void* ptrs[] = {tokens, positions, page_tables, ctx_lens, logits};
  for (const void* p : ptrs)
    if (!aligned256(p)) return fail(W4_EALIGN, "decode_step_device: device pointer not 256-byte aligned");
  StepInputs in{tokens, positions, page_tables, ctx_lens};
  return run_step(m, in, batch, logits, static_cast<hipStream_t>(stream), tokens);
}

W4_EXPORT int64_t w4_device_errors(w4_model* m, void* stream) {
  clear_error();
  if (!handle_live(m)) return -1;
  uint32_t v = 0;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return -1;
  if (hipMemcpy(&v, m->ws + m->L.err, 4, hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return v;
}

W4_EXPORT int decode_layer(w4_model* m, int32_t layer, const uint16_t* x_in, uint16_t* x_out,
                           const int32_t* positions, const int32_t* page_tables,
                           const int32_t* ctx_lens, int32_t batch, void* stream) {
  clear_error();
  int rc = check_model(m, batch);
  if (rc) return rc;
  if (layer < 0 || layer >= m->cfg.n_layers)
    return fail(W4_EINVAL, "decode_layer: layer %d outside [0, %d)", layer, m->cfg.n_layers);
  if (!x_in || !x_out || !positions || !page_tables || !ctx_lens)
    return fail(W4_EINVAL, "decode_layer: null pointer");
  if (!aligned256(x_in) || !aligned256(x_out))
    return fail(W4_EALIGN, "decode_layer: x_in/x_out not 256-byte aligned");
  rc = validate_inputs(m, nullptr, positions, page_tables, ctx_lens, batch);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = stage_inputs(m, nullptr, positions, page_tables, ctx_lens, batch, s);
  if (rc) return rc;
  rc = enqueue_plan(m, nullptr, staged(m), batch, s);
  if (rc) return rc;
  return enqueue_layer(m, layer, x_in, x_out, staged(m), batch, s);
}

// ------------------------------------------------------- standalone kernels

W4_EXPORT int w4_gemv(const void* packed, const uint16_t* x, uint16_t* y, int32_t n, int32_t k,
                      int32_t batch, void* stream) {
  clear_error();
  if (!packed || !x || !y) return fail(W4_EINVAL, "w4_gemv: null pointer");
  if (n <= 0 || k <= 0 || k % 8 || batch < 1 || batch > (1 << 20))
    return fail(W4_EINVAL, "w4_gemv: n=%d k=%d (multiple of 8) batch=%d (1..2^20)", n, k, batch);
  if (!aligned256(packed) || !aligned256(x) || !aligned256(y))
    return fail(W4_EALIGN, "w4_gemv: pointer not 256-byte aligned");
  GemvArgs a = gemv_args(packed, n, k, x, k, nullptr, 0.f, y, n, nullptr, batch);
  if (batch > 16) {
    W4_LAUNCH(launch_w4_gemm_prefill(EPI_STORE, a, static_cast<hipStream_t>(stream)));
    return W4_OK;
  }
  W4_LAUNCH(launch_w4_gemv(EPI_STORE, a, static_cast<hipStream_t>(stream)));
  return W4_OK;
}

W4_EXPORT int w4_gemv_variant(const void* packed, const uint16_t* x, uint16_t* y, int32_t n, int32_t k,
                              int32_t batch, int32_t int8_activations, void* stream) {
  clear_error();
  if (!packed || !x || !y) return fail(W4_EINVAL, "w4_gemv_variant: null pointer");
  if (n <= 0 || k <= 0 || k % 8 || batch < 1 || batch > 16)
    return fail(W4_EINVAL, "w4_gemv_variant: n=%d k=%d (multiple of 8) batch=%d (1..16)", n, k, batch);
  if (!aligned256(packed) || !aligned256(x) || !aligned256(y))
    return fail(W4_EALIGN, "w4_gemv_variant: pointer not 256-byte aligned");
  const size_t lds = w4ax_lds_bytes(w4_groups(k), batch, int8_activations != 0);
  if (lds > (size_t)160 * 1024)
    return fail(W4_EINVAL, "w4_gemv_variant: %d rows of %d columns need %zu bytes of LDS (at most 160 KiB)", batch,
                k, lds);
  W4AxArgs a{};
  a.w = static_cast<const uint8_t*>(packed);
  a.n = n;
  a.k = k;
  a.tiles = w4_tiles(n);
  a.groups = w4_groups(k);
  a.x = x;
  a.x_stride = k;
  a.y = y;
  a.y_stride = n;
  a.batch = batch;
  W4_LAUNCH(launch_w4ax_gemv(a, int8_activations != 0, static_cast<hipStream_t>(stream)));
  return W4_OK;
}

W4_EXPORT int w4_gemv_f16(const void* packed, const uint16_t* x, uint16_t* y, int32_t n, int32_t k,
                          int32_t batch, void* stream) {
  clear_error();
  if (!packed || !x || !y) return fail(W4_EINVAL, "w4_gemv_f16: null pointer");
  if (n <= 0 || k <= 0 || k % 8 || batch < 1 || batch > 16)
    return fail(W4_EINVAL, "w4_gemv_f16: n=%d k=%d (multiple of 8) batch=%d (1..16)", n, k, batch);
  if (!aligned256(packed) || !aligned256(x) || !aligned256(y))
    return fail(W4_EALIGN, "w4_gemv_f16: pointer not 256-byte aligned");
  F16GemvArgs f{};
  f.w = static_cast<const uint8_t*>(packed);
  f.n = n;
  f.k = k;
  f.tiles = w4_tiles(n);
  f.cblocks = ceil_div(k, 32);
  f.x = x;
  f.x_stride = k;
  f.y = y;
  f.y_stride = n;
  f.batch = batch;
  W4_LAUNCH(launch_f16_gemv(f, static_cast<hipStream_t>(stream)));
  return W4_OK;
}

static size_t attn_ws_layout(int batch, int n_heads, int n_kv_heads, int head_dim, int max_pages,
                             size_t* partials_off, int* max_splits, int* pps) {
  *pps = attention_pages_per_split(batch, n_kv_heads, max_pages);
  *max_splits = ceil_div(max_pages, *pps);
  // counters [batch][Hkv] then one invalid-index counter
  const size_t counters = round_up((size_t)batch * n_kv_heads * 4 + 4, 256);
  *partials_off = counters;
  return counters + round_up(attention_partial_floats(batch, n_kv_heads, *max_splits,
                                                      n_heads / n_kv_heads, head_dim) * 4, 256);
}

W4_EXPORT size_t paged_attention_workspace_bytes(int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                                 int32_t head_dim, int32_t max_pages) {
  if (batch < 1 || n_kv_heads < 1 || n_heads < 1 || n_heads % n_kv_heads || max_pages < 1 ||
      !attention_supported(head_dim, n_heads / n_kv_heads))
    return 0;
  size_t off;
  int ms, pps;
  return attn_ws_layout(batch, n_heads, n_kv_heads, head_dim, max_pages, &off, &ms, &pps);
}

namespace w4 {
// The standalone attention call on a scratch region ws of ws_bytes (the
// caller's workspace, or the allocation-free entry point's device array):
// validation, the counter clear, the launch. `who` names the entry point in
// messages.
int attention_standalone(const char* who, const uint16_t* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t num_pages,
                         int32_t max_pages, void* workspace, size_t ws_bytes, uint16_t* out,
                         void* stream) {
  if (!q || !k_pool || !v_pool || !page_tables || !ctx_lens || !workspace || !out)
    return fail(W4_EINVAL, "%s: null pointer", who);
  const size_t need = paged_attention_workspace_bytes(batch, n_heads, n_kv_heads, head_dim, max_pages);
  if (need == 0 || num_pages < 1)
    return fail(W4_EINVAL, "%s: unsupported shape batch=%d heads=%d/%d head_dim=%d max_pages=%d num_pages=%d",
                who, batch, n_heads, n_kv_heads, head_dim, max_pages, num_pages);
  if (ws_bytes < need)
    return fail(W4_EINVAL, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
  const void* ptrs[] = {q, k_pool, v_pool, page_tables, ctx_lens, workspace, out};
  for (const void* p : ptrs)
    if (!aligned256(p)) return fail(W4_EALIGN, "%s: pointer not 256-byte aligned", who);
  size_t poff;
  int max_splits, pps;
  attn_ws_layout(batch, n_heads, n_kv_heads, head_dim, max_pages, &poff, &max_splits, &pps);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  // counters start at zero; a small fill kernel (no memset node) keeps the
  // call safe inside a caller's graph capture
  W4_LAUNCH(launch_fill_u32(reinterpret_cast<uint32_t*>(ws), (size_t)batch * n_kv_heads + 1, 0u, s));
  AttnArgs at{};
  at.q = q;
  at.q_stride = n_heads * head_dim;
  at.k_pool = static_cast<const uint16_t*>(k_pool);
  at.v_pool = static_cast<const uint16_t*>(v_pool);
  at.page_tables = page_tables;
  at.ctx_lens = ctx_lens;
  at.batch = batch;
  at.max_pages = max_pages;
  at.num_pages = num_pages;
  at.n_heads = n_heads;
  at.n_kv_heads = n_kv_heads;
  at.pages_per_split = pps;
  at.max_splits = max_splits;
  at.partials = reinterpret_cast<float*>(ws + poff);
  at.counters = reinterpret_cast<uint32_t*>(ws);
  at.out = out;
  at.out_stride = n_heads * head_dim;
  at.err = reinterpret_cast<uint32_t*>(ws) + (size_t)batch * n_kv_heads;
  W4_LAUNCH(launch_attention(at, head_dim, n_heads / n_kv_heads, s));
  return W4_OK;
}
}  // namespace w4

W4_EXPORT int paged_attention_decode(const uint16_t* q, const void* k_pool, const void* v_pool,
                                     const int32_t* page_tables, const int32_t* ctx_lens,
                                     int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t num_pages, int32_t max_pages,
                                     void* workspace, size_t ws_bytes, uint16_t* out,
                                     void* stream) {
  clear_error();
  return attention_standalone("paged_attention_decode", q, k_pool, v_pool, page_tables, ctx_lens, batch,
                              n_heads, n_kv_heads, head_dim, num_pages, max_pages, workspace, ws_bytes, out,
                              stream);
}

// ------------------------------------------------------ per-operation access

W4_EXPORT int w4_model_stage(w4_model* m, const int32_t* tokens, const int32_t* positions,
                             const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                             void* stream) {
  clear_error();
  int rc = check_model(m, batch);
  if (rc) return rc;
  if (!positions || !page_tables || !ctx_lens) return fail(W4_EINVAL, "w4_model_stage: null pointer");
  rc = validate_inputs(m, tokens, positions, page_tables, ctx_lens, batch);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = stage_inputs(m, tokens, positions, page_tables, ctx_lens, batch, s);
  if (rc) return rc;
  return enqueue_plan(m, nullptr, staged(m), batch, s);
}

W4_EXPORT int w4_model_run_op(w4_model* m, int32_t op, int32_t layer, int32_t batch,
                              uint16_t* logits, void* stream) {
  clear_error();
  int rc = check_model(m, batch);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* x = m->at<uint16_t>(m->L.x);
  if (op == W4_OP_EMBED) {
    if (!m->weights.embed) return fail(W4_EINVAL, "w4_model_run_op: model has no embedding");
    return enqueue_plan(m, staged(m).tokens, staged(m), batch, s);
  }
  if (op == W4_OP_LM_HEAD) {
    if (!m->weights.lm_head || !m->weights.final_norm || !logits)
      return fail(W4_EINVAL, "w4_model_run_op: no lm_head / final norm / logits");
    if (!aligned256(logits)) return fail(W4_EALIGN, "w4_model_run_op: logits not 256-byte aligned");
    return enqueue_lm_head(m, x, batch, logits, s);
  }
  if (layer < 0 || layer >= m->cfg.n_layers)
    return fail(W4_EINVAL, "w4_model_run_op: layer %d outside [0, %d)", layer, m->cfg.n_layers);
  return enqueue_op(m, op, layer, x, x, staged(m), batch, s);
}

W4_EXPORT void* w4_model_buffer(w4_model* m, int32_t which, int32_t* row_stride) {
  if (!handle_live(m)) return nullptr;
  const WsLayout& L = m->L;
  const w4_config& c = m->cfg;
  size_t off;
  int stride;
  switch (which) {
    case W4_BUF_X: off = L.x; stride = c.hidden; break;
    case W4_BUF_Q: off = L.q; stride = c.n_heads * c.head_dim; break;
    case W4_BUF_O: off = L.o; stride = L.o_stride; break;
    case W4_BUF_H: off = L.h; stride = L.h_stride; break;
    case W4_BUF_XN: off = L.xn; stride = L.xn_stride; break;
    default: return nullptr;
  }
  if (row_stride) *row_stride = stride;
  return m->ws + off;
}

// Greedy generation: the token loop of "Building a Custom LLM Inference
// Runtime on H100" (Architecture Overview: the orchestrator drives the decode
// step and feeds each chosen token back). Every step grows each sequence's
// pages through the pool when its new position starts a page ("The Three
// Critical Bugs", Bug 1: logical position -> physical page), builds the page
// table, runs the step and takes the argmax of the logits on the device,
// straight into the staged token slot that the next step's embedding reads.
// Positions, and so page growth, do not depend on the chosen tokens: step
// s + 1's positions, page table and context lengths are validated and staged
// while step s still runs, and the host waits once per step only for the
// chosen tokens (to stop on a row with no choice before running another step).
W4_EXPORT int w4_generate_greedy(w4_model* m, w4_kv_pool* pool, const int32_t* seqs,
                                 const int32_t* first_tokens, const int32_t* first_positions,
                                 int32_t batch, int32_t n_steps, uint16_t* logits,
                                 int32_t* next_tokens, int32_t* out_tokens, int32_t* steps_done,
                                 void* stream) {
  clear_error();
  if (steps_done) *steps_done = 0;
  int rc = check_model(m, batch);
  if (rc) return rc;
  if (!pool || !seqs || !first_tokens || !first_positions || !logits || !next_tokens ||
      (n_steps > 0 && !out_tokens))
    return fail(W4_EINVAL, "w4_generate_greedy: null pointer");
  if (n_steps < 0) return fail(W4_EINVAL, "w4_generate_greedy: n_steps %d < 0", n_steps);
  if (!m->weights.embed || !m->weights.lm_head || !m->weights.final_norm)
    return fail(W4_EINVAL, "w4_generate_greedy: model has no embedding / final norm / lm_head");
  if (!aligned256(next_tokens) || !aligned256(logits))
    return fail(W4_EALIGN, "w4_generate_greedy: next_tokens or logits not 256-byte aligned");
  const int64_t cap = (int64_t)m->max_pages * kPage;
  for (int b = 0; b < batch; ++b) {
    const int32_t p0 = first_positions[b];
    if (p0 < 0 || (int64_t)p0 + n_steps > cap)
      return fail(W4_ERANGE, "w4_generate_greedy: sequence %d positions [%d, %lld) outside [0, %lld)",
                  b, p0, (long long)p0 + n_steps, (long long)cap);
    if (first_tokens[b] < 0 || first_tokens[b] >= m->cfg.vocab)
      return fail(W4_ERANGE, "w4_generate_greedy: first token %d of sequence %d outside [0, %d)",
                  first_tokens[b], b, m->cfg.vocab);
    const int32_t have = kv_seq_pages(pool, seqs[b]);
    if (have < 0) return fail(W4_ERANGE, "w4_generate_greedy: sequence id %d not in the pool", seqs[b]);
    if ((int64_t)have * kPage < p0)
      return fail(W4_ERANGE, "w4_generate_greedy: sequence %d holds %d pages, fewer than its %d prior tokens need",
                  seqs[b], have, p0);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_steps == 0) return W4_OK;
  // Each step's positions, context lengths and page tables go to the device
  // as one copy from a pinned image (stage_image / stage_commit), and the
  // chosen tokens come back into pinned memory: one copy each way per step,
  // asynchronous (pageable copies were five per step).
  const WsLayout& L = m->L;
  std::vector<int32_t> pos(first_positions, first_positions + batch);
  // validates and stages the next step's inputs while the current step runs;
  // the tokens are already in the staged slot after the first step (the
  // device argmax writes them there)
  auto stage_step = [&](const int32_t* tokens) -> int {
    StageImage im;
    int r = stage_image(m, im);
    if (r) return r;
    for (int b = 0; b < batch; ++b) {
      im.positions[b] = pos[b];
      im.ctx[b] = pos[b] + 1;
      r = kv_seq_reserve(pool, seqs[b], im.ctx[b]);
      if (r) return r;
    }
    r = page_table(pool, seqs, batch, m->max_pages, im.pt);
    if (r) return r;
    r = validate_inputs(m, tokens, im.positions, im.pt, im.ctx, batch);
    if (r) return r;
    if (tokens) std::memcpy(im.tokens, tokens, batch * 4);
    return stage_commit(m, im, tokens != nullptr, batch, s);
  };
  int32_t* tok_dev = m->at<int32_t>(L.tokens);
  // next_tokens gets the last chosen tokens once, on every return after a step
  auto finish = [&](int ret) -> int {
    if (hipMemcpyAsync(next_tokens, tok_dev, batch * sizeof(int32_t), hipMemcpyDeviceToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return ret ? ret : fail(W4_EHIP, "w4_generate_greedy: copy of the last tokens");
    return ret;
  };
  rc = stage_step(first_tokens);
  if (rc) return rc;
  for (int step = 0; step < n_steps; ++step) {
    rc = run_step(m, staged(m), batch, logits, s, nullptr);
    if (rc) return rc;
    W4_HIP(launch_argmax_f16(logits, batch, m->cfg.vocab, m->ws + L.amax, tok_dev, s));
    W4_HIP(hipMemcpyAsync(m->gen_tokens, tok_dev, batch * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    // the next step's inputs are staged while this step runs (the host work
    // and the copy, which the stream orders after this step's reads)
    int stage_rc = W4_OK;
    if (step + 1 < n_steps) {
      for (int b = 0; b < batch; ++b) ++pos[b];
      stage_rc = stage_step(nullptr);
    }
    W4_HIP(hipStreamSynchronize(s));
    int32_t* row = out_tokens + (size_t)step * batch;
    std::memcpy(row, m->gen_tokens, batch * sizeof(int32_t));
    for (int b = 0; b < batch; ++b)
      if (row[b] < 0)
        return finish(fail(W4_ERANGE, "w4_generate_greedy: step %d, sequence %d: every logit is NaN", step, b));
    if (steps_done) *steps_done = step + 1;
    if (stage_rc) return finish(stage_rc);
  }
  return finish(W4_OK);
}

// ------------------------------------------------------------------ prefill
// A prompt through the model at once ("How to build your own LLM runtime from
// scratch", Key performance metrics: time to first token of a 512-token
// prompt): every prompt row gets the decode step's arithmetic at its own
// position (the projections as M-row GEMMs on the matrix cores, RMSNorm per
// row, causal attention over the pages), every row's K/V goes into the
// sequence's pages, and the last row's logits come out.

namespace w4 {

struct PfLayout {
  size_t err, tokens, positions, pt, slot, rope, x, xn, q, o, h, lmxn, kpart, kcount, total;
  size_t kcount_words;
  int xn_stride, o_stride, h_stride;
};

static PfLayout pf_layout(const w4_config& c, int max_tokens, int max_pages) {
  PfLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  const size_t n = (size_t)max_tokens;
  L.xn_stride = (int)round_up(c.hidden, kGroup);
  L.o_stride = (int)round_up((size_t)c.n_heads * c.head_dim, kGroup);
  L.h_stride = (int)round_up(c.ffn, kGroup);
  L.err = take(256);
  L.tokens = take(n * 4);
  L.positions = take(n * 4);
  L.pt = take((size_t)max_pages * 4);
  L.slot = take(n * 4);
  L.rope = take(n * (c.head_dim / 2) * 2 * 4);
  L.x = take(n * c.hidden * 2);
  L.xn = take(n * L.xn_stride * 2);
  L.q = take(n * c.n_heads * c.head_dim * 2);
  L.o = take(n * L.o_stride * 2);
  L.h = take(n * L.h_stride * 2);
  L.lmxn = take((size_t)L.xn_stride * 2);
  // the prefill GEMMs' split sums and counters (the largest any projection uses)
  const int qkv_rows = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int proj[4][2] = {{qkv_rows, c.hidden}, {c.hidden, c.n_heads * c.head_dim}, {2 * c.ffn, c.hidden},
                          {c.hidden, c.ffn}};
  size_t kf = 0, kc = 0;
  for (const auto& pr : proj) {
    kf = std::max(kf, pf_split_floats(max_tokens, pr[0], pr[1]));
    kc = std::max(kc, pf_split_counters(max_tokens, pr[0], pr[1]));
  }
  L.kpart = take(kf * 4);
  L.kcount_words = kc;
  L.kcount = take(kc * 4);
  L.total = off;
  return L;
}

static int enqueue_prefill(w4_model* m, int n, int start, uint8_t* ws, const PfLayout& L, uint16_t* logits,
                           hipStream_t s) {
  const w4_config& c = m->cfg;
  auto at = [&](size_t off) { return ws + off; };
  uint16_t* x = reinterpret_cast<uint16_t*>(at(L.x));
  uint16_t* xn = reinterpret_cast<uint16_t*>(at(L.xn));
  uint16_t* q = reinterpret_cast<uint16_t*>(at(L.q));
  uint16_t* o = reinterpret_cast<uint16_t*>(at(L.o));
  uint16_t* h = reinterpret_cast<uint16_t*>(at(L.h));
  uint32_t* err = reinterpret_cast<uint32_t*>(at(L.err));
  W4_LAUNCH(launch_fill_u32(err, 1, 0u, s));
  // split counters start at zero; every split GEMM leaves them at zero
  float* kpart = reinterpret_cast<float*>(at(L.kpart));
  uint32_t* kcount = reinterpret_cast<uint32_t*>(at(L.kcount));
  W4_LAUNCH(launch_fill_u32(kcount, L.kcount_words, 0u, s));
  auto split = [&](GemvArgs g) {
    g.kpart = kpart;
    g.kcount = kcount;
    return g;
  };
  TokenPlanArgs p{};
  p.tokens = reinterpret_cast<const int32_t*>(at(L.tokens));
  p.table = m->weights.embed;
  p.vocab = c.vocab;
  p.hidden = c.hidden;
  p.x = x;
  p.positions = reinterpret_cast<const int32_t*>(at(L.positions));
  p.page_tables = reinterpret_cast<const int32_t*>(at(L.pt));
  p.pt_stride = 0;  // every row reads the one sequence's page table
  p.max_pages = m->max_pages;
  p.num_pages = m->num_pages;
  p.head_dim = c.head_dim;
  p.rope_base = c.rope_base;
  p.slot = reinterpret_cast<int32_t*>(at(L.slot));
  p.rope = reinterpret_cast<float*>(at(L.rope));
  p.batch = n;
  p.err = err;
  W4_LAUNCH(launch_embed_plan(p, s));
  const int qkv_rows = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  for (int l = 0; l < c.n_layers; ++l) {
    const w4_layer_weights& W = m->layers[l];
    W4_LAUNCH(launch_rmsnorm_rows(x, c.hidden, W.attn_norm, c.rms_eps, c.hidden, xn, L.xn_stride, n, s));
    GemvArgs a = gemv_args(W.qkv, qkv_rows, c.hidden, xn, L.xn_stride, nullptr, 0.f, nullptr, 0, nullptr, n);
    a.qkv.q_out = q;
    a.qkv.q_stride = c.n_heads * c.head_dim;
    a.qkv.k_pool = m->k_pool(l);
    a.qkv.v_pool = m->v_pool(l);
    a.qkv.bias = W.qkv_bias;
    a.qkv.slot = p.slot;
    a.qkv.rope = p.rope;
    a.qkv.n_heads = c.n_heads;
    a.qkv.n_kv_heads = c.n_kv_heads;
    a.qkv.head_dim = c.head_dim;
    W4_LAUNCH(launch_w4_gemm_prefill(EPI_QKV, split(a), s));
    PrefillAttnArgs pa{};
    pa.q = q;
    pa.q_stride = c.n_heads * c.head_dim;
    pa.k_pool = m->k_pool(l);
    pa.v_pool = m->v_pool(l);
    pa.page_table = p.page_tables;
    pa.max_pages = m->max_pages;
    pa.num_pages = m->num_pages;
    pa.start = start;
    pa.n = n;
    pa.n_heads = c.n_heads;
    pa.n_kv_heads = c.n_kv_heads;
    pa.out = o;
    pa.out_stride = L.o_stride;
    pa.err = err;
    W4_LAUNCH(launch_prefill_attention(pa, c.head_dim, c.n_heads / c.n_kv_heads, s));
    W4_LAUNCH(launch_w4_gemm_prefill(EPI_RESID, split(gemv_args(W.o, c.hidden, c.n_heads * c.head_dim, o,
                                                                L.o_stride, nullptr, 0.f, x, c.hidden, x, n)),
                                     s));
    W4_LAUNCH(launch_rmsnorm_rows(x, c.hidden, W.mlp_norm, c.rms_eps, c.hidden, xn, L.xn_stride, n, s));
    W4_LAUNCH(launch_w4_gemm_prefill(EPI_SILU, split(gemv_args(W.gate_up, 2 * c.ffn, c.hidden, xn, L.xn_stride,
                                                               nullptr, 0.f, h, L.h_stride, nullptr, n)),
                                     s));
    W4_LAUNCH(launch_w4_gemm_prefill(EPI_RESID, split(gemv_args(W.down, c.hidden, c.ffn, h, L.h_stride, nullptr,
                                                                0.f, x, c.hidden, x, n)),
                                     s));
  }
  F16GemvArgs f{};
  f.w = static_cast<const uint8_t*>(m->weights.lm_head);
  f.n = c.vocab;
  f.k = c.hidden;
  f.tiles = w4_tiles(c.vocab);
  f.cblocks = ceil_div(c.hidden, 32);
  f.x = x + (size_t)(n - 1) * c.hidden;  // the last prompt row
  f.x_stride = c.hidden;
  f.gamma = m->weights.final_norm;
  f.eps = c.rms_eps;
  f.y = logits;
  f.y_stride = c.vocab;
  f.xn_out = reinterpret_cast<uint16_t*>(at(L.lmxn));
  f.batch = 1;
  W4_LAUNCH(launch_f16_gemv(f, s));
  return W4_OK;
}

}  // namespace w4

W4_EXPORT size_t w4_prefill_workspace_bytes(const w4_config* cfg, int32_t max_tokens, int32_t max_pages) {
  if (check_config(cfg) || max_tokens < 1 || max_pages < 1 || max_pages > (1 << 26) || max_tokens > (1 << 22))
    return 0;
  return pf_layout(*cfg, max_tokens, max_pages).total;
}

W4_EXPORT int w4_prefill(w4_model* m, const int32_t* tokens, int32_t n_tokens, int32_t start,
                         const int32_t* page_table, void* workspace, size_t ws_bytes, uint16_t* logits,
                         void* stream) {
  clear_error();
  int rc = check_model(m, 1);
  if (rc) return rc;
  if (!tokens || !page_table || !workspace || !logits) return fail(W4_EINVAL, "w4_prefill: null pointer");
  if (!m->weights.embed || !m->weights.lm_head || !m->weights.final_norm)
    return fail(W4_EINVAL, "w4_prefill: model has no embedding / final norm / lm_head");
  if (n_tokens < 1 || n_tokens > (1 << 22)) return fail(W4_EINVAL, "w4_prefill: n_tokens %d outside [1, 2^22]", n_tokens);
  if (start < 0 || (int64_t)start + n_tokens > (int64_t)m->max_pages * kPage)
    return fail(W4_ERANGE, "w4_prefill: positions [%d, %lld) outside [0, %lld)", start,
                (long long)start + n_tokens, (long long)m->max_pages * kPage);
  if (!aligned256(workspace) || !aligned256(logits))
    return fail(W4_EALIGN, "w4_prefill: workspace or logits not 256-byte aligned");
  const PfLayout L = pf_layout(m->cfg, n_tokens, m->max_pages);
  if (ws_bytes < L.total) return fail(W4_EINVAL, "w4_prefill: workspace %zu < %zu bytes", ws_bytes, L.total);
  for (int i = 0; i < n_tokens; ++i)
    if (tokens[i] < 0 || tokens[i] >= m->cfg.vocab)
      return fail(W4_ERANGE, "w4_prefill: tokens[%d] = %d outside [0, %d)", i, tokens[i], m->cfg.vocab);
  for (int pg = 0; pg < ceil_div(start + n_tokens, kPage); ++pg)
    if (page_table[pg] < 0 || page_table[pg] >= m->num_pages)
      return fail(W4_ERANGE, "w4_prefill: page_table[%d] = %d outside [0, %d)", pg, page_table[pg], m->num_pages);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  std::vector<int32_t> pos(n_tokens);
  for (int i = 0; i < n_tokens; ++i) pos[i] = start + i;
  W4_HIP(hipMemcpyAsync(ws + L.tokens, tokens, (size_t)n_tokens * 4, hipMemcpyHostToDevice, s));
  W4_HIP(hipMemcpyAsync(ws + L.positions, pos.data(), (size_t)n_tokens * 4, hipMemcpyHostToDevice, s));
  W4_HIP(hipMemcpyAsync(ws + L.pt, page_table, (size_t)m->max_pages * 4, hipMemcpyHostToDevice, s));
  // the staged arrays must be on the device before the host vector goes away
  W4_HIP(hipStreamSynchronize(s));
  return enqueue_prefill(m, n_tokens, start, ws, L, logits, s);
}

W4_EXPORT int64_t w4_prefill_buffer(const w4_config* cfg, int32_t n_tokens, int32_t max_pages, int32_t which,
                                    int32_t* row_stride) {
  if (check_config(cfg) || n_tokens < 1 || max_pages < 1 || n_tokens > (1 << 22) || max_pages > (1 << 26)) return -1;
  const PfLayout L = pf_layout(*cfg, n_tokens, max_pages);
  size_t off;
  int stride;
  switch (which) {
    case W4_BUF_X: off = L.x; stride = cfg->hidden; break;
    case W4_BUF_Q: off = L.q; stride = cfg->n_heads * cfg->head_dim; break;
    case W4_BUF_O: off = L.o; stride = L.o_stride; break;
    case W4_BUF_H: off = L.h; stride = L.h_stride; break;
    case W4_BUF_XN: off = L.xn; stride = L.xn_stride; break;
    default: return -1;
  }
  if (row_stride) *row_stride = stride;
  return (int64_t)off;
}

// ------------------------------------------------------------ KV page copies

static int kv_copy(const char* who, const w4_config* cfg, void* kv_cache, int32_t num_pages, int32_t layer,
                   const int32_t* page_table, int32_t max_pages, int32_t start, int32_t n_tokens, uint16_t* k,
                   uint16_t* v, bool to_pages, void* stream) {
  clear_error();
  if (!cfg || !kv_cache || !page_table || !k || !v) return fail(W4_EINVAL, "%s: null pointer", who);
  if (cfg->n_kv_heads < 1 || (cfg->head_dim != 64 && cfg->head_dim != 128) || cfg->n_layers < 1)
    return fail(W4_EINVAL, "%s: unsupported n_kv_heads %d / head_dim %d", who, cfg->n_kv_heads, cfg->head_dim);
  if (layer < 0 || layer >= cfg->n_layers || num_pages < 1 || max_pages < 1 || start < 0 || n_tokens < 0)
    return fail(W4_EINVAL, "%s: layer %d (of %d), num_pages %d, max_pages %d, start %d, n_tokens %d", who, layer,
                cfg->n_layers, num_pages, max_pages, start, n_tokens);
  if ((int64_t)start + n_tokens > (int64_t)max_pages * kPage)
    return fail(W4_ERANGE, "%s: positions [%d, %lld) past the page table's %d pages", who, start,
                (long long)start + n_tokens, max_pages);
  const void* ptrs[] = {kv_cache, page_table, k, v};
  for (const void* p : ptrs)
    if (!aligned256(p)) return fail(W4_EALIGN, "%s: pointer not 256-byte aligned", who);
  KvCopyArgs a{};
  const size_t layer_elems = (size_t)num_pages * cfg->n_kv_heads * kPage * cfg->head_dim;
  a.k_pool = static_cast<uint16_t*>(kv_cache) + (size_t)(2 * layer) * layer_elems;
  a.v_pool = a.k_pool + layer_elems;
  a.page_table = page_table;
  a.num_pages = num_pages;
  a.n_kv_heads = cfg->n_kv_heads;
  a.head_dim = cfg->head_dim;
  a.start = start;
  a.n = n_tokens;
  a.k = k;
  a.v = v;
  a.to_pages = to_pages ? 1 : 0;
  W4_LAUNCH(launch_kv_pages(a, static_cast<hipStream_t>(stream)));
  return W4_OK;
}

W4_EXPORT int kv_write_pages(const w4_config* cfg, void* kv_cache, int32_t num_pages, int32_t layer,
                             const int32_t* page_table, int32_t max_pages, int32_t start, int32_t n_tokens,
                             const uint16_t* k, const uint16_t* v, void* stream) {
  return kv_copy("kv_write_pages", cfg, kv_cache, num_pages, layer, page_table, max_pages, start, n_tokens,
                 const_cast<uint16_t*>(k), const_cast<uint16_t*>(v), true, stream);
}

W4_EXPORT int kv_read_pages(const w4_config* cfg, const void* kv_cache, int32_t num_pages, int32_t layer,
                            const int32_t* page_table, int32_t max_pages, int32_t start, int32_t n_tokens,
                            uint16_t* k, uint16_t* v, void* stream) {
  return kv_copy("kv_read_pages", cfg, const_cast<void*>(kv_cache), num_pages, layer, page_table, max_pages,
                 start, n_tokens, k, v, false, stream);
}
