// Host side of libw4a16 that needs no GPU: error state, the weight packers
// and the KV page pool.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_set>
#include <vector>

#include "w4_internal.h"

namespace w4 {

static thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

// Never destroyed: handles may be released from static destructors or
// interpreter shutdown after this file's statics would be gone.
static std::mutex& handles_mu() {
  static auto* m = new std::mutex;
  return *m;
}
static std::unordered_set<const void*>& handles() {
  static auto* s = new std::unordered_set<const void*>;
  return *s;
}
void handle_register(const void* h) {
  std::lock_guard<std::mutex> g(handles_mu());
  handles().insert(h);
}
bool handle_release(const void* h) {
  std::lock_guard<std::mutex> g(handles_mu());
  return handles().erase(h) > 0;
}
bool handle_live(const void* h) {
  if (!h) return false;
  std::lock_guard<std::mutex> g(handles_mu());
  return handles().count(h) > 0;
}

// Runs f(begin, end) over [0, n) on up to hardware_concurrency threads.
template <class F>
static void parallel_for(int n, F f) {
  int threads = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n < 64 || threads == 1) {
    f(0, n);
    return;
  }
  threads = std::min(threads, n);
  std::vector<std::thread> pool;
  int chunk = ceil_div(n, threads);
  for (int i = 0; i < threads; ++i) {
    int b = i * chunk, e = std::min(n, b + chunk);
    if (b < e) pool.emplace_back(f, b, e);
  }
  for (auto& t : pool) t.join();
}

// Logical row stored at each physical row for a packing role (-1 = padding).
static int physical_to_logical(int prow, int n, uint32_t role, int head_dim) {
  if (prow >= n) return -1;
  if (role == W4_ROLE_QKV) {
    const int head = prow / head_dim, r = prow % head_dim;
    const int p = r / 16, i = r % 16;
    const int dim = i < 8 ? 8 * p + i : head_dim / 2 + 8 * p + (i - 8);
    return head * head_dim + dim;
  }
  if (role == W4_ROLE_GATE_UP) {
    const int f = n / 2, t = prow / 16, i = prow % 16;
    return i < 8 ? 8 * t + i : f + 8 * t + (i - 8);
  }
  return prow;
}

// Bit position of input-column offset e (0..7) inside a packed 32-bit word:
// even offsets fill the low half-word, odd ones the high half-word, so that
// (word >> 4i) & 0x000F000F holds offsets 2i and 2i+1 in its two halves.
static inline int nibble_bit(int e) { return (e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1); }

}  // namespace w4

using namespace w4;

W4_EXPORT const char* w4_last_error(void) { return g_error.c_str(); }
W4_EXPORT const char* w4_version(void) { return "w4a16-paged-kv-amd 0.1 (gfx950)"; }

W4_EXPORT size_t w4_packed_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)w4_tiles(n) * w4_groups(k) * (1024 + 32);
}

// Symmetric group-wise INT4 quantisation ("How to build your own LLM runtime
// from scratch", "Architectural decisions and optimizations": symmetric
// group-wise INT4, group 128). Per (row, group of 128 input columns): the
// scale is the fp16 value nearest to max|w| / 7 and each code the integer in
// [-8, 7] nearest to w / s, halves to even (the default rounding mode of
// nearbyint); a zero scale gives zero codes. w and s are fp16 values, so
// their quotient is never within double rounding of a halfway point unless
// it is one: the double division decides every code exactly.
W4_EXPORT int quantize_w4g128(const uint16_t* w, int32_t n, int32_t k, int8_t* q,
                              uint16_t* scales) {
  clear_error();
  if (!w || !q || !scales) return fail(W4_EINVAL, "quantize_w4g128: null pointer");
  if (n <= 0 || k <= 0) return fail(W4_EINVAL, "quantize_w4g128: bad shape n=%d k=%d", n, k);
  const size_t total = (size_t)n * k;
  for (size_t i = 0; i < total; ++i)
    if ((w[i] & 0x7c00u) == 0x7c00u)
      return fail(W4_ERANGE, "quantize_w4g128: w[%zu] is not finite", i);
  const int G = w4_groups(k);
  parallel_for(n, [&](int r0, int r1) {
    for (int r = r0; r < r1; ++r) {
      for (int g = 0; g < G; ++g) {
        const int lo = g * kGroup, hi = std::min(k, lo + kGroup);
        const uint16_t* wr = w + (size_t)r * k;
        double m = 0.0;
        for (int j = lo; j < hi; ++j) m = std::max(m, std::fabs((double)__builtin_bit_cast(_Float16, wr[j])));
        const _Float16 s16 = (_Float16)(m / 7.0);   // correctly rounded double -> fp16
        scales[(size_t)r * G + g] = __builtin_bit_cast(uint16_t, s16);
        const double s = (double)s16;
        for (int j = lo; j < hi; ++j) {
          double c = 0.0;
          if (s > 0.0) c = std::nearbyint((double)__builtin_bit_cast(_Float16, wr[j]) / s);
          q[(size_t)r * k + j] = (int8_t)std::min(7.0, std::max(-8.0, c));
        }
      }
    }
  });
  return W4_OK;
}

W4_EXPORT int pack_weights_w4g128(const int8_t* q, const uint16_t* scales, int32_t n, int32_t k,
                                  uint32_t role, int32_t head_dim, void* out, size_t out_bytes) {
  clear_error();
  if (!q || !scales || !out) return fail(W4_EINVAL, "pack_weights_w4g128: null pointer");
  if (n <= 0 || k <= 0) return fail(W4_EINVAL, "pack_weights_w4g128: bad shape n=%d k=%d", n, k);
  if (out_bytes < w4_packed_bytes(n, k))
    return fail(W4_EINVAL, "pack_weights_w4g128: out_bytes %zu < %zu", out_bytes,
                w4_packed_bytes(n, k));
  if (role == W4_ROLE_QKV) {
    if (head_dim <= 0 || head_dim % 16 != 0 || n % head_dim != 0)
      return fail(W4_EINVAL, "pack_weights_w4g128: QKV role needs head_dim %% 16 == 0 dividing n "
                  "(n=%d head_dim=%d)", n, head_dim);
  } else if (role == W4_ROLE_GATE_UP) {
    if (n % 16 != 0)
      return fail(W4_EINVAL, "pack_weights_w4g128: GATE_UP role needs n = 2F with F %% 8 == 0 (n=%d)", n);
  } else if (role != W4_ROLE_PLAIN) {
    return fail(W4_EINVAL, "pack_weights_w4g128: unknown role %u", role);
  }
  const size_t total = (size_t)n * k;
  for (size_t i = 0; i < total; ++i)
    if (q[i] < -8 || q[i] > 7)
      return fail(W4_ERANGE, "pack_weights_w4g128: q[%zu] = %d outside [-8, 7]", i, (int)q[i]);

  const int T = w4_tiles(n), G = w4_groups(k);
  uint8_t* nib = static_cast<uint8_t*>(out);
  uint16_t* sc = reinterpret_cast<uint16_t*>(nib + (size_t)T * G * 1024);
  parallel_for(T, [&](int t0, int t1) {
    for (int t = t0; t < t1; ++t) {
      int lrow[16];
      for (int i = 0; i < 16; ++i) lrow[i] = physical_to_logical(16 * t + i, n, role, head_dim);
      for (int g = 0; g < G; ++g) {
        uint8_t* blk = nib + ((size_t)t * G + g) * 1024;
        for (int lane = 0; lane < 64; ++lane) {
          const int lr = lrow[lane & 15];
          const int c0 = 128 * g + 32 * (lane >> 4);
          for (int j = 0; j < 4; ++j) {
            uint32_t word = 0;
            for (int e = 0; e < 8; ++e) {
              const int col = c0 + 8 * j + e;
              const uint32_t u = (lr >= 0 && col < k) ? (uint32_t)(q[(size_t)lr * k + col] + 8) : 8u;
              word |= u << nibble_bit(e);
            }
            uint8_t* dst = blk + 16 * lane + 4 * j;
            dst[0] = word & 255; dst[1] = (word >> 8) & 255;
            dst[2] = (word >> 16) & 255; dst[3] = word >> 24;
          }
        }
        for (int i = 0; i < 16; ++i)
          sc[((size_t)t * G + g) * 16 + i] = lrow[i] >= 0 ? scales[(size_t)lrow[i] * G + g] : 0;
      }
    }
  });
  return W4_OK;
}

W4_EXPORT size_t w4_packed_f16_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0) return 0;
  return (size_t)w4_tiles(n) * ceil_div(k, 32) * 1024;
}

W4_EXPORT int pack_weights_f16(const uint16_t* w, int32_t n, int32_t k, void* out, size_t out_bytes) {
  clear_error();
  if (!w || !out) return fail(W4_EINVAL, "pack_weights_f16: null pointer");
  if (n <= 0 || k <= 0) return fail(W4_EINVAL, "pack_weights_f16: bad shape n=%d k=%d", n, k);
  if (out_bytes < w4_packed_f16_bytes(n, k))
    return fail(W4_EINVAL, "pack_weights_f16: out_bytes %zu < %zu", out_bytes,
                w4_packed_f16_bytes(n, k));
  const int T = w4_tiles(n), C = ceil_div(k, 32);
  uint16_t* o = static_cast<uint16_t*>(out);
  parallel_for(T, [&](int t0, int t1) {
    for (int t = t0; t < t1; ++t)
      for (int c = 0; c < C; ++c) {
        uint16_t* blk = o + ((size_t)t * C + c) * 512;
        for (int lane = 0; lane < 64; ++lane) {
          const int row = 16 * t + (lane & 15);
          const int col = 32 * c + 8 * (lane >> 4);
          for (int e = 0; e < 8; ++e)
            blk[8 * lane + e] = (row < n && col + e < k) ? w[(size_t)row * k + col + e] : 0;
        }
      }
  });
  return W4_OK;
}

// ------------------------------------------------------------- KV page pool

struct w4_kv_pool {
  int32_t num_pages = 0;
  std::vector<int32_t> free_list;        // stack of free page ids
  std::vector<int32_t> owner;            // per page: -2 free, -1 allocated, >= 0 sequence
  std::vector<std::vector<int32_t>> seqs;
};

static constexpr int32_t kFree = -2, kLoose = -1;

static bool pool_ok(const w4_kv_pool* p) { return handle_live(p); }

W4_EXPORT int kv_pool_create(int32_t num_pages, int32_t max_seqs, w4_kv_pool** out) {
  clear_error();
  if (!out) return fail(W4_EINVAL, "kv_pool_create: null out");
  if (num_pages <= 0 || max_seqs <= 0)
    return fail(W4_EINVAL, "kv_pool_create: num_pages=%d max_seqs=%d", num_pages, max_seqs);
  auto* p = new w4_kv_pool;
  p->num_pages = num_pages;
  p->free_list.resize(num_pages);
  // pop order: page 0 first
  for (int32_t i = 0; i < num_pages; ++i) p->free_list[i] = num_pages - 1 - i;
  p->owner.assign(num_pages, kFree);
  p->seqs.resize(max_seqs);
  handle_register(p);
  *out = p;
  return W4_OK;
}

W4_EXPORT void kv_pool_destroy(w4_kv_pool* p) {
  if (!handle_release(p)) return;  // null, already destroyed or never created
  delete p;
}

static int take_pages(w4_kv_pool* p, int32_t n, int32_t owner, int32_t* out_ids) {
  if ((int64_t)p->free_list.size() < n)
    return fail(W4_ENOPAGES, "KV pool exhausted: %d pages requested, %zu free", n,
                p->free_list.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = p->free_list.back();
    p->free_list.pop_back();
    p->owner[id] = owner;
    out_ids[i] = id;
  }
  return W4_OK;
}

W4_EXPORT int kv_alloc_pages(w4_kv_pool* p, int32_t n, int32_t* out_ids) {
  clear_error();
  if (!pool_ok(p)) return fail(W4_ESTATE, "kv_alloc_pages: invalid pool");
  if (n < 0 || (n > 0 && !out_ids)) return fail(W4_EINVAL, "kv_alloc_pages: n=%d", n);
  return take_pages(p, n, kLoose, out_ids);
}

W4_EXPORT int kv_free_pages(w4_kv_pool* p, const int32_t* ids, int32_t n) {
  clear_error();
  if (!pool_ok(p)) return fail(W4_ESTATE, "kv_free_pages: invalid pool");
  if (n < 0 || (n > 0 && !ids)) return fail(W4_EINVAL, "kv_free_pages: n=%d", n);
  std::vector<char> seen(p->num_pages, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= p->num_pages)
      return fail(W4_ERANGE, "kv_free_pages: page id %d outside [0, %d)", id, p->num_pages);
    if (p->owner[id] != kLoose || seen[id])
      return fail(W4_ESTATE, "kv_free_pages: page %d is %s", id,
                  seen[id] ? "listed twice" : p->owner[id] == kFree ? "already free"
                                                                    : "owned by a sequence");
    seen[id] = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    p->owner[ids[i]] = kFree;
    p->free_list.push_back(ids[i]);
  }
  return W4_OK;
}

W4_EXPORT int32_t kv_free_count(const w4_kv_pool* p) {
  return pool_ok(p) ? (int32_t)p->free_list.size() : -1;
}

W4_EXPORT int kv_seq_reserve(w4_kv_pool* p, int32_t seq, int32_t ctx_len) {
  clear_error();
  if (!pool_ok(p)) return fail(W4_ESTATE, "kv_seq_reserve: invalid pool");
  if (seq < 0 || seq >= (int32_t)p->seqs.size())
    return fail(W4_ERANGE, "kv_seq_reserve: sequence %d outside [0, %zu)", seq, p->seqs.size());
  if (ctx_len < 0) return fail(W4_ERANGE, "kv_seq_reserve: ctx_len %d < 0", ctx_len);
  auto& list = p->seqs[seq];
  const int32_t need = ceil_div(ctx_len, kPage) - (int32_t)list.size();
  if (need <= 0) return W4_OK;
  std::vector<int32_t> ids(need);
  int rc = take_pages(p, need, seq, ids.data());
  if (rc) return rc;
  list.insert(list.end(), ids.begin(), ids.end());
  return W4_OK;
}

W4_EXPORT int kv_seq_release(w4_kv_pool* p, int32_t seq) {
  clear_error();
  if (!pool_ok(p)) return fail(W4_ESTATE, "kv_seq_release: invalid pool");
  if (seq < 0 || seq >= (int32_t)p->seqs.size())
    return fail(W4_ERANGE, "kv_seq_release: sequence %d outside [0, %zu)", seq, p->seqs.size());
  for (int32_t id : p->seqs[seq]) {
    p->owner[id] = kFree;
    p->free_list.push_back(id);
  }
  p->seqs[seq].clear();
  return W4_OK;
}

W4_EXPORT int32_t kv_seq_pages(const w4_kv_pool* p, int32_t seq) {
  if (!pool_ok(p) || seq < 0 || seq >= (int32_t)p->seqs.size()) return -1;
  return (int32_t)p->seqs[seq].size();
}

W4_EXPORT int page_table(const w4_kv_pool* p, const int32_t* seqs, int32_t batch, int32_t max_pages,
                         int32_t* out) {
  clear_error();
  if (!pool_ok(p)) return fail(W4_ESTATE, "page_table: invalid pool");
  if (batch < 0 || max_pages <= 0 || (batch > 0 && (!seqs || !out)))
    return fail(W4_EINVAL, "page_table: batch=%d max_pages=%d", batch, max_pages);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t s = seqs[b];
    if (s < 0 || s >= (int32_t)p->seqs.size())
      return fail(W4_ERANGE, "page_table: sequence %d outside [0, %zu)", s, p->seqs.size());
    if ((int32_t)p->seqs[s].size() > max_pages)
      return fail(W4_ERANGE, "page_table: sequence %d holds %zu pages > max_pages %d", s,
                  p->seqs[s].size(), max_pages);
  }
  for (int32_t b = 0; b < batch; ++b) {
    const auto& list = p->seqs[seqs[b]];
    int32_t* row = out + (size_t)b * max_pages;
    std::fill(row, row + max_pages, -1);
    std::copy(list.begin(), list.end(), row);
  }
  return W4_OK;
}

W4_EXPORT size_t kv_cache_bytes(const w4_config* cfg, int32_t num_pages) {
  if (!cfg || num_pages <= 0 || cfg->n_layers <= 0 || cfg->n_kv_heads <= 0 || cfg->head_dim <= 0)
    return 0;
  return (size_t)2 * cfg->n_layers * num_pages * cfg->n_kv_heads * kPage * cfg->head_dim * 2;
}
