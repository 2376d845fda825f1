/*
 * w4a16.h -- C ABI of libw4a16: the single-token decode step of a GQA
 * transformer with weight-only INT4 projections (W4A16) and a paged fp16 KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources (page title, section):
 *   [RT-arch]  "How to build your own LLM runtime from scratch" (aikraft.ru
 *              digest of a Towards Data Science article), "Architectural
 *              decisions and optimizations": symmetric group-wise INT4
 *              weights, group 128; RMSNorm and lm_head kept in FP16; GQA 7:1;
 *              16-token KV pages, 4 KiB per head slice; INT4 GEMVs for the
 *              gate/up/down projections.
 *   [H100-kv]  "Building a Custom LLM Inference Runtime on H100", "The KV
 *              Cache and PagedAttention": the KV cache split into pages and
 *              managed like virtual memory, so sequences grow without
 *              fragmentation.
 *   [H100-bug] same page, "The Three Critical Bugs": Bug 1 (logical token
 *              position -> physical block mapping), Bug 2 (aligned
 *              intermediate buffers from a custom allocator), Bug 3 (no
 *              asynchronous copy may be pending inside a captured graph).
 *   [H100-graph] same page, "CUDA Graph Capture": the steady decode step is
 *              captured once and replayed as one operation.
 *   [H100-guide] same page, "Implementation Guide: Step-by-Step": KV cache
 *              and activation buffers are allocated up front; an orchestrator
 *              drives graph execution.
 *
 * Conventions
 *   - Every int-returning call returns W4_OK (0) or a W4_E* code; on error
 *     w4_last_error() gives a message (thread-local, valid until the next
 *     call on the same thread). No C++ exception crosses this boundary.
 *   - fp16 values travel as uint16_t holding IEEE binary16 bits.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP
 *     device memory (for example a torch tensor's data_ptr()). Every device
 *     pointer must be 256-byte aligned (W4_EALIGN otherwise).
 *   - The caller owns every buffer. The library owns only the opaque
 *     handles (w4_kv_pool, w4_model) and what a model keeps inside: the
 *     graphs it captures, a capture stream, two events and pinned host
 *     memory for staging host inputs (hipHostMalloc: two images of about
 *     max_batch * (3 + max_pages_per_seq) * 4 bytes each), all released by
 *     the matching *_destroy. The library never allocates device
 *     memory: its scratch lives in the caller's workspace.
 *   - Device work is enqueued asynchronously on the caller's HIP stream
 *     (`stream` is a hipStream_t; NULL means the default stream). Outputs are
 *     valid once that stream has been synchronised.
 *   - Validation failures return before any device work is enqueued and
 *     change nothing.
 *   - A model handle must be used by one thread at a time.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
enum {
  W4_OK = 0,
  W4_EINVAL = 1,    /* null pointer or unsupported shape / argument          */
  W4_ERANGE = 2,    /* a value out of its range (q, page id, token, ctx ...) */
  W4_EALIGN = 3,    /* device pointer not 256-byte aligned                   */
  W4_ENOPAGES = 4,  /* KV page pool exhausted                                */
  W4_EHIP = 5,      /* HIP runtime error; destroy the model afterwards       */
  W4_ESTATE = 6     /* double free, unknown sequence, destroyed handle ...   */
};

/* Message for the last failing call on this thread ("" if none). */
const char* w4_last_error(void);
/* Library version string. */
const char* w4_version(void);

/* ------------------------------------------------------------ weight packing
 * INT4 packed format ("w4g128"). The quantisation is symmetric and
 * group-wise with group 128 along the input dimension [RT-arch]: the weight
 * of output row n, input column k is q[n,k] * s[n, k/128], q in [-8, 7],
 * s fp16. The packer only re-lays (q, s); it never rounds or rescales.
 *
 * Row order. `role` permutes logical rows into physical rows so that the
 * fused epilogues find related rows inside one 16-row tile:
 *   W4_ROLE_PLAIN    identity.
 *   W4_ROLE_QKV      n = (Hq + 2 Hkv) * head_dim rows (q heads, k heads, v
 *                    heads, each head head_dim rows). Inside every head,
 *                    physical tile p (p = 0 .. head_dim/16 - 1) holds logical
 *                    head rows [8p, 8p+8) followed by [head_dim/2 + 8p,
 *                    head_dim/2 + 8p + 8): the rotate-half RoPE pairs.
 *                    head_dim must be a multiple of 16 and divide n.
 *   W4_ROLE_GATE_UP  n = 2F rows: gate rows [0, F) then up rows [F, 2F).
 *                    Physical tile t holds gate rows [8t, 8t+8) followed by
 *                    up rows [F + 8t, F + 8t + 8). F must be a multiple of 8.
 *
 * Layout, with T = ceil(n/16) tiles and G = ceil(k/128) groups:
 *   nibble section, T*G blocks of 1024 bytes; block (t, g) starts at byte
 *   (t*G + g)*1024. In a block, lane l = 0..63 owns bytes [16l, 16l+16):
 *   physical row 16t + (l & 15), input columns c0 = 128g + 32(l >> 4) + [0,32).
 *   Those 16 bytes are four little-endian 32-bit words; word j holds columns
 *   c0 + 8j + e, e = 0..7, each as u = q + 8 (offset binary, 0..15) in the
 *   nibble at bit 4*(e/2) for even e and at bit 16 + 4*((e-1)/2) for odd e.
 *   Columns >= k and rows >= n hold u = 8 (q = 0).
 *   scale section, at byte T*G*1024: fp16 [T][G][16]; entry (t, g, i) is the
 *   scale of physical row 16t + i for group g (0 for rows >= n).
 *   Total size: w4_packed_bytes(n, k) = T*G*1024 + T*G*32.
 * A 64-lane wavefront thus reads each block with one fully coalesced
 * 16-byte-per-lane load, and the lane data of a block is also the B operand
 * of four 16x16x32 fp16 MFMAs after nibble expansion.
 */
enum { W4_ROLE_PLAIN = 0, W4_ROLE_QKV = 1, W4_ROLE_GATE_UP = 2 };

size_t w4_packed_bytes(int32_t n, int32_t k);

/* Pack q (host int8 [n*k], row-major, every value in [-8, 7]) and scales
 * (host fp16 [n * ceil(k/128)], row-major) into `out` (host, out_bytes >=
 * w4_packed_bytes(n, k)). Pure and deterministic. W4_ERANGE if some q is
 * outside [-8, 7]; W4_EINVAL on bad shapes or a role/head_dim mismatch.
 * head_dim is read only for W4_ROLE_QKV. */
int pack_weights_w4g128(const int8_t* q, const uint16_t* scales, int32_t n, int32_t k,
                        uint32_t role, int32_t head_dim, void* out, size_t out_bytes);

/* Symmetric group-wise INT4 quantisation [RT-arch] (the step before
 * pack_weights_w4g128). w: host fp16 [n*k] row-major, every value finite;
 * q: host int8 [n*k]; scales: host fp16 [n * ceil(k/128)]. Per row and
 * group of 128 input columns (the last group partial): s = the fp16 value
 * nearest to max|w| / 7; q = the integer in [-8, 7] nearest to w / s, halves
 * to even (so |w - q s| <= s / 2, and +-max|w| maps to +-7); s = 0 gives
 * q = 0. Pure and deterministic. W4_ERANGE on a non-finite weight (nothing
 * written), W4_EINVAL on null pointers or bad shapes. */
int quantize_w4g128(const uint16_t* w, int32_t n, int32_t k, int8_t* q, uint16_t* scales);

/* Packed fp16 format (lm_head, kept in FP16 [RT-arch]): T = ceil(n/16)
 * tiles, C = ceil(k/32) column blocks; block (t, c) of 1024 bytes starts at
 * (t*C + c)*1024; lane l owns bytes [16l, 16l+16) = the 8 fp16 values of row
 * 16t + (l & 15), columns 32c + 8(l >> 4) + [0, 8). Zero padded. */
size_t w4_packed_f16_bytes(int32_t n, int32_t k);
int pack_weights_f16(const uint16_t* w, int32_t n, int32_t k, void* out, size_t out_bytes);

/* ------------------------------------------------------------- KV page pool
 * Host-side bookkeeping of a paged KV cache [H100-kv]: pages of 16 tokens
 * [RT-arch], O(1) allocation from a free list, per-sequence page lists, and
 * dense page tables for the device. Page ids index the device KV cache.
 */
typedef struct w4_kv_pool w4_kv_pool;

/* Handles (pools here, models below) are tracked while live: a call with a
 * destroyed handle returns W4_ESTATE (counters: -1) and touches nothing, and
 * destroying a handle twice, or NULL, does nothing. (An address the library
 * later hands out again to a new handle is that new handle.) */
int  kv_pool_create(int32_t num_pages, int32_t max_seqs, w4_kv_pool** out);
void kv_pool_destroy(w4_kv_pool* pool);
/* Allocate n pages into out_ids[n] (host). All or nothing: W4_ENOPAGES if
 * fewer than n are free, and then nothing is allocated. */
int  kv_alloc_pages(w4_kv_pool* pool, int32_t n, int32_t* out_ids);
/* Return pages. W4_ESTATE (and nothing freed) if any id is not currently
 * allocated, is owned by a sequence, or repeats; W4_ERANGE if out of range. */
int  kv_free_pages(w4_kv_pool* pool, const int32_t* ids, int32_t n);
int32_t kv_free_count(const w4_kv_pool* pool);
/* Grow sequence `seq` (0 <= seq < max_seqs) to hold ctx_len tokens, i.e.
 * ceil(ctx_len/16) pages, appending pages to its list. Never shrinks.
 * All or nothing (W4_ENOPAGES). */
int  kv_seq_reserve(w4_kv_pool* pool, int32_t seq, int32_t ctx_len);
/* Free every page of `seq`. */
int  kv_seq_release(w4_kv_pool* pool, int32_t seq);
/* Number of pages held by `seq` (-1 if seq is out of range). */
int32_t kv_seq_pages(const w4_kv_pool* pool, int32_t seq);
/* Dense page table (host int32 [batch * max_pages]): row b lists the pages
 * of seqs[b] in logical order -- logical token t of that sequence lives in
 * page row[t / 16], slot t % 16 [H100-bug, Bug 1] -- padded with -1.
 * W4_ERANGE if a sequence holds more than max_pages pages. */
int  page_table(const w4_kv_pool* pool, const int32_t* seqs, int32_t batch, int32_t max_pages,
                int32_t* out);

/* ------------------------------------------------------------------- model */
typedef struct w4_config {
  int32_t hidden;      /* H                                              */
  int32_t n_heads;     /* Hq query heads                                 */
  int32_t n_kv_heads;  /* Hkv; Hq / Hkv (the GQA group) must be 1..8     */
  int32_t head_dim;    /* D: 64 or 128                                   */
  int32_t ffn;         /* F, multiple of 8                               */
  int32_t vocab;       /* V (lm_head rows / embedding rows)              */
  int32_t n_layers;    /* L                                              */
  float   rms_eps;     /* RMSNorm epsilon                                */
  float   rope_base;   /* RoPE base (rotate-half convention)             */
} w4_config;

/* Device KV cache: fp16 [L][2][P][Hkv][16 * D] -- for layer l, K pages then V
 * pages, each page holding one 4 KiB (for D = 128) slice per KV head
 * [RT-arch]. A K slice holds value (token t, dim d) at element ((d / 32) * 64
 * + 16 ((d / 8) % 4) + t) * 8 + d % 8: eight consecutive dims of one token
 * are one 16-byte operand of the attention's scores on the matrix cores, and
 * the 64 operands of one 32-dim step are 1 KiB of contiguous memory. A V
 * slice holds value (token t, dim d) at element ((d / 32) * 64 + d % 16 + 16
 * (t / 4)) * 8 + ((d / 16) % 2) * 4 + t % 4: four consecutive tokens of one
 * dimension are one operand of the attention's P V product, and a lane's
 * operands of two neighbouring 16-dim slices are 16 contiguous bytes.
 * kv_write_pages / kv_read_pages convert from and to natural [token][D]
 * rows. */
size_t kv_cache_bytes(const w4_config* cfg, int32_t num_pages);

typedef struct w4_layer_weights {
  const void*     qkv;        /* device, packed role QKV, n = (Hq+2Hkv)D, k = H */
  const void*     o;          /* device, packed role PLAIN, n = H, k = Hq D      */
  const void*     gate_up;    /* device, packed role GATE_UP, n = 2F, k = H      */
  const void*     down;       /* device, packed role PLAIN, n = H, k = F         */
  const uint16_t* attn_norm;  /* device fp16 [H]                                 */
  const uint16_t* mlp_norm;   /* device fp16 [H]                                 */
  const uint16_t* qkv_bias;   /* device fp16 [(Hq+2Hkv)D] logical order, or NULL */
} w4_layer_weights;

typedef struct w4_weights {
  const w4_layer_weights* layers;  /* host array [L]                              */
  const uint16_t* embed;           /* device fp16 [V][H] row-major (NULL: layers only) */
  const uint16_t* final_norm;      /* device fp16 [H] (NULL: layers only)          */
  const void*     lm_head;         /* device, pack_weights_f16, n = V, k = H (NULL: layers only) */
} w4_weights;

typedef struct w4_model w4_model;

/* Bytes of device workspace a model needs for batches up to max_batch and
 * page tables of max_pages_per_seq columns [H100-guide]. */
size_t w4_workspace_bytes(const w4_config* cfg, int32_t max_batch, int32_t max_pages_per_seq);

/* Bind weights, KV cache and workspace (all caller-owned device memory; the
 * pointers are kept, not copied) into a model: the KV cache and activation
 * buffers are allocated once, up front, by the caller [H100-guide], and
 * every pointer must be 256-byte aligned ([H100-bug], Bug 2: misaligned
 * intermediate buffers). The model is the decoder of [RT-arch]: per layer
 * an RMSNorm, the INT4 qkv projection, GQA attention over the paged cache,
 * the INT4 o projection, a second RMSNorm and the INT4 gate/up/down
 * projections, then an FP16 RMSNorm and lm_head. Zero-fills the workspace
 * with a kernel on the default stream and waits for it. num_pages and
 * max_pages_per_seq are at most 2^26 (W4_EINVAL otherwise). W4_EHIP if the
 * HIP runtime fails (no handle is returned). */
int  w4_model_create(const w4_config* cfg, const w4_weights* weights, void* kv_cache,
                     int32_t num_pages, void* workspace, size_t ws_bytes, int32_t max_batch,
                     int32_t max_pages_per_seq, w4_model** out);
/* Releases the model's captured graphs and its handle (the caller's device
 * memory is untouched). NULL or an already destroyed model: no-op. */
void w4_model_destroy(w4_model* model);
/* 1: decode_step captures its kernel sequence into a hipGraph on first use
 * (per batch size and output/input pointers) and replays it afterwards
 * [H100-graph]; 0: launch kernel by kernel. Default 1. */
int  w4_set_graph(w4_model* model, int enabled);

/* One decode step for `batch` sequences. tokens, positions, ctx_lens: host
 * int32 [batch]; page_tables: host int32 [batch * max_pages_per_seq].
 * Contract: ctx_lens[b] counts the token being decoded and positions[b] ==
 * ctx_lens[b] - 1; its K/V are written to every layer's cache at page
 * page_tables[b][positions[b] / 16], slot positions[b] % 16, before
 * attention reads tokens [0, ctx_lens[b]). logits: device fp16 [batch][V].
 * The host arrays are validated (W4_ERANGE) and copied into the workspace on
 * `stream` before any kernel runs, never inside a captured graph [H100-bug,
 * Bug 3]: on return they have been read (the caller may reuse them); their
 * values reach the device as one copy from one of two pinned host images of
 * the model, the call first waiting for the copy made from that image two
 * calls earlier (so the host runs at most two calls ahead of those copies),
 * or, while `stream` is being captured, as four pageable copies. */
int  decode_step(w4_model* model, const int32_t* tokens, const int32_t* positions,
                 const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                 uint16_t* logits, void* stream);
/* Same step with tokens/positions/page_tables/ctx_lens already in device
 * memory (same layouts). They cannot be validated on the host: kernels clamp
 * every index so no access leaves its buffer, skip the K/V write of a
 * token whose page id is invalid, and count such events; read the count with
 * w4_device_errors. */
int  decode_step_device(w4_model* model, const int32_t* tokens, const int32_t* positions,
                        const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                        uint16_t* logits, void* stream);
/* The host validation decode_step and decode_layer run before enqueueing
 * anything (pure host function, no device access): batch in [1, max_batch];
 * tokens[b] in [0, vocab) (tokens may be NULL to skip); ctx_lens[b] in
 * [1, 16 max_pages]; positions[b] == ctx_lens[b] - 1; page_tables[b][p] in
 * [0, num_pages) for p < ceil(ctx_lens[b]/16); and no two sequences write the
 * same (page, slot). Returns W4_OK, W4_EINVAL or W4_ERANGE. */
int  w4_validate_step(const w4_config* cfg, int32_t num_pages, int32_t max_batch, int32_t max_pages,
                      const int32_t* tokens, const int32_t* positions, const int32_t* page_tables,
                      const int32_t* ctx_lens, int32_t batch);
/* Synchronises `stream` and returns the number of invalid indices seen by
 * kernels since model creation (0 when every input was valid), or -1. */
int64_t w4_device_errors(w4_model* model, void* stream);

/* One decoder layer (no embedding, no lm_head): x_out = layer(x_in), with the
 * KV write of every sequence -- the layer of [RT-arch] (FP16 RMSNorm, INT4
 * group-128 projections, GQA 7:1 attention over 16-token pages through the
 * page table [H100-kv]). x_in, x_out: device fp16 [batch][H] (may be the
 * same buffer). positions/page_tables/ctx_lens: host, validated and staged
 * as for decode_step (W4_ERANGE / W4_EINVAL / W4_EALIGN as there). */
int  decode_layer(w4_model* model, int32_t layer, const uint16_t* x_in, uint16_t* x_out,
                  const int32_t* positions, const int32_t* page_tables, const int32_t* ctx_lens,
                  int32_t batch, void* stream);

/* ----------------------------------------------------------------- prefill
 * A prompt through the model at once, before decoding ("How to build your
 * own LLM runtime from scratch", Key performance metrics: time to first
 * token of a 512-token prompt). Prompt token i sits at position start + i of
 * one sequence; every prompt row gets the decode step's arithmetic at its
 * position (FP16 RMSNorm per row, INT4 group-128 projections as M-row GEMMs
 * on the matrix cores, RoPE, causal GQA attention over positions [0, its
 * own] read through the page table [H100-kv], SiLU-gated MLP, residuals),
 * its K/V is written into every layer's cache at page page_table[p / 16],
 * slot p % 16 [H100-bug, Bug 1], and the logits of the last prompt token
 * (after the FP16 final RMSNorm and lm_head) come out: decode_step then
 * continues at position start + n_tokens. Positions below start must
 * already hold the sequence's K/V (prior context, or nothing when start = 0).
 *
 * tokens: host int32 [n_tokens], each in [0, vocab); page_table: host int32
 * [max_pages_per_seq of the model], entries p < ceil((start + n_tokens) / 16)
 * in [0, num_pages) (W4_ERANGE otherwise; start + n_tokens <= 16
 * max_pages_per_seq); workspace: device, caller-owned, >=
 * w4_prefill_workspace_bytes(cfg, n_tokens, max_pages_per_seq) (every
 * row's residual, normalised, query and attention-output rows, its F-wide
 * MLP row and RoPE table: 67 KB per token for the Qwen2.5-7B shape);
 * logits: device fp16 [vocab]. The inputs are staged into
 * the workspace and the host waits for that copy (the call then returns with
 * the kernels enqueued on `stream`); it runs eagerly (no graph). */
size_t w4_prefill_workspace_bytes(const w4_config* cfg, int32_t max_tokens, int32_t max_pages_per_seq);
int  w4_prefill(w4_model* model, const int32_t* tokens, int32_t n_tokens, int32_t start,
                const int32_t* page_table, void* workspace, size_t ws_bytes, uint16_t* logits, void* stream);
/* For tests and profiling: the byte offset in a prefill workspace (sized for
 * n_tokens and max_pages_per_seq) of the fp16 rows [n_tokens][*row_stride]
 * the last w4_prefill left there: W4_BUF_X the final residual rows,
 * W4_BUF_Q / W4_BUF_O the last layer's queries (after RoPE) and attention
 * outputs, W4_BUF_H its MLP rows, W4_BUF_XN its second RMSNorm output; -1 on
 * bad arguments. */
int64_t w4_prefill_buffer(const w4_config* cfg, int32_t n_tokens, int32_t max_pages_per_seq, int32_t which,
                          int32_t* row_stride);

/* Copies between natural-layout K/V rows and one layer of a KV cache laid out
 * as above (K slices in the score operand order, V slices in the P V operand
 * order), so callers
 * can fill pages from K/V computed elsewhere or read them back ([H100-kv]:
 * the cache is addressed through the page table). Token i of the call sits
 * at position start + i, in page page_table[(start + i) / 16], slot
 * (start + i) % 16. k, v: device fp16 [n_tokens][Hkv][D]; page_table: device
 * int32 [max_pages], start + n_tokens <= 16 max_pages (W4_ERANGE otherwise);
 * kv_cache: device, the model's [L][2][num_pages][Hkv][16 D] cache; only
 * cfg->n_layers, n_kv_heads and head_dim (64 or 128) are read.
 * Device-resident page ids are not validated on the host: a token whose
 * page id is outside [0, num_pages) is skipped (nothing read or written).
 * Asynchronous on `stream`; W4_EINVAL / W4_EALIGN on bad arguments. */
int  kv_write_pages(const w4_config* cfg, void* kv_cache, int32_t num_pages, int32_t layer,
                    const int32_t* page_table, int32_t max_pages, int32_t start, int32_t n_tokens,
                    const uint16_t* k, const uint16_t* v, void* stream);
int  kv_read_pages(const w4_config* cfg, const void* kv_cache, int32_t num_pages, int32_t layer,
                   const int32_t* page_table, int32_t max_pages, int32_t start, int32_t n_tokens, uint16_t* k,
                   uint16_t* v, void* stream);

/* ---------------------------------------------------- per-operation access
 * For tests and profiling: run the step one operation at a time on the
 * model's own residual buffer (W4_BUF_X), with inputs staged by
 * w4_model_stage (host arrays, validated as decode_step). The operations,
 * in step order, are the embedding gather, then per layer the five fused
 * kernels of decode_layer, then the final RMSNorm + lm_head:
 *   W4_OP_QKV      RMSNorm, qkv projection, RoPE, K/V write of the token
 *   W4_OP_ATTN     paged attention -> W4_BUF_O
 *   W4_OP_OPROJ    x += W_o o
 *   W4_OP_GATE_UP  RMSNorm, gate/up projection, SiLU(gate) * up -> W4_BUF_H
 *   W4_OP_DOWN     x += W_down h
 * W4_BUF_XN holds the fp16 RMSNorm output of the last QKV, GATE_UP or
 * LM_HEAD operation.
 * w4_model_buffer returns the device address of a workspace buffer (fp16
 * rows of *row_stride elements, one per sequence) or NULL. */
enum { W4_OP_EMBED = 0, W4_OP_QKV = 1, W4_OP_ATTN = 2, W4_OP_OPROJ = 3, W4_OP_GATE_UP = 4,
       W4_OP_DOWN = 5, W4_OP_LM_HEAD = 6 };
enum { W4_BUF_X = 0, W4_BUF_Q = 1, W4_BUF_O = 2, W4_BUF_H = 3, W4_BUF_XN = 4 };
int   w4_model_stage(w4_model* model, const int32_t* tokens, const int32_t* positions,
                     const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                     void* stream);
/* layer is ignored for W4_OP_EMBED / W4_OP_LM_HEAD; logits (device fp16
 * [batch][V]) is used by W4_OP_LM_HEAD only. */
int   w4_model_run_op(w4_model* model, int32_t op, int32_t layer, int32_t batch,
                      uint16_t* logits, void* stream);
void* w4_model_buffer(w4_model* model, int32_t which, int32_t* row_stride);

/* ------------------------------------------------------- standalone kernels */
/* y = fp16(W x) for a w4g128-packed W (role PLAIN rows in physical order),
 * fp32 accumulation. x: device fp16 [batch][k]; y: device fp16 [batch][n];
 * 1 <= batch <= 2^20: batches 1..16 run the decode kernels, larger ones the
 * prefill GEMM (the projections of w4_prefill). */
int  w4_gemv(const void* packed, const uint16_t* x, uint16_t* y, int32_t n, int32_t k,
             int32_t batch, void* stream);
/* The W4A8 variant and its same-decomposition W4A16 twin (measurement of
 * the pages' finding that INT8 activations lost to the INT4 unpack on
 * Hopper, "How to build your own LLM runtime from scratch", Architectural
 * decisions and optimizations). y = W x for a w4g128-packed W (role PLAIN)
 * with one wavefront per 16-row tile; int8_activations = 1: each row of x is
 * quantised to INT8 (s_x = max|x| / 127, x_q = round-half-even(x / s_x) in
 * float32, clamped to +-127) and multiplied on the INT8 matrix cores with
 * exact integer group sums, y = fp16(s_x sum_g s_g sum q x_q); 0: the W4A16
 * arithmetic of w4_gemv (fp16 activations, fp32 accumulation). x: device fp16
 * [batch][k]; y: device fp16 [batch][n]; 1 <= batch <= 16 and the staged rows
 * must fit the LDS ((batch + 1) * ceil(k / 128) * 128 bytes, twice that for
 * fp16, at most about 160 KiB: W4_EINVAL otherwise). */
int  w4_gemv_variant(const void* packed, const uint16_t* x, uint16_t* y, int32_t n, int32_t k,
                     int32_t batch, int32_t int8_activations, void* stream);
/* y = fp16(W x) for a pack_weights_f16 W, fp32 accumulation, batch 1..16. */
int  w4_gemv_f16(const void* packed, const uint16_t* x, uint16_t* y, int32_t n, int32_t k,
                 int32_t batch, void* stream);

/* Paged-attention decode [H100-kv]: for each sequence b and query head h,
 * out[b][h] = fp16(sum_t softmax_t(q[b][h] . K_t / sqrt(D)) V_t) over tokens
 * t in [0, ctx_lens[b]), K_t/V_t read from KV head h / (Hq/Hkv) through the
 * page table. q: device fp16 [batch][Hq][D]; k_pool, v_pool: device fp16
 * [num_pages][Hkv][16 * D] (the KV cache's K and V slice layouts above);
 * page_tables: device int32 [batch][max_pages];
 * ctx_lens: device int32 [batch]; out: device fp16 [batch][Hq][D].
 * Device-resident indices are clamped like decode_step_device: a page id
 * outside [0, num_pages) contributes nothing, ctx_lens are clamped to
 * [0, 16 max_pages], and an empty context yields zeros. workspace: device,
 * >= paged_attention_workspace_bytes(...) (split partials and counters). */
size_t paged_attention_workspace_bytes(int32_t batch, int32_t n_heads, int32_t n_kv_heads,
                                       int32_t head_dim, int32_t max_pages);
int  paged_attention_decode(const uint16_t* q, const void* k_pool, const void* v_pool,
                            const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                            int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                            int32_t num_pages, int32_t max_pages, void* workspace,
                            size_t ws_bytes, uint16_t* out, void* stream);
/* paged_attention_decode for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and results, with no workspace argument. The
 * split partials, arrival counters and error count live in a device array
 * the library holds on each GPU it runs on, for the life of the process, of
 * paged_attention_noalloc_max_bytes() = 16 MiB; a call that needs more
 * (paged_attention_workspace_bytes(...) above that) fails with W4_EINVAL
 * before any device work. Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call. The counters are cleared by a fill kernel on
 * `stream` before each launch; the array keeps the last call's contents.
 * Every call on one GPU shares that GPU's array, so calls that overlap on
 * one GPU (other streams, other threads) race: serialise them. Other
 * arguments, layouts and errors as paged_attention_decode. */
size_t paged_attention_noalloc_max_bytes(void);
int  paged_attention_decode_noalloc(const uint16_t* q, const void* k_pool, const void* v_pool,
                                    const int32_t* page_tables, const int32_t* ctx_lens, int32_t batch,
                                    int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t num_pages, int32_t max_pages, uint16_t* out, void* stream);

/* ------------------------------------------------------ greedy generation
 * The token loop around the decode step ("Building a Custom LLM Inference
 * Runtime on H100", Architecture Overview: the orchestrator runs the
 * tokenization loop and feeds each chosen token back).
 *
 * w4_argmax_f16: out[b] = the index of the largest of logits[b][0..vocab),
 * the lowest index among equal maxima; values compare exactly (fp16 widened
 * to fp32); NaN is never chosen and a row of NaNs yields -1. logits: device
 * fp16 [batch][vocab]; out: device int32 [batch]; 1 <= batch <= 65535.
 * workspace: device, >= w4_argmax_workspace_bytes(batch, vocab) (per-chunk
 * partials; at most 512 bytes per row), caller-owned. Asynchronous on
 * `stream`; W4_EINVAL on a null pointer, a bad size or a short workspace,
 * W4_EALIGN if logits, workspace or out is not 256-byte aligned (rows of an
 * odd vocab start unaligned inside the buffer; that is handled). */
size_t w4_argmax_workspace_bytes(int32_t batch, int32_t vocab);   /* 0 on bad sizes */
int  w4_argmax_f16(const uint16_t* logits, int32_t batch, int32_t vocab, void* workspace,
                   size_t ws_bytes, int32_t* out, void* stream);
/* n_steps greedy decode steps for `batch` sequences of `pool` (whose page ids
 * index the model's KV cache). Sequence b (pool id seqs[b]) starts with token
 * first_tokens[b] at position first_positions[b]; its prior tokens
 * [0, first_positions[b]) must already be in the KV cache at the pages the
 * pool holds for it (W4_ERANGE otherwise), and first_positions[b] + n_steps
 * <= 16 * max_pages_per_seq. Step s decodes position p = first_positions[b]
 * + s with ctx_len p + 1: kv_seq_reserve grows the sequence by one page
 * whenever p starts a new page (W4_ENOPAGES when the pool is empty),
 * page_table rebuilds the table, and the step runs as decode_step would
 * (graph or eager as set by w4_set_graph); the w4_argmax_f16 kernels
 * (partials in the model's workspace) write each sequence's next token into
 * the model's staged token slot, which step s + 1 reads, and the host
 * copies it to out_tokens[s][b] (host int32 [n_steps][batch]) and to
 * next_tokens (device int32 [batch], 256-byte aligned, caller-owned: the
 * last chosen tokens on return). Step s + 1's positions and page table are
 * staged while step s runs; the host waits once per step for the chosen
 * tokens and stops with W4_ERANGE on a row with no non-NaN logit, before
 * running another step. logits: device fp16 [batch][vocab], 256-byte
 * aligned, holding the last step's logits on return. On an error,
 * *steps_done (optional) counts the steps whose tokens are in out_tokens;
 * pages already reserved stay with their sequences. */
int  w4_generate_greedy(w4_model* model, w4_kv_pool* pool, const int32_t* seqs,
                        const int32_t* first_tokens, const int32_t* first_positions,
                        int32_t batch, int32_t n_steps, uint16_t* logits, int32_t* next_tokens,
                        int32_t* out_tokens, int32_t* steps_done, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
