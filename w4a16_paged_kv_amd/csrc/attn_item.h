// Paged-attention decode as device code (one work item on one workgroup).
//
// The KV cache is split into 16-token pages addressed through a page table
// ("Building a Custom LLM Inference Runtime on H100", The KV Cache and
// PagedAttention; "How to build your own LLM runtime from scratch",
// Architectural decisions and optimizations: 16-token pages, 4 KiB per head
// slice, GQA 7:1). Logical token t of sequence b lives in page
// page_tables[b][t / 16], slot t % 16 (same page, The Three Critical Bugs,
// Bug 1).
//
// A work item is (split of consecutive pages, KV head, sequence). Each of
// eight wavefronts streams whole pages: one (page, KV head) K slice and V
// slice is read from HBM once and used for all GQ query heads of the group.
// Softmax is online, in fp32 and base 2. The item writes its un-normalised
// (o, m, l) partial; the last item of a (sequence, KV head) to finish merges
// all partials with a log-sum-exp reduction and writes fp16 o. Every barrier
// sits in uniform control flow (the same page's Bug list warns against
// barriers inside divergent branches).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "gemv_b1.h"

namespace w4 {

constexpr float kLog2e = 1.4426950408889634f;

constexpr int kAttnWaves = 8;  // wavefronts per workgroup, one page at a time each
constexpr int kPolicyNt = 2;    // buffer instruction cache-policy operand: nt (non-temporal)


// One work item (split of pages, KV head, sequence) on one workgroup of NT
// threads. The first kAttnWaves wavefronts stream pages; any further
// wavefronts only take part in the cooperative loops and the barriers, so
// every barrier stays in workgroup-uniform control flow (the item decides
// every early return). Queries and K/V are read coherently (they may have
// been written earlier in the same launch), outputs and partials are stored
// coherently.
// PF: keep the next page's K/V in flight while the current page is processed
// (two K/V register sets; without it the kernel fits a 1024-thread launch).
// EARLY: issue the wavefront's first page before the queries are staged
// (items of several pages per wavefront: their first pages then overlap the
// query staging; with one page per wavefront the queries are better first).
// NTL: read K/V with non-temporal loads (chosen by the launcher).
template <int D, int GQ, int NT, bool EARLY, bool NTL = false, bool PF = true>
__device__ void attn_item(const AttnArgs& a, int split, int kvh, int b) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(GQ >= 1 && GQ <= 8, "group");
  static_assert(NT >= kAttnWaves * 64 && NT % 64 == 0, "threads");
  constexpr int W = kAttnWaves;
  constexpr int NS = D / 16;          // 16-column slices of the P V product
  __shared__ float s_m[W][8], s_l[W][8];
  __shared__ __align__(16) float s_o[W][GQ][D];
  __shared__ __align__(16) uint16_t s_q[GQ * D];     // the group's query heads
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool pager = wave < W;  // this wavefront streams pages
  // The page table and context lengths are read-only here: read through the
  // constant address space they are scalar loads, so fetching the next page's
  // id does not wait behind the K/V loads in flight (with a vector load it
  // did, and a wavefront then had one page in flight at a time).
  typedef const __attribute__((address_space(4))) int32_t* cptr_t;
  const cptr_t pt = (cptr_t)(a.page_tables + (size_t)b * a.max_pages);
  // the context length, this wavefront's first two page ids and the queries
  // are independent: issue them together (page ids are validated below)
  const int pw0 = split * a.pages_per_split + wave;
  int pid_cur = pt[min(pw0, a.max_pages - 1)];
  int pid_nxt = pt[min(pw0 + W, a.max_pages - 1)];
  int ctx = ((cptr_t)a.ctx_lens)[b];
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(a.q + (size_t)b * a.q_stride + (size_t)kvh * GQ * D);
  u4_t qv[(GQ * D + NT * 8 - 1) / (NT * 8)];
#pragma unroll
  for (int r = 0; r < (GQ * D + NT * 8 - 1) / (NT * 8); ++r) {
    const int i = min((int)(threadIdx.x + r * NT) * 8, GQ * D - 8);
    qv[r] = ld128(rq, 2 * i);
  }
  ctx = ctx < 0 ? 0 : (ctx > a.max_pages * kPage ? a.max_pages * kPage : ctx);
  const int npages = (ctx + kPage - 1) / kPage;
  const int nsplit = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(npages, p_begin + a.pages_per_split);
  const int p_stop = pager ? p_end : pw0;  // non-page wavefronts skip the loop
  const size_t slice = (size_t)kPage * D;  // elements per (page, kv head)
  constexpr int NK = D / 32;               // MFMA k-steps per page
  const int lane_ = threadIdx.x & 63;
  // page p's id, validated (an invalid id is counted and read as page 0,
  // with no valid tokens)
  auto checked = [&](int p, int id, int& valid) {
    const bool bad = id < 0 || id >= a.num_pages;
    if (bad && lane_ == 0) atomicAdd(a.err, 1u);
    valid = bad ? 0 : min(kPage, ctx - p * kPage);
    return bad ? 0 : id;
  };
  u4_t kf[NK], kn[PF ? NK : 1];
  u4_t vf[NS / 2], vn[PF ? NS / 2 : 1];  // V operands of slice pairs (2i, 2i + 1)
  auto ld_kv = [](__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NTL ? kPolicyNt : 0));
  };
  auto load_kv = [&](int page, u4_t* kk, u4_t* vv) {
    page = __builtin_amdgcn_readfirstlane(page);  // one page per wavefront: keeps the resources scalar
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(a.k_pool + ((size_t)page * a.n_kv_heads + kvh) * slice);
    const __amdgpu_buffer_rsrc_t rv = buf_rsrc(a.v_pool + ((size_t)page * a.n_kv_heads + kvh) * slice);
#pragma unroll
    for (int i = 0; i < NK; ++i) kk[i] = ld_kv(rk, 16 * (64 * i + lane_));  // K slice in score operand order
#pragma unroll
    for (int i = 0; i < NS / 2; ++i) vv[i] = ld_kv(rv, 16 * (64 * i + lane_));
  };
  int valid_cur = 0, valid_nxt = 0;
  // (a split past the context has pw0 >= p_stop: no load, no id check)
  if (EARLY && pw0 < p_stop) load_kv(checked(pw0, pid_cur, valid_cur), kf, vf);
  uint16_t* out = a.out + (size_t)b * a.out_stride + (size_t)kvh * GQ * D;
  if (npages == 0) {  // empty context: zeros
    if (split == 0)
      for (int i = threadIdx.x; i < GQ * D; i += NT) st16_agent(out + i, 0);
    return;
  }
  if (split >= nsplit) return;

  // Scores on the matrix cores: S^T = K q^T with v_mfma_f32_16x16x32_f16, A =
  // the page's K (lane l: token l & 15, columns 32 kk + 8 (l >> 4) .. +8; the
  // K slice stores each step's 64 operands contiguously, k_slice_offset), B =
  // the group's queries (lane l: head l & 15, same columns; heads past GQ are
  // zero), so lane l ends with S[token 4 (l >> 4) + j][head l & 15], j < 4.
  // The queries pass through LDS once into that operand layout.
#pragma unroll
  for (int r = 0; r < (GQ * D + NT * 8 - 1) / (NT * 8); ++r) {
    const int i = (int)(threadIdx.x + r * NT) * 8;
    if (i < GQ * D) *reinterpret_cast<u4_t*>(&s_q[i]) = qv[r];
  }
  __syncthreads();
  const int qh = lane & 15, kc = 8 * (lane >> 4);
  const int qrow = min(qh, GQ - 1);        // heads past GQ read a real row and are zeroed

  const float scale = kLog2e / sqrtf((float)D);
  // P V on the matrix cores too: O^T = V^T P with v_mfma_f32_16x16x16_f16,
  // A = a 16-column slice of V^T (lane l: column 16 s + (l & 15), tokens
  // 4 (l >> 4) .. +4; the V page keeps them, for slices 2i and 2i + 1, in
  // 16 contiguous bytes per lane: v_slice_offset), B = P, which
  // the score step already left in B-operand order (lane l holds tokens
  // 4 (l >> 4) + j of head l & 15); lane l accumulates
  // O[head l & 15][16 s + 4 (l >> 4) + j], so each lane rescales only its
  // own head's values.
  float m_h = -INFINITY, l_h = 0.f;        // softmax state of head qh
  f4_t acc[NS];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) acc[sl] = (f4_t){0.f, 0.f, 0.f, 0.f};
  const int tk = 4 * (lane >> 4);          // this lane's tokens in the P V operands
  if (!EARLY && pw0 < p_stop) load_kv(checked(pw0, pid_cur, valid_cur), kf, vf);
  for (int p = pw0; p < p_stop; p += W) {
    const int valid = valid_cur;
    if (PF && p + W < p_stop) {
      load_kv(checked(p + W, pid_nxt, valid_nxt), kn, vn);
      pid_nxt = pt[min(p + 2 * W, a.max_pages - 1)];  // the page after, one step ahead
    }

    f4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      // the query operand is re-read from LDS per page (registers stay free)
      u4_t qb = *reinterpret_cast<const u4_t*>(&s_q[qrow * D + 32 * kk + kc]);
      if (qh >= GQ) qb = (u4_t){0u, 0u, 0u, 0u};
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, kf[kk]), __builtin_bit_cast(h8_t, qb), sc,
                                                  0, 0, 0);
    }
    // tokens past the context (and their NaN-poisoned slots) score -inf
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = 4 * (lane >> 4) + j < valid ? sc[j] * scale : -INFINITY;
    // page maximum and sum per head: four tokens in the lane, then the rows
    const float pm = rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const float n_h = fmaxf(m_h, pm);
    const float al = n_h == -INFINITY ? 1.f : exp2f(m_h - n_h);
    // the fp32 weights enter the product as two fp16 terms (hi + lo: about
    // 22 significant bits), so P V keeps fp32 accuracy on the fp16 MFMA
    float pj[4];
    h4_t ph, pl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pj[j] = n_h == -INFINITY ? 0.f : exp2f(sv[j] - n_h);
      ph[j] = (_Float16)pj[j];
      pl[j] = (_Float16)(pj[j] - (float)ph[j]);
    }
    l_h = l_h * al + rows_sum((pj[0] + pj[1]) + (pj[2] + pj[3]));
    m_h = n_h;

    // masked tokens contribute nothing even if their slots hold NaN
    if (valid < kPage) {
#pragma unroll
      for (int i = 0; i < NS / 2; ++i) {
        h8_t v8 = __builtin_bit_cast(h8_t, vf[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (tk + (j & 3) >= valid) v8[j] = (_Float16)0.f;
        vf[i] = __builtin_bit_cast(u4_t, v8);
      }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const u4_t vp = vf[i >> 1];
      const h4_t v4 = __builtin_bit_cast(h4_t, (i & 1) ? (u2_t){vp[2], vp[3]} : (u2_t){vp[0], vp[1]});
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v4, ph, acc[i] * al, 0, 0, 0);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x16f16(v4, pl, acc[i], 0, 0, 0);
    }
    if (PF) {
#pragma unroll
      for (int i = 0; i < NK; ++i) kf[i] = kn[PF ? i : 0];
#pragma unroll
      for (int i = 0; i < NS / 2; ++i) vf[i] = vn[PF ? i : 0];
      valid_cur = valid_nxt;
    } else if (p + W < p_stop) {
      load_kv(checked(p + W, pid_nxt, valid_cur), kf, vf);
      pid_nxt = pt[min(p + 2 * W, a.max_pages - 1)];
    }
  }
  if (pager && lane < 8) {
    s_m[wave][lane] = m_h;
    s_l[wave][lane] = l_h;
  }
  if (pager && qh < GQ)
#pragma unroll
    for (int i = 0; i < NS; ++i) *reinterpret_cast<f4_t*>(&s_o[wave][qh][16 * i + tk]) = acc[i];
  __syncthreads();

  // combine the wavefronts: this split's (o, m, l), or the output if one
  // split. Thread g < GQ D / 4 takes four consecutive dims of one head and
  // stores them with one 16-byte (partial) or 8-byte (output) store.
  constexpr int PS = D + 4;      // floats per (split, head) partial: o[D], m, l, 2 unused (16-byte rows)
  constexpr int NG = GQ * D / 4;  // four-dim groups of the item's output
  float* part = a.partials + (((size_t)b * a.n_kv_heads + kvh) * a.max_splits + split) * GQ * PS;
  const __amdgpu_buffer_rsrc_t rpart = buf_rsrc(part);
  const __amdgpu_buffer_rsrc_t rout = buf_rsrc(out);
  for (int g = threadIdx.x; g < NG; g += NT) {
    const int h = g / (D / 4), d0 = 4 * (g % (D / 4));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f;
    f4_t O = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = exp2f(s_m[w][h] - M);
        L += f * s_l[w][h];
        const f4_t o = *reinterpret_cast<const f4_t*>(&s_o[w][h][d0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) O[j] = fmaf(f, o[j], O[j]);
      }
    }
    if (nsplit == 1) {
      h4_t r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = (_Float16)(L > 0.f ? O[j] / L : 0.f);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, r), rout, 2 * (h * D + d0), 0, kPolicySc1);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, O), rpart, 4 * (h * PS + d0), 0, kPolicySc1);
      if (d0 == 0)
        __builtin_amdgcn_raw_buffer_store_b64((u2_t){(uint32_t)f_bits(M), (uint32_t)f_bits(L)}, rpart,
                                              4 * (h * PS + D), 0, kPolicySc1);
    }
  }
  if (nsplit == 1) return;
  // The last split to arrive merges (log-sum-exp over splits). Partials move
  // between workgroups, possibly on different XCDs, through device-scope
  // (coherent) stores and loads, so no L2 writeback or invalidate is needed:
  // each workgroup waits for its stores to complete before it counts itself.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* counter = a.counters + (size_t)b * a.n_kv_heads + kvh;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(nsplit - 1);
  __syncthreads();
  if (!s_last) return;
  // One pass: wavefront h < GQ loads (m, l) of head h for every split while
  // every thread's first kU partial outputs (16 bytes each) are in flight;
  // TPG threads share a four-dim group, thread part p taking the splits
  // p, p + TPG, ...; the wavefront h reduces (m, l) on the VALU and leaves
  // the merge weights w[h][s] = 2^(m_s - M) / sum_s' 2^(m_s' - M) l_s' in
  // LDS, the parts are summed in order through LDS.
  constexpr int kPool = kAttnWaves * 64;  // threads the split of the work is sized for (any NT >= it)
  constexpr int TPG = NG * 4 <= kPool ? 4 : NG * 2 <= kPool ? 2 : 1;
  constexpr int kU = 8;
  static_assert(GQ * 128 + (TPG - 1) * NG * 4 <= W * GQ * D, "merge scratch fits s_o");
  const float* pb = a.partials + ((size_t)b * a.n_kv_heads + kvh) * a.max_splits * GQ * PS;
  const __amdgpu_buffer_rsrc_t rp = buf_rsrc(pb);
  float* s_w = &s_o[0][0][0];                                  // reuse: [GQ][nsplit] (nsplit <= 128)
  f4_t* s_x = reinterpret_cast<f4_t*>(&s_o[0][0][0] + GQ * 128);  // [TPG - 1][NG]
  float mm[2] = {-INFINITY, -INFINITY}, ll[2] = {0.f, 0.f};
  if (wave < GQ) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sp = lane + 64 * r;
      if (sp < nsplit) {
        const u2_t ml = ld64_agent(rp, 4 * ((sp * GQ + wave) * PS + D));
        mm[r] = bits_f((int)ml[0]);
        ll[r] = bits_f((int)ml[1]);
      }
    }
  }
  const bool worker = (int)threadIdx.x < NG * TPG;
  const int gi = worker ? (int)threadIdx.x % NG : 0, pi = worker ? (int)threadIdx.x / NG : 0;
  const int mh = gi / (D / 4), md0 = 4 * (gi % (D / 4));
  auto ldo = [&](int sp) {  // split sp's four dims of the group (clamped: loads stay in the item)
    return __builtin_bit_cast(f4_t, ld128_agent(rp, 4 * ((min(sp, nsplit - 1) * GQ + mh) * PS + md0)));
  };
  f4_t v0[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) v0[u] = ldo(pi + TPG * u);
  if (wave < GQ) {
    float M = fmaxf(mm[0], mm[1]);
    M = fmaxf(M, ror4(M));
    M = fmaxf(M, ror8(M));
    M = fmaxf(M, dpp_xor1(M));
    M = fmaxf(M, dpp_xor2(M));
    M = rows_max(M);
    const float f0 = M == -INFINITY ? 0.f : exp2f(mm[0] - M);
    const float f1 = M == -INFINITY ? 0.f : exp2f(mm[1] - M);
    float L = f0 * ll[0] + f1 * ll[1];
    L += ror4(L);
    L += ror8(L);
    L += dpp_xor1(L);
    L += dpp_xor2(L);
    L = rows_sum(L);
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sp = lane + 64 * r;
      if (sp < nsplit) s_w[wave * nsplit + sp] = (r ? f1 : f0) * inv;
    }
  }
  __syncthreads();
  f4_t O = {0.f, 0.f, 0.f, 0.f};
  if (worker) {
    const float* wh = s_w + mh * nsplit;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int sp = pi + TPG * u;
      if (sp < nsplit)
#pragma unroll
        for (int j = 0; j < 4; ++j) O[j] = fmaf(wh[sp], v0[u][j], O[j]);
    }
    // splits past the first TPG kU: kU loads in flight, then their sums (in order)
    for (int sp0 = TPG * kU; sp0 < nsplit; sp0 += TPG * kU) {
      f4_t t8[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) t8[u] = ldo(sp0 + pi + TPG * u);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int sp = sp0 + pi + TPG * u;
        if (sp < nsplit)
#pragma unroll
          for (int j = 0; j < 4; ++j) O[j] = fmaf(wh[sp], t8[u][j], O[j]);
      }
    }
    if (pi > 0) s_x[(pi - 1) * NG + gi] = O;
  }
  __syncthreads();
  if (worker && pi == 0) {
#pragma unroll
    for (int p = 1; p < TPG; ++p) {
      const f4_t x = s_x[(p - 1) * NG + gi];
#pragma unroll
      for (int j = 0; j < 4; ++j) O[j] += x[j];
    }
    h4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (_Float16)O[j];
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, r), rout, 2 * (mh * D + md0), 0, kPolicySc1);
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace w4
