// libpkv C ABI: pool and page-table management, argument checks, dispatch.
//
// Paged KV cache and KV-gradient pools for chunk-recurrent training
// ("Out of the Memory Barrier", gist.science de, section 2.B; gist.science
// fr, technical summary 2.B; sciencestack.ai, Figures 3 and 4): every buffer
// is allocated once at pool creation, so appends never reallocate and the
// footprint is exactly the page bytes.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"
#include "pkv_pool.h"

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define PKV_HIP(expr, what)                      \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

namespace pkv {

pkv_status pool_fail(pkv_status st, const char* msg) { return fail(st, "%s", msg); }
pkv_status pool_hip_fail(hipError_t e, const char* what) { return hip_fail(e, what); }

LayerDev layer_view(pkv_pool* p, int layer) {
  LayerDev L;
  const pkv_pool_desc& d = p->desc;
  const int64_t tab_stride = (int64_t)d.n_kv_heads * d.max_logical_pages;
  L.reps = p->d_reps + (int64_t)layer * d.n_kv_heads * d.n_slots * d.head_dim;
  // host tier: the HBM window that holds the layer, reached through the
  // window's table (logical page -> window slot)
  const int64_t wl = d.host_tier ? p->window_of(layer) : layer;
  L.k = (char*)p->d_k + wl * p->dev_elems * p->kv_bytes;
  L.v = (char*)p->d_v + wl * p->dev_elems * p->kv_bytes;
  L.dk = p->d_dk + wl * p->dev_elems;
  L.dv = p->d_dv + wl * p->dev_elems;
  L.table = (d.host_tier ? p->d_wtable : p->d_table) + wl * tab_stride;
  return L;
}

LayerDev store_view(pkv_pool* p, int layer) {
  if (!p->desc.host_tier) return layer_view(p, layer);
  LayerDev L;
  L.k = p->m_k[layer];
  L.v = p->m_v[layer];
  L.dk = (float*)p->m_dk[layer];
  L.dv = (float*)p->m_dv[layer];
  L.reps = p->d_reps + (int64_t)layer * p->desc.n_kv_heads * p->desc.n_slots * p->desc.head_dim;
  L.table = p->d_table + (int64_t)layer * p->desc.n_kv_heads * p->desc.max_logical_pages;
  return L;
}

Geom geom(const pkv_pool* p) {
  Geom g;
  g.hkv = p->desc.n_kv_heads;
  g.d = p->desc.head_dim;
  g.page = p->desc.page_size;
  g.slots = p->desc.n_slots;
  g.max_logical = p->desc.max_logical_pages;
  return g;
}

Geom compute_geom(const pkv_pool* p) {
  Geom g = geom(p);
  if (p->desc.host_tier) g.slots = p->window_slots;
  return g;
}

pkv_status ensure_scratch(void** buf, int64_t* have, int64_t need) {
  if (*have >= need) return PKV_OK;
  if (*buf) {
    PKV_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize (scratch growth)");
    PKV_HIP(hipFree(*buf), "hipFree (scratch)");
    *buf = nullptr;
    *have = 0;
  }
  const int64_t bytes = ((need + 4095) / 4096) * 4096;
  if (hipMalloc(buf, bytes) != hipSuccess) {
    *buf = nullptr;
    return fail(PKV_ENOMEM, "scratch allocation of %lld bytes failed", (long long)bytes);
  }
  *have = bytes;
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

pkv_status pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out) {
  if (!desc || !out) return fail(PKV_EINVAL, "pkv_pool_create: null argument");
  *out = nullptr;
  const pkv_pool_desc& d = *desc;
  if (d.n_layers < 1 || d.n_kv_heads < 1 || d.page_size < 1 || d.max_logical_pages < 1 ||
      d.n_slots < d.max_logical_pages)
    return fail(PKV_EINVAL,
                "pkv_pool_create: need n_layers, n_kv_heads, page_size, max_logical_pages >= 1 "
                "and n_slots >= max_logical_pages");
  if (d.kv_dtype != PKV_F32 && d.kv_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "pkv_pool_create: kv_dtype must be PKV_F32 or PKV_BF16");
  if (d.kv_dtype == PKV_F32) {
    if ((d.head_dim != 64 && d.head_dim != 128) || d.page_size % 16)
      return fail(PKV_EUNSUPPORTED,
                  "pkv_pool_create: fp32 pools need head_dim 64 or 128 and page_size %% 16 == 0");
  } else {
    if (d.head_dim != 128 || d.page_size % 128)
      return fail(PKV_EUNSUPPORTED,
                  "pkv_pool_create: bf16 pools need head_dim 128 and page_size %% 128 == 0");
  }
  if (d.host_tier && d.host_grad_dtype != PKV_F32 && d.host_grad_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "pkv_pool_create: host_grad_dtype must be PKV_F32 or PKV_BF16");
  if (d.host_grad_accumulate != 0 && d.host_grad_accumulate != 1)
    return fail(PKV_EINVAL, "pkv_pool_create: host_grad_accumulate must be 0 or 1");
  if (d.host_grad_accumulate && !d.host_tier)
    return fail(PKV_EINVAL, "pkv_pool_create: host_grad_accumulate needs host_tier");
  if (d.window_slots < 0 || (d.window_slots && !d.host_tier))
    return fail(PKV_EINVAL, "pkv_pool_create: window_slots must be 0, or >= 1 with host_tier");

  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return fail(PKV_ENOMEM, "pkv_pool_create: out of host memory");
  p->desc = d;
  p->kv_bytes = d.kv_dtype == PKV_BF16 ? 2 : 4;
  p->accumulate = d.host_grad_accumulate != 0;
  p->layer_elems = (int64_t)d.n_kv_heads * d.n_slots * d.page_size * d.head_dim;
  p->window_slots = d.window_slots > 0 && d.window_slots < d.max_logical_pages
                        ? d.window_slots : d.max_logical_pages;
  p->dev_elems = d.host_tier
                     ? (int64_t)d.n_kv_heads * p->window_slots * d.page_size * d.head_dim
                     : p->layer_elems;
  p->length.assign(d.n_layers, 0);
  p->layer_ticket.assign(d.n_layers, 0);
  p->h_table.resize((size_t)d.n_layers * d.n_kv_heads * d.max_logical_pages);
  for (int l = 0; l < d.n_layers; ++l)
    for (int g = 0; g < d.n_kv_heads; ++g)
      for (int j = 0; j < d.max_logical_pages; ++j)
        p->h_table[((size_t)l * d.n_kv_heads + g) * d.max_logical_pages + j] = j;

  pkv_status st = pool_allocate(p);
  if (st != PKV_OK) {
    std::string keep = g_err;
    pool_release(p);
    delete p;
    g_err = keep;
    return st;
  }
  *out = p;
  return PKV_OK;
}

pkv_status pkv_pool_destroy(pkv_pool* pool) {
  if (!pool) return PKV_OK;
  pkv_status st = pool_release(pool);
  delete pool;
  return st;
}

pkv_status pkv_pool_bytes(const pkv_pool* pool, int64_t* device_bytes, int64_t* host_bytes) {
  if (!pool) return fail(PKV_EINVAL, "pkv_pool_bytes: null pool");
  if (device_bytes) *device_bytes = pool->device_bytes;
  if (host_bytes) *host_bytes = pool->host_bytes;
  return PKV_OK;
}

int64_t pkv_length(const pkv_pool* pool, int32_t layer) {
  if (!pool || layer < 0 || layer >= pool->desc.n_layers) return -1;
  return pool->length[layer];
}

pkv_status pkv_pool_reset(pkv_pool* pool, int32_t layer) {
  if (!pool) return fail(PKV_EINVAL, "pkv_pool_reset: null pool");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_pool_reset: layer %d out of range", layer);
  pool->length[layer] = 0;
  // a window holding the layer no longer covers any of its keys: attention
  // and appends need a new prefetch
  const int w = pool->window_of(layer);
  if (pool->desc.host_tier && pool->window_layer[w] == layer) pool->window_keys[w] = 0;
  return PKV_OK;
}

pkv_status pkv_page_table_set(pkv_pool* pool, int32_t layer, int32_t kv_head,
                              const int32_t* host_slots, int32_t n) {
  if (!pool || !host_slots) return fail(PKV_EINVAL, "pkv_page_table_set: null argument");
  const pkv_pool_desc& d = pool->desc;
  if (layer < 0 || layer >= d.n_layers || kv_head < 0 || kv_head >= d.n_kv_heads)
    return fail(PKV_EINVAL, "pkv_page_table_set: layer %d / kv_head %d out of range", layer,
                kv_head);
  if (n < 0 || n > d.max_logical_pages)
    return fail(PKV_ECAPACITY, "pkv_page_table_set: n=%d exceeds max_logical_pages=%d", n,
                d.max_logical_pages);
  if (pool->length[layer] != 0)
    return fail(PKV_ESTATE, "pkv_page_table_set: layer %d already holds tokens", layer);
  int32_t* row = &pool->h_table[((size_t)layer * d.n_kv_heads + kv_head) * d.max_logical_pages];
  std::vector<int32_t> next(row, row + d.max_logical_pages);
  for (int j = 0; j < n; ++j) next[j] = host_slots[j];
  std::vector<char> used(d.n_slots, 0);
  for (int j = 0; j < d.max_logical_pages; ++j) {
    const int32_t s = next[j];
    if (s < 0 || s >= d.n_slots)
      return fail(PKV_ECAPACITY, "pkv_page_table_set: slot %d of page %d outside [0, %d)", s, j,
                  d.n_slots);
    if (used[s]) return fail(PKV_EINVAL, "pkv_page_table_set: slot %d used twice", s);
    used[s] = 1;
  }
  std::memcpy(row, next.data(), sizeof(int32_t) * d.max_logical_pages);
  PKV_HIP(hipMemcpy(pool->d_table + ((size_t)layer * d.n_kv_heads + kv_head) * d.max_logical_pages,
                    row, sizeof(int32_t) * d.max_logical_pages, hipMemcpyHostToDevice),
          "pkv_page_table_set: hipMemcpy");
  return PKV_OK;
}

pkv_status pkv_append_kv(pkv_pool* pool, int32_t layer, int64_t pos0, int64_t n_tok,
                         const void* k, const void* v, hipStream_t stream) {
  if (!pool) return fail(PKV_EINVAL, "pkv_append_kv: null pool");
  const pkv_pool_desc& d = pool->desc;
  if (layer < 0 || layer >= d.n_layers)
    return fail(PKV_EINVAL, "pkv_append_kv: layer %d out of range", layer);
  if (n_tok < 0) return fail(PKV_EINVAL, "pkv_append_kv: n_tok < 0");
  if (n_tok == 0) return PKV_OK;
  if (!k || !v) return fail(PKV_EINVAL, "pkv_append_kv: null k or v");
  if (pos0 != pool->length[layer])
    return fail(PKV_ESTATE, "pkv_append_kv: pos0=%lld but layer %d holds %lld tokens",
                (long long)pos0, layer, (long long)pool->length[layer]);
  if (pos0 + n_tok > (int64_t)d.max_logical_pages * d.page_size)
    return fail(PKV_ECAPACITY, "pkv_append_kv: %lld tokens exceed %d pages of %d",
                (long long)(pos0 + n_tok), d.max_logical_pages, d.page_size);
  pkv_status st = pool_append(pool, layer, pos0, n_tok, k, v, stream);
  if (st != PKV_OK) return st;
  pool->length[layer] = pos0 + n_tok;
  return PKV_OK;
}

static pkv_status check_sel(const pkv_pool* pool, const pkv_sel* sel, int64_t n_q,
                            const char* who) {
  if (!sel) return PKV_OK;
  if (!sel->pages || !sel->count)
    return fail(PKV_EINVAL, "%s: selection with null pages/count", who);
  if (sel->n_qpages != cdiv(n_q, pool->desc.page_size))
    return fail(PKV_EINVAL, "%s: selection covers %d query pages, chunk has %lld", who,
                sel->n_qpages, (long long)cdiv(n_q, pool->desc.page_size));
  if (sel->stride < 1) return fail(PKV_EINVAL, "%s: selection stride < 1", who);
  return PKV_OK;
}

static pkv_status check_attn(const pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                             int32_t hq, const char* who) {
  if (!pool) return fail(PKV_EINVAL, "%s: null pool", who);
  const pkv_pool_desc& d = pool->desc;
  if (layer < 0 || layer >= d.n_layers) return fail(PKV_EINVAL, "%s: layer %d out of range", who, layer);
  if (hq < 1 || hq % d.n_kv_heads) return fail(PKV_EINVAL, "%s: n_q_heads=%d not a multiple of %d KV heads", who, hq, d.n_kv_heads);
  if (n_q < 0 || n_q > (1LL << 30)) return fail(PKV_EINVAL, "%s: n_q=%lld out of range", who, (long long)n_q);
  if (q_pos0 < 0 || q_pos0 % d.page_size)
    return fail(PKV_EINVAL, "%s: q_pos0=%lld must be a non-negative multiple of page_size %d",
                who, (long long)q_pos0, d.page_size);
  if (q_pos0 + n_q > pool->length[layer])
    return fail(PKV_ESTATE, "%s: queries up to %lld but layer %d holds %lld tokens", who,
                (long long)(q_pos0 + n_q), layer, (long long)pool->length[layer]);
  if ((int64_t)hq * n_q * d.head_dim > (1LL << 40)) return fail(PKV_EINVAL, "%s: chunk too large", who);
  return PKV_OK;
}

static AttnCall make_call(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q, int32_t hq,
                          float scale, const pkv_sel* sel) {
  AttnCall c;
  std::memset(&c, 0, sizeof c);
  c.L = layer_view(pool, layer);
  c.g = compute_geom(pool);
  c.hq = hq;
  c.q_pos0 = q_pos0;
  c.n_q = (int)n_q;
  c.scale = scale;
  if (sel) {
    c.sel.pages = sel->pages;
    c.sel.count = sel->count;
    c.sel.n_qpages = sel->n_qpages;
    c.sel.stride = sel->stride;
  }
  return c;
}

}  // extern "C"

namespace pkv {

// Scratch bytes of one backward call; *plan_off: where the dK/dV work list
// starts in it.
int64_t bwd_scratch_bytes(pkv_pool* pool, int64_t q_pos0, int64_t n_q, int32_t n_q_heads,
                          const pkv_sel* sel, int64_t* plan_off) {
  // D and lse2 ([hq][n_q] fp32 each), then the sparse dK/dV work list
  const int64_t dl_bytes = ((2 * (int64_t)n_q_heads * n_q * (int64_t)sizeof(float) + 255) / 256) * 256;
  *plan_off = dl_bytes;
  if (!sel || pool->desc.kv_dtype != PKV_BF16) return dl_bytes;
  return dl_bytes + dkdv_plan_layout(geom(pool), n_q_heads, q_pos0, (int)n_q, sel->stride).bytes;
}

// The backward behind pkv_attn_bwd (scratch == nullptr: the pool's own,
// grown on demand) and pkv_attn_bwd_noalloc (scratch: scratch_cap bytes the
// caller provides; a larger need is PKV_ECAPACITY).
pkv_status attn_bwd_impl(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                         int32_t n_q_heads, float scale, const void* q, const void* o,
                         const void* dout, const float* lse, const pkv_sel* sel, float* dq,
                         hipStream_t stream, void* scratch, int64_t scratch_cap, const char* who) {
  pkv_status st = check_attn(pool, layer, q_pos0, n_q, n_q_heads, who);
  if (st != PKV_OK) return st;
  if (n_q == 0) return PKV_OK;
  if (!q || !o || !dout || !lse || !dq) return fail(PKV_EINVAL, "%s: null q/o/dout/lse/dq", who);
  if ((st = check_sel(pool, sel, n_q, who)) != PKV_OK) return st;
  if (cdiv(n_q, pool->desc.page_size) > 1024)
    return fail(PKV_EUNSUPPORTED, "%s: chunks of more than 1024 pages", who);
  int64_t plan_off = 0;
  const int64_t need = bwd_scratch_bytes(pool, q_pos0, n_q, n_q_heads, sel, &plan_off);
  if (scratch) {
    // caller-provided scratch: nothing may be allocated, and kernel timing
    // creates events
    if (kernel_timing_on())
      return fail(PKV_ESTATE, "%s: not available while kernel timing is on", who);
    if (need > scratch_cap)
      return fail(PKV_ECAPACITY, "%s: the chunk needs %lld bytes of scratch, at most %lld",
                  who, (long long)need, (long long)scratch_cap);
  } else {
    if ((st = ensure_scratch(&pool->d_delta, &pool->delta_bytes, need)) != PKV_OK) return st;
    scratch = pool->d_delta;
  }
  if ((st = pool_before_compute(pool, layer, q_pos0 + n_q, stream, true)) != PKV_OK) return st;
  AttnCall c = make_call(pool, layer, q_pos0, n_q, n_q_heads, scale, sel);
  c.q = q;
  c.o = o;
  c.dout = dout;
  c.lse_in = lse;
  c.dq = dq;
  c.delta = (float*)scratch;
  c.lse2 = pool->desc.kv_dtype == PKV_BF16 ? c.delta + (int64_t)n_q_heads * n_q : nullptr;
  if (sel && pool->desc.kv_dtype == PKV_BF16) {
    DkvPlan pl = dkdv_plan_layout(geom(pool), n_q_heads, q_pos0, (int)n_q, sel->stride);
    pl.base = reinterpret_cast<int*>((char*)scratch + plan_off);
    c.plan = pl;
  }
  hipError_t e = pool->desc.kv_dtype == PKV_BF16
                     ? launch_bwd_bf16(c, stream, pool->s_aux, pool->ev_fork, pool->ev_join)
                     : launch_bwd_f32(c, stream);
  if (e != hipSuccess) return fail(PKV_EHIP, "%s: launch: %s", who, hipGetErrorString(e));
  return pool_after_compute(pool, layer, stream);
}

}  // namespace pkv

extern "C" {

pkv_status pkv_attn_fwd(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                        int32_t n_q_heads, float scale, const void* q, const pkv_sel* sel,
                        void* o, float* lse, hipStream_t stream) {
  pkv_status st = check_attn(pool, layer, q_pos0, n_q, n_q_heads, "pkv_attn_fwd");
  if (st != PKV_OK) return st;
  if (n_q == 0) return PKV_OK;
  if (!q || !o || !lse) return fail(PKV_EINVAL, "pkv_attn_fwd: null q/o/lse");
  if ((st = check_sel(pool, sel, n_q, "pkv_attn_fwd")) != PKV_OK) return st;
  if ((st = pool_before_compute(pool, layer, q_pos0 + n_q, stream, false)) != PKV_OK) return st;
  AttnCall c = make_call(pool, layer, q_pos0, n_q, n_q_heads, scale, sel);
  c.q = q;
  c.o_out = o;
  c.lse = lse;
  if (sel && pool->desc.kv_dtype == PKV_BF16) {
    // top-K: every unit attends about as many keys; split the last pass
    const int slots = 2 * pool->n_cus;
    TailSplit sp = plan_tail_split((int)cdiv(n_q, kFwdRows) * n_q_heads, slots);
    if (sp.n_split > 0) {
      const int64_t need = (int64_t)sp.n_split * 2 * 4 * kFwdPartWaveFloats * 4;
      if ((st = ensure_scratch(&pool->d_fsplit, &pool->fsplit_bytes, need)) != PKV_OK) return st;
      sp.part = (float*)pool->d_fsplit;
      c.split = sp;
    }
  }
  hipError_t e = pool->desc.kv_dtype == PKV_BF16 ? launch_fwd_bf16(c, stream) : launch_fwd_f32(c, stream);
  if (e != hipSuccess) return hip_fail(e, "pkv_attn_fwd: launch");
  return pool_after_compute(pool, layer, stream);
}

pkv_status pkv_attn_bwd(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                        int32_t n_q_heads, float scale, const void* q, const void* o,
                        const void* dout, const float* lse, const pkv_sel* sel, float* dq,
                        hipStream_t stream) {
  return attn_bwd_impl(pool, layer, q_pos0, n_q, n_q_heads, scale, q, o, dout, lse, sel, dq,
                       stream, nullptr, 0, "pkv_attn_bwd");
}

pkv_status pkv_measure_gather(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                              int32_t n_q_heads, const pkv_sel* sel, float* out,
                              hipStream_t stream) {
  pkv_status st = check_attn(pool, layer, q_pos0, n_q, n_q_heads, "pkv_measure_gather");
  if (st != PKV_OK) return st;
  if (pool->desc.kv_dtype != PKV_BF16 || pool->desc.host_tier)
    return fail(PKV_EUNSUPPORTED, "pkv_measure_gather: bf16 pools without a host tier only");
  if (n_q == 0) return PKV_OK;
  if (!out) return fail(PKV_EINVAL, "pkv_measure_gather: null out");
  if ((st = check_sel(pool, sel, n_q, "pkv_measure_gather")) != PKV_OK) return st;
  AttnCall c = make_call(pool, layer, q_pos0, n_q, n_q_heads, 1.f, sel);
  hipError_t e = launch_micro_gather(c, out, stream);
  if (e != hipSuccess) return hip_fail(e, "pkv_measure_gather: launch");
  return PKV_OK;
}

pkv_status pkv_measure_atomics(pkv_pool* pool, int32_t layer, int64_t n_keys, int32_t reps,
                               float value, hipStream_t stream) {
  if (!pool) return fail(PKV_EINVAL, "pkv_measure_atomics: null pool");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_measure_atomics: layer %d out of range", layer);
  if (pool->desc.kv_dtype != PKV_BF16 || pool->desc.host_tier)
    return fail(PKV_EUNSUPPORTED, "pkv_measure_atomics: bf16 pools without a host tier only");
  if (n_keys < 0 || n_keys > pool->length[layer] || reps < 0)
    return fail(PKV_EINVAL, "pkv_measure_atomics: n_keys=%lld (layer holds %lld), reps=%d",
                (long long)n_keys, (long long)pool->length[layer], reps);
  if (n_keys == 0 || reps == 0) return PKV_OK;
  AttnCall c = make_call(pool, layer, 0, n_keys, pool->desc.n_kv_heads, 1.f, nullptr);
  hipError_t e = launch_micro_atomics(c, reps, value, stream);
  if (e != hipSuccess) return hip_fail(e, "pkv_measure_atomics: launch");
  return PKV_OK;
}

pkv_status pkv_select_topk_pages(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                                 int32_t n_q_heads, const void* q, int32_t top_k,
                                 int32_t n_sink, int32_t n_local, int32_t* sel_pages,
                                 int32_t* sel_count, int32_t sel_stride, hipStream_t stream) {
  pkv_status st = check_attn(pool, layer, q_pos0, n_q, n_q_heads, "pkv_select_topk_pages");
  if (st != PKV_OK) return st;
  if (n_q == 0) return PKV_OK;
  if (!q || !sel_pages || !sel_count) return fail(PKV_EINVAL, "pkv_select_topk_pages: null argument");
  if (top_k < 0 || n_sink < 0 || n_local < 1)
    return fail(PKV_EINVAL, "pkv_select_topk_pages: need top_k >= 0, n_sink >= 0, n_local >= 1");
  if ((int64_t)sel_stride < (int64_t)top_k + n_sink + n_local)
    return fail(PKV_EINVAL, "pkv_select_topk_pages: sel_stride %d < top_k + n_sink + n_local",
                sel_stride);
  if (q_pos0 / pool->desc.page_size + cdiv(n_q, pool->desc.page_size) > 60000)
    return fail(PKV_EUNSUPPORTED, "pkv_select_topk_pages: more than 60000 pages");
  const Geom g = geom(pool);
  if ((st = ensure_scratch(&pool->d_select, &pool->select_bytes,
                           select_scratch_floats(g, q_pos0, (int)n_q, n_sink, n_local) * 4)) != PKV_OK)
    return st;
  hipError_t e = launch_select(store_view(pool, layer), g, pool->desc.kv_dtype == PKV_BF16,
                               n_q_heads, q_pos0, (int)n_q, q, top_k, n_sink, n_local, sel_pages,
                               sel_count, sel_stride, (float*)pool->d_select, stream);
  if (e != hipSuccess) return hip_fail(e, "pkv_select_topk_pages: launch");
  return PKV_OK;
}

pkv_status pkv_grad_zero(pkv_pool* pool, int32_t layer, hipStream_t stream) {
  if (!pool) return fail(PKV_EINVAL, "pkv_grad_zero: null pool");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_grad_zero: layer %d out of range", layer);
  return pool_grad_zero(pool, layer, stream);
}

pkv_status pkv_read_pages(pkv_pool* pool, int32_t layer, int32_t what, void* dst,
                          hipStream_t stream) {
  if (!pool || !dst) return fail(PKV_EINVAL, "pkv_read_pages: null argument");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_read_pages: layer %d out of range", layer);
  if (what < PKV_K || what > PKV_REPS) return fail(PKV_EINVAL, "pkv_read_pages: bad `what` %d", what);
  return pool_read(pool, layer, what, dst, stream);
}

pkv_status pkv_read_rows(pkv_pool* pool, int32_t layer, int32_t what, int64_t pos0,
                         int64_t n_tok, void* dst, hipStream_t stream) {
  if (!pool || !dst) return fail(PKV_EINVAL, "pkv_read_rows: null argument");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_read_rows: layer %d out of range", layer);
  if (what < PKV_K || what > PKV_DV) return fail(PKV_EINVAL, "pkv_read_rows: bad `what` %d", what);
  if (pos0 < 0 || n_tok < 0 || pos0 + n_tok > pool->length[layer])
    return fail(PKV_EINVAL, "pkv_read_rows: rows [%lld, %lld) outside the %lld appended",
                (long long)pos0, (long long)(pos0 + n_tok), (long long)pool->length[layer]);
  if (n_tok == 0) return PKV_OK;
  if (pool->desc.host_tier) {
    // from the HBM window that holds the layer (after its fetch; the next
    // prefetch into the window waits for this read)
    // gradient rows: the window must hold this visit's gradients (and their
    // zeroing, with host adds, must have run), as for an attention backward
    const bool grads = what == PKV_DK || what == PKV_DV;
    pkv_status st = pool_before_compute(pool, layer, pos0 + n_tok, stream, grads);
    if (st != PKV_OK) return st;
    hipError_t e;
    if (grads && pool->accumulate) {
      // the window holds this visit's contributions; the tier the sums of
      // the earlier visits once their host adds have run
      if ((e = pool->adder->wait(pool->layer_ticket[layer])) != hipSuccess)
        return hip_fail(e, "pkv_read_rows: host gradient adds");
      e = launch_grad_rows_sum(pool, layer, what, pos0, n_tok, (float*)dst, stream);
    } else {
      e = launch_export(layer_view(pool, layer), compute_geom(pool), what, pool->kv_bytes, n_tok,
                        dst, stream, pos0);
    }
    if (e != hipSuccess) return hip_fail(e, "pkv_read_rows: launch");
    return pool_after_compute(pool, layer, stream);
  }
  hipError_t e = launch_export(layer_view(pool, layer), geom(pool), what, pool->kv_bytes, n_tok,
                               dst, stream, pos0);
  if (e != hipSuccess) return hip_fail(e, "pkv_read_rows: launch");
  return PKV_OK;
}

pkv_status pkv_prefetch_pages(pkv_pool* pool, int32_t layer, const pkv_sel* sel,
                              int32_t with_grads, hipStream_t copy_stream, hipEvent_t ready) {
  if (!pool) return fail(PKV_EINVAL, "pkv_prefetch_pages: null pool");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_prefetch_pages: layer %d out of range", layer);
  if (!pool->desc.host_tier) {
    if (ready) PKV_HIP(hipEventRecord(ready, copy_stream), "pkv_prefetch_pages: hipEventRecord");
    return PKV_OK;
  }
  if (sel && (!sel->pages || !sel->count || sel->stride < 1 || sel->n_qpages < 0))
    return fail(PKV_EINVAL, "pkv_prefetch_pages: malformed selection");
  return pool_prefetch(pool, layer, sel, 0, with_grads != 0, copy_stream, ready);
}

pkv_status pkv_prefetch_prefix(pkv_pool* pool, int32_t layer, int64_t n_keys, int32_t with_grads,
                               hipStream_t copy_stream, hipEvent_t ready) {
  if (!pool) return fail(PKV_EINVAL, "pkv_prefetch_prefix: null pool");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_prefetch_prefix: layer %d out of range", layer);
  const int64_t cap = (int64_t)pool->desc.max_logical_pages * pool->desc.page_size;
  if (n_keys < 1 || n_keys > cap)
    return fail(PKV_EINVAL, "pkv_prefetch_prefix: n_keys=%lld outside [1, %lld]",
                (long long)n_keys, (long long)cap);
  if (!pool->desc.host_tier) {
    if (ready) PKV_HIP(hipEventRecord(ready, copy_stream), "pkv_prefetch_prefix: hipEventRecord");
    return PKV_OK;
  }
  return pool_prefetch(pool, layer, nullptr, n_keys, with_grads != 0, copy_stream, ready);
}

pkv_status pkv_offload_bytes(pkv_pool* pool, int64_t* fetched, int64_t* written) {
  if (!pool) return fail(PKV_EINVAL, "pkv_offload_bytes: null pool");
  return pool_copy_stats(pool, fetched, written);
}

pkv_status pkv_writeback_grads(pkv_pool* pool, int32_t layer, hipStream_t copy_stream,
                               hipEvent_t done) {
  if (!pool) return fail(PKV_EINVAL, "pkv_writeback_grads: null pool");
  if (layer < 0 || layer >= pool->desc.n_layers)
    return fail(PKV_EINVAL, "pkv_writeback_grads: layer %d out of range", layer);
  if (!pool->desc.host_tier) {
    if (done) PKV_HIP(hipEventRecord(done, copy_stream), "pkv_writeback_grads: hipEventRecord");
    return PKV_OK;
  }
  return pool_writeback(pool, layer, copy_stream, done);
}

}  // extern "C"
