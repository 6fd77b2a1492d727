// Pool allocation, appends, exports and the host tier (pinned host pools with
// a two-layer HBM window filled on a side stream).
//
// "Out of the Memory Barrier" (gist.science de, section 2.B: fixed-size
// pages, no reallocation on append; section 2.C and gist.science nl,
// "Methodologie": the KV cache and its gradients move asynchronously between
// pinned host memory and the GPU on separate streams, the next layer being
// fetched while the current one computes).
#include <hip/hip_runtime.h>
#include <sched.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>

#include "pkv_pool.h"

namespace pkv {
namespace {

// Test hook: PKV_FAIL_ALLOC_AT=n makes the n-th device or pinned allocation
// of a pool creation fail as if memory were exhausted, so that tests can
// check that a half-built pool is released completely.
bool injected_failure(pkv_pool* p) {
  const char* now = std::getenv("PKV_FAIL_ALLOC_AT");
  if (!now) return false;
  return ++p->allocs == std::atoi(now);
}

// Test hook: PKV_FAIL_COPY_AT=n makes the n-th host-link copy of a pool (the
// fetch of a prefetch, or a writeback) fail as if its launch had failed,
// before anything of it is enqueued, so that tests can check the pool's state
// after a failed transfer.
bool injected_copy_failure(pkv_pool* p) {
  const char* now = std::getenv("PKV_FAIL_COPY_AT");
  if (!now) return false;
  return ++p->copies == std::atoi(now);
}

pkv_status dev_alloc(pkv_pool* p, void** ptr, int64_t bytes, const char* what) {
  *ptr = nullptr;
  if (bytes <= 0) return PKV_OK;
  if (injected_failure(p)) return pool_fail(PKV_ENOMEM, "injected allocation failure (PKV_FAIL_ALLOC_AT)");
  hipError_t e = hipMalloc(ptr, (size_t)bytes);
  if (e != hipSuccess) {
    *ptr = nullptr;
    (void)hipGetLastError();
    return pool_fail(PKV_ENOMEM, what);
  }
  p->device_bytes += bytes;
  e = hipMemset(*ptr, 0, (size_t)bytes);
  if (e != hipSuccess) return pool_hip_fail(e, "hipMemset (pool init)");
  return PKV_OK;
}

pkv_status host_alloc(pkv_pool* p, void** hptr, void** dptr, int64_t bytes) {
  *hptr = *dptr = nullptr;
  if (injected_failure(p)) return pool_fail(PKV_ENOMEM, "injected allocation failure (PKV_FAIL_ALLOC_AT)");
  hipError_t e = hipHostMalloc(hptr, (size_t)bytes, hipHostMallocMapped);
  if (e != hipSuccess) {
    *hptr = nullptr;
    (void)hipGetLastError();
    return pool_fail(PKV_ENOMEM, "pinned host allocation for the host tier failed");
  }
  p->host_bytes += bytes;
  e = hipHostGetDevicePointer(dptr, *hptr, 0);
  if (e != hipSuccess) return pool_hip_fail(e, "hipHostGetDevicePointer");
  return PKV_OK;
}

int grad_host_bytes(const pkv_pool* p) { return p->desc.host_grad_dtype == PKV_BF16 ? 2 : 4; }

// Threads that add staged gradient contributions into the host tier: the
// environment variable PKV_HOST_ADD_THREADS, else min(16, CPUs this process
// may run on).
int host_add_threads() {
  if (const char* s = std::getenv("PKV_HOST_ADD_THREADS")) {
    const int n = std::atoi(s);
    return n < 1 ? 1 : (n > 64 ? 64 : n);
  }
  cpu_set_t set;
  CPU_ZERO(&set);
  const int cpus = sched_getaffinity(0, sizeof set, &set) == 0 ? CPU_COUNT(&set) : 8;
  return cpus < 1 ? 1 : (cpus > 16 ? 16 : cpus);
}

}  // namespace

pkv_status pool_allocate(pkv_pool* p) {
  const pkv_pool_desc& d = p->desc;
  const int copies = d.host_tier ? pkv_pool::kWindow : d.n_layers;
  pkv_status st;
  const int64_t kvb = p->dev_elems * p->kv_bytes * copies;
  const int64_t grb = p->dev_elems * 4 * copies;
  const int64_t repb = (int64_t)d.n_layers * d.n_kv_heads * d.n_slots * d.head_dim * 4;
  const int64_t tabb = (int64_t)d.n_layers * d.n_kv_heads * d.max_logical_pages * 4;
  // host tier: page maps and page-head lists (two buffers per window), and
  // the windows' tables
  const int64_t wtabb = d.host_tier ? (int64_t)pkv_pool::kWindow * d.n_kv_heads * d.max_logical_pages * 4 : 0;
  const int64_t needb = d.host_tier ? (int64_t)2 * pkv_pool::kWindow * d.n_kv_heads * d.max_logical_pages : 0;
  const int64_t itemb = d.host_tier ? (int64_t)8 * 2 * pkv_pool::kWindow * d.n_kv_heads * p->window_slots : 0;
  const int64_t countb = 4 * 2 * pkv_pool::kWindow;
  const int64_t base_b = 2 * kvb + 2 * grb + repb + tabb + wtabb + needb + itemb + countb + 16;
  if (d.host_tier && d.device_budget_bytes > 0 && base_b > d.device_budget_bytes)
    return pool_fail(PKV_ENOMEM, "host-tier window does not fit device_budget_bytes");
  // host accumulation: the device staging of the writeback, where the budget
  // leaves room for it (else the writeback kernel writes the pinned staging)
  const int64_t stage_heads = (int64_t)d.n_kv_heads * p->window_slots;
  const int64_t stageb = p->accumulate ? 2 * stage_heads * d.page_size * d.head_dim * grad_host_bytes(p) : 0;
  const bool with_stage = p->accumulate && (d.device_budget_bytes <= 0 || base_b + stageb <= d.device_budget_bytes);
  if ((st = dev_alloc(p, &p->d_k, kvb, "device allocation of the K pool failed")) != PKV_OK) return st;
  if ((st = dev_alloc(p, &p->d_v, kvb, "device allocation of the V pool failed")) != PKV_OK) return st;
  if ((st = dev_alloc(p, (void**)&p->d_dk, grb, "device allocation of the dK pool failed")) != PKV_OK) return st;
  if ((st = dev_alloc(p, (void**)&p->d_dv, grb, "device allocation of the dV pool failed")) != PKV_OK) return st;
  if ((st = dev_alloc(p, (void**)&p->d_reps, repb, "device allocation of the representatives failed")) != PKV_OK) return st;
  if ((st = dev_alloc(p, (void**)&p->d_table, tabb, "device allocation of the page tables failed")) != PKV_OK) return st;
  hipError_t e = hipMemcpy(p->d_table, p->h_table.data(), (size_t)tabb, hipMemcpyHostToDevice);
  if (e != hipSuccess) return pool_hip_fail(e, "hipMemcpy (page tables)");
  if ((e = hipStreamCreateWithFlags(&p->s_aux, hipStreamNonBlocking)) != hipSuccess)
    return pool_hip_fail(e, "hipStreamCreate");
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess ||
      (e = hipDeviceGetAttribute(&p->n_cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return pool_hip_fail(e, "hipDeviceGetAttribute (compute units)");
  if ((e = hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&p->ev_join, hipEventDisableTiming)) != hipSuccess)
    return pool_hip_fail(e, "hipEventCreate");
  if (d.host_tier) {
    if ((st = dev_alloc(p, (void**)&p->d_wtable, wtabb, "device allocation of the window tables failed")) != PKV_OK) return st;
    if ((st = dev_alloc(p, (void**)&p->d_need, needb, "device allocation of the window map failed")) != PKV_OK) return st;
    if ((st = dev_alloc(p, (void**)&p->d_items, itemb, "device allocation of the window list failed")) != PKV_OK) return st;
    if ((st = dev_alloc(p, (void**)&p->d_count, countb, "device allocation of the window list failed")) != PKV_OK) return st;
    if ((st = dev_alloc(p, (void**)&p->d_moved, 16, "device allocation of the copy counters failed")) != PKV_OK) return st;
    if (with_stage) {
      if ((st = dev_alloc(p, (void**)&p->d_stage, stageb, "device allocation of the writeback staging failed")) != PKV_OK)
        return st;
      p->stage_heads = stage_heads;
      if ((e = hipEventCreateWithFlags(&p->ev_stage, hipEventDisableTiming)) != hipSuccess)
        return pool_hip_fail(e, "hipEventCreate");
      for (int w = 0; w < pkv_pool::kWindow; ++w)
        if ((e = hipEventCreateWithFlags(&p->ev_count[w], hipEventDisableTiming)) != hipSuccess)
          return pool_hip_fail(e, "hipEventCreate");
    }
    for (int w = 0; w < pkv_pool::kWindow; ++w) {
      if ((e = hipEventCreateWithFlags(&p->ev_compute[w], hipEventDisableTiming)) != hipSuccess)
        return pool_hip_fail(e, "hipEventCreate");
      if ((e = hipEventCreateWithFlags(&p->ev_ready[w], hipEventDisableTiming)) != hipSuccess)
        return pool_hip_fail(e, "hipEventCreate");
      // the host adds' coordinator waits on this one: let it sleep, not spin
      const unsigned wb_flags =
          hipEventDisableTiming | (p->accumulate ? hipEventBlockingSync : 0u);
      if ((e = hipEventCreateWithFlags(&p->ev_wb[w], wb_flags)) != hipSuccess)
        return pool_hip_fail(e, "hipEventCreate");
      for (int b = 0; b < 2; ++b)
        if ((e = hipEventCreateWithFlags(&p->ev_list[w][b], hipEventDisableTiming)) != hipSuccess)
          return pool_hip_fail(e, "hipEventCreate");
    }
    const int64_t hkv = p->layer_elems * p->kv_bytes;
    const int64_t hgr = p->layer_elems * grad_host_bytes(p);
    p->h_k.assign(d.n_layers, nullptr);
    p->h_v.assign(d.n_layers, nullptr);
    p->h_dk.assign(d.n_layers, nullptr);
    p->h_dv.assign(d.n_layers, nullptr);
    p->m_k.assign(d.n_layers, nullptr);
    p->m_v.assign(d.n_layers, nullptr);
    p->m_dk.assign(d.n_layers, nullptr);
    p->m_dv.assign(d.n_layers, nullptr);
    for (int l = 0; l < d.n_layers; ++l) {
      if ((st = host_alloc(p, &p->h_k[l], &p->m_k[l], hkv)) != PKV_OK) return st;
      if ((st = host_alloc(p, &p->h_v[l], &p->m_v[l], hkv)) != PKV_OK) return st;
      if ((st = host_alloc(p, &p->h_dk[l], &p->m_dk[l], hgr)) != PKV_OK) return st;
      if ((st = host_alloc(p, &p->h_dv[l], &p->m_dv[l], hgr)) != PKV_OK) return st;
      // zero on the device through the mapping (fast, and never leaves NaN bit
      // patterns in rows that a tile reads past the appended length)
      if ((e = launch_fill_zero(p->m_k[l], hkv, nullptr)) != hipSuccess ||
          (e = launch_fill_zero(p->m_v[l], hkv, nullptr)) != hipSuccess ||
          (e = launch_fill_zero(p->m_dk[l], hgr, nullptr)) != hipSuccess ||
          (e = launch_fill_zero(p->m_dv[l], hgr, nullptr)) != hipSuccess)
        return pool_hip_fail(e, "host tier zero fill");
    }
    if (p->accumulate) {
      const int64_t need_w = (int64_t)d.n_kv_heads * d.max_logical_pages;
      for (int w = 0; w < pkv_pool::kWindow; ++w) {
        if ((st = host_alloc(p, &p->h_stage_dk[w], &p->m_stage_dk[w], hgr)) != PKV_OK) return st;
        if ((st = host_alloc(p, &p->h_stage_dv[w], &p->m_stage_dv[w], hgr)) != PKV_OK) return st;
        if (injected_failure(p))
          return pool_fail(PKV_ENOMEM, "injected allocation failure (PKV_FAIL_ALLOC_AT)");
        if ((e = hipHostMalloc((void**)&p->h_stage_need[w], (size_t)need_w, hipHostMallocDefault)) !=
            hipSuccess) {
          p->h_stage_need[w] = nullptr;
          (void)hipGetLastError();
          return pool_fail(PKV_ENOMEM, "pinned host allocation of the staging page map failed");
        }
        p->host_bytes += need_w;
        if (p->d_stage) {
          const int64_t lb = p->stage_heads * (int64_t)sizeof(int2);
          if (injected_failure(p))
            return pool_fail(PKV_ENOMEM, "injected allocation failure (PKV_FAIL_ALLOC_AT)");
          if ((e = hipHostMalloc((void**)&p->h_stage_items[w], (size_t)lb, hipHostMallocDefault)) !=
              hipSuccess) {
            p->h_stage_items[w] = nullptr;
            (void)hipGetLastError();
            return pool_fail(PKV_ENOMEM, "pinned host allocation of the staged page list failed");
          }
          p->host_bytes += lb;
        }
      }
      if (p->d_stage) {
        if (injected_failure(p))
          return pool_fail(PKV_ENOMEM, "injected allocation failure (PKV_FAIL_ALLOC_AT)");
        if ((e = hipHostMalloc((void**)&p->h_count, sizeof(int) * pkv_pool::kWindow,
                               hipHostMallocDefault)) != hipSuccess) {
          p->h_count = nullptr;
          (void)hipGetLastError();
          return pool_fail(PKV_ENOMEM, "pinned host allocation of the list lengths failed");
        }
        p->host_bytes += sizeof(int) * pkv_pool::kWindow;
      }
      try {
        p->adder = new HostAdder(host_add_threads());
      } catch (const std::exception&) {
        p->adder = nullptr;
        return pool_fail(PKV_ENOMEM, "could not start the host gradient add threads");
      }
    }
  }
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return pool_hip_fail(e, "hipDeviceSynchronize (pool init)");
  return PKV_OK;
}

pkv_status pool_release(pkv_pool* p) {
  pkv_status st = PKV_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) st = pool_hip_fail(e, "hipDeviceSynchronize (pool destroy)");
  delete p->adder;  // finishes the pending host adds
  p->adder = nullptr;
  for (int w = 0; w < pkv_pool::kWindow; ++w)
    for (void* x : {p->h_stage_dk[w], p->h_stage_dv[w], (void*)p->h_stage_need[w],
                    (void*)p->h_stage_items[w]})
      if (x) (void)hipHostFree(x);
  if (p->h_count) (void)hipHostFree(p->h_count);
  void* dev[] = {p->d_k, p->d_v, p->d_dk, p->d_dv, p->d_reps, p->d_table, p->d_wtable,
                 p->d_delta, p->d_select, p->d_fsplit, p->d_need, p->d_items, p->d_count,
                 p->d_moved, p->d_stage};
  for (void* x : dev)
    if (x) (void)hipFree(x);
  for (auto* v : {&p->h_k, &p->h_v, &p->h_dk, &p->h_dv})
    for (void* x : *v)
      if (x) (void)hipHostFree(x);
  if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
  if (p->ev_join) (void)hipEventDestroy(p->ev_join);
  if (p->s_aux) (void)hipStreamDestroy(p->s_aux);
  for (int w = 0; w < pkv_pool::kWindow; ++w) {
    if (p->ev_compute[w]) (void)hipEventDestroy(p->ev_compute[w]);
    if (p->ev_ready[w]) (void)hipEventDestroy(p->ev_ready[w]);
    if (p->ev_wb[w]) (void)hipEventDestroy(p->ev_wb[w]);
    for (int b = 0; b < 2; ++b)
      if (p->ev_list[w][b]) (void)hipEventDestroy(p->ev_list[w][b]);
    if (p->ev_count[w]) (void)hipEventDestroy(p->ev_count[w]);
  }
  if (p->ev_stage) (void)hipEventDestroy(p->ev_stage);
  return st;
}

pkv_status pool_append(pkv_pool* p, int layer, int64_t pos0, int64_t n_tok, const void* k,
                       const void* v, hipStream_t s) {
  const LayerDev L = store_view(p, layer);
  const Geom g = geom(p);
  hipError_t e;
  // A window's fetch may still be reading the partial last page that this
  // append writes: order the append after it.  (The window does not get the
  // new tokens; attention on them needs another prefetch, see
  // pool_before_compute.)
  const int w = p->window_of(layer);
  if (p->desc.host_tier && p->window_layer[w] == layer && p->ready_recorded[w] &&
      (e = hipStreamWaitEvent(s, p->ev_ready[w], 0)) != hipSuccess)
    return pool_hip_fail(e, "pkv_append_kv: hipStreamWaitEvent (window fetch)");
  e = launch_append(L, g, p->kv_bytes, pos0, n_tok, k, v, s);
  if (e != hipSuccess) return pool_hip_fail(e, "pkv_append_kv: append launch");
  const int64_t first = pos0 / g.page;
  const int64_t last = (pos0 + n_tok - 1) / g.page;
  e = launch_reps(L, g, p->desc.kv_dtype == PKV_BF16, first, last - first + 1, pos0 + n_tok, s);
  if (e != hipSuccess) return pool_hip_fail(e, "pkv_append_kv: representative launch");
  // A prefix prefetch that reserved the window's pages for these rows: write
  // them into the window as well (after its fetch, waited for above), so the
  // chunk can attend to its own keys without another prefetch.
  if (p->desc.host_tier && p->window_layer[w] == layer && pos0 + n_tok <= p->window_keys[w]) {
    e = launch_append(layer_view(p, layer), compute_geom(p), p->kv_bytes, pos0, n_tok, k, v, s);
    if (e != hipSuccess) {
      // the window lacks these rows now: it no longer holds the layer
      p->window_layer[w] = -1;
      p->window_grads[w] = false;
      p->window_keys[w] = 0;
      return pool_hip_fail(e, "pkv_append_kv: window append launch");
    }
    return pool_after_compute(p, layer, s);  // the next prefetch into the window waits for it
  }
  return PKV_OK;
}

pkv_status pool_grad_zero(pkv_pool* p, int layer, hipStream_t s) {
  hipError_t e;
  if (!p->desc.host_tier) {
    const LayerDev L = layer_view(p, layer);
    if ((e = launch_fill_zero(L.dk, p->layer_elems * 4, s)) != hipSuccess ||
        (e = launch_fill_zero(L.dv, p->layer_elems * 4, s)) != hipSuccess)
      return pool_hip_fail(e, "pkv_grad_zero");
    return PKV_OK;
  }
  // every transfer first: a writeback still in flight on a copy stream (or
  // an attention backward adding into the window) would otherwise land after
  // the zeros
  if ((e = hipDeviceSynchronize()) != hipSuccess) return pool_hip_fail(e, "pkv_grad_zero: sync");
  pkv_status st = pool_host_adds_wait(p);
  if (st != PKV_OK) return st;
  const int64_t hgr = p->layer_elems * grad_host_bytes(p);
  if ((e = launch_fill_zero(p->m_dk[layer], hgr, s)) != hipSuccess ||
      (e = launch_fill_zero(p->m_dv[layer], hgr, s)) != hipSuccess)
    return pool_hip_fail(e, "pkv_grad_zero (host tier)");
  const int w = p->window_of(layer);
  if (p->window_layer[w] == layer) {
    const LayerDev L = layer_view(p, layer);
    if ((e = launch_fill_zero(L.dk, p->dev_elems * 4, s)) != hipSuccess ||
        (e = launch_fill_zero(L.dv, p->dev_elems * 4, s)) != hipSuccess)
      return pool_hip_fail(e, "pkv_grad_zero (window)");
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return pool_hip_fail(e, "pkv_grad_zero: sync");
  return PKV_OK;
}

pkv_status pool_read(pkv_pool* p, int layer, int what, void* dst, hipStream_t s) {
  const Geom g = geom(p);
  const int64_t n_tok = p->length[layer];
  hipError_t e;
  if (!p->desc.host_tier || what == PKV_REPS) {
    e = launch_export(store_view(p, layer), g, what, p->kv_bytes, n_tok, dst, s);
  } else {
    if ((e = hipDeviceSynchronize()) != hipSuccess) return pool_hip_fail(e, "pkv_read_pages: sync");
    const pkv_status st = pool_host_adds_wait(p);
    if (st != PKV_OK) return st;
    if ((what == PKV_DK || what == PKV_DV) && p->desc.host_grad_dtype == PKV_BF16)
      e = launch_host_export(p, layer, what, n_tok, dst, s);
    else
      e = launch_export(store_view(p, layer), g, what, p->kv_bytes, n_tok, dst, s);
  }
  if (e != hipSuccess) return pool_hip_fail(e, "pkv_read_pages: launch");
  return PKV_OK;
}

// Zero the window's listed gradient pages on stream s if the visit still
// needs it (host accumulation), after the window's previous writeback.
static pkv_status zero_window_grads(pkv_pool* p, int layer, int w, hipStream_t s) {
  if (!p->zero_pending[w]) return PKV_OK;
  hipError_t e;
  if (p->wb_recorded[w] && (e = hipStreamWaitEvent(s, p->ev_wb[w], 0)) != hipSuccess)
    return pool_hip_fail(e, "hipStreamWaitEvent (window writeback)");
  if ((e = launch_window_grad_zero(p, layer, w, s)) != hipSuccess)
    return pool_hip_fail(e, "window gradient zero");
  p->zero_pending[w] = false;
  return PKV_OK;
}

pkv_status pool_before_compute(pkv_pool* p, int layer, int64_t q_end, hipStream_t s, bool grads) {
  if (!p->desc.host_tier) return PKV_OK;
  const int w = p->window_of(layer);
  if (p->window_layer[w] != layer)
    return pool_fail(PKV_ESTATE, "layer is not in the HBM window: call pkv_prefetch_pages first");
  if (q_end > p->window_keys[w])
    return pool_fail(PKV_ESTATE,
                     "queries reach past the keys the window's prefetch covered (tokens appended "
                     "after it, or a shorter prefix): call pkv_prefetch_pages again");
  // the backward adds into the window's gradients: they must be this
  // visit's (fetched, or zeroed for host adds) and not yet handed to a
  // writeback that ends the visit
  if (grads && !p->window_grads[w])
    return pool_fail(PKV_ESTATE,
                     "attention backward on a window whose gradients were not prefetched "
                     "(with_grads) or were already written back");
  if (p->ready_recorded[w]) {
    hipError_t e = hipStreamWaitEvent(s, p->ev_ready[w], 0);
    if (e != hipSuccess) return pool_hip_fail(e, "hipStreamWaitEvent (window ready)");
  }
  return grads ? zero_window_grads(p, layer, w, s) : PKV_OK;
}

pkv_status pool_after_compute(pkv_pool* p, int layer, hipStream_t s) {
  if (!p->desc.host_tier) return PKV_OK;
  const int w = p->window_of(layer);
  hipError_t e = hipEventRecord(p->ev_compute[w], s);
  if (e != hipSuccess) return pool_hip_fail(e, "hipEventRecord (window compute)");
  p->compute_recorded[w] = true;
  return PKV_OK;
}

pkv_status pool_prefetch(pkv_pool* p, int layer, const pkv_sel* sel, int64_t n_keys, bool with_grads,
                         hipStream_t cs, hipEvent_t ready) {
  const int w = p->window_of(layer);
  const pkv_pool_desc& d = p->desc;
  hipError_t e;
  // without a selection: the pages of keys 0 .. n_keys - 1 (n_keys = 0: every
  // appended key); n_keys may reach past the appended keys, whose pages the
  // window then holds for appends to come
  const int64_t n_avail = n_keys > 0 ? n_keys : p->length[layer];
  const int64_t n_pages = (n_avail + d.page_size - 1) / d.page_size;
  // the page-heads one KV head can need must fit the window's slots
  int64_t bound = n_pages;
  if (sel && (int64_t)sel->n_qpages * sel->stride < bound) bound = (int64_t)sel->n_qpages * sel->stride;
  if (bound > p->window_slots) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "prefetch could need %lld pages per KV head, the window holds %d (window_slots)",
             (long long)bound, p->window_slots);
    return pool_fail(PKV_ECAPACITY, msg);
  }
  // From here on the window's old content is given up (its table is
  // rewritten below): until this prefetch has been enqueued completely, no
  // layer is in the window, so that a prefetch that fails part-way leaves
  // attention on the window rejected (PKV_ESTATE) rather than reading pages
  // that were never fetched.
  p->window_layer[w] = -1;
  p->window_grads[w] = false;
  p->window_keys[w] = 0;
  p->zero_pending[w] = false;
  // K/V of the window are free once the attention calls on its last layer ran
  // and the window's previous fetch (possibly on another copy stream, and
  // possibly never used) has finished writing it
  if (p->compute_recorded[w]) {
    if ((e = hipStreamWaitEvent(cs, p->ev_compute[w], 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (window reuse)");
  }
  if (p->ready_recorded[w]) {
    if ((e = hipStreamWaitEvent(cs, p->ev_ready[w], 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (window's previous fetch)");
  }
  // build the other list buffer, once the writeback that last read it ran
  const int b = p->list_gen[w] ^ 1;
  if (p->list_recorded[w][b]) {
    if ((e = hipStreamWaitEvent(cs, p->ev_list[w][b], 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (window list)");
  }
  p->list_gen[w] = b;
  const int64_t nw = need_words(p);
  uint8_t* need = p->d_need + (int64_t)(w * 2 + b) * nw;
  if ((e = launch_need_clear(need, nw, cs)) != hipSuccess ||
      (e = launch_need_mark(need, sel, d.n_kv_heads, d.max_logical_pages, n_pages, cs)) != hipSuccess ||
      (e = launch_window_list(p, layer, w, n_pages, cs)) != hipSuccess)
    return pool_hip_fail(e, "pkv_prefetch_pages: page map");
  // the writeback sizes its staging copies by the list length
  if (p->d_stage) {
    if ((e = hipMemcpyAsync(p->h_count + w, p->d_count + (w * 2 + b), sizeof(int),
                            hipMemcpyDeviceToHost, cs)) != hipSuccess ||
        (e = hipEventRecord(p->ev_count[w], cs)) != hipSuccess)
      return pool_hip_fail(e, "pkv_prefetch_pages: list length");
  }
  // Gradients fetched into HBM (no host accumulation): one launch for K/V and
  // gradients after the window's last writeback has read its gradients.
  // Fetching K/V before that wait and the gradients after it ran the K/V
  // reads beside the writeback's host writes and made the 1M-token top-K
  // sweep slower.
  const bool grads_now = with_grads && !p->accumulate;
  if (grads_now && p->wb_recorded[w]) {
    if ((e = hipStreamWaitEvent(cs, p->ev_wb[w], 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (window writeback)");
  }
  if (injected_copy_failure(p)) return pool_hip_fail(hipErrorLaunchFailure,
                                                    "pkv_prefetch_pages: fetch (injected, PKV_FAIL_COPY_AT)");
  if ((e = launch_fetch(p, layer, w, cs, grads_now)) != hipSuccess)
    return pool_hip_fail(e, "pkv_prefetch_pages: fetch");
  p->window_layer[w] = layer;
  p->window_grads[w] = with_grads;
  p->window_keys[w] = n_avail;
  p->zero_pending[w] = with_grads && p->accumulate;
  if ((e = hipEventRecord(p->ev_ready[w], cs)) != hipSuccess)
    return pool_hip_fail(e, "hipEventRecord (window ready)");
  p->ready_recorded[w] = true;
  if (ready && (e = hipEventRecord(ready, cs)) != hipSuccess)
    return pool_hip_fail(e, "hipEventRecord (caller ready)");
  return PKV_OK;
}

pkv_status pool_writeback(pkv_pool* p, int layer, hipStream_t cs, hipEvent_t done) {
  const int w = p->window_of(layer);
  if (p->window_layer[w] != layer || !p->window_grads[w])
    return pool_fail(PKV_ESTATE,
                     "pkv_writeback_grads: the layer's gradients were not prefetched into the window");
  hipError_t e;
  if (p->compute_recorded[w]) {
    if ((e = hipStreamWaitEvent(cs, p->ev_compute[w], 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (writeback)");
  }
  // the prefetch filled the window on its own stream
  if (p->ready_recorded[w]) {
    if ((e = hipStreamWaitEvent(cs, p->ev_ready[w], 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (writeback after prefetch)");
  }
  if (p->accumulate) {
    // no attention backward since the prefetch: the contributions are zeros
    const pkv_status st = zero_window_grads(p, layer, w, cs);
    if (st != PKV_OK) return st;
    // the staging of window w is free once the adds of its last writeback ran
    if ((e = p->adder->wait(p->stage_ticket[w])) != hipSuccess)
      return pool_hip_fail(e, "host gradient adds: hipEventSynchronize");
  }
  if (injected_copy_failure(p)) return pool_hip_fail(hipErrorLaunchFailure,
                                                    "pkv_writeback_grads: (injected, PKV_FAIL_COPY_AT)");
  const pkv_pool_desc& d = p->desc;
  const int64_t need_w = need_words(p);
  const int b = p->list_gen[w];
  int n_staged = 0;
  if (p->d_stage) {
    // the list length the prefetch copied (long since on the host), and the
    // device staging once the previous staged writeback's copies read it
    if ((e = hipEventSynchronize(p->ev_count[w])) != hipSuccess)
      return pool_hip_fail(e, "hipEventSynchronize (window list length)");
    n_staged = p->h_count[w];
    n_staged = n_staged < 0 ? 0 : (n_staged > p->stage_heads ? (int)p->stage_heads : n_staged);
    if (p->stage_recorded && (e = hipStreamWaitEvent(cs, p->ev_stage, 0)) != hipSuccess)
      return pool_hip_fail(e, "hipStreamWaitEvent (writeback staging)");
    if ((e = launch_writeback_staged(p, w, n_staged, cs)) != hipSuccess)
      return pool_hip_fail(e, "pkv_writeback_grads: staging");
    if ((e = hipEventRecord(p->ev_stage, cs)) != hipSuccess)
      return pool_hip_fail(e, "hipEventRecord (writeback staging)");
    p->stage_recorded = true;
  } else {
    if ((e = launch_writeback_pages(p, layer, w, cs)) != hipSuccess)
      return pool_hip_fail(e, "pkv_writeback_grads: launch");
    if (p->accumulate &&
        (e = hipMemcpyAsync(p->h_stage_need[w], p->d_need + (int64_t)(w * 2 + b) * need_w,
                            (size_t)need_w, hipMemcpyDeviceToHost, cs)) != hipSuccess)
      return pool_hip_fail(e, "pkv_writeback_grads: page map copy");
  }
  if ((e = hipEventRecord(p->ev_list[w][b], cs)) != hipSuccess)
    return pool_hip_fail(e, "hipEventRecord (window list)");
  p->list_recorded[w][b] = true;
  if ((e = hipEventRecord(p->ev_wb[w], cs)) != hipSuccess)
    return pool_hip_fail(e, "hipEventRecord (writeback)");
  p->wb_recorded[w] = true;
  if (p->accumulate) {
    AddJob job;
    job.ready = p->ev_wb[w];
    if (p->d_stage) {
      job.list = p->h_stage_items[w];
      job.n_list = n_staged;
    }
    job.need = p->h_stage_need[w];
    const int32_t* tab = p->h_table.data() + (int64_t)layer * need_w;
    job.table.assign(tab, tab + need_w);
    job.hkv = d.n_kv_heads;
    job.max_logical = d.max_logical_pages;
    job.n_pages = (int)((p->length[layer] + d.page_size - 1) / d.page_size);
    job.slots = d.n_slots;
    job.page_elems = (int64_t)d.page_size * d.head_dim;
    job.bf16 = d.host_grad_dtype == PKV_BF16;
    job.src_dk = p->h_stage_dk[w];
    job.src_dv = p->h_stage_dv[w];
    job.dst_dk = p->h_dk[layer];
    job.dst_dv = p->h_dv[layer];
    p->stage_ticket[w] = p->adder->submit(job);
    p->layer_ticket[layer] = p->stage_ticket[w];
    p->window_grads[w] = false;  // a second writeback would add the same contributions again
  }
  if (done && (e = hipEventRecord(done, cs)) != hipSuccess)
    return pool_hip_fail(e, "hipEventRecord (writeback done)");
  return PKV_OK;
}

}  // namespace pkv

namespace pkv {

pkv_status pool_host_adds_wait(pkv_pool* p) {
  if (!p->adder) return PKV_OK;
  const hipError_t e = p->adder->drain();
  if (e != hipSuccess) return pool_hip_fail(e, "host gradient adds: hipEventSynchronize");
  return PKV_OK;
}

pkv_status pool_copy_stats(pkv_pool* p, int64_t* fetched, int64_t* written) {
  unsigned long long h[2] = {0, 0};
  if (p->d_moved) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return pool_hip_fail(e, "pkv_offload_bytes: sync");
    const pkv_status st = pool_host_adds_wait(p);
    if (st != PKV_OK) return st;
    e = hipMemcpy(h, p->d_moved, sizeof h, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return pool_hip_fail(e, "pkv_offload_bytes: copy");
  }
  if (fetched) *fetched = (int64_t)h[0];
  if (written) *written = (int64_t)h[1];
  return PKV_OK;
}

}  // namespace pkv
