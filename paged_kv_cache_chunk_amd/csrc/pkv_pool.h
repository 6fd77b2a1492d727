// The pool object behind the opaque pkv_pool handle, and the pool-level
// operations the C ABI dispatches to (pkv_pool.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "host_add.h"
#include "pkv.h"
#include "pkv_internal.h"

struct pkv_pool {
  pkv_pool_desc desc{};
  int kv_bytes = 2;          // bytes per K/V element
  int64_t layer_elems = 0;   // Hkv * n_slots * P * d: one layer of the pool (host tier: of the tier)
  // Host tier: HBM slots per KV head in each window (desc.window_slots, or a
  // whole layer's max_logical_pages), and the elements of one device copy of
  // K, V, dK or dV (a window with a host tier, a layer without)
  int window_slots = 0;
  int64_t dev_elems = 0;
  std::vector<int64_t> length;    // appended tokens per layer
  std::vector<int32_t> h_table;   // [layers][Hkv][max_logical], host mirror

  // Device buffers.  Without a host tier: n_layers copies of K, V, dK, dV
  // ([Hkv][n_slots][P][d] each).  With a host tier: kWindow windows of
  // [Hkv][window_slots][P][d] each, a window's pages reached through its
  // table d_wtable[w] ([Hkv][max_logical]: logical page -> window slot).
  void* d_k = nullptr;
  void* d_v = nullptr;
  float* d_dk = nullptr;
  float* d_dv = nullptr;
  float* d_reps = nullptr;        // [layers][Hkv][slots][d]
  int32_t* d_table = nullptr;     // [layers][Hkv][max_logical]
  int32_t* d_wtable = nullptr;    // host tier: [kWindow][Hkv][max_logical]
  void* d_delta = nullptr;        // attn_bwd scratch
  // attn_bwd (bf16) runs dQ and dK/dV side by side: dK/dV on this stream,
  // forked from and joined back to the caller's stream with the two events
  hipStream_t s_aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  int64_t delta_bytes = 0;
  void* d_select = nullptr;       // select scratch
  int64_t select_bytes = 0;
  // bf16 top-K forward: partial results of the tail split's parts
  void* d_fsplit = nullptr;
  int64_t fsplit_bytes = 0;
  int n_cus = 0;                  // compute units of the pool's device
  int64_t device_bytes = 0;
  int64_t host_bytes = 0;
  int allocs = 0;  // allocations made so far by pool creation (failure-injection hook)
  int copies = 0;  // host-link copies enqueued so far (failure-injection hook)

  // Host tier (pinned, device-mapped), per layer.
  static constexpr int kWindow = 2;
  std::vector<void*> h_k, h_v, h_dk, h_dv;      // host pointers
  std::vector<void*> m_k, m_v, m_dk, m_dv;      // device-visible aliases
  int window_layer[kWindow] = {-1, -1};
  bool window_grads[kWindow] = {false, false};  // grads of the needed pages were fetched
  // keys of the window's layer present when its last prefetch ran (a prefix
  // prefetch: the keys it names): attention needs queries below this, since
  // tokens appended later are not in the window
  int64_t window_keys[kWindow] = {0, 0};
  hipEvent_t ev_compute[kWindow] = {nullptr, nullptr};  // after the last attention call
  hipEvent_t ev_ready[kWindow] = {nullptr, nullptr};    // after the last prefetch
  hipEvent_t ev_wb[kWindow] = {nullptr, nullptr};       // after the last grad writeback
  bool wb_recorded[kWindow] = {false, false};
  bool compute_recorded[kWindow] = {false, false};
  bool ready_recorded[kWindow] = {false, false};
  // Page map and list of each window, double-buffered: a prefetch builds
  // buffer list_gen[w] ^ 1 while the window's last writeback may still read
  // buffer list_gen[w]; ev_list[w][b] is recorded after the writeback that
  // read buffer b.
  uint8_t* d_need = nullptr;      // [kWindow][2][Hkv][max_logical] page-heads held by the window
  // [kWindow][2][Hkv * window_slots] the listed page-heads: (tier page-head
  // g * n_slots + slot, window page-head g * window_slots + window slot)
  int2* d_items = nullptr;
  int* d_count = nullptr;         // [kWindow][2] list lengths
  int list_gen[kWindow] = {0, 0};
  hipEvent_t ev_list[kWindow][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
  bool list_recorded[kWindow][2] = {{false, false}, {false, false}};
  unsigned long long* d_moved = nullptr;  // [0] bytes fetched, [1] bytes written back

  // host_grad_accumulate: window gradients start at zero on every prefetch;
  // a writeback stages the visit's contributions (host gradient dtype) in
  // pinned memory, in window-list order with the window list (device
  // staging below) or indexed like the tier with the window's page map, and
  // `adder` adds them into the layer's host gradients.  stage_ticket[w] is
  // the add job that still reads window w's staging.
  bool accumulate = false;
  void* h_stage_dk[kWindow] = {nullptr, nullptr};
  void* h_stage_dv[kWindow] = {nullptr, nullptr};
  void* m_stage_dk[kWindow] = {nullptr, nullptr};   // device-visible aliases
  void* m_stage_dv[kWindow] = {nullptr, nullptr};
  uint8_t* h_stage_need[kWindow] = {nullptr, nullptr};
  int64_t stage_ticket[kWindow] = {0, 0};
  std::vector<int64_t> layer_ticket;  // per layer: ticket of its last add job (0: none)
  // With room in the HBM budget, the writeback converts the visit's
  // contributions into d_stage in window-list order (dK in the first
  // stage_heads page-heads, dV in the next), and one runtime copy each
  // (hipMemcpyAsync, made on a DMA engine) moves them, and the list, to the
  // window's pinned staging: that slows the copy kernels' host reads on the
  // link far less than kernel writes to mapped host memory do.
  // d_stage == nullptr: the writeback kernel writes the pinned staging
  // itself, indexed like the tier.  h_count[w] is the window list length of
  // w's last prefetch (copied after the list is built, ev_count[w]);
  // ev_stage follows the last staging copy, after which d_stage is free.
  char* d_stage = nullptr;
  int64_t stage_heads = 0;  // Hkv * window_slots
  hipEvent_t ev_stage = nullptr;
  bool stage_recorded = false;
  int* h_count = nullptr;
  hipEvent_t ev_count[kWindow] = {nullptr, nullptr};
  int2* h_stage_items[kWindow] = {nullptr, nullptr};
  // the window's gradient pages still have to be zeroed: done on the stream
  // of the first attention backward (or writeback) of the visit, so that the
  // prefetch stream never waits for the window's previous writeback
  bool zero_pending[kWindow] = {false, false};
  pkv::HostAdder* adder = nullptr;

  int window_of(int layer) const { return layer % kWindow; }
};

namespace pkv {

pkv_status pool_fail(pkv_status st, const char* msg);
pkv_status pool_hip_fail(hipError_t e, const char* what);
// What the attention kernels read and write for `layer`: its HBM pool, or
// with a host tier the window holding it (window table, window slots).
LayerDev layer_view(pkv_pool* p, int layer);
Geom compute_geom(const pkv_pool* p);
// The layer's own store: its HBM pool, or the device-mapped host tier; page
// table and representatives of the layer (slots = n_slots).
LayerDev store_view(pkv_pool* p, int layer);
Geom geom(const pkv_pool* p);
pkv_status ensure_scratch(void** buf, int64_t* have, int64_t need);

pkv_status pool_allocate(pkv_pool* p);
pkv_status pool_release(pkv_pool* p);
pkv_status pool_append(pkv_pool* p, int layer, int64_t pos0, int64_t n_tok, const void* k,
                       const void* v, hipStream_t s);
pkv_status pool_grad_zero(pkv_pool* p, int layer, hipStream_t s);
pkv_status pool_read(pkv_pool* p, int layer, int what, void* dst, hipStream_t s);
pkv_status pool_before_compute(pkv_pool* p, int layer, int64_t q_end, hipStream_t s, bool grads);
pkv_status pool_after_compute(pkv_pool* p, int layer, hipStream_t s);
pkv_status pool_prefetch(pkv_pool* p, int layer, const pkv_sel* sel, int64_t n_keys, bool with_grads,
                         hipStream_t copy_stream, hipEvent_t ready);
pkv_status pool_writeback(pkv_pool* p, int layer, hipStream_t copy_stream, hipEvent_t done);
pkv_status pool_copy_stats(pkv_pool* p, int64_t* fetched, int64_t* written);

// pkv_api.cpp: the attention backward with the pool's own scratch (scratch ==
// nullptr) or scratch_cap bytes of the caller's (no allocation)
pkv_status attn_bwd_impl(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                         int32_t n_q_heads, float scale, const void* q, const void* o,
                         const void* dout, const float* lse, const pkv_sel* sel, float* dq,
                         hipStream_t stream, void* scratch, int64_t scratch_cap, const char* who);

// offload.hip
hipError_t launch_need_clear(uint8_t* need, int64_t n, hipStream_t s);
hipError_t launch_need_mark(uint8_t* need, const pkv_sel* sel, int hkv, int max_logical,
                            int64_t n_pages_all, hipStream_t s);
int64_t need_words(const pkv_pool* p);  // Hkv * max_logical
hipError_t launch_window_list(const pkv_pool* p, int layer, int window, int64_t n_pages,
                              hipStream_t s);
hipError_t launch_fetch(const pkv_pool* p, int layer, int window, hipStream_t s,
                        bool with_grads);
hipError_t launch_window_grad_zero(const pkv_pool* p, int layer, int window, hipStream_t s);
hipError_t launch_writeback_pages(const pkv_pool* p, int layer, int window, hipStream_t s);
// Host accumulation with the device staging: the window list's first n
// page-heads into d_stage (list order), then DMA copies of the staging and
// the list to the window's pinned staging.
hipError_t launch_writeback_staged(const pkv_pool* p, int window, int n, hipStream_t s);
pkv_status pool_host_adds_wait(pkv_pool* p);
hipError_t launch_host_export(const pkv_pool* p, int layer, int what, int64_t n_tok, void* dst,
                              hipStream_t s);
// host_grad_accumulate: rows [t0, t0 + n_tok) of the layer's dK or dV as
// the window's contributions plus the host tier's sums (fp32 out); the host
// adds of the layer's earlier writebacks must have run.
hipError_t launch_grad_rows_sum(const pkv_pool* p, int layer, int what, int64_t t0, int64_t n_tok,
                                float* dst, hipStream_t s);

}  // namespace pkv
