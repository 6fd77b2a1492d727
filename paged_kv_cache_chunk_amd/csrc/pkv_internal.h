// Internal declarations shared by the host side of libpkv and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Device view of one layer's pools.
//   k, v    [Hkv][slots][P][d] in the pool's kv dtype
//   dk, dv  [Hkv][slots][P][d] fp32 (accumulated in place with atomics)
//   reps    [Hkv][slots][d] fp32 page representative (mean of the page's keys)
//   table   [Hkv][max_logical] int32 logical page -> slot
struct LayerDev {
  void* k;
  void* v;
  float* dk;
  float* dv;
  float* reps;
  const int32_t* table;
};

struct Geom {
  int hkv;
  int d;
  int page;
  int slots;
  int max_logical;
};

// Selection in device memory; pages == nullptr means dense.
struct SelDev {
  const int32_t* pages;
  const int32_t* count;
  int n_qpages;
  int stride;
};

// Work list of the sparse bf16 dK/dV kernel, built on the device by a planning
// kernel from the selection (int32 words at base):
//   [0]                  number of work items
//   cnt  [hkv][n_pages]  query pages whose selection holds key page p (head g)
//   mask [hkv][n_pages][mask_words]  those query pages as a bit mask
//   items[max_items]     two int4 each: {g, 128-key slab, first, end iteration}
//                        and {slot of the slab's page, query pages, mask words 0, 1}
struct DkvPlan {
  int* base;
  int n_pages;     // key pages of the chunk's context
  int qpi;         // query pages per work item (at most 1024)
  int mask_words;  // 32-bit words per (KV head, key page) query-page mask
  int64_t off_cnt, off_mask, off_items;
  int max_items;
  int64_t bytes;
};

// Tail split of a bf16 forward launch whose work units (128 query rows of one
// head) all cost about the same, as in top-K mode, where every query page
// attends the same number of pages.  The kernel fits two workgroups on a CU,
// so U units on S = 2 x CUs slots take ceil(U / S) passes of work although
// they hold U / S: with U = q S + r, the last pass leaves S - r slots idle.
// The last r units are therefore cut in two along their key tiles, a first
// part with the fraction cut_num / cut_den of the tiles (r / S, or 1/2 when
// r < S / 2) and a second part with the rest.  Dispatched after the q S whole
// units, the r first parts take r slots while the other S - r slots run the r
// second parts, so every slot finishes after about q + r / S units.  Each
// part stores its partial result (O unnormalised, the reference maximum and
// the row sums); a second kernel combines the two parts of every split unit
// and writes its O and log-sum-exp.
struct TailSplit {
  int n_whole = 0;   // units [0, n_whole) run whole
  int n_split = 0;   // units [n_whole, n_whole + n_split) run in two parts; 0: no split
  int cut_num = 1, cut_den = 2;
  float* part = nullptr;  // [n_split][2 parts][4 waves][kFwdPartWaveFloats]
};

// Query rows of one bf16 forward work unit (one workgroup, four waves).
constexpr int kFwdRows = 128;

// Floats of one wave's partial forward result: O (32 rows x 128 columns),
// then the reference maximum and the row sum of each of its 64 lanes.
constexpr int kFwdPartWaveFloats = 32 * 128 + 2 * 64;

// The split of a forward launch of `units` work units on a device with
// `slots` workgroup slots (part left unset).
TailSplit plan_tail_split(int units, int slots);

// Everything an attention launch needs.
struct AttnCall {
  LayerDev L;
  Geom g;
  int hq;
  int64_t q_pos0;
  int n_q;
  float scale;
  SelDev sel;
  const void* q;
  const void* o;
  const void* dout;
  void* o_out;
  float* lse;
  const float* lse_in;
  float* delta;  // D = rowsum(dO * O), [hq][n_q]
  float* lse2;   // lse * log2(e), [hq][n_q] (bf16 backward only)
  float* dq;
  DkvPlan plan;  // sparse bf16 backward only
  TailSplit split;  // sparse bf16 forward only
};

// Whether kernel timing (pkv_kernel_timing) is on.
bool kernel_timing_on();

// Brackets one kernel launch with timing events when kernel timing is on
// (pkv_kernel_timing); a no-op otherwise.
class KernelTimer {
 public:
  KernelTimer(int kind, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  int kind_;
  hipStream_t s_;
  void* start_;
};

enum { KT_APPEND = 0, KT_SELECT, KT_FWD, KT_DELTA, KT_DQ, KT_DKDV, KT_FETCH, KT_WRITEBACK, KT_COUNT };

// ---- kernels in kv_pages.hip
hipError_t launch_append(const LayerDev& L, const Geom& g, int elem_bytes, int64_t pos0,
                         int64_t n_tok, const void* k, const void* v, hipStream_t s);
hipError_t launch_reps(const LayerDev& L, const Geom& g, bool bf16, int64_t first_page,
                       int64_t n_pages, int64_t length, hipStream_t s);
hipError_t launch_export(const LayerDev& L, const Geom& g, int what, int elem_bytes,
                         int64_t n_tok, void* dst, hipStream_t s, int64_t t0 = 0);
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s);

// ---- kernels in select_topk.hip
hipError_t launch_select(const LayerDev& L, const Geom& g, bool bf16, int hq, int64_t q_pos0,
                         int n_q, const void* q, int top_k, int n_sink, int n_local,
                         int32_t* sel_pages, int32_t* sel_count, int sel_stride,
                         float* scratch, hipStream_t s);
int64_t select_scratch_floats(const Geom& g, int64_t q_pos0, int n_q, int n_sink, int n_local);

// ---- kernels in attn_f32.hip
hipError_t launch_fwd_f32(const AttnCall& c, hipStream_t s);
hipError_t launch_bwd_f32(const AttnCall& c, hipStream_t s);

// ---- kernels in attn_bf16_fwd.hip, attn_bf16_dq.hip, attn_bf16_dkdv.hip
hipError_t launch_fwd_bf16(const AttnCall& c, hipStream_t s);
// D, lse2, dQ, dK/dV; dK/dV runs on `aux` (forked from s after D / lse2 with
// ev_fork, joined back into s with ev_join) while dQ runs on s, so that the
// two kernels fill each other's last partial wave of workgroups.  aux may be
// null: everything on s.
hipError_t launch_bwd_bf16(const AttnCall& c, hipStream_t s, hipStream_t aux, hipEvent_t ev_fork,
                           hipEvent_t ev_join);
hipError_t launch_dq_bf16(const AttnCall& c, hipStream_t s);   // dQ only (D, lse2 written)
// Sizes of the sparse dK/dV work list for a chunk (base left null).
DkvPlan dkdv_plan_layout(const Geom& g, int hq, int64_t q_pos0, int n_q, int sel_stride);

// ---- measurement kernels in micro.hip (not used by the attention path)
hipError_t launch_micro_gather(const AttnCall& c, float* out, hipStream_t s);
hipError_t launch_micro_atomics(const AttnCall& c, int reps, float value, hipStream_t s);

// ---- kernels in attn_common.hip
hipError_t launch_delta(const AttnCall& c, bool bf16, hipStream_t s);

}  // namespace pkv
