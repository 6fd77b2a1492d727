// Per-kind kernel timing with HIP events on the launching stream.
#include <hip/hip_runtime.h>

#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

struct Pending {
  int kind;
  hipEvent_t a, b;
};

bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
double g_ms[KT_COUNT];
int64_t g_n[KT_COUNT];

hipEvent_t get_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void resolve() {
  for (const Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      g_ms[p.kind] += ms;
      g_n[p.kind] += 1;
    }
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.clear();
}

}  // namespace

bool kernel_timing_on() { return g_on; }

KernelTimer::KernelTimer(int kind, hipStream_t s) : kind_(kind), s_(s), start_(nullptr) {
  if (!g_on) return;
  hipEvent_t e = get_event();
  if (e && hipEventRecord(e, s) == hipSuccess) start_ = e;
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  hipEvent_t e = get_event();
  if (e && hipEventRecord(e, s_) == hipSuccess) {
    g_pending.push_back({kind_, (hipEvent_t)start_, e});
  } else {
    g_free.push_back((hipEvent_t)start_);
    if (e) g_free.push_back(e);
  }
}

}  // namespace pkv

extern "C" {

pkv_status pkv_kernel_timing(int32_t enable) {
  using namespace pkv;
  resolve();
  for (int k = 0; k < KT_COUNT; ++k) {
    g_ms[k] = 0.0;
    g_n[k] = 0;
  }
  g_on = enable != 0;
  return PKV_OK;
}

pkv_status pkv_kernel_times(int32_t n, double* total_ms, int64_t* launches) {
  using namespace pkv;
  resolve();
  for (int k = 0; k < n && k < KT_COUNT; ++k) {
    if (total_ms) total_ms[k] = g_ms[k];
    if (launches) launches[k] = g_n[k];
  }
  return PKV_OK;
}

}  // extern "C"
