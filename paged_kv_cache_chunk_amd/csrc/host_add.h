// Host-side accumulation of gradient contributions into the host tier
// (host_add.cpp).
//
// With host_grad_accumulate, a layer's window gradients start each visit at
// zero and its writeback stages only that visit's dK/dV contributions in
// pinned memory; this team of host threads then adds them into the layer's
// host gradient pages, so the gradients never travel host -> HBM.  Jobs run
// in submission order, one at a time, each split over the team by page-head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <thread>
#include <vector>

namespace pkv {

// The staged page-heads come either as a list (list != nullptr: staging
// page-head i goes to tier page-head list[i].x, the window list's entries)
// or as a page map with the layer's table (staging indexed like the tier).
struct AddJob {
  hipEvent_t ready = nullptr;      // recorded after the staging copies
  const int2* list = nullptr;      // [n_list] (tier page-head, window page-head), pinned
  int n_list = 0;
  const uint8_t* need = nullptr;   // [hkv][max_logical] staged page-heads (pinned)
  std::vector<int32_t> table;      // [hkv][max_logical] logical page -> slot, a copy
  int hkv = 0, max_logical = 0, n_pages = 0, slots = 0;
  int64_t page_elems = 0;
  bool bf16 = true;                // element type of staging and tier
  const void* src_dk = nullptr;    // staging
  const void* src_dv = nullptr;
  void* dst_dk = nullptr;          // host tier of the layer
  void* dst_dv = nullptr;
};

class HostAdder {
 public:
  explicit HostAdder(int n_threads);
  ~HostAdder();  // finishes every submitted job, then joins the team
  HostAdder(const HostAdder&) = delete;
  HostAdder& operator=(const HostAdder&) = delete;

  // Queue a job; returns its ticket (1, 2, ...).
  int64_t submit(const AddJob& job);
  // Block until job `ticket` (and every earlier one) is done; 0 returns at
  // once.  Returns the first HIP error a job met (its adds were skipped).
  hipError_t wait(int64_t ticket);
  hipError_t drain();

 private:
  void coordinator();
  void helper();
  void run_items();

  std::vector<std::thread> team_;
  std::thread coord_;
  std::mutex mu_;
  std::condition_variable cv_job_, cv_done_, cv_team_, cv_fin_;
  std::deque<std::pair<int64_t, AddJob>> q_;
  int64_t submitted_ = 0, done_ = 0;
  bool stop_ = false;
  hipError_t err_ = hipSuccess;
  // the job being split over the team
  AddJob cur_;
  // element offsets of the staged page-heads: in the staging, in the tier
  std::vector<std::pair<int64_t, int64_t>> items_;
  std::atomic<int64_t> next_{0};
  int64_t gen_ = 0;
  int pending_ = 0;             // helpers still working on generation gen_
};

}  // namespace pkv
