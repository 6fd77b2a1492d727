// Host-side accumulation of staged gradient contributions into the host
// tier: a coordinator thread takes jobs in order, waits for the staging
// copies' event, lists the staged page-heads (from the copied window list, or
// from the copied page map), and splits them over a small team of threads.  bf16 sums are rounded to
// nearest-even, as the device's conversion does.
#include "host_add.h"

#include <cstring>

// Host code only: the file is compiled as HIP, and the CPU feature builtins
// below have no meaning in the gfx950 pass.
#ifndef __HIP_DEVICE_COMPILE__

namespace pkv {
namespace {

inline __attribute__((always_inline)) void add_bf16_span(uint16_t* __restrict__ dst,
                                                         const uint16_t* __restrict__ src,
                                                         int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t a = (uint32_t)dst[i] << 16, b = (uint32_t)src[i] << 16;
    float fa, fb;
    std::memcpy(&fa, &a, 4);
    std::memcpy(&fb, &b, 4);
    const float s = fa + fb;
    uint32_t u;
    std::memcpy(&u, &s, 4);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet = (u >> 16) | 0x40u;  // NaN stays NaN
    dst[i] = (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
  }
}

inline __attribute__((always_inline)) void add_f32_span(float* __restrict__ dst,
                                                        const float* __restrict__ src,
                                                        int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] += src[i];
}

__attribute__((target("avx2"))) void add_bf16_avx2(uint16_t* dst, const uint16_t* src, int64_t n) {
  add_bf16_span(dst, src, n);
}
void add_bf16_base(uint16_t* dst, const uint16_t* src, int64_t n) { add_bf16_span(dst, src, n); }
__attribute__((target("avx2"))) void add_f32_avx2(float* dst, const float* src, int64_t n) {
  add_f32_span(dst, src, n);
}
void add_f32_base(float* dst, const float* src, int64_t n) { add_f32_span(dst, src, n); }

bool has_avx2() {
  static const bool v = (__builtin_cpu_init(), __builtin_cpu_supports("avx2"));
  return v;
}

void add(void* dst, int64_t d0, const void* src, int64_t s0, int64_t n, bool bf16) {
  const bool kAvx2 = has_avx2();
  if (bf16) {
    uint16_t* d = (uint16_t*)dst + d0;
    const uint16_t* s = (const uint16_t*)src + s0;
    kAvx2 ? add_bf16_avx2(d, s, n) : add_bf16_base(d, s, n);
  } else {
    float* d = (float*)dst + d0;
    const float* s = (const float*)src + s0;
    kAvx2 ? add_f32_avx2(d, s, n) : add_f32_base(d, s, n);
  }
}

}  // namespace

HostAdder::HostAdder(int n_threads) {
  if (n_threads < 1) n_threads = 1;
  coord_ = std::thread([this] { coordinator(); });
  for (int t = 1; t < n_threads; ++t) team_.emplace_back([this] { helper(); });
}

HostAdder::~HostAdder() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  cv_job_.notify_all();
  coord_.join();  // the coordinator finishes the queue before it leaves
  cv_team_.notify_all();
  for (auto& t : team_) t.join();
}

int64_t HostAdder::submit(const AddJob& job) {
  int64_t ticket;
  {
    std::lock_guard<std::mutex> lk(mu_);
    ticket = ++submitted_;
    q_.emplace_back(ticket, job);
  }
  cv_job_.notify_one();
  return ticket;
}

hipError_t HostAdder::wait(int64_t ticket) {
  std::unique_lock<std::mutex> lk(mu_);
  cv_done_.wait(lk, [&] { return done_ >= ticket; });
  return err_;
}

hipError_t HostAdder::drain() {
  int64_t last;
  {
    std::lock_guard<std::mutex> lk(mu_);
    last = submitted_;
  }
  return wait(last);
}

void HostAdder::run_items() {
  const int64_t n = (int64_t)items_.size();
  for (;;) {
    const int64_t i = next_.fetch_add(1, std::memory_order_relaxed);
    if (i >= n) break;
    const auto [src, dst] = items_[i];
    add(cur_.dst_dk, dst, cur_.src_dk, src, cur_.page_elems, cur_.bf16);
    add(cur_.dst_dv, dst, cur_.src_dv, src, cur_.page_elems, cur_.bf16);
  }
}

void HostAdder::coordinator() {
  for (;;) {
    std::pair<int64_t, AddJob> job;
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_job_.wait(lk, [&] { return stop_ || !q_.empty(); });
      if (q_.empty()) return;  // stopping, nothing left
      job = std::move(q_.front());
      q_.pop_front();
    }
    const hipError_t e = hipEventSynchronize(job.second.ready);
    if (e == hipSuccess) {
      cur_ = std::move(job.second);
      items_.clear();
      const int64_t tier_heads = (int64_t)cur_.hkv * cur_.slots;
      if (cur_.list) {
        for (int i = 0; i < cur_.n_list; ++i) {
          const int64_t h = cur_.list[i].x;
          if (h >= 0 && h < tier_heads)
            items_.emplace_back((int64_t)i * cur_.page_elems, h * cur_.page_elems);
        }
      } else {
        for (int g = 0; g < cur_.hkv; ++g)
          for (int j = 0; j < cur_.n_pages; ++j) {
            const int64_t at = (int64_t)g * cur_.max_logical + j;
            const int slot = cur_.table[at];
            if (cur_.need[at] && slot >= 0 && slot < cur_.slots) {
              const int64_t e = ((int64_t)g * cur_.slots + slot) * cur_.page_elems;
              items_.emplace_back(e, e);
            }
          }
      }
      next_.store(0, std::memory_order_relaxed);
      {
        std::lock_guard<std::mutex> lk(mu_);
        pending_ = (int)team_.size();
        ++gen_;
      }
      cv_team_.notify_all();
      run_items();
      std::unique_lock<std::mutex> lk(mu_);
      cv_fin_.wait(lk, [&] { return pending_ == 0; });
    }
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (e != hipSuccess && err_ == hipSuccess) err_ = e;
      done_ = job.first;
    }
    cv_done_.notify_all();
  }
}

void HostAdder::helper() {
  int64_t seen = 0;
  for (;;) {
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_team_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (gen_ == seen) return;  // stopping
      seen = gen_;
    }
    run_items();
    std::lock_guard<std::mutex> lk(mu_);
    if (--pending_ == 0) cv_fin_.notify_one();
  }
}

}  // namespace pkv

#endif  // __HIP_DEVICE_COMPILE__
