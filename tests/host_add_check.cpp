// CPU check of the host gradient-add team (csrc/host_add.cpp), built with
// g++ against a stand-in for hipEventSynchronize (no GPU is involved).
//
// It drives the team the way the pool's writeback does: two staging areas
// (one per window) used alternately, each refilled only after the add job
// that last read it has finished; random page maps, random page tables,
// random contributions.  Every other job hands its page-heads as a list
// (staging in list order, each entry naming its tier page-head, in a random
// order), the others as a page map (staging indexed like the tier).  The tier must end bit-identical to adding every
// job's contributions one job after the other, in submission order, with
// round-to-nearest-even to bf16 (or fp32 adds).
//
//   host_add_check <threads> <jobs> <bf16 0|1> <seed>
// prints "ok <jobs> <events>" or the first mismatch.
#include <atomic>
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "host_add.h"

static std::atomic<int> g_events{0};

// The stand-in: "the staging copies are done" after a short random delay.
extern "C" hipError_t hipEventSynchronize(hipEvent_t) {
  thread_local std::mt19937 r(12345);
  std::this_thread::sleep_for(std::chrono::microseconds(r() % 200));
  g_events.fetch_add(1);
  return hipSuccess;
}

static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Nearest bf16 of a finite float, ties to the even mantissa, found by
// comparing the two neighbouring bf16 values.
static uint16_t float_to_bf16_nearest(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint16_t down = (uint16_t)(u >> 16);  // toward zero
  const uint16_t up = (uint16_t)(down + 1);   // away from zero
  const double dd = std::fabs((double)f - (double)bf16_to_float(down));
  const double du = std::fabs((double)bf16_to_float(up) - (double)f);
  if (dd < du) return down;
  if (du < dd) return up;
  return (down & 1) ? up : down;
}

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const int threads = std::atoi(argv[1]), jobs = std::atoi(argv[2]);
  const bool bf16 = std::atoi(argv[3]) != 0;
  std::mt19937_64 rng((uint64_t)std::atoll(argv[4]));
  const int hkv = 2, max_logical = 48, n_pages = 40, slots = 56;
  const int64_t page_elems = 64;
  const int64_t elems = (int64_t)hkv * slots * page_elems;
  const int esz = bf16 ? 2 : 4;

  // [0] dK, [1] dV: tiers, serial references, and per window staging
  std::vector<char> tier[2], expect[2], stage[2][2];
  for (int x = 0; x < 2; ++x) {
    tier[x].resize(elems * esz);
    expect[x].resize(elems * esz);
    stage[0][x].resize(elems * esz);
    stage[1][x].resize(elems * esz);
  }
  std::vector<uint8_t> need[2] = {std::vector<uint8_t>(hkv * max_logical),
                                  std::vector<uint8_t>(hkv * max_logical)};
  std::vector<int2> list[2];
  std::normal_distribution<float> nd(0.f, 1.f);
  auto put = [&](std::vector<char>& b, int64_t i, float x) {
    if (bf16) {
      const uint16_t h = float_to_bf16_nearest(x);
      std::memcpy(b.data() + 2 * i, &h, 2);
    } else {
      std::memcpy(b.data() + 4 * i, &x, 4);
    }
  };
  auto get = [&](const std::vector<char>& b, int64_t i) {
    if (bf16) {
      uint16_t h;
      std::memcpy(&h, b.data() + 2 * i, 2);
      return bf16_to_float(h);
    }
    float x;
    std::memcpy(&x, b.data() + 4 * i, 4);
    return x;
  };
  for (int x = 0; x < 2; ++x)
    for (int64_t i = 0; i < elems; ++i) {
      put(tier[x], i, nd(rng));
      std::memcpy(expect[x].data() + i * esz, tier[x].data() + i * esz, esz);
    }

  int64_t ticket[2] = {0, 0};
  {
    pkv::HostAdder adder(threads);
    for (int t = 0; t < jobs; ++t) {
      const int w = t % 2;
      if (adder.wait(ticket[w]) != hipSuccess) return 3;  // staging w is free again
      std::vector<int32_t> table(hkv * max_logical, -1);
      for (int g = 0; g < hkv; ++g) {
        std::vector<int32_t> perm(slots);
        for (int s = 0; s < slots; ++s) perm[s] = s;
        std::shuffle(perm.begin(), perm.end(), rng);
        for (int j = 0; j < max_logical; ++j) table[g * max_logical + j] = perm[j];
      }
      const double density = 0.1 + 0.8 * (double)(rng() % 1000) / 1000.0;
      const bool as_list = t % 4 >= 2;  // alternate per window
      list[w].clear();
      for (int g = 0; g < hkv; ++g)
        for (int j = 0; j < max_logical; ++j) {
          const bool on = j < n_pages && (double)(rng() % 1000) / 1000.0 < density;
          need[w][g * max_logical + j] = on ? 1 : 0;
          if (on) list[w].push_back(make_int2(g * slots + table[g * max_logical + j], 0));
        }
      if (as_list) std::shuffle(list[w].begin(), list[w].end(), rng);
      for (size_t i = 0; i < list[w].size(); ++i) {
        const int64_t e0 = (int64_t)list[w][i].x * page_elems;         // tier
        const int64_t s0 = as_list ? (int64_t)i * page_elems : e0;      // staging
        for (int x = 0; x < 2; ++x)
          for (int64_t e = 0; e < page_elems; ++e) {
            put(stage[w][x], s0 + e, 0.25f * nd(rng));
            // the serial reference: one rounded add per element and job
            const float sum = get(expect[x], e0 + e) + get(stage[w][x], s0 + e);
            put(expect[x], e0 + e, sum);
          }
      }
      pkv::AddJob job;
      job.ready = nullptr;
      if (as_list) {
        job.list = list[w].data();
        job.n_list = (int)list[w].size();
      }
      job.need = need[w].data();
      job.table = table;
      job.hkv = hkv;
      job.max_logical = max_logical;
      job.n_pages = n_pages;
      job.slots = slots;
      job.page_elems = page_elems;
      job.bf16 = bf16;
      job.src_dk = stage[w][0].data();
      job.src_dv = stage[w][1].data();
      job.dst_dk = tier[0].data();
      job.dst_dv = tier[1].data();
      ticket[w] = adder.submit(job);
    }
    if (adder.drain() != hipSuccess) return 3;
  }
  for (int x = 0; x < 2; ++x)
    for (int64_t i = 0; i < elems; ++i)
      if (std::memcmp(tier[x].data() + i * esz, expect[x].data() + i * esz, esz) != 0) {
        std::printf("mismatch in %s at element %lld: got %.9g expected %.9g\n", x ? "dV" : "dK",
                    (long long)i, (double)get(tier[x], i), (double)get(expect[x], i));
        return 1;
      }
  std::printf("ok %d %d\n", jobs, g_events.load());
  return 0;
}
