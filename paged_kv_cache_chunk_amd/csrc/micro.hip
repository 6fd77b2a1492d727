// Measurement kernels: the data movement of two phases of the bf16 path
// without their arithmetic, to set the attention kernels' rates beside the
// rate of their memory traffic alone.
//   gather:  the forward's K/V tile stream (global_load_lds into two LDS
//            buffers per workgroup, the same grid, tile walk, page-table
//            lookups and waits), no MFMA;
//   atomics: the dK/dV kernel's epilogue (one fp32 atomic add per gradient
//            element of every 128-key slab, the same grid and lane pattern),
//            repeated, no MFMA.
// Neither is called by the attention path.
#include "attn_bf16_tiles.h"

namespace pkv {
namespace {

constexpr int MB_BNT = 64;  // keys per tile, as the forward kernel

// grid nqb * hq, 256 threads (4 waves) as the forward kernel.  out[bid] gets
// one LDS word so that the copies have a consumer.
__global__ void __launch_bounds__(256) gather_kernel(AttnCall c, int n_qblocks, float* out) {
  constexpr int TB = MB_BNT * ROWB;
  __shared__ __align__(1024) char sm[2][2 * TB];
  const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
  const int G = c.hq / c.g.hkv;
  const int bid = blockIdx.x;
  const int g = uni(bid % c.g.hkv), m = uni(bid / c.g.hkv);
  const int qb = n_qblocks - 1 - m / G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  int n_tiles;
  TileWalk<MB_BNT> walk = make_walk<MB_BNT>(c, g, r0, rlast, &n_tiles);
  TileDma<MB_BNT, 4> dma;
  dma.init(w, lane);
  auto issue = [&](int b, const KeyTile& t) {
    dma.issue(sm[b], w, key_rows<MB_BNT>(c, c.L.k, g, t), ROWB);
    dma.issue(sm[b] + TB, w, key_rows<MB_BNT>(c, c.L.v, g, t), ROWB);
  };
  if (n_tiles > 0) issue(0, walk.next());
  wait_dma_and_sync();
  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) issue((j + 1) & 1, walk.next());
    wait_dma_and_sync();
  }
  if (tid == 0) out[bid] = *reinterpret_cast<const float*>(sm[n_tiles & 1]);
}

// grid n_slabs * hkv, 256 threads: wave w adds `value` to the dK and dV of
// keys 32 w .. 32 w + 31 of its slab, `reps` times, with the dK/dV kernel's
// element order.
__global__ void __launch_bounds__(256) atomics_kernel(AttnCall c, int reps, float value) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int g = blockIdx.x % c.g.hkv, slab = blockIdx.x / c.g.hkv;
  const int P = c.g.page;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int64_t wk0 = (int64_t)slab * 128 + 32 * w;
  const int slot = uni(c.L.table[(int64_t)g * c.g.max_logical + wk0 / P]);
  float* dkp = c.L.dk + (((int64_t)g * c.g.slots + slot) * P + (wk0 % P)) * D + l32;
  float* dvp = c.L.dv + (((int64_t)g * c.g.slots + slot) * P + (wk0 % P)) * D + l32;
  for (int rep = 0; rep < reps; ++rep) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int srel = 8 * (r >> 2) + 4 * half + (r & 3);
      if (wk0 + srel >= n_keys) continue;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        unsafeAtomicAdd(dkp + srel * D + 32 * dt, value);
        unsafeAtomicAdd(dvp + srel * D + 32 * dt, value);
      }
    }
  }
}

}  // namespace

hipError_t launch_micro_gather(const AttnCall& c, float* out, hipStream_t s) {
  const int nqb = (c.n_q + BM - 1) / BM;
  hipLaunchKernelGGL(gather_kernel, dim3(nqb * c.hq), dim3(256), 0, s, c, nqb, out);
  return hipGetLastError();
}

hipError_t launch_micro_atomics(const AttnCall& c, int reps, float value, hipStream_t s) {
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int n_slabs = (int)((n_keys + 127) / 128);
  hipLaunchKernelGGL(atomics_kernel, dim3(n_slabs * c.g.hkv), dim3(256), 0, s, c, reps, value);
  return hipGetLastError();
}

}  // namespace pkv
