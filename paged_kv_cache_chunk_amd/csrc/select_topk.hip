// Page-level top-K selection.
//
// "Out of the Memory Barrier" (gist.science de, section 2.D; gist.science nl,
// "Methodologie", page-level sparse attention; sciencestack.ai, Figure 5):
// for dense-attention models each query page retrieves the most relevant key
// pages, scored through one representative vector per page, and attends only
// to those.  Here:
//   qbar(i, g)  = fp32 mean of q over query page i's tokens and group g's heads
//   score(i, j) = fp32 dot(qbar(i, g), rep(j, g)), candidates j in
//                 [n_sink, i - n_local]
//   kept        = top_k scores, ties to the lower page index (exact radix
//                 select on an order-preserving 32-bit key, then an ordered
//                 scan over the ties)
//   list        = sinks U local window U kept, ascending.
// Three kernels: query means, scores, and selection (one workgroup per
// (query page, KV head), wavefront ballots for the ordered scans).
#include "pkv_internal.h"

namespace pkv {
namespace {

__device__ __forceinline__ float ld(const void* p, int64_t i, bool bf16) {
  if (bf16) {
    const unsigned short u = reinterpret_cast<const unsigned short*>(p)[i];
    return __uint_as_float(((unsigned)u) << 16);
  }
  return reinterpret_cast<const float*>(p)[i];
}

// grid (n_qpages, hkv), block 1024.  Thread (part p = tid / 32, lane j =
// tid % 32) sums columns j*E .. j*E+E-1 (E = d / 32) over the (token, head)
// pairs p, p + 32, .. of the page's group in that order; the 32 partial
// sums are then added in part order.  Fixed order, so reruns are
// bit-identical.  The loads of four pairs are issued before their adds (which
// keep the pair order), so that their latencies overlap.
template <int DD, bool BF16>
__global__ void __launch_bounds__(1024) qmean_kernel(const void* __restrict__ q,
                                                     float* __restrict__ qbar, int hq, int hkv,
                                                     int page, int n_q) {
  constexpr int E = DD / 32;
  constexpr int NP = 32;
  constexpr int U = 4;  // pairs loaded ahead of their adds
  __shared__ float red[NP][DD];
  const int il = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int part = tid >> 5, j = tid & 31;
  const int G = hq / hkv;
  const int t0 = il * page;
  int t1 = t0 + page;
  if (t1 > n_q) t1 = n_q;
  const int n_pairs = (t1 - t0) * G;
  // this thread's E values of pair pr, widened to fp32
  auto load = [&](int pr, float (&x)[E]) {
    const int t = t0 + pr / G, h = g * G + pr % G;
    const int64_t base = ((int64_t)t * hq + h) * DD + j * E;
    if (BF16) {
      // E consecutive bf16 values (4 or 2): one 8- or 4-byte load
      const unsigned short* p = reinterpret_cast<const unsigned short*>(q) + base;
      if (E == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        const unsigned w[4] = {v.x << 16, v.x & 0xffff0000u, v.y << 16, v.y & 0xffff0000u};
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = __uint_as_float(w[e]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = __uint_as_float(((unsigned)p[e]) << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = reinterpret_cast<const float*>(q)[base + e];
    }
  };
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  int pr = part;
  for (; pr + (U - 1) * NP < n_pairs; pr += U * NP) {
    float x[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) load(pr + u * NP, x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += x[u][e];
  }
  for (; pr < n_pairs; pr += NP) {
    float x[E];
    load(pr, x);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[part][j * E + e] = acc[e];
  __syncthreads();
  if (tid < DD) {
    float sum = 0.f;
#pragma unroll
    for (int x = 0; x < NP; ++x) sum += red[x][tid];
    qbar[((int64_t)il * hkv + g) * DD + tid] = sum / (float)n_pairs;
  }
}

// grid (n_qpages, hkv, ceil(max_cand / 256)), block 256.  Sequential fma over d.
__global__ void score_kernel(const float* __restrict__ qbar, const float* __restrict__ reps,
                             const int32_t* __restrict__ table, float* __restrict__ scores,
                             int hkv, int d, int slots, int max_logical, int first_qpage,
                             int n_sink, int n_local, int max_cand) {
  __shared__ float qs[128];
  const int il = blockIdx.x, g = blockIdx.y;
  const int i = first_qpage + il;
  for (int e = threadIdx.x; e < d; e += blockDim.x) qs[e] = qbar[((int64_t)il * hkv + g) * d + e];
  __syncthreads();
  const int c = blockIdx.z * blockDim.x + threadIdx.x;
  const int nc = i - n_local - n_sink + 1;
  if (c >= nc || c >= max_cand) return;
  const int j = n_sink + c;
  const int slot = table[(int64_t)g * max_logical + j];
  const float4* r = reinterpret_cast<const float4*>(reps + ((int64_t)g * slots + slot) * d);
  float acc = 0.f;
  for (int e4 = 0; e4 < d / 4; ++e4) {
    const float4 x = r[e4];
    acc = fmaf(qs[4 * e4 + 0], x.x, acc);
    acc = fmaf(qs[4 * e4 + 1], x.y, acc);
    acc = fmaf(qs[4 * e4 + 2], x.z, acc);
    acc = fmaf(qs[4 * e4 + 3], x.w, acc);
  }
  scores[((int64_t)il * hkv + g) * max_cand + c] = acc;
}

__device__ __forceinline__ unsigned fkey(float x) {
  if (x == 0.f) x = 0.f;  // -0 and +0 compare equal; give them one key
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTB = 256;  // threads per selection workgroup

// Inclusive prefix sum of x across the workgroup in thread order (wavefront
// shuffles, then the 4 wave totals through LDS).
__device__ int block_incl_scan(int x, int* wave_tot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[w] = x;
  __syncthreads();
  int before = 0;
  for (int v = 0; v < w; ++v) before += wave_tot[v];
  __syncthreads();
  return x + before;
}

// Exclusive prefix of `flag` across the workgroup in thread order; returns the
// prefix and writes the workgroup total to *total.  Uses wavefront ballots.
__device__ int block_excl_scan(bool flag, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[w] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
  for (int x = 0; x < kTB / 64; ++x) {
    if (x < w) before += wave_tot[x];
    all += wave_tot[x];
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

// grid (n_qpages, hkv), block kTB, dynamic LDS: one byte per page [0, i].
__global__ void __launch_bounds__(kTB) topk_kernel(const float* __restrict__ scores,
                                                   int max_cand, int hkv, int first_qpage,
                                                   int top_k, int n_sink, int n_local,
                                                   int32_t* __restrict__ sel_pages,
                                                   int32_t* __restrict__ sel_count,
                                                   int stride) {
  extern __shared__ unsigned char flag[];
  __shared__ unsigned hist[256];
  __shared__ int s_digit, s_k;
  __shared__ int wave_tot[kTB / 64];
  const int il = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int i = first_qpage + il;
  int nc = i - n_local - n_sink + 1;
  if (nc < 0) nc = 0;
  const float* sc = scores + ((int64_t)il * hkv + g) * max_cand;
  const int kk = top_k < nc ? top_k : nc;

  for (int p = tid; p <= i; p += kTB) flag[p] = 0;
  __syncthreads();
  // forced pages: sinks and the local window (the query page itself included)
  for (int p = tid; p <= i; p += kTB)
    if (p < n_sink || p > i - n_local) flag[p] = 1;

  if (kk == nc) {
    for (int c = tid; c < nc; c += kTB) flag[n_sink + c] = 1;
  } else if (kk > 0) {
    // Radix select of the kk-th largest key, 8 bits at a time from the top.
    unsigned prefix = 0u, mask = 0u;
    int k = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kTB) hist[b] = 0u;
      __syncthreads();
      for (int c = tid; c < nc; c += kTB) {
        const unsigned key = fkey(sc[c]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // suffix sums over the bins: S(b) = count of digits >= b; the digit of
      // the k-th largest is the b with S(b) >= k > S(b + 1)
      {
        const int b = 255 - tid;  // tid < 256 == kTB
        const int above = block_incl_scan((int)hist[b], wave_tot) - (int)hist[b];  // S(b + 1)
        const int at = above + (int)hist[b];                                          // S(b)
        if (at >= k && above < k) {
          s_digit = b;
          s_k = k - above;
        }
      }
      __syncthreads();
      prefix |= ((unsigned)s_digit) << shift;
      mask |= 255u << shift;
      k = s_k;
      __syncthreads();
    }
    const unsigned T = prefix;  // the kk-th largest key
    const int take_eq = k;      // how many keys equal to T are kept (lowest page first)
    int taken = 0;
    for (int base = 0; base < nc; base += kTB) {
      const int c = base + tid;
      bool gt = false, eq = false;
      if (c < nc) {
        const unsigned key = fkey(sc[c]);
        gt = key > T;
        eq = key == T;
      }
      int tot;
      const int pos = block_excl_scan(eq, wave_tot, &tot);
      if (gt || (eq && taken + pos < take_eq)) flag[n_sink + c] = 1;
      taken += tot;
    }
  }
  __syncthreads();

  // Compact the flags into an ascending list.
  int32_t* out = sel_pages + ((int64_t)il * hkv + g) * stride;
  int written = 0;
  for (int base = 0; base <= i; base += kTB) {
    const int p = base + tid;
    const bool f = (p <= i) && flag[p];
    int tot;
    const int pos = block_excl_scan(f, wave_tot, &tot);
    if (f && written + pos < stride) out[written + pos] = p;
    written += tot;
  }
  for (int x = written + tid; x < stride; x += kTB) out[x] = -1;
  if (tid == 0) sel_count[(int64_t)il * hkv + g] = written < stride ? written : stride;
}

}  // namespace

int64_t select_scratch_floats(const Geom& g, int64_t q_pos0, int n_q, int n_sink, int n_local) {
  const int nqp = (n_q + g.page - 1) / g.page;
  const int64_t last = q_pos0 / g.page + nqp - 1;
  int64_t max_cand = last - n_local - n_sink + 1;
  if (max_cand < 1) max_cand = 1;
  return (int64_t)nqp * g.hkv * g.d + (int64_t)nqp * g.hkv * max_cand;
}

hipError_t launch_select(const LayerDev& L, const Geom& g, bool bf16, int hq, int64_t q_pos0,
                         int n_q, const void* q, int top_k, int n_sink, int n_local,
                         int32_t* sel_pages, int32_t* sel_count, int sel_stride,
                         float* scratch, hipStream_t s) {
  const int nqp = (n_q + g.page - 1) / g.page;
  const int first = (int)(q_pos0 / g.page);
  int max_cand = first + nqp - 1 - n_local - n_sink + 1;
  if (max_cand < 1) max_cand = 1;
  KernelTimer t(KT_SELECT, s);
  float* qbar = scratch;
  float* scores = scratch + (int64_t)nqp * g.hkv * g.d;
  const dim3 qgrid(nqp, g.hkv);
  if (g.d == 64 && bf16)
    hipLaunchKernelGGL((qmean_kernel<64, true>), qgrid, dim3(1024), 0, s, q, qbar, hq, g.hkv, g.page, n_q);
  else if (g.d == 64)
    hipLaunchKernelGGL((qmean_kernel<64, false>), qgrid, dim3(1024), 0, s, q, qbar, hq, g.hkv, g.page, n_q);
  else if (bf16)
    hipLaunchKernelGGL((qmean_kernel<128, true>), qgrid, dim3(1024), 0, s, q, qbar, hq, g.hkv, g.page, n_q);
  else
    hipLaunchKernelGGL((qmean_kernel<128, false>), qgrid, dim3(1024), 0, s, q, qbar, hq, g.hkv, g.page, n_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_kernel, dim3(nqp, g.hkv, (max_cand + 255) / 256), dim3(256), 0, s,
                     (const float*)qbar, (const float*)L.reps, L.table, scores, g.hkv, g.d,
                     g.slots, g.max_logical, first, n_sink, n_local, max_cand);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = ((size_t)(first + nqp) + 15) & ~(size_t)15;
  hipLaunchKernelGGL(topk_kernel, dim3(nqp, g.hkv), dim3(kTB), lds, s, (const float*)scores,
                     max_cand, g.hkv, first, top_k, n_sink, n_local, sel_pages, sel_count,
                     sel_stride);
  return hipGetLastError();
}

}  // namespace pkv
