// Host tier: moves the page-heads a layer needs between pinned host memory
// and the HBM window, with kernels that read / write the device-mapped host
// pools on a side stream.
//
// "Out of the Memory Barrier" (gist.science de, section 2.C; gist.science
// nl, "Methodologie", asynchronous CPU offloading; de 2.D: page-level
// sparsity also shrinks the offload traffic, because only the selected pages
// move).  The union of the pages a selection names is marked in a per-window
// byte map, which one small kernel turns into a list of page-heads and the
// window's table: the window holds a fixed number of slots per KV head and
// each visit packs its pages into the first ones, so its size bounds the
// pages of one visit, not the context.  The copy kernels stream over the
// list.  Gradients travel as the host gradient dtype and live in HBM as
// fp32 while the layer computes; with host accumulation they are not
// fetched but zeroed in the window, and the writeback sends the window's
// contributions to a pinned staging area instead of the tier.  Two device
// counters add up the bytes fetched and written back.
#include "pkv_pool.h"

namespace pkv {
namespace {

__global__ void need_clear_kernel(uint8_t* need, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    need[i] = 0;
}

// grid (n_qpages, hkv)
__global__ void need_mark_sel_kernel(uint8_t* need, const int32_t* pages, const int32_t* count,
                                     int stride, int hkv, int max_logical) {
  const int il = blockIdx.x, g = blockIdx.y;
  int cnt = count[(int64_t)il * hkv + g];
  cnt = cnt < 0 ? 0 : (cnt > stride ? stride : cnt);
  const int32_t* lst = pages + ((int64_t)il * hkv + g) * stride;
  for (int u = threadIdx.x; u < cnt; u += blockDim.x) {
    const int j = lst[u];
    if (j >= 0 && j < max_logical) need[(int64_t)g * max_logical + j] = 1;
  }
}

// grid (ceil(n_pages / 256), hkv)
__global__ void need_mark_all_kernel(uint8_t* need, int max_logical, int64_t n_pages) {
  const int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (j < n_pages) need[(int64_t)blockIdx.y * max_logical + j] = 1;
}

// The marked page-heads of a window as a dense list, and the window's table:
// one workgroup, one block scan over the map per KV head.  The j-th marked
// page of head g (in page order) takes window slot j of that head; a list
// entry holds the page-head's index in the tier (g * n_slots + its slot in
// the layer's table) and in the window (g * wslots + window slot), so the
// copy kernels stream over the list without touching the map or a table
// again.  Pages the window does not hold map to window slot 0 of their head
// (a selection that names only listed pages never reaches them).  The host
// checks before the launch that no head marks more than wslots pages; a
// page past that bound would be left out, never written out of bounds.
__global__ void __launch_bounds__(1024) need_compact_kernel(
    const uint8_t* __restrict__ need, const int32_t* __restrict__ table, int max_logical,
    int n_slots, int hkv, int n_pages, int wslots, int2* __restrict__ items,
    int* __restrict__ count, int32_t* __restrict__ wtable) {
  __shared__ int s_sum[1024];
  __shared__ int s_base;
  const int tid = threadIdx.x, T = blockDim.x;
  const int per = (n_pages + T - 1) / T;
  const int lo = tid * per < n_pages ? tid * per : n_pages;
  const int hi = lo + per < n_pages ? lo + per : n_pages;
  if (tid == 0) s_base = 0;
  for (int g = 0; g < hkv; ++g) {
    const uint8_t* ng = need + (int64_t)g * max_logical;
    int c = 0;
    for (int j = lo; j < hi; ++j) c += ng[j] != 0;
    __syncthreads();  // s_base of the previous head is in place
    const int base = s_base;
    s_sum[tid] = c;
    __syncthreads();
    for (int off = 1; off < T; off <<= 1) {
      const int add = tid >= off ? s_sum[tid - off] : 0;
      __syncthreads();
      s_sum[tid] += add;
      __syncthreads();
    }
    int pos = s_sum[tid] - c;
    int32_t* wt = wtable + (int64_t)g * max_logical;
    for (int j = lo; j < hi; ++j) {
      int ws = 0;
      if (ng[j]) {
        if (pos < wslots) {
          items[base + pos] = make_int2(g * n_slots + table[(int64_t)g * max_logical + j],
                                        g * wslots + pos);
          ws = pos;
        }
        ++pos;
      }
      wt[j] = ws;
    }
    for (int j = n_pages + tid; j < max_logical; j += T) wt[j] = 0;
    __syncthreads();
    if (tid == T - 1) s_base = base + (s_sum[T - 1] < wslots ? s_sum[T - 1] : wslots);
  }
  __syncthreads();
  if (tid == 0) *count = s_base;
}

__device__ __forceinline__ float4 lo4(uint4 a) {
  return make_float4(__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xffff0000u),
                     __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xffff0000u));
}
__device__ __forceinline__ float4 hi4(uint4 a) {
  return make_float4(__uint_as_float(a.z << 16), __uint_as_float(a.z & 0xffff0000u),
                     __uint_as_float(a.w << 16), __uint_as_float(a.w & 0xffff0000u));
}

// A small persistent grid does the host-link copies (kFetchBlocks workgroups
// host -> HBM, kCopyBlocks HBM -> host), so that they occupy a few CUs next to
// the attention kernels instead of flooding the whole GPU.  Each workgroup
// copies whole page-heads from the list (its next list entry loaded one
// page-head ahead).  Host-mapped memory answers after microseconds, so a
// workgroup's bandwidth is its bytes in flight over that latency: every thread
// keeps kInflight 16-byte loads in flight.  (A flat stream of 16-byte units
// over all listed page-heads was slower on the host link: 38 vs 42 GB/s host
// -> HBM, 41 vs 50 back.)  The fetch's grid is sized against a writeback made
// by the DMA engines at the same time: on the 1M-token top-K stack, 24 fetch
// workgroups reach ~39 GB/s, 32 reach ~48 GB/s with the writeback still at
// ~48 GB/s, and 36 or 40 take the writeback down to 36-41 GB/s.
constexpr int kFetchBlocks = 32;
constexpr int kCopyBlocks = 24;
constexpr int kInflight = 8;

// Copies `bytes` (a multiple of 16 * blockDim).
__device__ __forceinline__ void copy_bytes(char* __restrict__ dst, const char* __restrict__ src,
                                           int64_t bytes) {
  const int64_t step = (int64_t)blockDim.x * 16;
  for (int64_t i = threadIdx.x * 16; i < bytes; i += kInflight * step) {
    uint4 v[kInflight];
#pragma unroll
    for (int u = 0; u < kInflight; ++u)
      if (i + u * step < bytes) v[u] = *reinterpret_cast<const uint4*>(src + i + u * step);
#pragma unroll
    for (int u = 0; u < kInflight; ++u)
      if (i + u * step < bytes) *reinterpret_cast<uint4*>(dst + i + u * step) = v[u];
  }
}

// bf16 [n] -> fp32 [n], n a multiple of 8 * blockDim.
__device__ __forceinline__ void widen(float* __restrict__ dst, const unsigned short* __restrict__ src,
                                      int64_t n) {
  const int64_t n8 = n / 8;
  for (int64_t i = threadIdx.x; i < n8; i += kInflight * (int64_t)blockDim.x) {
    uint4 a[kInflight];
#pragma unroll
    for (int u = 0; u < kInflight; ++u)
      if (i + u * blockDim.x < n8) a[u] = reinterpret_cast<const uint4*>(src)[i + u * blockDim.x];
#pragma unroll
    for (int u = 0; u < kInflight; ++u)
      if (i + u * blockDim.x < n8) {
        float4* d = reinterpret_cast<float4*>(dst + 8 * (i + u * blockDim.x));
        d[0] = lo4(a[u]);
        d[1] = hi4(a[u]);
      }
  }
}

// Host -> window for every listed page-head: K and V (with_kv), and dK/dV
// with grad_mode 1 (bf16 host gradients, widened to fp32) or 2 (fp32).
__global__ void __launch_bounds__(256) fetch_kernel(
    const int2* __restrict__ items, const int* __restrict__ count, int64_t page_elems,
    bool with_kv, int kv_bytes, const char* __restrict__ hk, const char* __restrict__ hv,
    char* __restrict__ wk, char* __restrict__ wv, int grad_mode, const char* __restrict__ hdk,
    const char* __restrict__ hdv, float* __restrict__ wdk, float* __restrict__ wdv,
    unsigned long long* __restrict__ moved) {
  const int n = *count;
  const int64_t per = (with_kv ? 2 * page_elems * kv_bytes : 0) +
                      (grad_mode ? 2 * page_elems * (grad_mode == 1 ? 2 : 4) : 0);
  int it = blockIdx.x;
  int2 e0 = it < n ? items[it] : make_int2(0, 0);
  for (; it < n; it += gridDim.x) {
    const int2 e_next = it + (int)gridDim.x < n ? items[it + gridDim.x] : make_int2(0, 0);
    const int64_t eh = e0.x * page_elems, ew = e0.y * page_elems;  // tier, window
    if (with_kv) {
      copy_bytes(wk + ew * kv_bytes, hk + eh * kv_bytes, page_elems * kv_bytes);
      copy_bytes(wv + ew * kv_bytes, hv + eh * kv_bytes, page_elems * kv_bytes);
    }
    if (grad_mode == 1) {
      widen(wdk + ew, (const unsigned short*)hdk + eh, page_elems);
      widen(wdv + ew, (const unsigned short*)hdv + eh, page_elems);
    } else if (grad_mode == 2) {
      copy_bytes((char*)(wdk + ew), hdk + eh * 4, page_elems * 4);
      copy_bytes((char*)(wdv + ew), hdv + eh * 4, page_elems * 4);
    }
    e0 = e_next;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && n) atomicAdd(moved, (unsigned long long)n * per);
}

// Zero the window's fp32 dK/dV of every listed page-head (host gradient
// accumulation: each visit starts from zero).  HBM-only work, so a full grid
// rather than the copy kernels' small one, which keeps the host link's
// workgroups on host reads.
__global__ void __launch_bounds__(256) window_grad_zero_kernel(
    const int2* __restrict__ items, const int* __restrict__ count, int64_t page_elems,
    float* __restrict__ wdk, float* __restrict__ wdv) {
  const int64_t per = page_elems / 4;  // float4 per page-head
  const int64_t total = (int64_t)*count * per;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t it = u / per, e = items[it].y * page_elems + (u - it * per) * 4;
    *reinterpret_cast<float4*>(wdk + e) = z;
    *reinterpret_cast<float4*>(wdv + e) = z;
  }
}

__device__ __forceinline__ unsigned to_bf16(float x) {
  return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)x);
}

// Window fp32 dK/dV of the listed page-heads -> host gradient dtype (the
// tier, or the staging of host accumulation, indexed alike), whole
// page-heads per workgroup as in the fetch.
__global__ void __launch_bounds__(256) writeback_kernel(
    const int2* __restrict__ items, const int* __restrict__ count, int64_t page_elems,
    bool grad_bf16, char* __restrict__ hdk, char* __restrict__ hdv,
    const float* __restrict__ wdk, const float* __restrict__ wdv,
    unsigned long long* __restrict__ moved) {
  const int n = *count;
  int it = blockIdx.x;
  int2 e0 = it < n ? items[it] : make_int2(0, 0);
  for (; it < n; it += gridDim.x) {
    const int2 e_next = it + (int)gridDim.x < n ? items[it + gridDim.x] : make_int2(0, 0);
    const int64_t eh = e0.x * page_elems, ew = e0.y * page_elems;  // tier, window
    if (!grad_bf16) {
      copy_bytes(hdk + eh * 4, (const char*)(wdk + ew), page_elems * 4);
      copy_bytes(hdv + eh * 4, (const char*)(wdv + ew), page_elems * 4);
    } else {
      uint4* dk = reinterpret_cast<uint4*>(hdk + eh * 2);
      uint4* dv = reinterpret_cast<uint4*>(hdv + eh * 2);
      for (int64_t i = threadIdx.x; i < page_elems / 8; i += blockDim.x) {
        const float4* a = reinterpret_cast<const float4*>(wdk + ew + 8 * i);
        const float4* b = reinterpret_cast<const float4*>(wdv + ew + 8 * i);
        const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
        dk[i] = make_uint4(to_bf16(a0.x) | (to_bf16(a0.y) << 16), to_bf16(a0.z) | (to_bf16(a0.w) << 16),
                           to_bf16(a1.x) | (to_bf16(a1.y) << 16), to_bf16(a1.z) | (to_bf16(a1.w) << 16));
        dv[i] = make_uint4(to_bf16(b0.x) | (to_bf16(b0.y) << 16), to_bf16(b0.z) | (to_bf16(b0.w) << 16),
                           to_bf16(b1.x) | (to_bf16(b1.y) << 16), to_bf16(b1.z) | (to_bf16(b1.w) << 16));
      }
    }
    e0 = e_next;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && n)
    atomicAdd(moved, (unsigned long long)n * 2 * page_elems * (grad_bf16 ? 2 : 4));
}

// Host accumulation with the device staging: window fp32 dK/dV of the first
// n listed page-heads (n = min(count, cap)) -> the staging in list order,
// page-head i of the list to staging page-head i, in the host gradient
// dtype (dK in the first cap page-heads, dV in the next).  HBM only, so a
// full grid; one runtime copy per tensor (on a DMA engine) then carries the
// staging over the host link.
__global__ void __launch_bounds__(256) stage_grads_kernel(
    const int2* __restrict__ items, const int* __restrict__ count, int cap, int64_t page_elems,
    bool grad_bf16, char* __restrict__ stage, const float* __restrict__ wdk,
    const float* __restrict__ wdv, unsigned long long* __restrict__ moved) {
  const int n = *count < cap ? *count : cap;
  const int64_t per = page_elems / 8;  // 8 elements per step
  const int64_t total = (int64_t)n * per;
  const int gb = grad_bf16 ? 2 : 4;
  char* sdk = stage;
  char* sdv = stage + (int64_t)cap * page_elems * gb;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t it = u / per, off = (u - it * per) * 8;
    const int64_t src = items[it].y * page_elems + off, dst = it * page_elems + off;
    const float4* a = reinterpret_cast<const float4*>(wdk + src);
    const float4* b = reinterpret_cast<const float4*>(wdv + src);
    const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
    if (grad_bf16) {
      *reinterpret_cast<uint4*>(sdk + dst * 2) =
          make_uint4(to_bf16(a0.x) | (to_bf16(a0.y) << 16), to_bf16(a0.z) | (to_bf16(a0.w) << 16),
                     to_bf16(a1.x) | (to_bf16(a1.y) << 16), to_bf16(a1.z) | (to_bf16(a1.w) << 16));
      *reinterpret_cast<uint4*>(sdv + dst * 2) =
          make_uint4(to_bf16(b0.x) | (to_bf16(b0.y) << 16), to_bf16(b0.z) | (to_bf16(b0.w) << 16),
                     to_bf16(b1.x) | (to_bf16(b1.y) << 16), to_bf16(b1.z) | (to_bf16(b1.w) << 16));
    } else {
      float4* dk = reinterpret_cast<float4*>(sdk + dst * 4);
      float4* dv = reinterpret_cast<float4*>(sdv + dst * 4);
      dk[0] = a0;
      dk[1] = a1;
      dv[0] = b0;
      dv[1] = b1;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && n)
    atomicAdd(moved, (unsigned long long)n * 2 * page_elems * gb);
}

// dst[t][g][:] (fp32) = bf16 host gradient of token t
__global__ void export_bf16_grad_kernel(const unsigned short* __restrict__ src,
                                        float* __restrict__ dst, const int32_t* __restrict__ table,
                                        int hkv, int page, int slots, int max_logical, int d,
                                        int64_t n_tok) {
  const int64_t total = n_tok * hkv * d;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx % d);
    const int64_t tg = idx / d;
    const int g = (int)(tg % hkv);
    const int64_t t = tg / hkv;
    const int slot = table[(int64_t)g * max_logical + t / page];
    const unsigned short u = src[(((int64_t)g * slots + slot) * page + t % page) * d + e];
    dst[idx] = __uint_as_float(((unsigned)u) << 16);
  }
}

// dst[t][g][:] (fp32) = window gradient + host-tier gradient of token
// t0 + t: the complete sum of a gradient row while the host adds the window's
// contributions into the tier (host_grad_accumulate).  Four elements per
// thread; the tier is read through its device-mapped alias (bf16 or fp32).
__global__ void grad_rows_sum_kernel(const float* __restrict__ win, const int32_t* __restrict__ wtab,
                                     int wslots, const void* __restrict__ tier,
                                     const int32_t* __restrict__ ttab, int tslots, bool tier_bf16,
                                     float* __restrict__ dst, int hkv, int page, int max_logical,
                                     int d, int64_t t0, int64_t n_tok) {
  const int q = d / 4;
  const int64_t total = n_tok * hkv * q;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int e = 4 * (int)(idx % q);
    const int64_t tg = idx / q;
    const int g = (int)(tg % hkv);
    const int64_t t = t0 + tg / hkv;
    const int64_t pg = t / page;
    const int64_t row = t % page;
    const int64_t wo = (((int64_t)g * wslots + wtab[(int64_t)g * max_logical + pg]) * page + row) * d + e;
    const int64_t to = (((int64_t)g * tslots + ttab[(int64_t)g * max_logical + pg]) * page + row) * d + e;
    float4 a = *reinterpret_cast<const float4*>(win + wo);
    float b[4];
    if (tier_bf16) {
      const uint2 u = *reinterpret_cast<const uint2*>((const unsigned short*)tier + to);
      b[0] = __uint_as_float(u.x << 16);
      b[1] = __uint_as_float(u.x & 0xffff0000u);
      b[2] = __uint_as_float(u.y << 16);
      b[3] = __uint_as_float(u.y & 0xffff0000u);
    } else {
      const float4 v = *reinterpret_cast<const float4*>((const float*)tier + to);
      b[0] = v.x;
      b[1] = v.y;
      b[2] = v.z;
      b[3] = v.w;
    }
    a.x += b[0];
    a.y += b[1];
    a.z += b[2];
    a.w += b[3];
    *reinterpret_cast<float4*>(dst + tg * d + e) = a;
  }
}

int grid_of(int64_t work) {
  int64_t b = (work + 255) / 256;
  if (b > 65536) b = 65536;
  return b < 1 ? 1 : (int)b;
}

}  // namespace

hipError_t launch_need_clear(uint8_t* need, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(need_clear_kernel, dim3(grid_of(n)), dim3(256), 0, s, need, n);
  return hipGetLastError();
}

hipError_t launch_need_mark(uint8_t* need, const pkv_sel* sel, int hkv, int max_logical,
                            int64_t n_pages_all, hipStream_t s) {
  if (sel) {
    if (sel->n_qpages <= 0) return hipSuccess;
    hipLaunchKernelGGL(need_mark_sel_kernel, dim3(sel->n_qpages, hkv), dim3(128), 0, s, need,
                       sel->pages, sel->count, sel->stride, hkv, max_logical);
  } else {
    if (n_pages_all <= 0) return hipSuccess;
    hipLaunchKernelGGL(need_mark_all_kernel, dim3((unsigned)((n_pages_all + 255) / 256), hkv),
                       dim3(256), 0, s, need, max_logical, n_pages_all);
  }
  return hipGetLastError();
}

int64_t need_words(const pkv_pool* p) {
  return (int64_t)p->desc.n_kv_heads * p->desc.max_logical_pages;
}

namespace {

struct WindowList {
  const uint8_t* need;
  int2* items;
  int* count;
};

// The page map and list buffer the window's last prefetch built.
WindowList window_list(const pkv_pool* p, int window) {
  const int64_t nw = need_words(p);
  const int64_t ni = (int64_t)p->desc.n_kv_heads * p->window_slots;
  const int b = window * 2 + p->list_gen[window];
  return {p->d_need + b * nw, p->d_items + b * ni, p->d_count + b};
}

int64_t pages_of(const pkv_pool* p, int layer) {
  return (p->length[layer] + p->desc.page_size - 1) / p->desc.page_size;
}

}  // namespace

hipError_t launch_window_list(const pkv_pool* p, int layer, int window, int64_t n_pages,
                              hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const WindowList L = window_list(p, window);
  const int32_t* table = p->d_table + (int64_t)layer * need_words(p);
  // pages the map can mark: the appended ones, or those a prefix reserves
  int64_t np = pages_of(p, layer) > n_pages ? pages_of(p, layer) : n_pages;
  if (np > d.max_logical_pages) np = d.max_logical_pages;
  hipLaunchKernelGGL(need_compact_kernel, dim3(1), dim3(1024), 0, s, L.need, table,
                     d.max_logical_pages, d.n_slots, d.n_kv_heads, (int)np,
                     p->window_slots, L.items, L.count, p->d_wtable + window * need_words(p));
  return hipGetLastError();
}

hipError_t launch_fetch(const pkv_pool* p, int layer, int window, hipStream_t s,
                        bool with_grads) {
  const pkv_pool_desc& d = p->desc;
  const WindowList L = window_list(p, window);
  const int grad_mode = with_grads ? (d.host_grad_dtype == PKV_BF16 ? 1 : 2) : 0;
  KernelTimer t(KT_FETCH, s);
  hipLaunchKernelGGL(fetch_kernel, dim3(kFetchBlocks), dim3(256), 0, s, L.items, L.count,
                     (int64_t)d.page_size * d.head_dim, true, p->kv_bytes,
                     (const char*)p->m_k[layer], (const char*)p->m_v[layer],
                     (char*)p->d_k + window * p->dev_elems * p->kv_bytes,
                     (char*)p->d_v + window * p->dev_elems * p->kv_bytes, grad_mode,
                     (const char*)p->m_dk[layer], (const char*)p->m_dv[layer],
                     p->d_dk + window * p->dev_elems, p->d_dv + window * p->dev_elems,
                     p->d_moved);
  return hipGetLastError();
}

hipError_t launch_window_grad_zero(const pkv_pool* p, int layer, int window, hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const WindowList L = window_list(p, window);
  hipLaunchKernelGGL(window_grad_zero_kernel, dim3(2048), dim3(256), 0, s, L.items, L.count,
                     (int64_t)d.page_size * d.head_dim, p->d_dk + window * p->dev_elems,
                     p->d_dv + window * p->dev_elems);
  return hipGetLastError();
}

hipError_t launch_writeback_pages(const pkv_pool* p, int layer, int window, hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const WindowList L = window_list(p, window);
  // the page-heads the window's last prefetch listed; their gradients go to
  // the tier itself, or to the window's staging (same indexing) for host adds
  void* dst_dk = p->accumulate ? p->m_stage_dk[window] : p->m_dk[layer];
  void* dst_dv = p->accumulate ? p->m_stage_dv[window] : p->m_dv[layer];
  KernelTimer t(KT_WRITEBACK, s);
  hipLaunchKernelGGL(writeback_kernel, dim3(kCopyBlocks), dim3(256), 0, s, L.items, L.count,
                     (int64_t)d.page_size * d.head_dim, d.host_grad_dtype == PKV_BF16,
                     (char*)dst_dk, (char*)dst_dv,
                     (const float*)(p->d_dk + window * p->dev_elems),
                     (const float*)(p->d_dv + window * p->dev_elems), p->d_moved + 1);
  return hipGetLastError();
}

hipError_t launch_writeback_staged(const pkv_pool* p, int window, int n, hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const WindowList L = window_list(p, window);
  const int64_t page_elems = (int64_t)d.page_size * d.head_dim;
  const int gb = d.host_grad_dtype == PKV_BF16 ? 2 : 4;
  const int cap = (int)p->stage_heads;
  const size_t bytes = (size_t)n * page_elems * gb;
  KernelTimer t(KT_WRITEBACK, s);  // the conversion and the copies over the link
  hipLaunchKernelGGL(stage_grads_kernel, dim3(2048), dim3(256), 0, s, L.items, L.count, cap,
                     page_elems, gb == 2, p->d_stage, (const float*)(p->d_dk + window * p->dev_elems),
                     (const float*)(p->d_dv + window * p->dev_elems), p->d_moved + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  if ((e = hipMemcpyAsync(p->h_stage_dk[window], p->d_stage, bytes, hipMemcpyDeviceToHost, s)) !=
          hipSuccess ||
      (e = hipMemcpyAsync(p->h_stage_dv[window], p->d_stage + (size_t)cap * page_elems * gb, bytes,
                          hipMemcpyDeviceToHost, s)) != hipSuccess)
    return e;
  return hipMemcpyAsync(p->h_stage_items[window], L.items, (size_t)n * sizeof(int2),
                        hipMemcpyDeviceToHost, s);
}

hipError_t launch_grad_rows_sum(const pkv_pool* p, int layer, int what, int64_t t0, int64_t n_tok,
                                float* dst, hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  if (n_tok <= 0) return hipSuccess;
  if (d.head_dim % 4) return hipErrorInvalidValue;
  const int64_t tab_stride = (int64_t)d.n_kv_heads * d.max_logical_pages;
  const int w = p->window_of(layer);
  const float* win = (what == PKV_DK ? p->d_dk : p->d_dv) + (int64_t)w * p->dev_elems;
  const int32_t* wtab = p->d_wtable + w * tab_stride;
  const void* tier = what == PKV_DK ? p->m_dk[layer] : p->m_dv[layer];
  const int32_t* ttab = p->d_table + (int64_t)layer * tab_stride;
  hipLaunchKernelGGL(grad_rows_sum_kernel, dim3(grid_of(n_tok * d.n_kv_heads * (d.head_dim / 4))),
                     dim3(256), 0, s, win, wtab, p->window_slots, tier, ttab, d.n_slots,
                     d.host_grad_dtype == PKV_BF16, dst, d.n_kv_heads, d.page_size,
                     d.max_logical_pages, d.head_dim, t0, n_tok);
  return hipGetLastError();
}

hipError_t launch_host_export(const pkv_pool* p, int layer, int what, int64_t n_tok, void* dst,
                              hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const int32_t* table = p->d_table + (int64_t)layer * d.n_kv_heads * d.max_logical_pages;
  const unsigned short* src = (const unsigned short*)(what == PKV_DK ? p->m_dk[layer] : p->m_dv[layer]);
  hipLaunchKernelGGL(export_bf16_grad_kernel, dim3(grid_of(n_tok * d.n_kv_heads * d.head_dim)),
                     dim3(256), 0, s, src, (float*)dst, table, d.n_kv_heads, d.page_size,
                     d.n_slots, d.max_logical_pages, d.head_dim, n_tok);
  return hipGetLastError();
}

}  // namespace pkv
