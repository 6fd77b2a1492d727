// Host tier: moves the page-heads a layer needs between pinned host memory
// and the HBM window, with kernels that read / write the device-mapped host
// pools on a side stream.
//
// "Out of the Memory Barrier" (gist.science de, section 2.C; gist.science
// nl, "Methodologie", asynchronous CPU offloading; de 2.D: page-level
// sparsity also shrinks the offload traffic, because only the selected pages
// move).  The union of the pages a selection names is marked in a per-window
// byte map; one workgroup per (page, KV head) then copies that page-head if
// marked.  Gradients travel as the host gradient dtype and live in HBM as
// fp32 while the layer computes.  Two device counters add up the bytes
// fetched and written back.
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

// Copies `bytes` (a multiple of 4 KiB) with every thread keeping kInflight
// 16-byte loads in flight (host-mapped sources answer after microseconds, so
// a workgroup's bandwidth is its bytes in flight over that latency).
constexpr int kInflight = 8;
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

__device__ __forceinline__ float4 lo4(uint4 a) {
  return make_float4(__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xffff0000u),
                     __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xffff0000u));
}
__device__ __forceinline__ float4 hi4(uint4 a) {
  return make_float4(__uint_as_float(a.z << 16), __uint_as_float(a.z & 0xffff0000u),
                     __uint_as_float(a.w << 16), __uint_as_float(a.w & 0xffff0000u));
}

// bf16 [n] -> fp32 [n], n a multiple of 8 * blockDim; kInflight 16-byte
// loads in flight per thread.
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

// Work items are (page, KV head) pairs; a small persistent grid (kCopyBlocks
// workgroups) walks them so that the copies occupy a few CUs next to the
// attention kernels instead of flooding the whole GPU.
constexpr int kCopyBlocks = 24;

__global__ void __launch_bounds__(256) fetch_kernel(
    const uint8_t* __restrict__ need, const int32_t* __restrict__ table, int max_logical,
    int slots, int hkv, int n_pages, int64_t page_elems, int kv_bytes,
    const char* __restrict__ hk, const char* __restrict__ hv, char* __restrict__ wk,
    char* __restrict__ wv, bool with_grads, bool grad_bf16, const void* __restrict__ hdk,
    const void* __restrict__ hdv, float* __restrict__ wdk, float* __restrict__ wdv,
    unsigned long long* __restrict__ moved) {
  unsigned long long mine = 0;
  for (int item = blockIdx.x; item < n_pages * hkv; item += gridDim.x) {
    const int g = item % hkv, j = item / hkv;
    if (!need[(int64_t)g * max_logical + j]) continue;
    const int slot = table[(int64_t)g * max_logical + j];
    const int64_t e0 = ((int64_t)g * slots + slot) * page_elems;
    copy_bytes(wk + e0 * kv_bytes, hk + e0 * kv_bytes, page_elems * kv_bytes);
    copy_bytes(wv + e0 * kv_bytes, hv + e0 * kv_bytes, page_elems * kv_bytes);
    mine += 2 * page_elems * kv_bytes;
    if (!with_grads) continue;
    if (!grad_bf16) {
      copy_bytes((char*)(wdk + e0), (const char*)hdk + e0 * 4, page_elems * 4);
      copy_bytes((char*)(wdv + e0), (const char*)hdv + e0 * 4, page_elems * 4);
      mine += 2 * page_elems * 4;
    } else {
      widen(wdk + e0, (const unsigned short*)hdk + e0, page_elems);
      widen(wdv + e0, (const unsigned short*)hdv + e0, page_elems);
      mine += 2 * page_elems * 2;
    }
  }
  if (threadIdx.x == 0 && mine) atomicAdd(moved, mine);
}

__device__ __forceinline__ unsigned to_bf16(float x) {
  return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)x);
}

// window fp32 grads -> host gradient dtype, same persistent walk.
__global__ void __launch_bounds__(256) writeback_kernel(
    const uint8_t* __restrict__ need, const int32_t* __restrict__ table, int max_logical,
    int slots, int hkv, int n_pages, int64_t page_elems, bool grad_bf16, void* __restrict__ hdk,
    void* __restrict__ hdv, const float* __restrict__ wdk, const float* __restrict__ wdv,
    unsigned long long* __restrict__ moved) {
  unsigned long long mine = 0;
  for (int item = blockIdx.x; item < n_pages * hkv; item += gridDim.x) {
    const int g = item % hkv, j = item / hkv;
    if (!need[(int64_t)g * max_logical + j]) continue;
    const int slot = table[(int64_t)g * max_logical + j];
    const int64_t e0 = ((int64_t)g * slots + slot) * page_elems;
    if (!grad_bf16) {
      copy_bytes((char*)hdk + e0 * 4, (const char*)(wdk + e0), page_elems * 4);
      copy_bytes((char*)hdv + e0 * 4, (const char*)(wdv + e0), page_elems * 4);
      mine += 2 * page_elems * 4;
      continue;
    }
    uint4* dk = reinterpret_cast<uint4*>((unsigned short*)hdk + e0);
    uint4* dv = reinterpret_cast<uint4*>((unsigned short*)hdv + e0);
    for (int64_t i = threadIdx.x; i < page_elems / 8; i += blockDim.x) {
      const float4* a = reinterpret_cast<const float4*>(wdk + e0 + 8 * i);
      const float4* b = reinterpret_cast<const float4*>(wdv + e0 + 8 * i);
      const float4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
      dk[i] = make_uint4(to_bf16(a0.x) | (to_bf16(a0.y) << 16), to_bf16(a0.z) | (to_bf16(a0.w) << 16),
                         to_bf16(a1.x) | (to_bf16(a1.y) << 16), to_bf16(a1.z) | (to_bf16(a1.w) << 16));
      dv[i] = make_uint4(to_bf16(b0.x) | (to_bf16(b0.y) << 16), to_bf16(b0.z) | (to_bf16(b0.w) << 16),
                         to_bf16(b1.x) | (to_bf16(b1.y) << 16), to_bf16(b1.z) | (to_bf16(b1.w) << 16));
    }
    mine += 2 * page_elems * 2;
  }
  if (threadIdx.x == 0 && mine) atomicAdd(moved, mine);
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

hipError_t launch_fetch_pages(const pkv_pool* p, int layer, int window, bool with_grads,
                              hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const int64_t n_pages = (p->length[layer] + d.page_size - 1) / d.page_size;
  if (n_pages <= 0) return hipSuccess;
  const int64_t page_elems = (int64_t)d.page_size * d.head_dim;
  const uint8_t* need = p->d_need + (int64_t)window * d.n_kv_heads * d.max_logical_pages;
  const int32_t* table = p->d_table + (int64_t)layer * d.n_kv_heads * d.max_logical_pages;
  KernelTimer t(KT_FETCH, s);
  hipLaunchKernelGGL(fetch_kernel, dim3(kCopyBlocks), dim3(256), 0, s, need,
                     table, d.max_logical_pages, d.n_slots, d.n_kv_heads, (int)n_pages, page_elems,
                     p->kv_bytes,
                     (const char*)p->m_k[layer], (const char*)p->m_v[layer],
                     (char*)p->d_k + window * p->layer_elems * p->kv_bytes,
                     (char*)p->d_v + window * p->layer_elems * p->kv_bytes, with_grads,
                     d.host_grad_dtype == PKV_BF16, (const void*)p->m_dk[layer],
                     (const void*)p->m_dv[layer], p->d_dk + window * p->layer_elems,
                     p->d_dv + window * p->layer_elems, p->d_moved);
  return hipGetLastError();
}

hipError_t launch_writeback_pages(const pkv_pool* p, int layer, int window, hipStream_t s) {
  const pkv_pool_desc& d = p->desc;
  const int64_t n_pages = (p->length[layer] + d.page_size - 1) / d.page_size;
  if (n_pages <= 0) return hipSuccess;
  const int64_t page_elems = (int64_t)d.page_size * d.head_dim;
  const uint8_t* need = p->d_need + (int64_t)window * d.n_kv_heads * d.max_logical_pages;
  const int32_t* table = p->d_table + (int64_t)layer * d.n_kv_heads * d.max_logical_pages;
  KernelTimer t(KT_WRITEBACK, s);
  hipLaunchKernelGGL(writeback_kernel, dim3(kCopyBlocks), dim3(256), 0, s,
                     need, table, d.max_logical_pages, d.n_slots, d.n_kv_heads, (int)n_pages,
                     page_elems, d.host_grad_dtype == PKV_BF16, p->m_dk[layer], p->m_dv[layer],
                     (const float*)(p->d_dk + window * p->layer_elems),
                     (const float*)(p->d_dv + window * p->layer_elems), p->d_moved + 1);
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
