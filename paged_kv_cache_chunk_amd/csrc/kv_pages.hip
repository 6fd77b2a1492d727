// Page writes and reads of the KV pool: append (scatter a chunk's K/V into
// page slots through the page table), page representatives, logical-order
// export and zero fill.  All of these move bytes; they are HBM-bound.
//
// "Out of the Memory Barrier" (gist.science de, section 2.B): the KV cache is
// kept in fixed-size pages so that appending a chunk's key/value pairs needs
// no reallocation.  (gist.science nl, "Methodologie"): one representative
// vector per page is what page retrieval scores.
#include "pkv_internal.h"

namespace pkv {
namespace {

// One thread moves 16 bytes.  Rows of d elements are 16-byte aligned
// (d * elem_bytes is a multiple of 16 for every supported shape).
__global__ void append_kernel(char* __restrict__ kpool, char* __restrict__ vpool,
                              const char* __restrict__ k, const char* __restrict__ v,
                              const int32_t* __restrict__ table, int hkv, int page,
                              int slots, int max_logical, int row_bytes, int64_t pos0,
                              int64_t n_tok) {
  const int vec_per_row = row_bytes / 16;
  const int64_t total = n_tok * hkv * vec_per_row;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % vec_per_row);
    const int64_t tg = idx / vec_per_row;
    const int g = (int)(tg % hkv);
    const int64_t t = tg / hkv;
    const int64_t s = pos0 + t;
    const int slot = table[(int64_t)g * max_logical + s / page];
    const int64_t dst = (((int64_t)g * slots + slot) * page + s % page) * row_bytes + c * 16;
    const int64_t src = tg * row_bytes + c * 16;
    *reinterpret_cast<uint4*>(kpool + dst) = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(vpool + dst) = *reinterpret_cast<const uint4*>(v + src);
  }
}

__device__ __forceinline__ float load_elem(const void* p, int64_t i, bool bf16) {
  if (bf16) {
    const unsigned short u = reinterpret_cast<const unsigned short*>(p)[i];
    return __uint_as_float(((unsigned)u) << 16);
  }
  return reinterpret_cast<const float*>(p)[i];
}

// Mean of the keys present in each page, fp32.  grid (n_pages, hkv), block
// 8 x d threads: part p sums rows p, p + 8, .. of its column, then the 8
// partial sums are added in part order (fixed order).
__global__ void __launch_bounds__(1024) reps_kernel(const void* __restrict__ kpool,
                                                    float* __restrict__ reps,
                                                    const int32_t* __restrict__ table, int page,
                                                    int slots, int max_logical, int d, bool bf16,
                                                    int64_t first_page, int64_t length) {
  __shared__ float red[8][128];
  const int64_t j = first_page + blockIdx.x;
  const int g = blockIdx.y;
  const int e = threadIdx.x % d, part = threadIdx.x / d;
  const int slot = table[(int64_t)g * max_logical + j];
  int64_t n = length - j * page;
  if (n > page) n = page;
  const int64_t base = (((int64_t)g * slots + slot) * page) * d + e;
  float acc = 0.f;
  for (int r = part; r < n; r += 8) acc += load_elem(kpool, base + (int64_t)r * d, bf16);
  red[part][e] = acc;
  __syncthreads();
  if (part == 0) {
    float sum = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) sum += red[x][e];
    reps[((int64_t)g * slots + slot) * d + e] = sum / (float)n;
  }
}

// Logical-order export of K / V / dK / dV: dst[t][g][:] = pool[g][slot][t % P][:].
__global__ void export_rows_kernel(const char* __restrict__ pool, char* __restrict__ dst,
                                   const int32_t* __restrict__ table, int hkv, int page,
                                   int slots, int max_logical, int row_bytes, int64_t t0,
                                   int64_t n_tok) {
  const int vec_per_row = row_bytes / 16;
  const int64_t total = n_tok * hkv * vec_per_row;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % vec_per_row);
    const int64_t tg = idx / vec_per_row;
    const int g = (int)(tg % hkv);
    const int64_t t = t0 + tg / hkv;
    const int slot = table[(int64_t)g * max_logical + t / page];
    const int64_t src = (((int64_t)g * slots + slot) * page + t % page) * row_bytes + c * 16;
    *reinterpret_cast<uint4*>(dst + tg * row_bytes + c * 16) =
        *reinterpret_cast<const uint4*>(pool + src);
  }
}

// dst[j][g][:] = reps[g][slot(j)][:]
__global__ void export_reps_kernel(const float* __restrict__ reps, float* __restrict__ dst,
                                   const int32_t* __restrict__ table, int hkv, int slots,
                                   int max_logical, int d, int64_t n_pages) {
  const int64_t total = n_pages * hkv * d;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx % d);
    const int64_t jg = idx / d;
    const int g = (int)(jg % hkv);
    const int64_t j = jg / hkv;
    const int slot = table[(int64_t)g * max_logical + j];
    dst[idx] = reps[((int64_t)g * slots + slot) * d + e];
  }
}

__global__ void zero_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void zero_tail_kernel(char* __restrict__ p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

int grid_for(int64_t work, int block) {
  int64_t b = (work + block - 1) / block;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_append(const LayerDev& L, const Geom& g, int elem_bytes, int64_t pos0,
                         int64_t n_tok, const void* k, const void* v, hipStream_t s) {
  const int row_bytes = g.d * elem_bytes;
  const int64_t work = n_tok * g.hkv * (row_bytes / 16);
  KernelTimer t(KT_APPEND, s);
  hipLaunchKernelGGL(append_kernel, dim3(grid_for(work, 256)), dim3(256), 0, s,
                     (char*)L.k, (char*)L.v, (const char*)k, (const char*)v, L.table, g.hkv,
                     g.page, g.slots, g.max_logical, row_bytes, pos0, n_tok);
  return hipGetLastError();
}

hipError_t launch_reps(const LayerDev& L, const Geom& g, bool bf16, int64_t first_page,
                       int64_t n_pages, int64_t length, hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  KernelTimer t(KT_APPEND, s);
  hipLaunchKernelGGL(reps_kernel, dim3((unsigned)n_pages, g.hkv), dim3(8 * g.d), 0, s,
                     (const void*)L.k, L.reps, L.table, g.page, g.slots, g.max_logical, g.d,
                     bf16, first_page, length);
  return hipGetLastError();
}

hipError_t launch_export(const LayerDev& L, const Geom& g, int what, int elem_bytes,
                         int64_t n_tok, void* dst, hipStream_t s, int64_t t0) {
  if (n_tok <= 0) return hipSuccess;
  if (what == 4) {
    const int64_t n_pages = (n_tok + g.page - 1) / g.page;
    hipLaunchKernelGGL(export_reps_kernel, dim3(grid_for(n_pages * g.hkv * g.d, 256)),
                       dim3(256), 0, s, (const float*)L.reps, (float*)dst, L.table, g.hkv,
                       g.slots, g.max_logical, g.d, n_pages);
    return hipGetLastError();
  }
  const char* src = nullptr;
  int row_bytes = g.d * elem_bytes;
  switch (what) {
    case 0: src = (const char*)L.k; break;
    case 1: src = (const char*)L.v; break;
    case 2: src = (const char*)L.dk; row_bytes = g.d * 4; break;
    default: src = (const char*)L.dv; row_bytes = g.d * 4; break;
  }
  const int64_t work = n_tok * g.hkv * (row_bytes / 16);
  hipLaunchKernelGGL(export_rows_kernel, dim3(grid_for(work, 256)), dim3(256), 0, s, src,
                     (char*)dst, L.table, g.hkv, g.page, g.slots, g.max_logical, row_bytes,
                     t0, n_tok);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 > 0) {
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n16, 256)), dim3(256), 0, s, (uint4*)p, n16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t tail = bytes - n16 * 16;
  if (tail > 0) {
    hipLaunchKernelGGL(zero_tail_kernel, dim3(1), dim3(16), 0, s, (char*)p + n16 * 16, tail);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace pkv
