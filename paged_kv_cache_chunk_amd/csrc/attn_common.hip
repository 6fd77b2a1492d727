// D = rowsum(dO * O) per (query head, row): the correction term of the
// softmax backward (dS = P * (dP - D)), "Out of the Memory Barrier"
// (gist.science de, section 2.A: the backward recomputes the forward's
// probabilities instead of storing them).  fp32 accumulation of the stored
// O and dO values, 16-byte loads.  Also writes the log-sum-exp in base 2
// (lse * log2 e), the form the bf16 backward kernels use with v_exp_f32.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Sum over 8 consecutive elements of o * dO starting at element i.
__device__ __forceinline__ float dot8(const void* o, const void* dO, int64_t i, bool bf16) {
  float acc = 0.f;
  if (bf16) {  // 16 bytes per operand: 8 bf16 values
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned short*>(o) + i);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned short*>(dO) + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(__uint_as_float(a[k] << 16), __uint_as_float(b[k] << 16), acc);
      acc = fmaf(__uint_as_float(a[k] & 0xffff0000u), __uint_as_float(b[k] & 0xffff0000u), acc);
    }
  } else {  // 2 x 16 bytes per operand: 8 fp32 values
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(o) + i + 4 * h);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(dO) + i + 4 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = fmaf(a[k], b[k], acc);
    }
  }
  return acc;
}

// 16 lanes per row; lane j sums elements 8 j .. 8 j + 7 (d = 128; d = 64
// leaves lanes 8-15 idle), then the 16 partial sums are added in a tree.
__global__ void __launch_bounds__(256) delta_kernel(const void* __restrict__ o,
                                                    const void* __restrict__ dO,
                                                    const float* __restrict__ lse,
                                                    float* __restrict__ delta,
                                                    float* __restrict__ lse2, int hq, int n_q,
                                                    int d, bool bf16) {
  const int64_t row = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;  // row = t * hq + h
  const int lane = threadIdx.x % 16;
  const int64_t n_rows = (int64_t)n_q * hq;
  float acc = 0.f;
  if (row < n_rows && 8 * lane < d) acc = dot8(o, dO, row * d + 8 * lane, bf16);
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (row < n_rows && lane == 0) {
    const int64_t t = row / hq;
    const int h = (int)(row % hq);
    delta[(int64_t)h * n_q + t] = acc;
    if (lse2) lse2[(int64_t)h * n_q + t] = lse[(int64_t)h * n_q + t] * 1.4426950408889634f;
  }
}

}  // namespace

hipError_t launch_delta(const AttnCall& c, bool bf16, hipStream_t s) {
  const int64_t n_rows = (int64_t)c.n_q * c.hq;
  KernelTimer t(KT_DELTA, s);
  hipLaunchKernelGGL(delta_kernel, dim3((unsigned)((n_rows + 15) / 16)), dim3(256), 0, s,
                     c.o, c.dout, c.lse_in, c.delta, c.lse2, c.hq, c.n_q, c.g.d, bf16);
  return hipGetLastError();
}

}  // namespace pkv
