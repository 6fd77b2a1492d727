// D = rowsum(dO * O) per (query head, row): the correction term of the
// softmax backward (dS = P * (dP - D)), "Out of the Memory Barrier"
// (gist.science de, section 2.A: the backward recomputes the forward's
// probabilities instead of storing them).  fp32 accumulation of the stored
// O and dO values.  16 lanes per row.  Also writes the log-sum-exp in base 2
// (lse * log2 e), the form the bf16 backward kernels use with v_exp_f32.
#include "pkv_internal.h"

namespace pkv {
namespace {

__device__ __forceinline__ float ldv(const void* p, int64_t i, bool bf16) {
  if (bf16) {
    const unsigned short u = reinterpret_cast<const unsigned short*>(p)[i];
    return __uint_as_float(((unsigned)u) << 16);
  }
  return reinterpret_cast<const float*>(p)[i];
}

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
  if (row < n_rows) {
    for (int e = lane; e < d; e += 16)
      acc = fmaf(ldv(o, row * d + e, bf16), ldv(dO, row * d + e, bf16), acc);
  }
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
