// fp32 paged attention (forward, dQ, dK/dV), the library's fp32 mode.
//
// Plain fp32 VALU arithmetic with expf/logf; a team of 4 lanes owns one row
// (query row or key row) and holds d/4 of its elements.  K/V (forward, dQ) or
// Q/dO (dK/dV) tiles are staged in LDS and read by every team.  Definitions:
// "Out of the Memory Barrier" (gist.science de, sections 2.A, 2.B, 2.D;
// sciencestack.ai, Figure 3): exact causal softmax attention of a query chunk
// over the paged cache, recompute-backward, dK/dV added in place with atomics.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kTeam = 4;                // lanes per row
constexpr int kRows = 64 / kTeam;       // rows per 64-thread workgroup
constexpr int kKT = 32;                 // keys (or queries) per LDS tile

__device__ __forceinline__ float team_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Key enumeration of one query page range: dense = keys 0..n_virtual-1;
// sparse = the pages of `list` (ascending), P keys each.
struct KeySeq {
  const int32_t* list;  // nullptr: dense
  int page;
  int max_logical;      // list entries are clamped into [0, max_logical)
  __device__ __forceinline__ int64_t key(int64_t v) const {
    if (!list) return v;
    int pg = list[v / page];
    pg = pg < 0 ? 0 : (pg >= max_logical ? max_logical - 1 : pg);
    return (int64_t)pg * page + v % page;
  }
};

__device__ __forceinline__ int sel_count(const AttnCall& c, int il, int g) {
  const int n = c.sel.count[(int64_t)il * c.g.hkv + g];
  return n < 0 ? 0 : (n > c.sel.stride ? c.sel.stride : n);
}

template <int D>
__global__ void __launch_bounds__(64) fwd_f32_kernel(AttnCall c) {
  constexpr int E = D / kTeam;
  __shared__ float Ks[kKT][D];
  __shared__ float Vs[kKT][D];
  __shared__ int64_t Ss[kKT];
  const int tid = threadIdx.x, part = tid % kTeam, rloc = tid / kTeam;
  const int h = blockIdx.y;
  const int G = c.hq / c.g.hkv, g = h / G;
  const int r0 = blockIdx.x * kRows;
  const int r = r0 + rloc;
  const bool valid = r < c.n_q;
  const int rr = valid ? r : c.n_q - 1;
  const int64_t t = c.q_pos0 + rr;
  int rmax = r0 + kRows - 1;
  if (rmax >= c.n_q) rmax = c.n_q - 1;
  const int64_t tmax = c.q_pos0 + rmax;

  KeySeq ks{nullptr, c.g.page, c.g.max_logical};
  int64_t n_virtual = tmax + 1;
  if (c.sel.pages) {
    const int il = r0 / c.g.page;
    ks.list = c.sel.pages + ((int64_t)il * c.g.hkv + g) * c.sel.stride;
    n_virtual = (int64_t)sel_count(c, il, g) * c.g.page;
  }

  const float* q = reinterpret_cast<const float*>(c.q) + ((int64_t)rr * c.hq + h) * D;
  float qr[E], o[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    qr[i] = q[part + kTeam * i];
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float* kp = reinterpret_cast<const float*>(c.L.k);
  const float* vp = reinterpret_cast<const float*>(c.L.v);
  const int32_t* tab = c.L.table + (int64_t)g * c.g.max_logical;

  for (int64_t v0 = 0; v0 < n_virtual; v0 += kKT) {
    __syncthreads();
    for (int x = tid; x < kKT * D; x += 64) {
      const int kr = x / D, e = x % D;
      const int64_t vv = v0 + kr;
      int64_t s = -1;
      float kv = 0.f, vvv = 0.f;
      if (vv < n_virtual) {
        s = ks.key(vv);
        if (s <= tmax) {
          const int slot = tab[s / c.g.page];
          const int64_t off = (((int64_t)g * c.g.slots + slot) * c.g.page + s % c.g.page) * D + e;
          kv = kp[off];
          vvv = vp[off];
        } else {
          s = -1;
        }
      }
      Ks[kr][e] = kv;
      Vs[kr][e] = vvv;
      if (e == 0) Ss[kr] = s;
    }
    __syncthreads();
    for (int kr = 0; kr < kKT; ++kr) {
      const int64_t s = Ss[kr];
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) dot = fmaf(qr[i], Ks[kr][part + kTeam * i], dot);
      dot = team_sum(dot);
      if (s < 0 || s > t) continue;
      const float x = dot * c.scale;
      const float mn = fmaxf(m, x);
      const float corr = expf(m - mn);
      const float p = expf(x - mn);
      l = l * corr + p;
#pragma unroll
      for (int i = 0; i < E; ++i) o[i] = fmaf(p, Vs[kr][part + kTeam * i], o[i] * corr);
      m = mn;
    }
  }
  if (!valid) return;
  float* out = reinterpret_cast<float*>(c.o_out) + ((int64_t)r * c.hq + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < E; ++i) out[part + kTeam * i] = o[i] * inv;
  if (part == 0) c.lse[(int64_t)h * c.n_q + r] = m + logf(l);
}

template <int D>
__global__ void __launch_bounds__(64) dq_f32_kernel(AttnCall c) {
  constexpr int E = D / kTeam;
  __shared__ float Ks[kKT][D];
  __shared__ float Vs[kKT][D];
  __shared__ int64_t Ss[kKT];
  const int tid = threadIdx.x, part = tid % kTeam, rloc = tid / kTeam;
  const int h = blockIdx.y;
  const int G = c.hq / c.g.hkv, g = h / G;
  const int r0 = blockIdx.x * kRows;
  const int r = r0 + rloc;
  const bool valid = r < c.n_q;
  const int rr = valid ? r : c.n_q - 1;
  const int64_t t = c.q_pos0 + rr;
  int rmax = r0 + kRows - 1;
  if (rmax >= c.n_q) rmax = c.n_q - 1;
  const int64_t tmax = c.q_pos0 + rmax;

  KeySeq ks{nullptr, c.g.page, c.g.max_logical};
  int64_t n_virtual = tmax + 1;
  if (c.sel.pages) {
    const int il = r0 / c.g.page;
    ks.list = c.sel.pages + ((int64_t)il * c.g.hkv + g) * c.sel.stride;
    n_virtual = (int64_t)sel_count(c, il, g) * c.g.page;
  }
  const float* q = reinterpret_cast<const float*>(c.q) + ((int64_t)rr * c.hq + h) * D;
  const float* dO = reinterpret_cast<const float*>(c.dout) + ((int64_t)rr * c.hq + h) * D;
  float qr[E], dor[E], dq[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    qr[i] = q[part + kTeam * i];
    dor[i] = dO[part + kTeam * i];
    dq[i] = 0.f;
  }
  const float lse = c.lse_in[(int64_t)h * c.n_q + rr];
  const float Dt = c.delta[(int64_t)h * c.n_q + rr];
  const float* kp = reinterpret_cast<const float*>(c.L.k);
  const float* vp = reinterpret_cast<const float*>(c.L.v);
  const int32_t* tab = c.L.table + (int64_t)g * c.g.max_logical;

  for (int64_t v0 = 0; v0 < n_virtual; v0 += kKT) {
    __syncthreads();
    for (int x = tid; x < kKT * D; x += 64) {
      const int kr = x / D, e = x % D;
      const int64_t vv = v0 + kr;
      int64_t s = -1;
      float kv = 0.f, vvv = 0.f;
      if (vv < n_virtual) {
        s = ks.key(vv);
        if (s <= tmax) {
          const int slot = tab[s / c.g.page];
          const int64_t off = (((int64_t)g * c.g.slots + slot) * c.g.page + s % c.g.page) * D + e;
          kv = kp[off];
          vvv = vp[off];
        } else {
          s = -1;
        }
      }
      Ks[kr][e] = kv;
      Vs[kr][e] = vvv;
      if (e == 0) Ss[kr] = s;
    }
    __syncthreads();
    for (int kr = 0; kr < kKT; ++kr) {
      const int64_t s = Ss[kr];
      float dot = 0.f, dpv = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        dot = fmaf(qr[i], Ks[kr][part + kTeam * i], dot);
        dpv = fmaf(dor[i], Vs[kr][part + kTeam * i], dpv);
      }
      dot = team_sum(dot);
      dpv = team_sum(dpv);
      if (s < 0 || s > t) continue;
      const float p = expf(dot * c.scale - lse);
      const float ds = p * (dpv - Dt);
#pragma unroll
      for (int i = 0; i < E; ++i) dq[i] = fmaf(ds, Ks[kr][part + kTeam * i], dq[i]);
    }
  }
  if (!valid) return;
  float* out = c.dq + ((int64_t)r * c.hq + h) * D;
#pragma unroll
  for (int i = 0; i < E; ++i) out[part + kTeam * i] = dq[i] * c.scale;
}

// grid (ceil(n_keys / kRows), hkv).  Each team owns one key row s; loops over
// every (query row, head of the group) of the chunk that may attend to s.
template <int D>
__global__ void __launch_bounds__(64) dkdv_f32_kernel(AttnCall c) {
  constexpr int E = D / kTeam;
  __shared__ float Qs[kKT][D];
  __shared__ float Os[kKT][D];
  __shared__ float Ls[kKT], Dl[kKT];
  __shared__ unsigned char qp_ok[1024];
  const int tid = threadIdx.x, part = tid % kTeam, kloc = tid / kTeam;
  const int g = blockIdx.y;
  const int G = c.hq / c.g.hkv;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int64_t s0 = (int64_t)blockIdx.x * kRows;  // kRows divides page
  const int64_t s = s0 + kloc;
  const bool valid = s < n_keys;
  const int64_t ss = valid ? s : n_keys - 1;
  const int P = c.g.page;
  const int64_t kpage = s0 / P;
  const int nqp = (c.n_q + P - 1) / P;
  const int first_qp = (int)(c.q_pos0 / P);

  // Which query pages of the chunk attend to this key page.
  if (c.sel.pages) {
    for (int il = tid; il < nqp; il += 64) {
      const int32_t* lst = c.sel.pages + ((int64_t)il * c.g.hkv + g) * c.sel.stride;
      const int cnt = sel_count(c, il, g);
      bool ok = false;
      for (int u = 0; u < cnt; ++u) ok |= (lst[u] == kpage);
      qp_ok[il] = ok;
    }
  } else {
    for (int il = tid; il < nqp; il += 64) qp_ok[il] = (first_qp + il >= kpage);
  }
  __syncthreads();

  const int slot = c.L.table[(int64_t)g * c.g.max_logical + ss / P];
  const int64_t poff = (((int64_t)g * c.g.slots + slot) * P + ss % P) * D;
  const float* kp = reinterpret_cast<const float*>(c.L.k) + poff;
  const float* vp = reinterpret_cast<const float*>(c.L.v) + poff;
  float kr[E], vr[E], dk[E], dv[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    kr[i] = kp[part + kTeam * i];
    vr[i] = vp[part + kTeam * i];
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  // first query row that can see s0
  int rstart = (int)(s0 - c.q_pos0);
  if (rstart < 0) rstart = 0;
  rstart -= rstart % kKT;
  for (int h = g * G; h < (g + 1) * G; ++h) {
    for (int q0 = rstart; q0 < c.n_q; q0 += kKT) {
      if (!qp_ok[q0 / P] && !qp_ok[(q0 + kKT - 1 < c.n_q ? q0 + kKT - 1 : c.n_q - 1) / P]) continue;
      __syncthreads();
      const float* qg = reinterpret_cast<const float*>(c.q);
      const float* dg = reinterpret_cast<const float*>(c.dout);
      for (int x = tid; x < kKT * D; x += 64) {
        const int rq = x / D, e = x % D;
        const int row = q0 + rq;
        float a = 0.f, b = 0.f;
        if (row < c.n_q) {
          a = qg[((int64_t)row * c.hq + h) * D + e];
          b = dg[((int64_t)row * c.hq + h) * D + e];
        }
        Qs[rq][e] = a;
        Os[rq][e] = b;
      }
      for (int rq = tid; rq < kKT; rq += 64) {
        const int row = q0 + rq;
        Ls[rq] = row < c.n_q ? c.lse_in[(int64_t)h * c.n_q + row] : 0.f;
        Dl[rq] = row < c.n_q ? c.delta[(int64_t)h * c.n_q + row] : 0.f;
      }
      __syncthreads();
      for (int rq = 0; rq < kKT; ++rq) {
        const int row = q0 + rq;
        float dot = 0.f, dpv = 0.f;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          dot = fmaf(Qs[rq][part + kTeam * i], kr[i], dot);
          dpv = fmaf(Os[rq][part + kTeam * i], vr[i], dpv);
        }
        dot = team_sum(dot);
        dpv = team_sum(dpv);
        if (row >= c.n_q || !qp_ok[row / P] || s > c.q_pos0 + row || !valid) continue;
        const float p = expf(dot * c.scale - Ls[rq]);
        const float ds = p * (dpv - Dl[rq]);
#pragma unroll
        for (int i = 0; i < E; ++i) {
          dk[i] = fmaf(ds, Qs[rq][part + kTeam * i], dk[i]);
          dv[i] = fmaf(p, Os[rq][part + kTeam * i], dv[i]);
        }
      }
    }
  }
  if (!valid) return;
  float* dkp = c.L.dk + poff;
  float* dvp = c.L.dv + poff;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    unsafeAtomicAdd(dkp + part + kTeam * i, dk[i] * c.scale);
    unsafeAtomicAdd(dvp + part + kTeam * i, dv[i]);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const AttnCall& c, hipStream_t s) {
  const dim3 grid((c.n_q + kRows - 1) / kRows, c.hq);
  KernelTimer t(KT_FWD, s);
  if (c.g.d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, s, c);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const AttnCall& c, hipStream_t s) {
  hipError_t e = launch_delta(c, false, s);
  if (e != hipSuccess) return e;
  const dim3 gq((c.n_q + kRows - 1) / kRows, c.hq);
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const dim3 gk((unsigned)((n_keys + kRows - 1) / kRows), c.g.hkv);
  {
    KernelTimer t(KT_DQ, s);
    if (c.g.d == 64)
      hipLaunchKernelGGL(dq_f32_kernel<64>, gq, dim3(64), 0, s, c);
    else
      hipLaunchKernelGGL(dq_f32_kernel<128>, gq, dim3(64), 0, s, c);
  }
  {
    KernelTimer t(KT_DKDV, s);
    if (c.g.d == 64)
      hipLaunchKernelGGL(dkdv_f32_kernel<64>, gk, dim3(64), 0, s, c);
    else
      hipLaunchKernelGGL(dkdv_f32_kernel<128>, gk, dim3(64), 0, s, c);
  }
  return hipGetLastError();
}

}  // namespace pkv
