// bf16 paged attention dK/dV for gfx950 (tile layout, swizzle and operand
// layouts are described in attn_bf16_tiles.h), and the backward launcher.
//
// Backward of one query chunk, key side ("Out of the Memory Barrier",
// gist.science de, sections 2.B and 2.D): every key that the chunk's rows can
// see receives dK = scale * dS^T Q and dV = P^T dO from those rows, added with
// fp32 atomics into the paged gradient pool, where the contributions of all
// later chunks accumulate.
#include "attn_bf16_tiles.h"

namespace pkv {
namespace {

template <int BQT>
struct __align__(1024) DkvSmem {
  char q[2][BQT * ROWB];
  char o[2][BQT * ROWB];
  float lsd[2][2 * BQT];  // per buffer: LSE of the BQT rows, then D of the BQT rows
  int qpl[1024];
  int n_qpl;
};

// grid ceil(n_keys / 128) * hkv * splits.  BQT: query rows per tile (32 or
// 64); OCC: waves per SIMD the register budget is sized for.
template <int OCC, int BQT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
dkdv_bf16_kernel(AttnCall c, int splits) {
  constexpr int ST = BQT / 32;  // 32-row sub-tiles per tile
  __shared__ DkvSmem<BQT> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  // Workgroup -> (KV head, slab, split): bid % Hkv = KV head keeps a head's
  // workgroups on the same XCDs; the earliest slabs (the most query rows)
  // first.
  const int bid = blockIdx.x;
  const int g = bid % c.g.hkv;
  const int m = bid / c.g.hkv;
  const int slab = m / splits, zsplit = m % splits;
  const int G = c.hq / c.g.hkv;
  const int P = c.g.page;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int64_t s_base = (int64_t)slab * 128;
  const int64_t kpage = s_base / P;
  const int64_t wk0 = s_base + 32 * w;            // this wave's first key
  const int s_rel = (int)(wk0 + l32 - c.q_pos0);  // this lane's key, relative to q_pos0
  const int nqp = (c.n_q + P - 1) / P;
  const int tiles_pp = P / BQT;

  // Row tiles (BQT query rows) of the chunk that can see this key slab.
  int n_rt, r_first = 0;
  if (c.sel.pages) {
    if (tid == 0) {
      int n = 0;
      for (int il = 0; il < nqp; ++il) {
        const int32_t* lst = c.sel.pages + ((int64_t)il * c.g.hkv + g) * c.sel.stride;
        const int cnt = sel_count(c, il, g);
        int lo = 0, hi = cnt;
        while (lo < hi) {  // ascending list: binary search for kpage
          const int mid = (lo + hi) >> 1;
          if (lst[mid] < kpage) lo = mid + 1; else hi = mid;
        }
        if (lo < cnt && lst[lo] == kpage) sm.qpl[n++] = il;
      }
      sm.n_qpl = n;
    }
    __syncthreads();
    n_rt = sm.n_qpl * tiles_pp;
  } else {
    r_first = (int)(s_base - c.q_pos0);
    if (r_first < 0) r_first = 0;
    r_first -= r_first % BQT;
    n_rt = (c.n_q - r_first + BQT - 1) / BQT;
  }
  const int total = n_rt * G;
  const int it0 = (int)((int64_t)total * zsplit / splits);
  const int it1 = (int)((int64_t)total * (zsplit + 1) / splits);
  if (it0 >= it1) return;

  bf16x8 kf[8], vf[8];
  const int slot = uni(c.L.table[(int64_t)g * c.g.max_logical + kpage]);
  const int64_t prow = ((int64_t)g * c.g.slots + slot) * P + ((wk0 + l32) % P);
  {
    const u16* kr = reinterpret_cast<const u16*>(c.L.k) + prow * D + 8 * half;
    const u16* vr = reinterpret_cast<const u16*>(c.L.v) + prow * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = as_bf16x8(ld16(kr + 16 * ks));
      vf[ks] = as_bf16x8(ld16(vr + 16 * ks));
    }
  }
  f32x16 kacc[4], vacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    kacc[dt] = f32x16{};
    vacc[dt] = f32x16{};
  }
  const float c2 = c.scale * kLog2e;

  auto tile_row0 = [&](int it, int* hh) -> int {
    *hh = g * G + it / n_rt;
    const int rt = it % n_rt;
    if (c.sel.pages) return sm.qpl[rt / tiles_pp] * P + (rt % tiles_pp) * BQT;
    return r_first + rt * BQT;
  };
  // Q and dO rows of the tile straight into LDS (rows past the chunk repeat its
  // last row and are masked); log2-scaled LSE and D of the rows by wave 0.
  TileDma<BQT, 4> dma;
  dma.init(w, lane);
  const int qrow_b = c.hq * ROWB;
  auto issue = [&](int b, int it) {
    int hh;
    const int row0 = tile_row0(it, &hh);
    const int64_t off = ((int64_t)row0 * c.hq + hh) * ROWB;
    const char* qb = reinterpret_cast<const char*>(c.q) + off;
    const char* ob = reinterpret_cast<const char*>(c.dout) + off;
    if (row0 + BQT <= c.n_q) {
      dma.issue(sm.q[b], w, qb, qrow_b);
      dma.issue(sm.o[b], w, ob, qrow_b);
    } else {
      dma.issue_clamped(sm.q[b], w, qb, qrow_b, c.n_q - 1 - row0);
      dma.issue_clamped(sm.o[b], w, ob, qrow_b, c.n_q - 1 - row0);
    }
    if (w == 0) {
#pragma unroll
      for (int x = 0; x < BQT / 32; ++x) {  // 64 values per instruction
        const int v = 64 * x + lane;         // value index in lsd[b]
        const bool is_d = v >= BQT;
        const int rr = row0 + (is_d ? v - BQT : v);
        const int rc = rr < c.n_q ? rr : c.n_q - 1;
        const float* src = (is_d ? c.delta : c.lse2) + (int64_t)hh * c.n_q + rc;
        __builtin_amdgcn_global_load_lds((const GLB_AS void*)src, (LDS_AS void*)(sm.lsd[b] + 64 * x),
                                         4, 0, 0);
      }
    }
  };

  issue(0, it0);
  wait_dma_and_sync();
  for (int it = it0; it < it1; ++it) {
    const int b = (it - it0) & 1;
    if (it + 1 < it1) issue(b ^ 1, it + 1);
    int hh;
    const int row0 = tile_row0(it, &hh);
    const int64_t t_min = c.q_pos0 + row0;
    const int64_t t_max = t_min + BQT - 1;
    if (wk0 <= t_max) {
      const char* qt = sm.q[b];
      const char* ot = sm.o[b];
      f32x16 sacc[ST], pacc[ST];
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        sacc[st] = f32x16{};
        pacc[st] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int st = 0; st < ST; ++st) {
          sacc[st] = mfma(frag_row(qt, 32 * st + l32, ks, half), kf[ks], sacc[st]);
          pacc[st] = mfma(frag_row(ot, 32 * st + l32, ks, half), vf[ks], pacc[st]);
        }
      }
      // keys past a row (causal) and rows past the chunk get probability 0
      const float* lse_b = sm.lsd[b];
      const float* dl_b = sm.lsd[b] + BQT;
      auto pass = [&](auto masked) {
        constexpr bool MASK = decltype(masked)::value;
#pragma unroll
        for (int kk = 0; kk < 2 * ST; ++kk) {
          // tile rows 16 kk .. 16 kk + 15: sub-tile kk / 2, entries 8 (kk % 2) ..
          const int st = kk >> 1;
          float p[8], ds[8];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j4 = 2 * (kk & 1) + jj;
            const int rb = 32 * st + 8 * j4 + 4 * half;  // first of the 4 rows
            const float4 L4 = *reinterpret_cast<const float4*>(lse_b + rb);
            const float4 D4 = *reinterpret_cast<const float4*>(dl_b + rb);
            const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
            const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              float sv = sacc[st][4 * j4 + x];
              if (MASK) {
                const int tr = row0 + rb + x;
                if (s_rel > tr || tr >= c.n_q) sv = -INFINITY;
              }
              const float pr = ex2(fmaf(sv, c2, -Lr[x]));
              p[4 * jj + x] = pr;
              ds[4 * jj + x] = pr * (pacc[st][4 * j4 + x] - Dr[x]);
            }
          }
          u32x4 pv, dv;
          pv.x = pack2(p[0], p[1]);
          pv.y = pack2(p[2], p[3]);
          pv.z = pack2(p[4], p[5]);
          pv.w = pack2(p[6], p[7]);
          dv.x = pack2(ds[0], ds[1]);
          dv.y = pack2(ds[2], ds[3]);
          dv.z = pack2(ds[4], ds[5]);
          dv.w = pack2(ds[6], ds[7]);
          const bf16x8 pa = as_bf16x8(pv), da = as_bf16x8(dv);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            vacc[dt] = mfma(pa, frag_tr(ot, 16 * kk, 32 * dt, lane), vacc[dt]);
            kacc[dt] = mfma(da, frag_tr(qt, 16 * kk, 32 * dt, lane), kacc[dt]);
          }
        }
      };
      if ((wk0 + 31 > t_min) || (row0 + BQT > c.n_q))
        pass(std::true_type{});
      else
        pass(std::false_type{});
    }
    wait_dma_and_sync();
  }

  // One fp32 atomic add per gradient element into the pool.
  float* dkp = c.L.dk + (((int64_t)g * c.g.slots + slot) * P + (wk0 % P)) * D + l32;
  float* dvp = c.L.dv + (((int64_t)g * c.g.slots + slot) * P + (wk0 % P)) * D + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int srel = 8 * (r >> 2) + 4 * half + (r & 3);
    if (wk0 + srel >= n_keys) continue;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      unsafeAtomicAdd(dkp + srel * D + 32 * dt, kacc[dt][r] * c.scale);
      unsafeAtomicAdd(dvp + srel * D + 32 * dt, vacc[dt][r]);
    }
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const AttnCall& c, hipStream_t s) {
  hipError_t e = launch_delta(c, true, s);
  if (e != hipSuccess) return e;
  e = launch_dq_bf16(c, s);
  if (e != hipSuccess) return e;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int n_slabs = (int)((n_keys + 127) / 128);
  int splits = (2048 + n_slabs * c.g.hkv - 1) / (n_slabs * c.g.hkv);
  if (splits < 1) splits = 1;
  if (splits > 16) splits = 16;
  // PKV_DKDV: "1x32" / "1x64" (32- or 64-row query tiles)
  static const bool rows32 = [] {
    const char* v = getenv("PKV_DKDV");
    return v && !strcmp(v, "1x32");
  }();
  KernelTimer t(KT_DKDV, s);
  const dim3 grid(n_slabs * c.g.hkv * splits);
  if (rows32)
    hipLaunchKernelGGL((dkdv_bf16_kernel<1, 32>), grid, dim3(256), 0, s, c, splits);
  else
    hipLaunchKernelGGL((dkdv_bf16_kernel<1, 64>), grid, dim3(256), 0, s, c, splits);
  return hipGetLastError();
}

}  // namespace pkv
