// bf16 paged attention dQ for gfx950 (tile layout, swizzle and operand
// layouts are described in attn_bf16_tiles.h).
//
// Backward of one query chunk, query side ("Out of the Memory Barrier",
// gist.science de, section 2.B): the probabilities are recomputed from the
// forward's log-sum-exp and dQ = scale * dS K is written per row.
#include "attn_bf16_tiles.h"

namespace pkv {
namespace {

template <int NT, int BNT>
__global__ void __launch_bounds__(256 / NT) __attribute__((amdgpu_waves_per_eu(2, 2))) dq_bf16_kernel(AttnCall c, int n_qblocks) {
  constexpr int NW = 4 / NT;
  constexpr int MT = BNT / 32;
  constexpr int TB = BNT * ROWB;
  __shared__ __align__(1024) char sm[2][2 * TB];  // [buffer][K tile | V tile]
  const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int G = c.hq / c.g.hkv;
  const int bid = blockIdx.x;
  const int g = uni(bid % c.g.hkv), m = uni(bid / c.g.hkv);
  const int qb = n_qblocks - 1 - m / G;
  const int h = g * G + m % G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const int rw0 = r0 + 32 * NT * w;
  const int tw_min = rw0 < rlast ? rw0 : rlast;
  const int tw_max = rw0 + 32 * NT - 1 < rlast ? rw0 + 32 * NT - 1 : rlast;

  bf16x8 qf[NT][8], df[NT][8];
  int t_rel[NT];
  float lse2[NT], Dl[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int r = rw0 + 32 * nt + l32;
    r = r < rlast ? r : rlast;
    t_rel[nt] = r;
    const int64_t off = ((int64_t)r * c.hq + h) * D + 8 * half;
    const u16* qrow = reinterpret_cast<const u16*>(c.q) + off;
    const u16* drow = reinterpret_cast<const u16*>(c.dout) + off;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[nt][ks] = as_bf16x8(ld16(qrow + 16 * ks));
      df[nt][ks] = as_bf16x8(ld16(drow + 16 * ks));
    }
    lse2[nt] = c.lse2[(int64_t)h * c.n_q + r];
    Dl[nt] = c.delta[(int64_t)h * c.n_q + r];
  }
  const float c2 = c.scale * kLog2e;

  int n_tiles;
  TileAhead<BNT> walk = make_ahead<BNT>(c, g, r0, rlast, &n_tiles);
  TileDma<BNT, NW> dma;
  dma.init(w, lane);
  auto issue = [&](int b, const KeyTile& t, int slot) {
    dma.issue_direct(sm[b], w, key_rows_at<BNT>(c, c.L.k, g, t, slot), ROWB);
    dma.issue_direct(sm[b] + TB, w, key_rows_at<BNT>(c, c.L.v, g, t, slot), ROWB);
  };

  f32x16 qacc[4][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) qacc[dt][nt] = f32x16{};

  KeyTile t_cur{0, 0, 0};
  if (n_tiles > 0) {
    int slot;
    t_cur = walk.take(&slot);
    issue(0, t_cur, slot);
  }
  wait_dma_and_sync();

  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    KeyTile t_next{0, 0, 0};
    if (j + 1 < n_tiles) {
      int slot;
      t_next = walk.take(&slot);
      issue(b ^ 1, t_next, slot);
    }
    const char* kt = sm[b];
    const char* vt = sm[b] + TB;
    const int srel0 = t_cur.srel0;
    if (srel0 <= tw_max) {
      f32x16 sacc[MT][NT], pacc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          sacc[mt][nt] = f32x16{};
          pacc[mt][nt] = f32x16{};
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 ak = frag_row(kt, 32 * mt + l32, ks, half);
          const bf16x8 av = frag_row(vt, 32 * mt + l32, ks, half);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            sacc[mt][nt] = mfma(ak, qf[nt][ks], sacc[mt][nt]);
            pacc[mt][nt] = mfma(av, df[nt][ks], pacc[mt][nt]);
          }
        }
      }
      if (srel0 + BNT - 1 > tw_min) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int sr = srel0 + 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
              if (sr > t_rel[nt]) sacc[mt][nt][r] = -INFINITY;
            }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float nl = -lse2[nt];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = ex2(fmaf(sacc[mt][nt][r], c2, nl));
            sacc[mt][nt][r] = p * (pacc[mt][nt][r] - Dl[nt]);
          }
        }
#pragma unroll
      for (int kk = 0; kk < 2 * MT; ++kk) {
        bf16x8 bfr[NT];
        const int mt = kk >> 1, rb = 8 * (kk & 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 pv;
          pv.x = pack2(sacc[mt][nt][rb + 0], sacc[mt][nt][rb + 1]);
          pv.y = pack2(sacc[mt][nt][rb + 2], sacc[mt][nt][rb + 3]);
          pv.z = pack2(sacc[mt][nt][rb + 4], sacc[mt][nt][rb + 5]);
          pv.w = pack2(sacc[mt][nt][rb + 6], sacc[mt][nt][rb + 7]);
          bfr[nt] = as_bf16x8(pv);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 a = frag_tr(kt, 16 * kk, 32 * dt, lane);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) qacc[dt][nt] = mfma(a, bfr[nt], qacc[dt][nt]);
        }
      }
    }
    t_cur = t_next;
    wait_dma_and_sync();
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int my_r = rw0 + 32 * nt + l32;
    if (my_r <= rlast) {
      float* out = c.dq + ((int64_t)my_r * c.hq + h) * D + 4 * half;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          float4 v;
          v.x = qacc[dt][nt][4 * j4 + 0] * c.scale;
          v.y = qacc[dt][nt][4 * j4 + 1] * c.scale;
          v.z = qacc[dt][nt][4 * j4 + 2] * c.scale;
          v.w = qacc[dt][nt][4 * j4 + 3] * c.scale;
          *reinterpret_cast<float4*>(out + 32 * dt + 8 * j4) = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_dq_bf16(const AttnCall& c, hipStream_t s) {
  const int nqb = (c.n_q + BM - 1) / BM;
  KernelTimer t(KT_DQ, s);
  hipLaunchKernelGGL((dq_bf16_kernel<1, 64>), dim3(nqb * c.hq), dim3(256), 0, s, c, nqb);
  return hipGetLastError();
}

}  // namespace pkv
