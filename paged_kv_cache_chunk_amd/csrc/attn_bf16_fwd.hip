// bf16 paged attention forward for gfx950 (tile layout, swizzle and operand
// layouts are described in attn_bf16_tiles.h).
//
// Per query chunk and head, the online-softmax forward of exact causal
// attention over the paged keys ("Out of the Memory Barrier", gist.science
// de, sections 2.A and 2.B): O and the log-sum-exp of every row.
#include "attn_bf16_tiles.h"

namespace pkv {
namespace {

// NT: 32-row column tiles per wave (a wave owns 32*NT query rows);
// BNT: keys per tile.  A workgroup owns 128 rows of one query head: a whole
// work unit, or one part of a tail-split unit (TailSplit).
template <int NT, int BNT>
__global__ void __launch_bounds__(256 / NT) __attribute__((amdgpu_waves_per_eu(2, 2))) fwd_bf16_kernel(AttnCall c, int n_qblocks) {
  constexpr int NW = 4 / NT;          // waves per workgroup
  constexpr int MT = BNT / 32;        // 32-key m-tiles per tile
  constexpr int TB = BNT * ROWB;      // bytes per K or V tile
  static_assert(NT == 1, "the tail split's partial layout holds 32 rows per wave");
  static_assert(BM == kFwdRows, "work unit rows");
  __shared__ __align__(1024) char sm[2][2 * TB];  // [buffer][K tile | V tile]
  const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  // Workgroup -> work unit (and part): units [0, n_whole) first, then the
  // first parts of the split units, then their second parts.
  int bid = blockIdx.x, part = -1;
  if (c.split.n_split > 0 && bid >= c.split.n_whole) {
    const int j = bid - c.split.n_whole;
    part = j >= c.split.n_split ? 1 : 0;
    bid = c.split.n_whole + (part ? j - c.split.n_split : j);
  }
  // Work unit -> (query block, head): workgroups are dealt to the 8 XCDs
  // round-robin, so unit % Hkv = KV head keeps every head's workgroups on the
  // same XCDs (sharing their L2 for that head's K/V); longest rows first.
  const int G = c.hq / c.g.hkv;
  const int g = uni(bid % c.g.hkv), m = uni(bid / c.g.hkv);
  const int qb = n_qblocks - 1 - m / G;
  const int h = g * G + m % G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const int rw0 = r0 + 32 * NT * w;   // wave's first row (relative to q_pos0)
  const int tw_min = rw0 < rlast ? rw0 : rlast;
  const int tw_max = rw0 + 32 * NT - 1 < rlast ? rw0 + 32 * NT - 1 : rlast;

  bf16x8 qf[NT][8];
  int t_rel[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int r = rw0 + 32 * nt + l32;
    r = r < rlast ? r : rlast;
    t_rel[nt] = r;
    const u16* qrow = reinterpret_cast<const u16*>(c.q) + ((int64_t)r * c.hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }

  int n_tiles;
  TileAhead<BNT> walk = make_ahead<BNT>(c, g, r0, rlast, &n_tiles, part);
  TileDma<BNT, NW> dma;
  dma.init(w, lane);
  auto issue = [&](int b, const KeyTile& t, int slot) {
    dma.issue_direct(sm[b], w, key_rows_at<BNT>(c, c.L.k, g, t, slot), ROWB);
    dma.issue_direct(sm[b] + TB, w, key_rows_at<BNT>(c, c.L.v, g, t, slot), ROWB);
  };

  f32x16 oacc[4][NT];
  float m_ref[NT], l_i[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt][nt] = f32x16{};
    m_ref[nt] = -INFINITY;
    l_i[nt] = 0.f;
  }
  const float c2 = c.scale * kLog2e;

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
    const int srel0 = t_cur.srel0;  // tile's first key, relative to q_pos0
    if (srel0 <= tw_max) {
      // S^T = K Q^T for this tile; keys past a row get -inf on tiles that
      // cross this wave's causal diagonal
      f32x16 sacc[MT][NT];
      auto scores = [&]() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 a = frag_row(kt, 32 * mt + l32, ks, half);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = mfma(a, qf[nt][ks], sacc[mt][nt]);
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
      };
      // Probabilities 2^(s c2 - m_ref) of column tile nt, packed to bf16 in
      // MFMA B-operand order (pk[kk] = rows 16 kk .. 16 kk + 15 of the tile);
      // returns their sum, taken over the packed values (v_dot2c with ones),
      // i.e. over exactly the weights the P V product uses.
      u32x4 pk[2 * MT][NT];
      auto probs = [&](int nt) -> float {
        const float mneg = -m_ref[nt];
        float rs = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2 * MT; ++kk) {
          const int mt = kk >> 1, rb = 8 * (kk & 1);
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = ex2(fmaf(sacc[mt][nt][rb + e], c2, mneg));
          u32x4 v;
          v.x = pack2(p[0], p[1]);
          v.y = pack2(p[2], p[3]);
          v.z = pack2(p[4], p[5]);
          v.w = pack2(p[6], p[7]);
          pk[kk][nt] = v;
#pragma unroll
          for (int e = 0; e < 4; ++e) rs = dot2_ones(v[e], rs);
        }
        return rs;
      };
      scores();
      // Lazy rescale: the reference maximum m_ref is kept while every
      // probability stays <= 2^8 (exact enough in fp32, representable in
      // bf16).  The probabilities are computed against it; if a row's sum
      // over the tile exceeds 2^8 (which any probability above 2^8 implies;
      // also inf or NaN, as on a wave's first tile, where m_ref = -inf), the
      // reference moves to the running row maximum, O and l are rescaled and
      // the probabilities are computed again.  On i.i.d. scores the first
      // tile's maximum is rarely exceeded by 8 (base 2), so the per-tile
      // maximum search is skipped on almost every tile.
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float rs, alpha = 1.f;
        bool moved = false;
#pragma nounroll
        for (int pass = 0;; ++pass) {
          rs = probs(nt);
          if (pass == 1 || !__any(!(rs <= 256.f))) break;
          float mx = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][nt][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
          const float mr = fmaxf(m_ref[nt], mx);
          alpha = ex2(m_ref[nt] - mr);
          m_ref[nt] = mr;
          moved = true;
        }
        if (moved) {
          l_i[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt][nt] *= alpha;
        }
        l_i[nt] += rs;
      }
#pragma unroll
      for (int kk = 0; kk < 2 * MT; ++kk) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 a = frag_tr(vt, 16 * kk, 32 * dt, lane);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = mfma(a, as_bf16x8(pk[kk][nt]), oacc[dt][nt]);
        }
      }
    }
    t_cur = t_next;
    wait_dma_and_sync();
  }

  if (part >= 0) {
    // Store this part's partial, lane-major (each store instruction writes
    // 1 KB of a wave): O as 16 float4 per lane, then m_ref and l_i per lane;
    // fwd_merge_kernel combines the two parts.
    const int s_unit = bid - c.split.n_whole;
    float* mine = c.split.part + ((int64_t)(2 * s_unit + part) * NW + w) * kFwdPartWaveFloats;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        float4 v;
        v.x = oacc[dt][0][4 * j4 + 0];
        v.y = oacc[dt][0][4 * j4 + 1];
        v.z = oacc[dt][0][4 * j4 + 2];
        v.w = oacc[dt][0][4 * j4 + 3];
        *reinterpret_cast<float4*>(mine + (dt * 4 + j4) * 256 + 4 * lane) = v;
      }
    mine[4096 + lane] = m_ref[0];
    mine[4096 + 64 + lane] = l_i[0];
    return;
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int my_r = rw0 + 32 * nt + l32;
    const float lt = l_i[nt] + __shfl_xor(l_i[nt], 32);
    if (my_r <= rlast) {
      const float inv = 1.f / lt;
      u16* orow = reinterpret_cast<u16*>(c.o_out) + ((int64_t)my_r * c.hq + h) * D + 4 * half;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          u32x2 v;
          v.x = pack2(oacc[dt][nt][4 * j4 + 0] * inv, oacc[dt][nt][4 * j4 + 1] * inv);
          v.y = pack2(oacc[dt][nt][4 * j4 + 2] * inv, oacc[dt][nt][4 * j4 + 3] * inv);
          st8(orow + 32 * dt + 8 * j4, v);
        }
      }
      if (half == 0) c.lse[(int64_t)h * c.n_q + my_r] = (m_ref[nt] + __log2f(lt)) * kLn2;
    }
  }
}

// One workgroup per split unit, its waves over the rows the forward's waves
// own: the two parts' partials combined as the online softmax combines two
// blocks of keys (both rescaled to the larger reference maximum), then O and
// the log-sum-exp written as the forward writes them.  The parts are taken in
// order (part 0's terms first), and the merge runs after the forward kernel
// has finished, so its reads need no synchronisation of their own.
__global__ void __launch_bounds__(256) fwd_merge_kernel(AttnCall c, int n_qblocks) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int s_unit = blockIdx.x;
  const int unit = c.split.n_whole + s_unit;
  const int G = c.hq / c.g.hkv;
  const int g = unit % c.g.hkv, m = unit / c.g.hkv;
  const int qb = n_qblocks - 1 - m / G;
  const int h = g * G + m % G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const float* p0 = c.split.part + ((int64_t)(2 * s_unit) * 4 + w) * kFwdPartWaveFloats;
  const float* p1 = p0 + 4 * kFwdPartWaveFloats;
  const float m0 = p0[4096 + lane], m1 = p1[4096 + lane];
  const float mx = fmaxf(m0, m1);
  const float base = mx == -INFINITY ? 0.f : mx;  // both parts empty: every weight 0
  const float a0 = ex2(m0 - base), a1 = ex2(m1 - base);
  const float l = p0[4096 + 64 + lane] * a0 + p1[4096 + 64 + lane] * a1;
  const float lt = l + __shfl_xor(l, 32);
  const int my_r = r0 + 32 * w + l32;
  if (my_r > rlast) return;
  const float inv = 1.f / lt;
  u16* orow = reinterpret_cast<u16*>(c.o_out) + ((int64_t)my_r * c.hq + h) * D + 4 * half;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const float4 x = *reinterpret_cast<const float4*>(p0 + (dt * 4 + j4) * 256 + 4 * lane);
      const float4 y = *reinterpret_cast<const float4*>(p1 + (dt * 4 + j4) * 256 + 4 * lane);
      u32x2 v;
      v.x = pack2((x.x * a0 + y.x * a1) * inv, (x.y * a0 + y.y * a1) * inv);
      v.y = pack2((x.z * a0 + y.z * a1) * inv, (x.w * a0 + y.w * a1) * inv);
      st8(orow + 32 * dt + 8 * j4, v);
    }
  if (half == 0) c.lse[(int64_t)h * c.n_q + my_r] = (mx + __log2f(lt)) * kLn2;
}

}  // namespace

TailSplit plan_tail_split(int units, int slots) {
  TailSplit sp;
  if (slots <= 0 || units < slots) return sp;  // a single pass (or less)
  const int r = units % slots;
  // no split when the last pass is full or nearly so
  if (r == 0 || 10 * r > 9 * slots) return sp;
  sp.n_whole = units - r;
  sp.n_split = r;
  if (2 * r >= slots) {
    sp.cut_num = r;
    sp.cut_den = slots;
  }
  return sp;
}

hipError_t launch_fwd_bf16(const AttnCall& c, hipStream_t s) {
  const int nqb = (c.n_q + BM - 1) / BM;
  const int units = nqb * c.hq;
  if (c.split.n_split > 0 && (c.split.n_whole + c.split.n_split != units || !c.split.part ||
                              c.split.cut_den <= 0))
    return hipErrorInvalidValue;
  const int grid = c.split.n_split > 0 ? units + c.split.n_split : units;
  KernelTimer t(KT_FWD, s);  // the merge counts as part of the forward
  hipLaunchKernelGGL((fwd_bf16_kernel<1, 64>), dim3(grid), dim3(256), 0, s, c, nqb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.split.n_split == 0) return e;
  hipLaunchKernelGGL(fwd_merge_kernel, dim3(c.split.n_split), dim3(256), 0, s, c, nqb);
  return hipGetLastError();
}

}  // namespace pkv
