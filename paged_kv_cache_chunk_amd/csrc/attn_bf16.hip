// bf16 paged attention for gfx950: forward, dQ and dK/dV, bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// What is computed ("Out of the Memory Barrier", gist.science de, sections
// 2.A, 2.B, 2.D; sciencestack.ai, Figure 3): exact causal softmax attention of
// one query chunk over every earlier key plus its own causal prefix, with K/V
// read page by page through the page table; the backward recomputes the
// probabilities from the forward's log-sum-exp, writes dQ, and adds dK/dV into
// the paged gradient pool with fp32 atomics.  In sparse mode a query page only
// visits the key pages of its selection.
//
// Layout of the work (d = 128, page size a multiple of 128):
//   forward / dQ: one workgroup = 128 query rows of one query head (four
//     waves x 32 rows).  K/V tiles of 64 keys are gathered through the page
//     table into LDS (double-buffered) and shared by the four waves.  Each wave
//     computes S^T = K Q^T so that a lane owns one query column: the softmax
//     statistics are per lane, the probabilities feed the next MFMA as its B
//     operand without any lane shuffle, and O^T / dQ^T accumulate per lane.
//     The second product needs V^T (forward) or K^T (dQ); the tile loader
//     writes that transposed copy into LDS.
//   dK/dV: one workgroup = 128 keys (one page slab) of one KV head; the four
//     waves own 32 keys each and hold K, V as MFMA B operands in registers.
//     They loop over the 32-row query tiles of all G query heads of the group
//     that can see the slab (in sparse mode: the query pages whose selection
//     holds the page), optionally split over several workgroups, and finish
//     with one fp32 atomic add per gradient element into the pool.
//
// MFMA 32x32x16 operand layout used below (lane l, half = l / 32, e = 0..7,
// r = 0..15):  A[m = l % 32][k = 8 * half + e];  B[k = 8 * half + e][n = l % 32];
// C[m = 8 * (r / 4) + 4 * half + r % 4][n = l % 32].
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int BM = 128;       // query rows per forward / dQ workgroup
constexpr int BN = 64;        // keys per K/V tile
constexpr int KSTR = D + 8;   // LDS row stride (elements) of row-major [row][d] tiles
constexpr int TSTR = BN + 4;  // LDS row stride of transposed [d][key] tiles
constexpr int BQ = 32;        // query rows per dK/dV tile
constexpr int QTSTR = BQ + 4; // LDS row stride of transposed [d][query] tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 cat8(u32x2 lo, u32x2 hi) {
  u32x4 v;
  v.x = lo.x;
  v.y = lo.y;
  v.z = hi.x;
  v.w = hi.y;
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ unsigned bf16_bits(float x) {
  return (unsigned)__builtin_bit_cast(u16, (__bf16)x);
}
__device__ __forceinline__ unsigned pack2(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }

// 16-bit element e (0..7) of a 16-byte register group.
__device__ __forceinline__ unsigned elem(u32x4 v, int e) {
  const unsigned w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Write 4 rows x 8 columns (one 16-byte group per row) transposed: row c of
// the destination gets the 4 values of column c, 8 bytes.
__device__ __forceinline__ void st_transposed(u16* dst, int stride, const u32x4 (&r)[4]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x2 v;
    v.x = elem(r[0], e) | (elem(r[1], e) << 16);
    v.y = elem(r[2], e) | (elem(r[3], e) << 16);
    st8(dst + e * stride, v);
  }
}

// The sequence of 64-key tiles a query block visits: dense = keys 0.. in
// order; sparse = the pages of the block's selection list, ascending.
struct Tiles {
  const int32_t* list;  // nullptr: dense
  int per_page;         // page / BN
  int page;
  int max_logical;      // list entries are clamped into [0, max_logical)
  __device__ __forceinline__ int64_t key0(int j) const {
    if (!list) return (int64_t)j * BN;
    int pg = list[j / per_page];
    pg = pg < 0 ? 0 : (pg >= max_logical ? max_logical - 1 : pg);
    return (int64_t)pg * page + (int64_t)(j % per_page) * BN;
  }
};

__device__ __forceinline__ int sel_count(const AttnCall& c, int il, int g) {
  const int n = c.sel.count[(int64_t)il * c.g.hkv + g];
  return n < 0 ? 0 : (n > c.sel.stride ? c.sel.stride : n);
}

__device__ __forceinline__ Tiles make_tiles(const AttnCall& c, int g, int r0, int64_t tmax_blk,
                                            int* n_tiles) {
  Tiles T{nullptr, c.g.page / BN, c.g.page, c.g.max_logical};
  if (!c.sel.pages) {
    *n_tiles = (int)((tmax_blk + BN) / BN);
    return T;
  }
  const int il = r0 / c.g.page;
  T.list = c.sel.pages + ((int64_t)il * c.g.hkv + g) * c.sel.stride;
  int n = sel_count(c, il, g) * T.per_page;
  while (n > 0 && T.key0(n - 1) > tmax_blk) --n;
  *n_tiles = n;
  return T;
}

__device__ __forceinline__ const u16* tile_src(const AttnCall& c, const void* pool, int g,
                                               int64_t s0) {
  const int slot = c.L.table[(int64_t)g * c.g.max_logical + s0 / c.g.page];
  return reinterpret_cast<const u16*>(pool) +
         (((int64_t)g * c.g.slots + slot) * c.g.page + s0 % c.g.page) * D;
}

// ------------------------------------------------------------------ forward
struct __align__(16) FwdSmem {
  u16 k[2][BN * KSTR];
  u16 vt[2][D * TSTR];
};

__global__ void __launch_bounds__(256, 2) fwd_bf16_kernel(AttnCall c, int n_qblocks) {
  __shared__ FwdSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int qb = n_qblocks - 1 - (int)blockIdx.x;  // longest rows first
  const int h = blockIdx.y;
  const int G = c.hq / c.g.hkv, g = h / G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const int64_t tmax_blk = c.q_pos0 + rlast;
  const int rw0 = r0 + 32 * w;
  const int my_r = rw0 + l32;
  const bool row_valid = my_r < c.n_q;
  const int my_rr = row_valid ? my_r : c.n_q - 1;
  const int64_t my_t = c.q_pos0 + my_rr;
  const int64_t tw_min = c.q_pos0 + (rw0 < c.n_q ? rw0 : c.n_q - 1);
  const int64_t tw_max = c.q_pos0 + (rw0 + 31 < c.n_q ? rw0 + 31 : c.n_q - 1);

  bf16x8 qf[8];
  {
    const u16* qrow = reinterpret_cast<const u16*>(c.q) + ((int64_t)my_rr * c.hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }

  int n_tiles;
  const Tiles T = make_tiles(c, g, r0, tmax_blk, &n_tiles);

  const int dc = tid & 15, sg = tid >> 4;
  u32x4 kreg[4], vreg[4];
  auto gload = [&](int j) {
    const int64_t s0 = T.key0(j);
    const u16* kb = tile_src(c, c.L.k, g, s0) + (4 * sg) * D + 8 * dc;
    const u16* vb = tile_src(c, c.L.v, g, s0) + (4 * sg) * D + 8 * dc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kreg[i] = ld16(kb + i * D);
      vreg[i] = ld16(vb + i * D);
    }
  };
  auto swrite = [&](int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(&sm.k[b][(4 * sg + i) * KSTR + 8 * dc], kreg[i]);
    st_transposed(&sm.vt[b][(8 * dc) * TSTR + 4 * sg], TSTR, vreg);
  };

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  float m_i = -INFINITY, l_i = 0.f;
  const float c2 = c.scale * kLog2e;

  if (n_tiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    if (j + 1 < n_tiles) gload(j + 1);
    const int64_t s0 = T.key0(j);
    if (s0 <= tw_max) {
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = f32x16{};
        const u16* krow = &sm.k[b][(32 * mt + l32) * KSTR + 8 * half];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) sacc[mt] = mfma(as_bf16x8(ld16(krow + 16 * ks)), qf[ks], sacc[mt]);
      }
      const bool need_mask = s0 + BN - 1 > tw_min;
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[mt][r] * c2;
          if (need_mask) {
            const int64_t s = s0 + 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
            if (s > my_t) x = -INFINITY;
          }
          sacc[mt][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_i, mx);
      const float alpha = exp2f(m_i - m_new);
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(sacc[mt][r] - m_new);
          sacc[mt][r] = p;
          rs += p;
        }
      }
      rs += __shfl_xor(rs, 32);
      l_i = l_i * alpha + rs;
      m_i = m_new;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 pv;
        const int mt = kk >> 1, rb = 8 * (kk & 1);
        pv.x = pack2(sacc[mt][rb + 0], sacc[mt][rb + 1]);
        pv.y = pack2(sacc[mt][rb + 2], sacc[mt][rb + 3]);
        pv.z = pack2(sacc[mt][rb + 4], sacc[mt][rb + 5]);
        pv.w = pack2(sacc[mt][rb + 6], sacc[mt][rb + 7]);
        const bf16x8 pf = as_bf16x8(pv);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u16* vrow = &sm.vt[b][(32 * dt + l32) * TSTR + 16 * kk + 4 * half];
          oacc[dt] = mfma(cat8(ld8(vrow), ld8(vrow + 8)), pf, oacc[dt]);
        }
      }
    }
    if (j + 1 < n_tiles) swrite((j + 1) & 1);
    __syncthreads();
  }

  if (row_valid) {
    const float inv = 1.f / l_i;
    u16* orow = reinterpret_cast<u16*>(c.o_out) + ((int64_t)my_r * c.hq + h) * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        u32x2 v;
        v.x = pack2(oacc[dt][4 * j4 + 0] * inv, oacc[dt][4 * j4 + 1] * inv);
        v.y = pack2(oacc[dt][4 * j4 + 2] * inv, oacc[dt][4 * j4 + 3] * inv);
        st8(orow + 32 * dt + 8 * j4, v);
      }
    }
    if (half == 0) c.lse[(int64_t)h * c.n_q + my_r] = (m_i + __log2f(l_i)) * kLn2;
  }
}

// ----------------------------------------------------------------------- dQ
struct __align__(16) DqSmem {
  u16 k[2][BN * KSTR];
  u16 v[2][BN * KSTR];
  u16 kt[2][D * TSTR];
};

__global__ void __launch_bounds__(256, 1) dq_bf16_kernel(AttnCall c, int n_qblocks) {
  __shared__ DqSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int qb = n_qblocks - 1 - (int)blockIdx.x;
  const int h = blockIdx.y;
  const int G = c.hq / c.g.hkv, g = h / G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const int64_t tmax_blk = c.q_pos0 + rlast;
  const int rw0 = r0 + 32 * w;
  const int my_r = rw0 + l32;
  const bool row_valid = my_r < c.n_q;
  const int my_rr = row_valid ? my_r : c.n_q - 1;
  const int64_t my_t = c.q_pos0 + my_rr;
  const int64_t tw_min = c.q_pos0 + (rw0 < c.n_q ? rw0 : c.n_q - 1);
  const int64_t tw_max = c.q_pos0 + (rw0 + 31 < c.n_q ? rw0 + 31 : c.n_q - 1);

  bf16x8 qf[8], df[8];
  {
    const int64_t off = ((int64_t)my_rr * c.hq + h) * D + 8 * half;
    const u16* qrow = reinterpret_cast<const u16*>(c.q) + off;
    const u16* drow = reinterpret_cast<const u16*>(c.dout) + off;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
      df[ks] = as_bf16x8(ld16(drow + 16 * ks));
    }
  }
  const float lse2 = c.lse_in[(int64_t)h * c.n_q + my_rr] * kLog2e;
  const float Dl = c.delta[(int64_t)h * c.n_q + my_rr];
  const float c2 = c.scale * kLog2e;

  int n_tiles;
  const Tiles T = make_tiles(c, g, r0, tmax_blk, &n_tiles);

  const int dc = tid & 15, sg = tid >> 4;
  u32x4 kreg[4], vreg[4];
  auto gload = [&](int j) {
    const int64_t s0 = T.key0(j);
    const u16* kb = tile_src(c, c.L.k, g, s0) + (4 * sg) * D + 8 * dc;
    const u16* vb = tile_src(c, c.L.v, g, s0) + (4 * sg) * D + 8 * dc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kreg[i] = ld16(kb + i * D);
      vreg[i] = ld16(vb + i * D);
    }
  };
  auto swrite = [&](int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st16(&sm.k[b][(4 * sg + i) * KSTR + 8 * dc], kreg[i]);
      st16(&sm.v[b][(4 * sg + i) * KSTR + 8 * dc], vreg[i]);
    }
    st_transposed(&sm.kt[b][(8 * dc) * TSTR + 4 * sg], TSTR, kreg);
  };

  f32x16 qacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) qacc[dt] = f32x16{};

  if (n_tiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    if (j + 1 < n_tiles) gload(j + 1);
    const int64_t s0 = T.key0(j);
    if (s0 <= tw_max) {
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = f32x16{};
        pacc[mt] = f32x16{};
        const u16* krow = &sm.k[b][(32 * mt + l32) * KSTR + 8 * half];
        const u16* vrow = &sm.v[b][(32 * mt + l32) * KSTR + 8 * half];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          sacc[mt] = mfma(as_bf16x8(ld16(krow + 16 * ks)), qf[ks], sacc[mt]);
          pacc[mt] = mfma(as_bf16x8(ld16(vrow + 16 * ks)), df[ks], pacc[mt]);
        }
      }
      const bool need_mask = s0 + BN - 1 > tw_min;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2f(sacc[mt][r] * c2 - lse2);
          if (need_mask) {
            const int64_t s = s0 + 32 * mt + 8 * (r >> 2) + 4 * half + (r & 3);
            if (s > my_t) p = 0.f;
          }
          sacc[mt][r] = p * (pacc[mt][r] - Dl);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 pv;
        const int mt = kk >> 1, rb = 8 * (kk & 1);
        pv.x = pack2(sacc[mt][rb + 0], sacc[mt][rb + 1]);
        pv.y = pack2(sacc[mt][rb + 2], sacc[mt][rb + 3]);
        pv.z = pack2(sacc[mt][rb + 4], sacc[mt][rb + 5]);
        pv.w = pack2(sacc[mt][rb + 6], sacc[mt][rb + 7]);
        const bf16x8 dsf = as_bf16x8(pv);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u16* krow = &sm.kt[b][(32 * dt + l32) * TSTR + 16 * kk + 4 * half];
          qacc[dt] = mfma(cat8(ld8(krow), ld8(krow + 8)), dsf, qacc[dt]);
        }
      }
    }
    if (j + 1 < n_tiles) swrite((j + 1) & 1);
    __syncthreads();
  }

  if (row_valid) {
    float* out = c.dq + ((int64_t)my_r * c.hq + h) * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        float4 v;
        v.x = qacc[dt][4 * j4 + 0] * c.scale;
        v.y = qacc[dt][4 * j4 + 1] * c.scale;
        v.z = qacc[dt][4 * j4 + 2] * c.scale;
        v.w = qacc[dt][4 * j4 + 3] * c.scale;
        *reinterpret_cast<float4*>(out + 32 * dt + 8 * j4) = v;
      }
    }
  }
}

// -------------------------------------------------------------------- dK/dV
struct __align__(16) DkvSmem {
  u16 q[2][BQ * KSTR];
  u16 qt[2][D * QTSTR];
  u16 o[2][BQ * KSTR];
  u16 ot[2][D * QTSTR];
  float lse[2][BQ];
  float dl[2][BQ];
  int qpl[1024];
  int n_qpl;
};

// grid (ceil(n_keys / 128), hkv, splits)
__global__ void __launch_bounds__(256, 1) dkdv_bf16_kernel(AttnCall c, int splits) {
  __shared__ DkvSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int g = blockIdx.y;
  const int G = c.hq / c.g.hkv;
  const int P = c.g.page;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int64_t s_base = (int64_t)blockIdx.x * 128;
  const int64_t kpage = s_base / P;
  const int64_t wk0 = s_base + 32 * w;        // this wave's first key
  const int64_t my_s = wk0 + l32;
  const int first_qp = (int)(c.q_pos0 / P);
  const int nqp = (c.n_q + P - 1) / P;
  const int tiles_pp = P / BQ;

  // Row tiles (32 query rows) of the chunk that can see this key slab.
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
    r_first -= r_first % BQ;
    n_rt = (c.n_q - r_first + BQ - 1) / BQ;
  }
  const int total = n_rt * G;
  const int it0 = (int)((int64_t)total * blockIdx.z / splits);
  const int it1 = (int)((int64_t)total * (blockIdx.z + 1) / splits);
  if (it0 >= it1) return;

  bf16x8 kf[8], vf[8];
  const int slot = c.L.table[(int64_t)g * c.g.max_logical + kpage];
  const int64_t prow = ((int64_t)g * c.g.slots + slot) * P + (my_s % P);
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
    if (c.sel.pages) return sm.qpl[rt / tiles_pp] * P + (rt % tiles_pp) * BQ;
    return r_first + rt * BQ;
  };

  // Loader: threads 0-127 load Q, 128-255 load dO; 4 rows x 16 bytes each.
  const int t2 = tid & 127, dc = t2 & 15, sg = t2 >> 4;
  const bool is_q = tid < 128;
  u32x4 reg[4];
  float aux = 0.f;
  auto gload = [&](int it) {
    int hh;
    const int row0 = tile_row0(it, &hh);
    const u16* src = reinterpret_cast<const u16*>(is_q ? c.q : c.dout);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + 4 * sg + i;
      if (row < c.n_q)
        reg[i] = ld16(src + ((int64_t)row * c.hq + hh) * D + 8 * dc);
      else
        reg[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 2 * BQ) {
      const int row = row0 + (tid & (BQ - 1));
      if (tid < BQ)
        aux = row < c.n_q ? c.lse_in[(int64_t)hh * c.n_q + row] * kLog2e : INFINITY;
      else
        aux = row < c.n_q ? c.delta[(int64_t)hh * c.n_q + row] : 0.f;
    }
  };
  auto swrite = [&](int b) {
    u16* rm = is_q ? sm.q[b] : sm.o[b];
    u16* tr = is_q ? sm.qt[b] : sm.ot[b];
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(&rm[(4 * sg + i) * KSTR + 8 * dc], reg[i]);
    st_transposed(&tr[(8 * dc) * QTSTR + 4 * sg], QTSTR, reg);
    if (tid < BQ) sm.lse[b][tid] = aux;
    else if (tid < 2 * BQ) sm.dl[b][tid - BQ] = aux;
  };

  gload(it0);
  swrite(0);
  __syncthreads();
  for (int it = it0; it < it1; ++it) {
    const int b = (it - it0) & 1;
    if (it + 1 < it1) gload(it + 1);
    int hh;
    const int row0 = tile_row0(it, &hh);
    const int64_t t_min = c.q_pos0 + row0;
    const int64_t t_max = t_min + BQ - 1;
    if (wk0 <= t_max) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const u16* qrow = &sm.q[b][l32 * KSTR + 8 * half];
      const u16* orow = &sm.o[b][l32 * KSTR + 8 * half];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sacc = mfma(as_bf16x8(ld16(qrow + 16 * ks)), kf[ks], sacc);
        pacc = mfma(as_bf16x8(ld16(orow + 16 * ks)), vf[ks], pacc);
      }
      const bool need_mask = wk0 + 31 > t_min;
      float p[16], ds[16];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const float4 L4 = *reinterpret_cast<const float4*>(&sm.lse[b][8 * j4 + 4 * half]);
        const float4 D4 = *reinterpret_cast<const float4*>(&sm.dl[b][8 * j4 + 4 * half]);
        const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
        const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * j4 + x;
          float pr = exp2f(sacc[r] * c2 - Lr[x]);
          if (need_mask) {
            const int64_t t = t_min + 8 * j4 + 4 * half + x;
            if (my_s > t) pr = 0.f;
          }
          p[r] = pr;
          ds[r] = pr * (pacc[r] - Dr[x]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pv, dv;
        pv.x = pack2(p[8 * kk + 0], p[8 * kk + 1]);
        pv.y = pack2(p[8 * kk + 2], p[8 * kk + 3]);
        pv.z = pack2(p[8 * kk + 4], p[8 * kk + 5]);
        pv.w = pack2(p[8 * kk + 6], p[8 * kk + 7]);
        dv.x = pack2(ds[8 * kk + 0], ds[8 * kk + 1]);
        dv.y = pack2(ds[8 * kk + 2], ds[8 * kk + 3]);
        dv.z = pack2(ds[8 * kk + 4], ds[8 * kk + 5]);
        dv.w = pack2(ds[8 * kk + 6], ds[8 * kk + 7]);
        const bf16x8 pa = as_bf16x8(pv), da = as_bf16x8(dv);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u16* otr = &sm.ot[b][(32 * dt + l32) * QTSTR + 16 * kk + 4 * half];
          const u16* qtr = &sm.qt[b][(32 * dt + l32) * QTSTR + 16 * kk + 4 * half];
          vacc[dt] = mfma(pa, cat8(ld8(otr), ld8(otr + 8)), vacc[dt]);
          kacc[dt] = mfma(da, cat8(ld8(qtr), ld8(qtr + 8)), kacc[dt]);
        }
      }
    }
    if (it + 1 < it1) swrite((it + 1 - it0) & 1);
    __syncthreads();
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

hipError_t launch_fwd_bf16(const AttnCall& c, hipStream_t s) {
  const int nqb = (c.n_q + BM - 1) / BM;
  KernelTimer t(KT_FWD, s);
  hipLaunchKernelGGL(fwd_bf16_kernel, dim3(nqb, c.hq), dim3(256), 0, s, c, nqb);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const AttnCall& c, hipStream_t s) {
  hipError_t e = launch_delta(c, true, s);
  if (e != hipSuccess) return e;
  const int nqb = (c.n_q + BM - 1) / BM;
  {
    KernelTimer t(KT_DQ, s);
    hipLaunchKernelGGL(dq_bf16_kernel, dim3(nqb, c.hq), dim3(256), 0, s, c, nqb);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int n_slabs = (int)((n_keys + 127) / 128);
  int splits = (2048 + n_slabs * c.g.hkv - 1) / (n_slabs * c.g.hkv);
  if (splits < 1) splits = 1;
  if (splits > 16) splits = 16;
  KernelTimer t(KT_DKDV, s);
  hipLaunchKernelGGL(dkdv_bf16_kernel, dim3(n_slabs, c.g.hkv, splits), dim3(256), 0, s, c,
                     splits);
  return hipGetLastError();
}

}  // namespace pkv
