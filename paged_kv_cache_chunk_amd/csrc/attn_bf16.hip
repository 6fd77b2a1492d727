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
// Data movement (d = 128, page size a multiple of 128):
//   * every tile (K/V rows of one page, or Q/dO rows of one head) is copied
//     from HBM straight into LDS with global_load_lds (16 bytes per lane, no
//     staging registers), row-major, 256 bytes per row, the 16-byte chunks of
//     row r XOR-swizzled by swz(r) so that both access patterns below are
//     free of bank conflicts;
//   * MFMA operands whose reduction dimension runs along d are read as rows
//     (ds_read_b128); operands whose reduction runs along the rows (P V,
//     dS K, P^T dO, dS^T Q) are read with the gfx950 transpose load
//     ds_read_b64_tr_b16 from the same row-major tile, so no transposed copy
//     is ever written.
// Work split:
//   forward / dQ: a workgroup owns 128 query rows of one query head; a wave
//     owns 32*NT of them and computes S^T = K Q^T, so a lane owns one query
//     column: softmax statistics are per lane and the probabilities are the
//     next MFMA's B operand without any lane shuffle.
//   dK/dV: a workgroup owns 128 keys (a page slab) of one KV head; a wave
//     owns 32 keys with K, V held as MFMA B operands in registers, loops over
//     the 32-row query tiles of all G query heads of the group that can see
//     the slab (in sparse mode: the query pages whose selection holds the
//     page), optionally split over several workgroups, and ends with one fp32
//     atomic add per gradient element into the pool.
//
// MFMA 32x32x16 operand layout used below (lane l, half = l / 32, e = 0..7,
// r = 0..15):  A[m = l % 32][k = 8 * half + e];  B[k = 8 * half + e][n = l % 32];
// C[m = 8 * (r / 4) + 4 * half + r % 4][n = l % 32].
// ds_read_b64_tr_b16 (per 16-lane group, lane j): element e of lane j is
// element j % 4 of the 8 bytes addressed by lane j / 4 + 4 e of the group.
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

constexpr int D = 128;
constexpr int ROWB = 256;     // bytes of one tile row (d bf16 values)
constexpr int BM = 128;       // query rows per forward / dQ workgroup
constexpr int BQ = 32;        // query rows per dK/dV tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ unsigned bf16_bits(float x) {
  return (unsigned)__builtin_bit_cast(u16, (__bf16)x);
}
__device__ __forceinline__ unsigned pack2(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }

// Raw v_exp_f32 (2^x); arguments are <= 8 or -inf here.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte chunk c of tile row r lives at chunk c ^ swz(r): 16 consecutive
// rows read at one logical chunk hit 16 different chunks, and the 4 rows x 4
// chunks of a transpose read hit 4 different 64-byte bank groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int toff(int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); }

// Row fragment: lane reads 8 values of row `row`, columns 16 ks + 8 half ..
__device__ __forceinline__ bf16x8 frag_row(const char* tile, int row, int ks, int half) {
  return as_bf16x8(ld16(tile + toff(row, 2 * ks + half)));
}

// Transposed fragment of a row-major tile M: lane l receives, as elements
// e = 0..7, M[row0 + 8 (e / 4) + 4 half + e % 4][col0 + l % 32].
__device__ __forceinline__ bf16x8 frag_tr(const char* tile, int row0, int col0, int lane) {
  const int half = lane >> 5, q2 = (lane >> 4) & 1, j = lane & 15;
  const int col = col0 + 16 * q2 + 4 * (lane & 3);
  const int c = col >> 3, sub = (col & 7) << 1;
  const int ra = row0 + 4 * half + (j >> 2);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tile + toff(ra, c) + sub));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(tile + toff(ra + 8, c) + sub));
  const i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Copy R rows of 256 bytes into a swizzled LDS tile with NW waves; row r
// comes from rowptr(r).  One 1 KB global_load_lds per 4 rows.
template <int R, int NW, typename F>
__device__ __forceinline__ void dma_tile(char* tile, int w, int lane, F rowptr) {
  static_assert((R / 4) % NW == 0, "rows must split evenly over the waves");
#pragma unroll
  for (int x = 0; x < R / 4 / NW; ++x) {
    const int u = w + x * NW;
    const int p = 64 * u + lane;
    const int row = p >> 4;
    const int c = (p & 15) ^ swz(row);
    const char* src = rowptr(row) + (c << 4);
    __builtin_amdgcn_global_load_lds((const GLB_AS void*)src, (LDS_AS void*)(tile + 1024 * u), 16,
                                     0, 0);
  }
}

__device__ __forceinline__ int sel_count(const AttnCall& c, int il, int g) {
  const int n = c.sel.count[(int64_t)il * c.g.hkv + g];
  return n < 0 ? 0 : (n > c.sel.stride ? c.sel.stride : n);
}

// Walks the key tiles (BNT keys each) a query block visits: dense = keys
// 0.. in order; sparse = the pages of the block's selection list, ascending,
// P / BNT tiles per page.  List entries are clamped into [0, max_logical) so
// that a malformed selection cannot address outside the pool.
template <int BNT>
struct TileWalk {
  const int32_t* list;  // nullptr: dense
  int tpp;              // tiles per page
  int page;
  int max_logical;
  int u, sub;           // position of the next tile
  int64_t dense_next;
  __device__ __forceinline__ int64_t next() {
    if (!list) {
      const int64_t s0 = dense_next;
      dense_next += BNT;
      return s0;
    }
    int pg = list[u];
    pg = pg < 0 ? 0 : (pg >= max_logical ? max_logical - 1 : pg);
    const int64_t s0 = (int64_t)pg * page + (int64_t)sub * BNT;
    if (++sub == tpp) {
      sub = 0;
      ++u;
    }
    return s0;
  }
};

// Tiles of a query block whose last row is at absolute position tmax_blk,
// and a walker positioned on the first tile.
template <int BNT>
__device__ __forceinline__ TileWalk<BNT> make_walk(const AttnCall& c, int g, int r0,
                                                   int64_t tmax_blk, int* n_tiles) {
  TileWalk<BNT> W;
  W.list = nullptr;
  W.page = c.g.page;
  W.tpp = c.g.page / BNT;
  W.max_logical = c.g.max_logical;
  W.u = W.sub = 0;
  W.dense_next = 0;
  if (!c.sel.pages) {
    *n_tiles = (int)((tmax_blk + BNT) / BNT);
    return W;
  }
  const int il = r0 / c.g.page;
  W.list = c.sel.pages + ((int64_t)il * c.g.hkv + g) * c.sel.stride;
  const int n_list = sel_count(c, il, g);
  // the last listed page is the query page: drop its tiles past the block's last row
  int n = n_list * W.tpp;
  if (n_list > 0) {
    int pg = W.list[n_list - 1];
    pg = pg < 0 ? 0 : (pg >= W.max_logical ? W.max_logical - 1 : pg);
    const int64_t base = (int64_t)pg * c.g.page;
    int keep = W.tpp;
    while (keep > 0 && base + (int64_t)(keep - 1) * BNT > tmax_blk) --keep;
    n = (n_list - 1) * W.tpp + keep;
  }
  *n_tiles = n;
  return W;
}

// Source of row 0 of a key tile starting at absolute key s0 (inside one page).
__device__ __forceinline__ const char* key_rows(const AttnCall& c, const void* pool, int g,
                                                int64_t s0) {
  const int slot = c.L.table[(int64_t)g * c.g.max_logical + s0 / c.g.page];
  return reinterpret_cast<const char*>(pool) +
         (((int64_t)g * c.g.slots + slot) * c.g.page + s0 % c.g.page) * ROWB;
}

__device__ __forceinline__ void wait_dma_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// ------------------------------------------------------------------ forward
// NT: 32-row column tiles per wave (a wave owns 32*NT query rows);
// BNT: keys per tile.  A workgroup owns 128 rows of one query head.
template <int NT, int BNT>
__global__ void __launch_bounds__(256 / NT) __attribute__((amdgpu_waves_per_eu(2, 2))) fwd_bf16_kernel(AttnCall c, int n_qblocks) {
  constexpr int NW = 4 / NT;          // waves per workgroup
  constexpr int MT = BNT / 32;        // 32-key m-tiles per tile
  constexpr int TB = BNT * ROWB;      // bytes per K or V tile
  __shared__ __align__(1024) char sm[2][2 * TB];  // [buffer][K tile | V tile]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int qb = n_qblocks - 1 - (int)blockIdx.x;  // longest rows first
  const int h = blockIdx.y;
  const int G = c.hq / c.g.hkv, g = h / G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const int64_t tmax_blk = c.q_pos0 + rlast;
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
  TileWalk<BNT> walk = make_walk<BNT>(c, g, r0, tmax_blk, &n_tiles);
  auto issue = [&](int b, int64_t s0) {
    const char* kb = key_rows(c, c.L.k, g, s0);
    const char* vb = key_rows(c, c.L.v, g, s0);
    dma_tile<BNT, NW>(sm[b], w, lane, [&](int r) { return kb + r * ROWB; });
    dma_tile<BNT, NW>(sm[b] + TB, w, lane, [&](int r) { return vb + r * ROWB; });
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

  int64_t s_cur = 0;
  if (n_tiles > 0) {
    s_cur = walk.next();
    issue(0, s_cur);
  }
  wait_dma_and_sync();

  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    int64_t s_next = 0;
    if (j + 1 < n_tiles) {
      s_next = walk.next();
      issue(b ^ 1, s_next);
    }
    const char* kt = sm[b];
    const char* vt = sm[b] + TB;
    const int srel0 = (int)(s_cur - c.q_pos0);  // tile's first key, relative to q_pos0
    if (srel0 <= tw_max) {
      f32x16 sacc[MT][NT];
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
      if (srel0 + BNT - 1 > tw_min) {  // tile crosses the causal diagonal of this wave
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
      for (int nt = 0; nt < NT; ++nt) {
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][nt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
        // Lazy rescale: keep the reference maximum unless a row's maximum
        // grew by more than 2^8 (probabilities stay <= 256, exact enough in
        // fp32 and representable in bf16).
        if (__any(mx > m_ref[nt] + 8.f)) {
          const float mr = fmaxf(m_ref[nt], mx);
          const float alpha = ex2(m_ref[nt] - mr);
          l_i[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt][nt] *= alpha;
          m_ref[nt] = mr;
        }
        const float mneg = -m_ref[nt];
        float rs = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = ex2(fmaf(sacc[mt][nt][r], c2, mneg));
            sacc[mt][nt][r] = p;
            rs += p;
          }
        l_i[nt] += rs;
      }
#pragma unroll
      for (int kk = 0; kk < 2 * MT; ++kk) {
        bf16x8 pf[NT];
        const int mt = kk >> 1, rb = 8 * (kk & 1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          u32x4 pv;
          pv.x = pack2(sacc[mt][nt][rb + 0], sacc[mt][nt][rb + 1]);
          pv.y = pack2(sacc[mt][nt][rb + 2], sacc[mt][nt][rb + 3]);
          pv.z = pack2(sacc[mt][nt][rb + 4], sacc[mt][nt][rb + 5]);
          pv.w = pack2(sacc[mt][nt][rb + 6], sacc[mt][nt][rb + 7]);
          pf[nt] = as_bf16x8(pv);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 a = frag_tr(vt, 16 * kk, 32 * dt, lane);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = mfma(a, pf[nt], oacc[dt][nt]);
        }
      }
    }
    s_cur = s_next;
    wait_dma_and_sync();
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

// ----------------------------------------------------------------------- dQ
template <int NT, int BNT>
__global__ void __launch_bounds__(256 / NT) __attribute__((amdgpu_waves_per_eu(2, 2))) dq_bf16_kernel(AttnCall c, int n_qblocks) {
  constexpr int NW = 4 / NT;
  constexpr int MT = BNT / 32;
  constexpr int TB = BNT * ROWB;
  __shared__ __align__(1024) char sm[2][2 * TB];  // [buffer][K tile | V tile]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int qb = n_qblocks - 1 - (int)blockIdx.x;
  const int h = blockIdx.y;
  const int G = c.hq / c.g.hkv, g = h / G;
  const int r0 = qb * BM;
  const int rlast = (r0 + BM < c.n_q ? r0 + BM : c.n_q) - 1;
  const int64_t tmax_blk = c.q_pos0 + rlast;
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
    lse2[nt] = c.lse_in[(int64_t)h * c.n_q + r] * kLog2e;
    Dl[nt] = c.delta[(int64_t)h * c.n_q + r];
  }
  const float c2 = c.scale * kLog2e;

  int n_tiles;
  TileWalk<BNT> walk = make_walk<BNT>(c, g, r0, tmax_blk, &n_tiles);
  auto issue = [&](int b, int64_t s0) {
    const char* kb = key_rows(c, c.L.k, g, s0);
    const char* vb = key_rows(c, c.L.v, g, s0);
    dma_tile<BNT, NW>(sm[b], w, lane, [&](int r) { return kb + r * ROWB; });
    dma_tile<BNT, NW>(sm[b] + TB, w, lane, [&](int r) { return vb + r * ROWB; });
  };

  f32x16 qacc[4][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) qacc[dt][nt] = f32x16{};

  int64_t s_cur = 0;
  if (n_tiles > 0) {
    s_cur = walk.next();
    issue(0, s_cur);
  }
  wait_dma_and_sync();

  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    int64_t s_next = 0;
    if (j + 1 < n_tiles) {
      s_next = walk.next();
      issue(b ^ 1, s_next);
    }
    const char* kt = sm[b];
    const char* vt = sm[b] + TB;
    const int srel0 = (int)(s_cur - c.q_pos0);
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
    s_cur = s_next;
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

// -------------------------------------------------------------------- dK/dV
struct __align__(1024) DkvSmem {
  char q[2][BQ * ROWB];
  char o[2][BQ * ROWB];
  float lsd[2][2 * BQ];  // per buffer: LSE of the 32 rows, then D of the 32 rows
  int qpl[1024];
  int n_qpl;
};

// grid (ceil(n_keys / 128), hkv, splits); OCC: waves per SIMD the register
// budget is sized for.
template <int OCC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
dkdv_bf16_kernel(AttnCall c, int splits) {
  __shared__ DkvSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int g = blockIdx.y;
  const int G = c.hq / c.g.hkv;
  const int P = c.g.page;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int64_t s_base = (int64_t)blockIdx.x * 128;
  const int64_t kpage = s_base / P;
  const int64_t wk0 = s_base + 32 * w;            // this wave's first key
  const int s_rel = (int)(wk0 + l32 - c.q_pos0);  // this lane's key, relative to q_pos0
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
    if (c.sel.pages) return sm.qpl[rt / tiles_pp] * P + (rt % tiles_pp) * BQ;
    return r_first + rt * BQ;
  };
  // Q and dO rows of the tile straight into LDS (rows past the chunk repeat its
  // last row and are masked); the 32 LSE and 32 D values by wave 0.
  auto issue = [&](int b, int it) {
    int hh;
    const int row0 = tile_row0(it, &hh);
    const char* qb = reinterpret_cast<const char*>(c.q);
    const char* ob = reinterpret_cast<const char*>(c.dout);
    dma_tile<BQ, 4>(sm.q[b], w, lane, [&](int r) {
      const int rr = row0 + r < c.n_q ? row0 + r : c.n_q - 1;
      return qb + ((int64_t)rr * c.hq + hh) * ROWB;
    });
    dma_tile<BQ, 4>(sm.o[b], w, lane, [&](int r) {
      const int rr = row0 + r < c.n_q ? row0 + r : c.n_q - 1;
      return ob + ((int64_t)rr * c.hq + hh) * ROWB;
    });
    if (w == 0) {
      const int rr = row0 + l32;
      const int rc = rr < c.n_q ? rr : c.n_q - 1;
      const float* src = half == 0 ? c.lse_in + (int64_t)hh * c.n_q + rc
                                   : c.delta + (int64_t)hh * c.n_q + rc;
      __builtin_amdgcn_global_load_lds((const GLB_AS void*)src, (LDS_AS void*)sm.lsd[b], 4, 0, 0);
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
    const int64_t t_max = t_min + BQ - 1;
    if (wk0 <= t_max) {
      const char* qt = sm.q[b];
      const char* ot = sm.o[b];
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sacc = mfma(frag_row(qt, l32, ks, half), kf[ks], sacc);
        pacc = mfma(frag_row(ot, l32, ks, half), vf[ks], pacc);
      }
      // keys past a row (causal) and rows past the chunk get probability 0
      const bool need_mask = (wk0 + 31 > t_min) || (row0 + BQ > c.n_q);
      const float* lse_b = sm.lsd[b];
      const float* dl_b = sm.lsd[b] + BQ;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // rows 16 kk .. 16 kk + 15 of the tile: accumulator entries 8 kk .. 8 kk + 7
        float p[8], ds[8];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j4 = 2 * kk + jj;
          const float4 L4 = *reinterpret_cast<const float4*>(lse_b + 8 * j4 + 4 * half);
          const float4 D4 = *reinterpret_cast<const float4*>(dl_b + 8 * j4 + 4 * half);
          const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
          const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int tr = row0 + 8 * j4 + 4 * half + x;
            float sv = sacc[4 * j4 + x];
            if (need_mask && (s_rel > tr || tr >= c.n_q)) sv = -INFINITY;
            const float pr = ex2(fmaf(sv, c2, -Lr[x] * kLog2e));
            p[4 * jj + x] = pr;
            ds[4 * jj + x] = pr * (pacc[4 * j4 + x] - Dr[x]);
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

// Tile shape of the forward and dQ kernels: NT x 32 query rows per wave,
// BNT keys per LDS tile.  PKV_FWD_TILE / PKV_DQ_TILE ("1x64", "2x32", "2x64")
// override the defaults for tuning.
static int tile_choice(const char* env, int dflt) {
  const char* v = getenv(env);
  if (!v) return dflt;
  if (!strcmp(v, "1x64")) return 0;
  if (!strcmp(v, "2x32")) return 1;
  if (!strcmp(v, "2x64")) return 2;
  return dflt;
}

hipError_t launch_fwd_bf16(const AttnCall& c, hipStream_t s) {
  const int nqb = (c.n_q + BM - 1) / BM;
  static const int choice = tile_choice("PKV_FWD_TILE", 0);
  KernelTimer t(KT_FWD, s);
  switch (choice) {
    case 1:
      hipLaunchKernelGGL((fwd_bf16_kernel<2, 32>), dim3(nqb, c.hq), dim3(128), 0, s, c, nqb);
      break;
    case 2:
      hipLaunchKernelGGL((fwd_bf16_kernel<2, 64>), dim3(nqb, c.hq), dim3(128), 0, s, c, nqb);
      break;
    default:
      hipLaunchKernelGGL((fwd_bf16_kernel<1, 64>), dim3(nqb, c.hq), dim3(256), 0, s, c, nqb);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const AttnCall& c, hipStream_t s) {
  hipError_t e = launch_delta(c, true, s);
  if (e != hipSuccess) return e;
  const int nqb = (c.n_q + BM - 1) / BM;
  static const int choice = tile_choice("PKV_DQ_TILE", 0);
  {
    KernelTimer t(KT_DQ, s);
    switch (choice) {
      case 1:
        hipLaunchKernelGGL((dq_bf16_kernel<2, 32>), dim3(nqb, c.hq), dim3(128), 0, s, c, nqb);
        break;
      case 2:
        hipLaunchKernelGGL((dq_bf16_kernel<2, 64>), dim3(nqb, c.hq), dim3(128), 0, s, c, nqb);
        break;
      default:
        hipLaunchKernelGGL((dq_bf16_kernel<1, 64>), dim3(nqb, c.hq), dim3(256), 0, s, c, nqb);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int n_slabs = (int)((n_keys + 127) / 128);
  int splits = (2048 + n_slabs * c.g.hkv - 1) / (n_slabs * c.g.hkv);
  if (splits < 1) splits = 1;
  if (splits > 16) splits = 16;
  static const int occ = getenv("PKV_DKDV_OCC") && !strcmp(getenv("PKV_DKDV_OCC"), "2") ? 2 : 1;
  KernelTimer t(KT_DKDV, s);
  if (occ == 2)
    hipLaunchKernelGGL(dkdv_bf16_kernel<2>, dim3(n_slabs, c.g.hkv, splits), dim3(256), 0, s, c,
                       splits);
  else
    hipLaunchKernelGGL(dkdv_bf16_kernel<1>, dim3(n_slabs, c.g.hkv, splits), dim3(256), 0, s, c,
                       splits);
  return hipGetLastError();
}

}  // namespace pkv
