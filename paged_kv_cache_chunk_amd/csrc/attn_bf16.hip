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

#include <type_traits>

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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

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

// Copy R rows of 256 bytes into a swizzled LDS tile with NW waves: one
// 1 KB global_load_lds per 4 rows; wave w issues instructions w, w + NW, ..
// Lane l of instruction u moves 16-byte chunk c = ((64 u + l) % 16) ^ swz(row)
// of row (64 u + l) / 16, so that it lands at its swizzled place.
template <int R, int NW>
struct TileDma {
  static constexpr int NX = R / 4 / NW;
  static_assert((R / 4) % NW == 0, "rows must split evenly over the waves");
  int row[NX];       // source row of this lane, per instruction
  int chunk_b[NX];   // byte offset of its chunk within the row
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int p = 64 * (w + x * NW) + lane;
      row[x] = p >> 4;
      chunk_b[x] = ((p & 15) ^ swz(p >> 4)) << 4;
    }
  }
  // rows of `row_bytes` stride starting at base (byte offsets fit 32 bits)
  __device__ __forceinline__ void issue(char* tile, int w, const char* base, int row_bytes) const {
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const char* src = base + (row[x] * row_bytes + chunk_b[x]);
      __builtin_amdgcn_global_load_lds((const GLB_AS void*)src,
                                       (LDS_AS void*)(tile + 1024 * (w + x * NW)), 16, 0, 0);
    }
  }
  // same, with source rows clamped to [0, last_row]
  __device__ __forceinline__ void issue_clamped(char* tile, int w, const char* base, int row_bytes,
                                                int last_row) const {
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int r = row[x] < last_row ? row[x] : last_row;
      const char* src = base + (r * row_bytes + chunk_b[x]);
      __builtin_amdgcn_global_load_lds((const GLB_AS void*)src,
                                       (LDS_AS void*)(tile + 1024 * (w + x * NW)), 16, 0, 0);
    }
  }
};

__device__ __forceinline__ int sel_count(const AttnCall& c, int il, int g) {
  const int n = c.sel.count[(int64_t)il * c.g.hkv + g];
  return n < 0 ? 0 : (n > c.sel.stride ? c.sel.stride : n);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// One key tile: logical page, BNT-row sub-tile inside it, and its first key
// relative to the chunk's first query.
struct KeyTile {
  int pg;
  int sub;
  int srel0;
};

// Walks the key tiles (BNT keys each) a query block visits: dense = pages
// 0, 1, .. in order; sparse = the pages of the block's selection list,
// ascending; P / BNT tiles per page.  List entries are clamped into
// [0, max_logical) so that a malformed selection cannot address outside the
// pool.  Everything here is wave-uniform and kept in scalar registers.
template <int BNT>
struct TileWalk {
  const int32_t* list;  // nullptr: dense
  int tpp;              // tiles per page
  int page;
  int max_logical;
  int rel;              // -q_pos0 (keys relative to the chunk)
  int u, sub;           // position of the next tile (u: list index or page)
  __device__ __forceinline__ KeyTile next() {
    int pg = u;
    if (list) {
      pg = list[u];
      pg = pg < 0 ? 0 : (pg >= max_logical ? max_logical - 1 : pg);
      pg = uni(pg);
    }
    KeyTile t{pg, sub, pg * page + sub * BNT + rel};
    if (++sub == tpp) {
      sub = 0;
      ++u;
    }
    return t;
  }
};

// Tiles of a query block whose last row is rlast (relative to q_pos0), and a
// walker positioned on the first tile.
template <int BNT>
__device__ __forceinline__ TileWalk<BNT> make_walk(const AttnCall& c, int g, int r0, int rlast,
                                                   int* n_tiles) {
  TileWalk<BNT> W;
  W.list = nullptr;
  W.page = c.g.page;
  W.tpp = c.g.page / BNT;
  W.max_logical = c.g.max_logical;
  W.rel = (int)(-c.q_pos0);
  W.u = W.sub = 0;
  const int64_t tmax_blk = c.q_pos0 + rlast;
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
  *n_tiles = uni(n);
  return W;
}

// Row 0 of key tile t of KV head g in `pool`.
template <int BNT>
__device__ __forceinline__ const char* key_rows(const AttnCall& c, const void* pool, int g,
                                                const KeyTile& t) {
  const int slot = uni(c.L.table[(int64_t)g * c.g.max_logical + t.pg]);
  return reinterpret_cast<const char*>(pool) +
         (((int64_t)g * c.g.slots + slot) * c.g.page + t.sub * BNT) * ROWB;
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
  const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  // Workgroup -> (query block, head): workgroups are dealt to the 8 XCDs
  // round-robin, so bid % Hkv = KV head keeps every head's workgroups on the
  // same XCDs (sharing their L2 for that head's K/V); longest rows first.
  const int G = c.hq / c.g.hkv;
  const int bid = blockIdx.x;
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
  TileWalk<BNT> walk = make_walk<BNT>(c, g, r0, rlast, &n_tiles);
  TileDma<BNT, NW> dma;
  dma.init(w, lane);
  auto issue = [&](int b, const KeyTile& t) {
    dma.issue(sm[b], w, key_rows<BNT>(c, c.L.k, g, t), ROWB);
    dma.issue(sm[b] + TB, w, key_rows<BNT>(c, c.L.v, g, t), ROWB);
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
    t_cur = walk.next();
    issue(0, t_cur);
  }
  wait_dma_and_sync();

  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    KeyTile t_next{0, 0, 0};
    if (j + 1 < n_tiles) {
      t_next = walk.next();
      issue(b ^ 1, t_next);
    }
    const char* kt = sm[b];
    const char* vt = sm[b] + TB;
    const int srel0 = t_cur.srel0;  // tile's first key, relative to q_pos0
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
    t_cur = t_next;
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
  TileWalk<BNT> walk = make_walk<BNT>(c, g, r0, rlast, &n_tiles);
  TileDma<BNT, NW> dma;
  dma.init(w, lane);
  auto issue = [&](int b, const KeyTile& t) {
    dma.issue(sm[b], w, key_rows<BNT>(c, c.L.k, g, t), ROWB);
    dma.issue(sm[b] + TB, w, key_rows<BNT>(c, c.L.v, g, t), ROWB);
  };

  f32x16 qacc[4][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) qacc[dt][nt] = f32x16{};

  KeyTile t_cur{0, 0, 0};
  if (n_tiles > 0) {
    t_cur = walk.next();
    issue(0, t_cur);
  }
  wait_dma_and_sync();

  for (int j = 0; j < n_tiles; ++j) {
    const int b = j & 1;
    KeyTile t_next{0, 0, 0};
    if (j + 1 < n_tiles) {
      t_next = walk.next();
      issue(b ^ 1, t_next);
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

// -------------------------------------------------------------------- dK/dV
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
      hipLaunchKernelGGL((fwd_bf16_kernel<2, 32>), dim3(nqb * c.hq), dim3(128), 0, s, c, nqb);
      break;
    case 2:
      hipLaunchKernelGGL((fwd_bf16_kernel<2, 64>), dim3(nqb * c.hq), dim3(128), 0, s, c, nqb);
      break;
    default:
      hipLaunchKernelGGL((fwd_bf16_kernel<1, 64>), dim3(nqb * c.hq), dim3(256), 0, s, c, nqb);
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
        hipLaunchKernelGGL((dq_bf16_kernel<2, 32>), dim3(nqb * c.hq), dim3(128), 0, s, c, nqb);
        break;
      case 2:
        hipLaunchKernelGGL((dq_bf16_kernel<2, 64>), dim3(nqb * c.hq), dim3(128), 0, s, c, nqb);
        break;
      default:
        hipLaunchKernelGGL((dq_bf16_kernel<1, 64>), dim3(nqb * c.hq), dim3(256), 0, s, c, nqb);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int64_t n_keys = c.q_pos0 + c.n_q;
  const int n_slabs = (int)((n_keys + 127) / 128);
  int splits = (2048 + n_slabs * c.g.hkv - 1) / (n_slabs * c.g.hkv);
  if (splits < 1) splits = 1;
  if (splits > 16) splits = 16;
  // PKV_DKDV: "1x32" (one wave per SIMD, 32-row query tiles), "1x64", "2x32"
  static const int kind = [] {
    const char* v = getenv("PKV_DKDV");
    if (v && !strcmp(v, "1x32")) return 0;
    if (v && !strcmp(v, "2x32")) return 2;
    return 1;
  }();
  KernelTimer t(KT_DKDV, s);
  const dim3 grid(n_slabs * c.g.hkv * splits);
  if (kind == 0)
    hipLaunchKernelGGL((dkdv_bf16_kernel<1, 32>), grid, dim3(256), 0, s, c, splits);
  else if (kind == 2)
    hipLaunchKernelGGL((dkdv_bf16_kernel<2, 32>), grid, dim3(256), 0, s, c, splits);
  else
    hipLaunchKernelGGL((dkdv_bf16_kernel<1, 64>), grid, dim3(256), 0, s, c, splits);
  return hipGetLastError();
}

}  // namespace pkv
