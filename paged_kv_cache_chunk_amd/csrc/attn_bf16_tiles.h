// bf16 paged attention for gfx950, shared tile machinery of the forward, dQ
// and dK/dV kernels (attn_bf16_fwd.hip, attn_bf16_dq.hip, attn_bf16_dkdv.hip):
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
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
#pragma once
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

// acc + (sum of the two bf16 values packed in w), one v_dot2c_f32_bf16 with
// (1, 1): the products are exact, the sum is taken in fp32.
__device__ __forceinline__ float dot2_ones(unsigned w, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
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

// Tile copies issued directly (global_load_lds_dwordx4, saddr form: a
// wave-uniform 64-bit base plus a per-lane 32-bit byte offset; lane l's 16
// bytes land at lds + 16 l).  The compiler does not see them as LDS writes,
// so it does not guard later LDS reads of other buffers with waits for them
// (it cannot tell the buffers apart and would wait for a copy issued for the
// next tile); the kernels order the copies themselves: s_waitcnt + barrier
// before a copied buffer is read (wait_dma_and_sync).  M0 holds the LDS
// address; one wait state separates its write from the copy.  The host pass
// of the compiler sees no instructions.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(unsigned, (const LDS_AS void*)p);
#else
  (void)p;
  return 0;
#endif
}
__device__ __forceinline__ void copy16(const void* base, unsigned off, unsigned lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  // readfirstlane returns int: widen through unsigned, never sign-extend
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
  const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
  const unsigned lu = (unsigned)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lu), "v"(off), "s"(bu)
               : "memory", "m0");
#else
  (void)base;
  (void)off;
  (void)lds;
#endif
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
  // same, issued directly (copy16); base wave-uniform, offsets non-negative
  __device__ __forceinline__ void issue_direct(char* tile, int w, const char* base,
                                               int row_bytes) const {
#pragma unroll
    for (int x = 0; x < NX; ++x)
      copy16(base, (unsigned)(row[x] * row_bytes + chunk_b[x]), lds_addr(tile + 1024 * (w + x * NW)));
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

// Key tiles in the order of TileWalk, with their page-table lookups done
// ahead: when tile j is taken (its copy is about to be issued), the slot of
// tile j+1 has been loaded since the previous take and the list entry of
// tile j+2 since the one before.  Both lookups are global loads whose
// results are first used a whole tile later, so their latency overlaps that
// tile's MFMAs instead of stalling the copy.  Reads past the walk's end stay
// inside the list and the table (positions and pages are clamped); those
// tiles are never taken.
template <int BNT>
struct TileAhead {
  const int32_t* list;   // nullptr: dense
  const int32_t* table;  // page table row of the KV head
  int tpp, page, max_logical, rel, n_list;
  int pu, psub;          // walk position of the next list lookup
  int b_raw, b_sub;      // tile after next: list entry (or page), sub-tile
  int a_pg, a_sub;       // next tile: page, sub-tile
  int a_slot;            // its slot (loaded ahead)
  __device__ __forceinline__ int clamp_pg(int p) const {
    return p < 0 ? 0 : (p >= max_logical ? max_logical - 1 : p);
  }
  __device__ __forceinline__ void lookup_list() {
    if (list) {
      const int i = pu < n_list ? pu : n_list - 1;
      b_raw = list[i < 0 ? 0 : i];
    } else {
      b_raw = pu;
    }
    b_sub = psub;
    if (++psub == tpp) {
      psub = 0;
      ++pu;
    }
  }
  // the tile after next becomes the next one: its page is known now (the
  // list entry was loaded a tile ago) and its slot lookup starts; the list
  // lookup of the following tile starts
  __device__ __forceinline__ void advance() {
    a_pg = uni(clamp_pg(b_raw));
    a_sub = b_sub;
    a_slot = table[a_pg];
    lookup_list();
  }
  // the next tile, with its slot; then advance
  __device__ __forceinline__ KeyTile take(int* slot) {
    KeyTile t{a_pg, a_sub, a_pg * page + a_sub * BNT + rel};
    *slot = uni(a_slot);
    advance();
    return t;
  }
};

// The look-ahead walker of a query block (the tiles of make_walk).  part 0 /
// 1 of a tail-split unit: only the first floor(n cut_num / cut_den) of its n
// tiles / the rest (*n_tiles is then the part's count).
template <int BNT>
__device__ __forceinline__ TileAhead<BNT> make_ahead(const AttnCall& c, int g, int r0, int rlast,
                                                     int* n_tiles, int part = -1) {
  const TileWalk<BNT> W = make_walk<BNT>(c, g, r0, rlast, n_tiles);
  int t0 = 0;
  if (part >= 0) {
    const int n = *n_tiles;
    const int cut = uni((int)((int64_t)n * c.split.cut_num / c.split.cut_den));
    t0 = part ? cut : 0;
    *n_tiles = part ? n - cut : cut;
  }
  TileAhead<BNT> A;
  A.list = W.list;
  A.table = c.L.table + (int64_t)g * c.g.max_logical;
  A.tpp = W.tpp;
  A.page = W.page;
  A.max_logical = W.max_logical;
  A.rel = W.rel;
  A.n_list = W.list ? uni(sel_count(c, r0 / c.g.page, g)) : 0;
  A.pu = uni(t0 / W.tpp);
  A.psub = uni(t0 % W.tpp);
  A.lookup_list();  // tile t0
  A.advance();      // tile t0 next (slot loading), tile t0 + 1's list entry loading
  return A;
}

// Row 0 of key tile t (slot looked up already) of KV head g in `pool`.
template <int BNT>
__device__ __forceinline__ const char* key_rows_at(const AttnCall& c, const void* pool, int g,
                                                   const KeyTile& t, int slot) {
  return reinterpret_cast<const char*>(pool) +
         (((int64_t)g * c.g.slots + slot) * c.g.page + t.sub * BNT) * ROWB;
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

}  // namespace
}  // namespace pkv
