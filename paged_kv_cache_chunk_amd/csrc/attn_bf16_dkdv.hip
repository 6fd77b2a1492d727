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
};

// Work list of the sparse dK/dV kernel (layout in DkvPlan), one workgroup of
// 1024 threads.  The selection is inverted: for every (KV head g, key page p)
// a bit mask of the query pages of the chunk whose selection holds p (bit il
// % 32 of word il / 32; a page listed twice counts once) and its population
// count.  A key page that many query pages selected (the sink pages, pages
// every query scores high) would otherwise leave one workgroup with all their
// rows while the rest of the grid idles; here its work is cut into items of
// at most qpi query pages.  Items are ordered by size, largest first, so the
// workgroups dealt out last are the short ones.  An item is two int4: (g,
// 128-key slab, first iteration, end iteration) and (page-table slot of the
// slab's page, number of query pages, mask words 0 and 1), so that a
// workgroup has everything it needs after one set of loads when the chunk
// has at most 64 query pages.  Every phase runs over all entries at once: no
// step is sequential over the query pages.
__global__ void __launch_bounds__(1024) dkdv_plan_kernel(SelDev sel, int hkv, int G, int page,
                                                         int tiles_pp, const int32_t* table,
                                                         int max_logical, DkvPlan pl) {
  __shared__ int s_scan[1024];
  __shared__ int s_next[1025];  // per item size (query pages): item count, then next free index
  const int tid = threadIdx.x;
  int* cnt = pl.base + pl.off_cnt;
  unsigned* mask = reinterpret_cast<unsigned*>(pl.base + pl.off_mask);
  int4* items = reinterpret_cast<int4*>(pl.base + pl.off_items);
  const int W = pl.mask_words;
  const int qpi = pl.qpi;
  const int64_t E = (int64_t)hkv * pl.n_pages;
  const int subs = page / 128;
  for (int64_t x = tid; x < E * W; x += 1024) mask[x] = 0u;
  for (int q = tid; q <= qpi; q += 1024) s_next[q] = 0;
  __threadfence();
  __syncthreads();
  // mark: every (query page, KV head, list entry) in parallel, atomics at L2
  const int per_qp = hkv * sel.stride;
  const int64_t n_ent = (int64_t)sel.n_qpages * per_qp;
  for (int64_t x = tid; x < n_ent; x += 1024) {
    const int il = (int)(x / per_qp);
    const int r = (int)(x % per_qp);
    const int g = r / sel.stride, j = r % sel.stride;
    int n = sel.count[(int64_t)il * hkv + g];
    n = n < 0 ? 0 : (n > sel.stride ? sel.stride : n);
    if (j < n && il < 32 * W) {
      const int p = sel.pages[((int64_t)il * hkv + g) * sel.stride + j];
      if (p >= 0 && p < pl.n_pages)
        atomicOr(&mask[((int64_t)g * pl.n_pages + p) * W + (il >> 5)], 1u << (il & 31));
    }
  }
  __threadfence();
  __syncthreads();
  // counts and item counts per size; thread t owns a contiguous run of
  // entries.  The masks were written by atomics (at L2): read past the L1.
  const int64_t run = (E + 1023) / 1024;
  const int64_t e0 = tid * run < E ? tid * run : E;
  const int64_t e1 = e0 + run < E ? e0 + run : E;
  for (int64_t e = e0; e < e1; ++e) {
    int cv = 0;
    for (int w = 0; w < W; ++w)
      cv += __popc(__hip_atomic_load(&mask[e * W + w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    cnt[e] = cv;
    if (cv > 0) {
      if (cv >= qpi) atomicAdd(&s_next[qpi], (cv / qpi) * subs);
      if (cv % qpi) atomicAdd(&s_next[cv % qpi], subs);
    }
  }
  __syncthreads();
  // first index of each size, largest size first: inclusive scan over
  // t = qpi - size (Hillis-Steele)
  const int hv = tid < qpi ? s_next[qpi - tid] : 0;
  s_scan[tid] = hv;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  if (tid < qpi) s_next[qpi - tid] = s_scan[tid] - hv;
  if (tid == 0) pl.base[0] = s_scan[1023] < pl.max_items ? s_scan[1023] : pl.max_items;
  __syncthreads();
  for (int64_t e = e0; e < e1; ++e) {
    const int cv = cnt[e];  // written by this thread above
    if (cv == 0) continue;
    const int g = (int)(e / pl.n_pages), p = (int)(e % pl.n_pages);
    const int slot = table[(int64_t)g * max_logical + p];
    const int m0 = (int)__hip_atomic_load(&mask[e * W], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int m1 = W > 1 ? (int)__hip_atomic_load(&mask[e * W + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    const int per_page = tiles_pp * G;  // iterations per query page
    const int it_total = cv * per_page;
    const int it_step = qpi * per_page;
    for (int i0 = 0; i0 < it_total; i0 += it_step) {
      const int i1 = i0 + it_step < it_total ? i0 + it_step : it_total;
      const int size = (i1 - i0) / per_page;
      for (int sub = 0; sub < subs; ++sub) {
        const int b = atomicAdd(&s_next[size], 1);
        if (b < pl.max_items) {
          items[2 * (int64_t)b] = make_int4(g, p * subs + sub, i0, i1);
          items[2 * (int64_t)b + 1] = make_int4(slot, cv, m0, m1);
        }
      }
    }
  }
}

// Dense: grid ceil(n_keys / 128) * hkv * splits, workgroup -> (KV head, slab,
// split) with bid % Hkv = KV head (a head's workgroups share XCDs) and the
// earliest slabs (the most query rows) first.  Sparse: grid = the work list's
// capacity, workgroup b takes item b (or exits).  BQT: query rows per tile (32
// or 64); OCC: waves per SIMD the register budget is sized for.
template <int OCC, int BQT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
dkdv_bf16_kernel(AttnCall c, int splits) {
  constexpr int ST = BQT / 32;  // 32-row sub-tiles per tile
  __shared__ DkvSmem<BQT> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int bid = blockIdx.x;
  const int G = c.hq / c.g.hkv;
  const int P = c.g.page;
  const int tiles_pp = P / BQT;
  const int64_t n_keys = c.q_pos0 + c.n_q;

  // This workgroup's KV head, 128-key slab and range [it0, it1) of its
  // iterations; iteration it = head (it / n_rt) x row tile (it % n_rt) over the
  // n_rt row tiles (BQT query rows) of the chunk that can see the slab.
  int g, slab, it0, it1, n_rt, r_first = 0, slot = 0;
  if (c.sel.pages) {
    // the item's two int4 (bid is below the grid, the list's capacity) and the
    // item count, loaded together
    const int* pb = c.plan.base;
    const int4* rec = reinterpret_cast<const int4*>(pb + c.plan.off_items) + 2 * (int64_t)bid;
    const int4 r0 = rec[0], r1 = rec[1];
    if (bid >= pb[0]) return;
    g = uni(r0.x);
    slab = uni(r0.y);
    it0 = uni(r0.z);
    it1 = uni(r0.w);
    slot = uni(r1.x);
    if (g < 0 || g >= c.g.hkv || slab < 0 || (int64_t)slab * 128 >= (int64_t)c.plan.n_pages * P ||
        it0 < 0 || slot < 0 || slot >= c.g.slots)
      return;  // not a valid item (cannot happen for a plan written by dkdv_plan_kernel)
    const int W = c.plan.mask_words;  // <= 32 (chunks of at most 1024 pages)
    int n = uni(r1.y);
    n = n < 32 * W ? n : 32 * W;
    // the query pages of the mask, ascending: lane t < W expands word t after
    // the population counts of the words before it (words 0 and 1 come with
    // the item)
    if (w == 0) {
      unsigned bits = lane == 0 ? (unsigned)r1.z : (lane == 1 && W > 1 ? (unsigned)r1.w : 0u);
      if (W > 2) {
        const int e = g * c.plan.n_pages + (int)((int64_t)slab * 128 / P);
        const unsigned* mw = reinterpret_cast<const unsigned*>(pb + c.plan.off_mask) + (int64_t)e * W;
        if (lane >= 2 && lane < W) bits = mw[lane];
      }
      int pos = __popc(bits);
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(pos, d);
        if (lane >= d) pos += v;
      }
      pos -= __popc(bits);
      while (bits) {
        sm.qpl[pos++] = 32 * lane + __ffs(bits) - 1;
        bits &= bits - 1;
      }
    }
    __syncthreads();
    n_rt = n * tiles_pp;
    if (it1 > n_rt * G) it1 = n_rt * G;
  } else {
    g = bid % c.g.hkv;
    const int m = bid / c.g.hkv;
    slab = m / splits;
    const int zsplit = m % splits;
    r_first = (int)((int64_t)slab * 128 - c.q_pos0);
    if (r_first < 0) r_first = 0;
    r_first -= r_first % BQT;
    n_rt = (c.n_q - r_first + BQT - 1) / BQT;
    const int total = n_rt * G;
    it0 = (int)((int64_t)total * zsplit / splits);
    it1 = (int)((int64_t)total * (zsplit + 1) / splits);
  }
  if (it0 >= it1) return;
  const int64_t s_base = (int64_t)slab * 128;
  const int64_t kpage = s_base / P;
  const int64_t wk0 = s_base + 32 * w;            // this wave's first key
  const int s_rel = (int)(wk0 + l32 - c.q_pos0);  // this lane's key, relative to q_pos0

  bf16x8 kf[8], vf[8];
  if (!c.sel.pages) slot = uni(c.L.table[(int64_t)g * c.g.max_logical + kpage]);
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
  // K and V stay in accumulation registers (AGPRs; MFMA reads its A/B
  // operands from there), so that the S/dP and dV/dK accumulators, built
  // with -amdgpu-mfma-vgpr-form, take the VGPRs and the softmax reads S and
  // dP without 64 v_accvgpr_read per tile.  Placed after the first wait, so
  // the K/V loads overlap the first tile's copy.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));
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

  // One fp32 atomic add per gradient element into the pool (measured faster
  // than a plain read-add-write even where the workgroup owns the element).
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

// Query pages per work item of the sparse dK/dV kernel (PKV_DKDV_QPI overrides).
static int dkdv_qpi() {
  static const int q = [] {
    const char* v = getenv("PKV_DKDV_QPI");
    const int x = v ? atoi(v) : 0;
    return x >= 1 && x <= 1024 ? x : 8;
  }();
  return q;
}

DkvPlan dkdv_plan_layout(const Geom& g, int hq, int64_t q_pos0, int n_q, int sel_stride) {
  (void)hq;
  DkvPlan pl{};
  const int64_t n_keys = q_pos0 + n_q;
  pl.n_pages = (int)((n_keys + g.page - 1) / g.page);
  pl.qpi = dkdv_qpi();
  const int64_t nqp = (n_q + g.page - 1) / g.page;
  pl.mask_words = (int)((nqp + 31) / 32);
  const int64_t E = (int64_t)g.hkv * pl.n_pages;
  const int64_t H = nqp * g.hkv * (sel_stride > 0 ? sel_stride : 0);  // list entries
  pl.off_cnt = 64;
  pl.off_mask = pl.off_cnt + E;
  pl.off_items = ((pl.off_mask + E * pl.mask_words + 3) / 4) * 4;
  const int64_t bound = (H + pl.qpi - 1) / pl.qpi + (H < E ? H : E);
  pl.max_items = (int)((H < bound ? H : bound) * (g.page / 128));
  pl.bytes = (pl.off_items + 8 * (int64_t)pl.max_items) * 4;
  return pl;
}

// PKV_BWD_STREAMS=1 runs dQ and dK/dV one after the other on the caller's
// stream.
static bool bwd_one_stream() {
  static const bool r = [] {
    const char* v = getenv("PKV_BWD_STREAMS");
    return v && !strcmp(v, "1");
  }();
  return r;
}

static hipError_t launch_dkdv(const AttnCall& c, hipStream_t s);

hipError_t launch_bwd_bf16(const AttnCall& c, hipStream_t s, hipStream_t aux, hipEvent_t ev_fork,
                           hipEvent_t ev_join) {
  hipError_t e = launch_delta(c, true, s);
  if (e != hipSuccess) return e;
  // with kernel timing on, one after the other, so that each kernel's events
  // bracket its own work only
  if (!aux || bwd_one_stream() || kernel_timing_on()) {
    if ((e = launch_dq_bf16(c, s)) != hipSuccess) return e;
    return launch_dkdv(c, s);
  }
  // fork: dK/dV (the longer kernel) first on aux, dQ on s, then join
  if ((e = hipEventRecord(ev_fork, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(aux, ev_fork, 0)) != hipSuccess) return e;
  if ((e = launch_dkdv(c, aux)) != hipSuccess) return e;
  if ((e = launch_dq_bf16(c, s)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev_join, aux)) != hipSuccess) return e;
  return hipStreamWaitEvent(s, ev_join, 0);
}

static hipError_t launch_dkdv(const AttnCall& c, hipStream_t s) {
  hipError_t e = hipSuccess;
  constexpr int kBQT = 64;  // query rows per dK/dV tile
  const int G = c.hq / c.g.hkv;
  int splits = 1;
  dim3 grid;
  KernelTimer t(KT_DKDV, s);  // the planning kernel counts as part of dK/dV
  if (c.sel.pages) {
    if (c.plan.max_items == 0) return hipSuccess;  // nothing selected
    hipLaunchKernelGGL(dkdv_plan_kernel, dim3(1), dim3(1024), 0, s, c.sel, c.g.hkv, G, c.g.page,
                       c.g.page / kBQT, c.L.table, c.g.max_logical, c.plan);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    grid = dim3(c.plan.max_items);
  } else {
    const int64_t n_keys = c.q_pos0 + c.n_q;
    const int n_slabs = (int)((n_keys + 127) / 128);
    splits = (2048 + n_slabs * c.g.hkv - 1) / (n_slabs * c.g.hkv);
    if (splits < 1) splits = 1;
    if (splits > 16) splits = 16;
    grid = dim3(n_slabs * c.g.hkv * splits);
  }
  hipLaunchKernelGGL((dkdv_bf16_kernel<1, kBQT>), grid, dim3(256), 0, s, c, splits);
  return hipGetLastError();
}

}  // namespace pkv
