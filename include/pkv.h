/*
 * pkv.h -- paged-KV chunk attention for one MI355X (gfx950).
 *
 * The operations follow "Out of the Memory Barrier: A Highly Memory Efficient
 * Training System for LLMs with Million-Token Contexts" as summarised on
 * gist.science (de: sections 2.A-2.D; fr: technical summary 2.B-2.D;
 * nl: "Methodologie") and sciencestack.ai (abstract, Figures 3 and 5):
 *   - the sequence is processed in query chunks; each chunk's K/V are appended
 *     to a paged cache made of fixed-size pages, without reallocation
 *     (de 2.B, "Paged Memory Management");
 *   - custom kernels run attention forward and backward directly on the paged
 *     cache; the cache is not an autograd activation, and the gradients of
 *     the cached K/V are accumulated in place with atomic adds into a paged
 *     gradient pool (de 2.B; fr 2.B; sciencestack Figure 3);
 *   - activations are recomputed in the backward (de 2.A), so the backward
 *     takes the forward's log-sum-exp and rebuilds the probabilities;
 *   - for dense-attention models, each query page attends only to the top-K
 *     key pages scored through one representative vector per page
 *     (de 2.D; nl "Methodologie"; sciencestack Figure 5);
 *   - the cache and its gradients can live in pinned host memory and move
 *     asynchronously on a side stream while compute runs (de 2.C; nl
 *     "Methodologie", asynchronous CPU offloading).
 *
 * Conventions shared by every call
 *   Hq query heads, Hkv KV heads (Hq % Hkv == 0, G = Hq / Hkv; query head h
 *   uses KV head h / G), head dim d, page size P tokens.  Positions are
 *   absolute token indices.  Query/output tensors of a chunk are
 *   [n_q][Hq][d] row-major; K/V handed to append are [n_tok][Hkv][d].
 *   The log-sum-exp is [Hq][n_q] fp32, natural log.
 *   A query at absolute position t attends to keys s <= t (every earlier page
 *   plus the causal part of its own chunk); in sparse mode additionally only
 *   to keys whose page is in the selection of t's query page.
 *
 *   Device pointers are raw HIP device addresses (for example
 *   torch.Tensor.data_ptr()).  They stay owned by the caller and must remain
 *   valid until the enqueued work has completed; the library never keeps
 *   them after a call returns.  Every call that takes a stream enqueues its
 *   work on that stream and returns without synchronising the device, unless
 *   stated otherwise.
 *
 * Errors
 *   Argument and state checks run on the host before anything is enqueued;
 *   a failing check returns a non-zero pkv_status and enqueues nothing.
 *   A failing HIP call returns PKV_EHIP.  pkv_last_error() returns a
 *   thread-local description of the last non-OK status.  Faults that happen
 *   inside kernels surface at the caller's next stream synchronisation.
 *   No C++ exception crosses this interface.  A pool is not thread-safe:
 *   drive each pool from one host thread.
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,      /* bad argument (null pointer, size, alignment, range) */
  PKV_ENOMEM = 2,      /* device or pinned host allocation failed / over budget */
  PKV_ECAPACITY = 3,   /* a page table entry or an append exceeds the pool */
  PKV_ESTATE = 4,      /* call out of order (e.g. attention past the appended length) */
  PKV_EHIP = 5,        /* a HIP runtime call failed */
  PKV_EUNSUPPORTED = 6 /* shape or dtype combination without a kernel */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* What pkv_read_pages exports. */
typedef enum { PKV_K = 0, PKV_V = 1, PKV_DK = 2, PKV_DV = 3, PKV_REPS = 4 } pkv_what;

typedef struct pkv_pool pkv_pool; /* opaque; owned by the library */

/*
 * Pool descriptor.  One pool holds, for each of n_layers layers and each KV
 * head, n_slots page slots of P x d elements for K, V, dK and dV, one page
 * table (logical page -> slot) and one representative vector per slot.
 *
 *   kv_dtype     storage type of K/V and of the query/output tensors of the
 *                attention calls (PKV_F32 or PKV_BF16).  Gradients (dK, dV,
 *                dQ) are always fp32 on the device.
 *   page_size    tokens per page.  PKV_F32 needs page_size % 16 == 0;
 *                PKV_BF16 needs page_size % 128 == 0.
 *   head_dim     PKV_F32: 64 or 128.  PKV_BF16: 128.
 *   max_logical_pages  pages per layer per KV head (context / page_size).
 *   n_slots      slots per layer per KV head (>= max_logical_pages).
 *   host_tier    0: all pools in HBM.  1: K, V, dK, dV of every layer live in
 *                pinned host memory (K/V in kv_dtype, gradients in
 *                host_grad_dtype) and HBM holds two windows (layers of
 *                even / odd index) that pkv_prefetch_pages fills;
 *                representatives and page tables stay in HBM.
 *   window_slots host-tier only (else 0): page slots per KV head in each
 *                HBM window; 0 means max_logical_pages (a whole layer).  A
 *                prefetch places the page-heads it brings in the first free
 *                slots of its window, so the window bounds the pages one
 *                visit can hold, not the context: HBM use is then
 *                2 x Hkv x window_slots x P x d x (2 kv bytes + 8) (with
 *                host_grad_accumulate, and room in the budget, plus the
 *                writeback staging below) plus the representatives and
 *                page tables, whatever
 *                max_logical_pages is ("Out of the Memory Barrier",
 *                gist.science de, section 4: memory grows by ~10 MB per 10K
 *                tokens; section 2.D: with page top-K only the selected
 *                pages move).  A prefetch whose pages could exceed it is
 *                rejected (PKV_ECAPACITY; see pkv_prefetch_pages).
 *   host_grad_dtype  host-tier gradient storage (PKV_F32 or PKV_BF16).
 *   host_grad_accumulate  host-tier only (else PKV_EINVAL).  0: a prefetch
 *                with grads brings the pages' accumulated dK/dV into HBM
 *                and pkv_writeback_grads writes the sums back.  1: the
 *                window's gradient pages start at zero on every prefetch
 *                with grads (nothing is read from the host for them),
 *                pkv_writeback_grads stages only that visit's contributions
 *                (in host_grad_dtype) in pinned memory, and threads of the
 *                library add them into the host tier.  The host link then
 *                carries K/V one way and contributions the other, instead
 *                of K/V + gradients one way and gradients the other.  Costs
 *                pinned staging of two layers' dK/dV (host_grad_dtype) and,
 *                with bf16 host gradients, one more bf16 rounding per visit
 *                (contribution and sum are both rounded).  Where the
 *                device budget leaves room, the writeback first gathers the
 *                contributions into a device staging of
 *                2 x Hkv x window_slots x P x d host-gradient elements, in
 *                the order of the window's page list, and one runtime copy
 *                per tensor (hipMemcpyAsync, which the runtime makes on a
 *                DMA engine) moves them over the host link: that slows the
 *                prefetch's host reads far less than the writeback kernel's
 *                writes to mapped host memory.  Without room, the writeback
 *                kernel writes the pinned staging.  The adds finish
 *                asynchronously; every call that reads or zeroes the host
 *                gradients waits for them (pkv_read_rows of dK/dV returns
 *                the window's contributions plus the tier's sums).  Thread count: environment
 *                variable PKV_HOST_ADD_THREADS, else min(16, CPUs the
 *                process may run on).
 *   device_budget_bytes  host-tier only: cap on the library's HBM use; pool
 *                creation fails with PKV_ENOMEM if the window does not fit
 *                (0 = no cap).
 */
typedef struct {
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_logical_pages;
  int32_t n_slots;
  int32_t kv_dtype;        /* pkv_dtype */
  int32_t host_tier;       /* 0 or 1 */
  int32_t host_grad_dtype; /* pkv_dtype, host-tier only */
  int32_t host_grad_accumulate; /* 0 or 1, host-tier only */
  int32_t window_slots;    /* host-tier only: HBM slots per KV head per window */
  int64_t device_budget_bytes;
} pkv_pool_desc;

/*
 * A page selection (device memory), as written by pkv_select_topk_pages:
 *   pages  int32 [n_qpages][Hkv][stride]: ascending absolute key-page ids of
 *          each (query page, KV head), entries past count are ignored;
 *   count  int32 [n_qpages][Hkv].
 * Query page i of a chunk that starts at q_pos0 is absolute page
 * q_pos0 / P + i.  Every list must contain the query page itself (so that
 * every query sees at least its own key), ascend strictly, and hold only
 * pages <= the query page; entries outside [0, max_logical_pages) are
 * clamped into it, so a malformed list cannot make a kernel read outside
 * the pool (its results are then unspecified).
 */
typedef struct {
  const int32_t* pages;
  const int32_t* count;
  int32_t n_qpages;
  int32_t stride;
} pkv_sel;

/* Create a pool (allocates every buffer up front; never reallocates, so the
 * pool's footprint is exactly the page bytes -- de 2.B: no reallocation or
 * fragmentation when pages are appended).  Page tables start as the
 * identity (logical page j -> slot j), gradients start at zero.
 * Synchronous.  *out receives the pool. */
pkv_status pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out);

/* Destroy a pool: synchronises the device, then frees everything.  NULL is
 * accepted and ignored.  (Support call: the pages allocate the paged cache
 * once per training run, de 2.B; this releases it.) */
pkv_status pkv_pool_destroy(pkv_pool* pool);

/* Set the page table of (layer, kv_head) from host memory: host_slots[j] is
 * the slot of logical page j, for j < n (n <= max_logical_pages; the rest of
 * the table is left as is).  Entries must be distinct and in [0, n_slots).
 * Must be called before any append to that layer.  Synchronous.  (The
 * logical-to-physical page mapping of the paged cache, de 2.B "Paged Memory
 * Management"; results do not depend on it, which tests use with permuted
 * tables.) */
pkv_status pkv_page_table_set(pkv_pool* pool, int32_t layer, int32_t kv_head,
                              const int32_t* host_slots, int32_t n);

/* Number of tokens appended so far to `layer` (host value; -1 on bad args).
 * (Support call: the chunk-recurrent driver appends one chunk after another,
 * de 2.A, and takes the next chunk's first position from here.) */
int64_t pkv_length(const pkv_pool* pool, int32_t layer);

/* Append n_tok tokens at positions [pos0, pos0 + n_tok) to `layer`:
 * k, v are device [n_tok][Hkv][d] in kv_dtype.  pos0 must equal the current
 * length (no overwrite), and the pages must fit the table.  Token s goes to
 * slot table[g][s / P], row s % P.  The representative vector of every page
 * the call writes is recomputed as the fp32 mean of that page's keys present
 * so far (nl "Methodologie": one representative vector per page). */
pkv_status pkv_append_kv(pkv_pool* pool, int32_t layer, int64_t pos0, int64_t n_tok,
                         const void* k, const void* v, hipStream_t stream);

/* Forward attention of one query chunk over the paged cache of `layer`
 * (de 2.B custom kernels; sciencestack Figure 3).
 *   q_pos0  absolute position of the chunk's first query; q_pos0 % P == 0 and
 *           q_pos0 + n_q <= pkv_length(layer) (the chunk's own K/V are
 *           appended first).
 *   scale   softmax scale (1/sqrt(d) for standard attention).
 *   q       device [n_q][n_q_heads][d], kv_dtype.
 *   sel     NULL for dense causal attention, else a selection covering the
 *           chunk's query pages (sel->n_qpages == ceil(n_q / P)).
 *   o       device [n_q][n_q_heads][d], kv_dtype (written).
 *   lse     device [n_q_heads][n_q] fp32 (written), natural log.
 * Accumulation is fp32 (bf16 inputs go through bf16 MFMA with fp32
 * accumulate; fp32 inputs use fp32 arithmetic).  With a selection on a bf16
 * pool, where every 128-row block of a head attends about as many keys, the
 * last pass of workgroups (when the blocks do not fill whole passes of two
 * per compute unit) is cut in two along the keys; each part's partial
 * softmax state goes to a library-owned scratch buffer of the pool and a
 * second kernel combines the parts (135 KB per split block; the buffer is
 * grown with hipMalloc, after a device synchronisation, when a larger chunk
 * arrives, so forward calls of one pool on different streams must not
 * overlap, and a call under HIP graph capture needs an earlier call of at
 * least the same size outside it). */
pkv_status pkv_attn_fwd(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                        int32_t n_q_heads, float scale, const void* q, const pkv_sel* sel,
                        void* o, float* lse, hipStream_t stream);

/* Recompute-backward of one query chunk (de 2.A recomputation, 2.B in-place
 * atomic gradient accumulation; sciencestack Figure 3).  Takes the forward's
 * q, o and lse, the upstream gradient dout (device [n_q][n_q_heads][d],
 * kv_dtype) and the same sel as the forward.  Writes dq (device
 * [n_q][n_q_heads][d] fp32, overwritten) and ADDS dK, dV into the layer's
 * gradient pool with fp32 atomics (dK/dV of a multi-chunk run are the sum
 * of every chunk's contribution).  Uses a library-owned scratch buffer for
 * D = rowsum(dO * O), the log-sum-exp in base 2 and, with a selection, the
 * dK/dV work list (the selection inverted per key page); it is grown with
 * hipMalloc (after a device synchronisation) when a larger chunk arrives.
 * The scratch is one per pool: backward calls of one pool on different
 * streams must not overlap.  Chunks of more than 1024 pages are rejected
 * (PKV_EUNSUPPORTED).  bf16
 * pools run the dQ and dK/dV kernels side by side on a second, library-owned
 * stream forked from and joined back into `stream` with events (capturable
 * into a HIP graph); the call's work is complete, as seen from `stream`, when
 * the join is reached. */
pkv_status pkv_attn_bwd(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                        int32_t n_q_heads, float scale, const void* q, const void* o,
                        const void* dout, const float* lse, const pkv_sel* sel, float* dq,
                        hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * backward as pkv_attn_bwd (same arguments, checks, kernels and results), but
 * its scratch (D, the base-2 log-sum-exp and the top-K dK/dV work list) is a
 * fixed 16 MiB device array of the library instead of pool memory grown with
 * hipMalloc; the call allocates nothing.  Each GPU holds its own array (on
 * the current device, which must be the pool's) from the first call until
 * the process ends.  A chunk whose scratch exceeds 16 MiB, 2 x n_q_heads x
 * n_q x 4 bytes rounded up to 256 plus, with a top-K selection on a bf16
 * pool, the work list (about 4 x Hkv x context pages x (1 + ceil(n_q / P /
 * 32)) + 32 x (P / 128) x n_qpages x Hkv x stride bytes; 1.5 MB for chunks
 * of 8192 tokens at a 1M-token context), returns PKV_ECAPACITY; while
 * kernel timing is on it returns PKV_ESTATE.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * pools, other threads) race and must be ordered by the caller.  Nothing in
 * the array needs to start at zero. */
pkv_status pkv_attn_bwd_noalloc(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                                int32_t n_q_heads, float scale, const void* q, const void* o,
                                const void* dout, const float* lse, const pkv_sel* sel,
                                float* dq, hipStream_t stream);

/* Page-level top-K selection for every query page of one chunk (de 2.D; nl
 * "Methodologie"; sciencestack Figure 5).  For query page i (absolute) and
 * KV head g:
 *   qbar = fp32 mean of q over the page's tokens in the chunk and the G query
 *          heads of group g;  kbar_j = the page's representative vector;
 *   score_j = fp32 dot(qbar, kbar_j) for candidates
 *          j in [n_sink, i - n_local] (the pages between the sinks and the
 *          local window);
 *   kept = the top_k candidates by score, ties to the lower page index;
 *   written list = {0 .. n_sink-1} U {i-n_local+1 .. i} U kept, ascending,
 *          clipped to [0, i].
 * q is device [n_q][n_q_heads][d] in kv_dtype.  sel_pages is device
 * [ceil(n_q/P)][Hkv][sel_stride] int32 with sel_stride >=
 * top_k + n_sink + n_local (unused entries set to -1); sel_count is device
 * [ceil(n_q/P)][Hkv] int32.  Uses library-owned scratch for the scores (one
 * per pool: selection calls of one pool on different streams must not
 * overlap).  Contexts beyond 60000 pages are rejected (PKV_EUNSUPPORTED). */
pkv_status pkv_select_topk_pages(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                                 int32_t n_q_heads, const void* q, int32_t top_k,
                                 int32_t n_sink, int32_t n_local, int32_t* sel_pages,
                                 int32_t* sel_count, int32_t sel_stride, hipStream_t stream);

/* Host-tier pools only (PKV_OK and no work otherwise): bring the pages of
 * `layer` that `sel` names (every query page, every KV head; sel == NULL:
 * every appended page) from pinned host memory into the HBM window, on
 * copy_stream, without a host synchronisation (de 2.C: prefetch of the next
 * layer while the current one computes).  with_grads != 0 also brings the
 * pages' dK/dV (host gradient dtype -> fp32); with host_grad_accumulate it
 * instead zeroes them in the window, on the stream of the layer's first
 * attention backward (or writeback) after the prefetch.  The window slot
 * the layer lands in is not overwritten before earlier attention calls that
 * read it and the slot's previous fetch (on any copy stream) have finished,
 * nor its gradients before the window's previous pkv_writeback_grads has
 * read them (the library orders this with events; that writeback must have
 * been called before this prefetch).  `ready`, if
 * not NULL, is recorded on copy_stream when the copies are done; attention
 * calls on this layer wait for it on their own stream automatically.
 * The window then covers the keys appended so far: attention calls on the
 * layer whose queries reach past them (tokens appended after the prefetch)
 * return PKV_ESTATE until the layer is prefetched again, and a backward
 * after a prefetch without gradients (or after the visit's
 * pkv_writeback_grads) returns PKV_ESTATE.  With a window smaller than a
 * layer, the pages a selection can name per KV head, min(n_qpages x stride,
 * pages appended), must fit window_slots, else PKV_ECAPACITY and nothing
 * is enqueued.  A prefetch that fails after those checks (a HIP call
 * failing: PKV_EHIP) leaves the window holding no layer: attention on the
 * window's layers returns PKV_ESTATE until a prefetch succeeds, and the
 * prefetch can simply be called again.  (Test hook: PKV_FAIL_COPY_AT=n in
 * the environment makes the n-th host-link copy of a pool, a prefetch's
 * fetch or a writeback, fail this way before it is enqueued.) */
pkv_status pkv_prefetch_pages(pkv_pool* pool, int32_t layer, const pkv_sel* sel,
                              int32_t with_grads, hipStream_t copy_stream, hipEvent_t ready);

/* Host-tier pools only (PKV_OK and no work otherwise): as pkv_prefetch_pages
 * for a dense chunk whose last query is key n_keys - 1: brings the pages of
 * keys 0 .. n_keys - 1 of `layer` (and with_grads != 0: their dK/dV), the
 * only pages causal attention of that chunk reads or whose gradients it
 * changes (de 2.C: prefetch of the next layer's KV; the chunk attends to
 * every earlier page plus its own, de 2.A).  pkv_writeback_grads then writes
 * back the same pages.  1 <= n_keys <= max_logical_pages x P, else
 * PKV_EINVAL; ceil(n_keys / P) pages must fit window_slots, else
 * PKV_ECAPACITY.  n_keys may reach past the keys appended so far: the window
 * then holds the pages of the keys to come, and a later pkv_append_kv of
 * rows below n_keys writes them into the window as well as the host tier
 * (on its stream, after the fetch), so the next layer of a forward sweep can
 * be prefetched before its chunk is appended (de 2.C: the next layer is
 * fetched while the current one computes). */
pkv_status pkv_prefetch_prefix(pkv_pool* pool, int32_t layer, int64_t n_keys, int32_t with_grads,
                               hipStream_t copy_stream, hipEvent_t ready);

/* Host-tier pools only: write the dK/dV pages of `layer` that the last
 * prefetch with grads brought in back to host memory (fp32 -> host gradient
 * dtype) on copy_stream, after the attention calls on `layer` issued so far
 * have finished (de 2.C and nl "Methodologie": the KV gradients are
 * offloaded to CPU memory asynchronously, like the cache itself).  `done`, if not NULL, is recorded when the copies finish.
 * With host_grad_accumulate the copies go to the window's pinned staging,
 * `done` means they are staged, and the library's host threads then add
 * them into the host tier; the call first waits (on the host) until the adds
 * of the window's previous writeback have finished, since they read the
 * same staging, and a second writeback of one prefetch is PKV_ESTATE (it
 * would add the same contributions twice).  A writeback whose copies fail
 * to enqueue (PKV_EHIP) leaves the window's gradients in place, and calling
 * it again writes them back. */
pkv_status pkv_writeback_grads(pkv_pool* pool, int32_t layer, hipStream_t copy_stream,
                               hipEvent_t done);

/* Host-tier pools: total bytes moved so far by pkv_prefetch_pages (host ->
 * HBM, K/V and gradients) and by pkv_writeback_grads (HBM -> host), counted
 * on the device by the copy kernels (measurement support: de 2.D, sparsity
 * shrinks the offload traffic; these are the bytes that show it).  Synchronises the device and waits
 * for pending host gradient adds.  Both are 0 without a host tier. */
pkv_status pkv_offload_bytes(pkv_pool* pool, int64_t* fetched, int64_t* written);

/* Zero the dK/dV pool of `layer` (all slots; the host tier too in host-tier
 * mode, synchronously, after all work on the device, pending writebacks
 * included, and any pending host adds).  (Support call: the
 * gradient pool accumulates in place over the chunks of a training step, de
 * 2.B; a new step starts it from zero.) */
pkv_status pkv_grad_zero(pkv_pool* pool, int32_t layer, hipStream_t stream);

/* Export (copy, never alias) pool contents of `layer` in logical order, for
 * tests and tooling (support call: it undoes the paging of de 2.B so results
 * can be compared in token order):
 *   PKV_K, PKV_V   -> dst device [n_tok][Hkv][d] kv_dtype;
 *   PKV_DK, PKV_DV -> dst device [n_tok][Hkv][d] fp32;
 *   PKV_REPS       -> dst device [n_pages][Hkv][d] fp32;
 * where n_tok = pkv_length(layer) and n_pages = ceil(n_tok / P).  In
 * host-tier mode K/V/dK/dV are read from the host tier (synchronises the
 * device first, and waits for pending host adds). */
pkv_status pkv_read_pages(pkv_pool* pool, int32_t layer, int32_t what, void* dst,
                          hipStream_t stream);

/* The rows [pos0, pos0 + n_tok) of one pool tensor of `layer` in logical
 * order (copy, never alias): PKV_K, PKV_V -> dst device [n_tok][Hkv][d]
 * kv_dtype; PKV_DK, PKV_DV -> dst device [n_tok][Hkv][d] fp32.  A
 * chunk-recurrent backward reads its own chunk's completed dK/dV this way to
 * carry them back through the K/V projections (sciencestack Figure 3: the
 * pool's gradients leave the attention outside the autograd graph).  The
 * rows must have been appended (else PKV_EINVAL).  Host-tier pools: read
 * from the HBM window holding the layer, on `stream` after the window's
 * fetch, so the rows must lie below the keys its last prefetch covered
 * (else PKV_ESTATE, also when the layer is not in its window, or for dK/dV
 * when the window holds no gradients of the layer) and their pages must be
 * among those it fetched: a chunk's own pages are, for any selection of
 * pkv_select_topk_pages (its query page is always kept) and for a prefix
 * prefetch up to the chunk's end.  dK/dV are the accumulated sums: the
 * window's when the prefetch fetched them; with host_grad_accumulate the
 * window's contributions of this visit plus the host tier's sums of the
 * earlier ones (the call first waits on the host for the adds of the
 * layer's last writeback, then reads the tier rows through its device-mapped
 * alias). */
pkv_status pkv_read_rows(pkv_pool* pool, int32_t layer, int32_t what, int64_t pos0,
                         int64_t n_tok, void* dst, hipStream_t stream);

/* Forget the tokens of `layer` (length back to 0) so that a new sequence can
 * be appended; no memory is freed or cleared (gradients are left as they
 * are: pkv_grad_zero clears them; a host-tier window holding the layer then
 * covers no keys until the next prefetch).  Host-only, immediate.  (Support
 * call: the pages are allocated once and reused, de 2.B; a new training
 * sequence reuses them.) */
pkv_status pkv_pool_reset(pkv_pool* pool, int32_t layer);

/* Kernel timing (measurement support: the per-kernel times behind the
 * rates of the hot path's steps, de 2.B and 2.D).  While enabled, every kernel the library launches is
 * bracketed by two HIP events recorded on the stream it is launched on, and
 * its duration is added to the counter of its kind.  Kinds: */
typedef enum {
  PKV_KT_APPEND = 0,    /* append_kv scatter + page representatives */
  PKV_KT_SELECT = 1,    /* select_topk_pages (query means, scores, top-K) */
  PKV_KT_FWD = 2,       /* attention forward */
  PKV_KT_DELTA = 3,     /* backward: D = rowsum(dO * O) */
  PKV_KT_DQ = 4,        /* backward: dQ */
  PKV_KT_DKDV = 5,      /* backward: dK/dV with atomics into the pool */
  PKV_KT_FETCH = 6,     /* host tier: page fetch into the HBM window */
  PKV_KT_WRITEBACK = 7, /* host tier: gradient writeback */
  PKV_KT_COUNT = 8
} pkv_kernel_kind;

/* enable != 0: clear the counters and start timing; 0: stop timing.  While
 * timing is on, pkv_attn_bwd runs its dQ and dK/dV kernels one after the other
 * (otherwise side by side on a library stream) so that each kernel's events
 * bracket its own work only. */
pkv_status pkv_kernel_timing(int32_t enable);

/* Wait for the recorded events, then write per-kind totals: total_ms[k] and
 * launches[k] for k < n (n <= PKV_KT_COUNT).  Either array may be NULL. */
pkv_status pkv_kernel_times(int32_t n, double* total_ms, int64_t* launches);

/* Bytes the pool holds on the device and in pinned host memory.
 * (Measurement support: the pool's footprint is exactly its page bytes,
 * sciencestack Figure 4, and its HBM side bounds the memory growth per
 * context length that de 4 reports.) */
pkv_status pkv_pool_bytes(const pkv_pool* pool, int64_t* device_bytes, int64_t* host_bytes);

/* ---- Measurement kernels (not used by the attention path).  They move the
 * data of one phase of the bf16 path without its arithmetic, so that the
 * attention kernels' rates can be set beside the rate of their memory
 * traffic alone.  bf16 pools without a host tier (else PKV_EUNSUPPORTED).
 *
 * pkv_measure_gather: streams into LDS exactly the K/V tiles that
 * pkv_attn_fwd(layer, q_pos0, n_q, n_q_heads, sel) reads (same tile walk,
 * page-table lookups and double buffering, and the forward's grid of one
 * workgroup per 128 query rows and head; with a selection, the forward may
 * cut its last pass of workgroups in two, which this kernel does not; "Out of the Memory
 * Barrier", gist.science de, section 2.B: attention reads K/V page by page
 * through the table) and computes nothing.  out: caller-owned device buffer
 * of ceil(n_q / 128) * n_q_heads floats (one word per workgroup, contents
 * unspecified).  Same argument checks as pkv_attn_fwd.
 *
 * pkv_measure_atomics: adds `value` `reps` times to every dK and dV element
 * of keys [0, n_keys) of `layer` with the lane pattern of the dK/dV kernel's
 * fp32 atomic epilogue (de section 2.B: in-place atomic accumulation of the
 * KV gradients).  Modifies the gradient pool (zero it afterwards with
 * pkv_grad_zero); n_keys <= pkv_length(layer), reps >= 0. */
pkv_status pkv_measure_gather(pkv_pool* pool, int32_t layer, int64_t q_pos0, int64_t n_q,
                              int32_t n_q_heads, const pkv_sel* sel, float* out,
                              hipStream_t stream);
pkv_status pkv_measure_atomics(pkv_pool* pool, int32_t layer, int64_t n_keys, int32_t reps,
                               float value, hipStream_t stream);

/* Thread-local message of the last non-OK status returned on this thread
 * (support call: error reporting of the interface, see Errors above). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
