/* Drives the C ABI's host-side logic under AddressSanitizer (built with
 * tests/test_abi_asan.py): every entry point with a null pool or malformed
 * arguments must return its documented status and leave a message; pool
 * creation must either succeed (a GPU is present) and be destroyed, or fail
 * with a status (no GPU: the allocations fail) after releasing whatever it
 * had allocated.  ASan reports any invalid access or leak on these paths.
 * Prints "ok <checks>" and exits 0 when every status is as expected. */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static int g_checks, g_bad;

static void expect(const char* what, pkv_status got, pkv_status want) {
  ++g_checks;
  if (got != want) {
    ++g_bad;
    printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, pkv_last_error());
  } else if (want != PKV_OK && pkv_last_error()[0] == '\0') {
    ++g_bad;
    printf("FAIL %s: no error message\n", what);
  }
}

static pkv_pool_desc desc_bf16(void) {
  pkv_pool_desc d;
  memset(&d, 0, sizeof d);
  d.n_layers = 2;
  d.n_kv_heads = 4;
  d.head_dim = 128;
  d.page_size = 128;
  d.max_logical_pages = 16;
  d.n_slots = 16;
  d.kv_dtype = PKV_BF16;
  return d;
}

int main(void) {
  pkv_pool* pool = NULL;
  pkv_pool_desc d = desc_bf16();
  int dummy = 0;
  float f = 0.f;
  pkv_sel sel = {(const int32_t*)&dummy, (const int32_t*)&dummy, 1, 1};

  expect("create(null)", pkv_pool_create(NULL, &pool), PKV_EINVAL);
  expect("create(null out)", pkv_pool_create(&d, NULL), PKV_EINVAL);
  d.n_slots = 8;
  expect("create(slots < pages)", pkv_pool_create(&d, &pool), PKV_EINVAL);
  d = desc_bf16();
  d.head_dim = 96;
  expect("create(bf16 d 96)", pkv_pool_create(&d, &pool), PKV_EUNSUPPORTED);
  d = desc_bf16();
  d.kv_dtype = 7;
  expect("create(bad dtype)", pkv_pool_create(&d, &pool), PKV_EINVAL);
  d = desc_bf16();
  d.host_grad_accumulate = 1;
  expect("create(accumulate without tier)", pkv_pool_create(&d, &pool), PKV_EINVAL);
  d = desc_bf16();
  d.window_slots = 4;
  expect("create(window without tier)", pkv_pool_create(&d, &pool), PKV_EINVAL);

  expect("destroy(null)", pkv_pool_destroy(NULL), PKV_OK);
  expect("table_set(null)", pkv_page_table_set(NULL, 0, 0, &dummy, 1), PKV_EINVAL);
  expect("append(null)", pkv_append_kv(NULL, 0, 0, 1, &dummy, &dummy, NULL), PKV_EINVAL);
  expect("fwd(null)", pkv_attn_fwd(NULL, 0, 0, 1, 28, 1.f, &dummy, NULL, &dummy, &f, NULL), PKV_EINVAL);
  expect("bwd(null)", pkv_attn_bwd(NULL, 0, 0, 1, 28, 1.f, &dummy, &dummy, &dummy, &f, &sel, &f, NULL),
         PKV_EINVAL);
  expect("select(null)", pkv_select_topk_pages(NULL, 0, 0, 1, 28, &dummy, 4, 1, 2, &dummy, &dummy, 7, NULL),
         PKV_EINVAL);
  expect("prefetch(null)", pkv_prefetch_pages(NULL, 0, NULL, 0, NULL, NULL), PKV_EINVAL);
  expect("prefetch_prefix(null)", pkv_prefetch_prefix(NULL, 0, 1, 0, NULL, NULL), PKV_EINVAL);
  expect("writeback(null)", pkv_writeback_grads(NULL, 0, NULL, NULL), PKV_EINVAL);
  expect("grad_zero(null)", pkv_grad_zero(NULL, 0, NULL), PKV_EINVAL);
  expect("read_pages(null)", pkv_read_pages(NULL, 0, PKV_K, &dummy, NULL), PKV_EINVAL);
  expect("read_rows(null)", pkv_read_rows(NULL, 0, PKV_K, 0, 1, &dummy, NULL), PKV_EINVAL);
  expect("reset(null)", pkv_pool_reset(NULL, 0), PKV_EINVAL);
  expect("bytes(null)", pkv_pool_bytes(NULL, NULL, NULL), PKV_EINVAL);
  expect("offload_bytes(null)", pkv_offload_bytes(NULL, NULL, NULL), PKV_EINVAL);
  expect("gather(null)", pkv_measure_gather(NULL, 0, 0, 1, 28, NULL, &f, NULL), PKV_EINVAL);
  expect("atomics(null)", pkv_measure_atomics(NULL, 0, 1, 1, 0.f, NULL), PKV_EINVAL);
  ++g_checks;
  if (pkv_length(NULL, 0) != -1) {
    ++g_bad;
    printf("FAIL length(null)\n");
  }
  expect("timing on", pkv_kernel_timing(1), PKV_OK);
  expect("timing off", pkv_kernel_timing(0), PKV_OK);
  expect("times", pkv_kernel_times(PKV_KT_COUNT, NULL, NULL), PKV_OK);

  /* a real pool: created and destroyed with a GPU, a clean failure without */
  for (int tier = 0; tier < 2; ++tier) {
    d = desc_bf16();
    d.host_tier = tier;
    d.host_grad_dtype = PKV_BF16;
    pool = NULL;
    const pkv_status st = pkv_pool_create(&d, &pool);
    ++g_checks;
    if (st == PKV_OK) {
      expect("table_set(dup slots)", pkv_page_table_set(pool, 0, 0, (const int32_t[]){1, 1}, 2),
             PKV_EINVAL);
      expect("append(at 5)", pkv_append_kv(pool, 0, 5, 1, &dummy, &dummy, NULL), PKV_ESTATE);
      expect("destroy", pkv_pool_destroy(pool), PKV_OK);
    } else if (pool != NULL || pkv_last_error()[0] == '\0') {
      ++g_bad;
      printf("FAIL create(tier %d) failed (%d) without a message or left a pool\n", tier, (int)st);
    }
  }
  if (g_bad) return 1;
  printf("ok %d\n", g_checks);
  return 0;
}
