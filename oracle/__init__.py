"""fp64 CPU oracle for paged-KV chunk attention.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package.  The GPU library never calls it, shares
no code with it, and this package imports nothing of the library.

What it computes (plain definitions, fp64, numpy):
  * de-paging a KV pool through its page table;
  * exact causal softmax attention of one query chunk over every earlier
    key plus its own causal prefix, forward (O, LSE) and backward
    (dQ, dK, dV), with dK/dV of a multi-chunk run being the sum of the
    per-chunk contributions;
  * page-level top-K selection from per-page mean vectors, and attention
    restricted to the selected pages.

Sources, all titled "Out of the Memory Barrier: A Highly Memory Efficient
Training System for LLMs with Million-Token Contexts":
  gist.science (de) summary, sections 2.A (chunk-recurrent training with
  recomputation), 2.B (paged KV cache and gradients, in-place atomic
  accumulation, custom forward/backward kernels), 2.D (top-K page retrieval
  from representative vectors); gist.science (nl) summary, "Methodologie",
  page-level sparse attention (one representative vector per page);
  sciencestack.ai page, Figure 3 (kernel updates KV gradients in place) and
  Figure 5 (key pages retrieved per query page).

Readings where the pages are silent are listed in the repository's design
notes; each function states the one it uses.

Parity status: every function is pinned by tests under tests/ (brute force,
finite differences, an independent library routine, closed forms,
invariants).  No function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    depage, page_in, attn_fwd, attn_bwd, run_chunks, rows_fwd_bwd,
    key_grads_sampled, chunk_page_grads, allowed_pages_matrix,
)
from .select import key_page_means, query_page_means, select_pages  # noqa: F401
from .brute import attn_brute  # noqa: F401
