"""Planted mistakes in the fp64 oracle must fail its pins.  CPU only.

Each case rewrites one line of an oracle function (a dropped scale or term, a
flipped sign, an off-by-one causal boundary or page mask, a wrong head-to-group
mapping, a transposed or swapped operand, a reversed tie order, a misplaced or
missing forced page, one page too many, ...), puts
the rewritten function in place of the original for the duration of the case,
and runs every pin of tests/test_oracle_pins.py against it; at least one pin
must fail.  The pure-loop brute force (oracle/brute.py), the hand-worked and
golden fixtures and torch's CPU attention are the references the pins compare
with; no case touches them.
"""
import inspect
import textwrap

import pytest

import oracle
import oracle.attention as OA
import oracle.select as OS
import test_oracle_pins as P

PINS = {
    "brute_dense_2_1": lambda: P.test_brute_dense(2, 1),
    "brute_dense_4_2": lambda: P.test_brute_dense(4, 2),
    "brute_sparse": P.test_brute_sparse,
    "select_vs_sorted": P.test_select_vs_sorted,
    "select_golden_ties": P.test_select_golden_ties,
    "fd_every_coordinate": lambda: P.test_finite_differences_every_coordinate(False),
    "fd_every_coordinate_sparse": lambda: P.test_finite_differences_every_coordinate(True),
    "fd_directional": P.test_finite_differences_directional_tiny_config,
    "torch_sdpa": P.test_against_torch_sdpa_tiny_config,
    "chunked_equals_full": P.test_chunked_equals_full_sequence,
    "permutation": P.test_page_table_permutation_invariance,
    "topk_all_equals_dense": P.test_topk_all_pages_equals_dense,
    "sum_identities": lambda: P.test_gradient_sum_identities(None),
    "sum_identities_sparse": lambda: P.test_gradient_sum_identities(dict(top_k=2)),
    "closed_forms": P.test_closed_forms,
    "hand_worked": P.test_hand_worked_two_tokens,
    "sampled_helpers": lambda: P.test_sampled_helpers_match_full(None),
    "sampled_helpers_sparse": lambda: P.test_sampled_helpers_match_full(dict(top_k=2)),
    "chunk_page_grads": P.test_chunk_page_grads_against_brute_force_and_masked_form,
}

# (module, function, exact source text, replacement)
MUTANTS = {
    "dq_without_scale": (OA, "_rows", "dq=scale * (dS @ k)", "dq=(dS @ k)"),
    "dk_without_scale": (OA, "_chunk", 'dk[:nk, g] += scale * (res["dS"].T', 'dk[:nk, g] += (res["dS"].T'),
    "ds_sign_flipped": (OA, "_rows", "dS = P * (dP - D)", "dS = P * (D - dP)"),
    "ds_without_D": (OA, "_rows", "dS = P * (dP - D)", "dS = P * dP"),
    "lse_without_max": (OA, "_rows", "lse = (m + np.log(Z))[:, 0]", "lse = np.log(Z)[:, 0]"),
    "causal_strict": (OA, "_mask", "m = s[None, :] <= t_abs[:, None]", "m = s[None, :] < t_abs[:, None]"),
    "causal_one_ahead": (OA, "_mask", "m = s[None, :] <= t_abs[:, None]", "m = s[None, :] <= t_abs[:, None] + 1"),
    "gqa_interleaved": (OA, "_chunk", "g = h // G", "g = h % hkv"),
    "dv_from_dq_side": (OA, "_chunk", 'dv[:nk, g] += res["P"].T @ do[r0:r1, h]', 'dv[:nk, g] += res["P"].T @ q[r0:r1, h]'),
    "pv_with_keys": (OA, "_rows", "O = P @ v", "O = P @ k"),
    "tie_to_higher_page": (OS, "select_pages", "order = np.lexsort((cand, -s.astype(np.float64)))",
                           "order = np.lexsort((-cand, -s.astype(np.float64)))"),
    "ascending_scores": (OS, "select_pages", "order = np.lexsort((cand, -s.astype(np.float64)))",
                         "order = np.lexsort((cand, s.astype(np.float64)))"),
    "local_window_short": (OS, "select_pages", "set(range(max(0, i - n_local + 1), i + 1))",
                           "set(range(max(0, i - n_local + 2), i + 1))"),
    "candidates_overlap_local": (OS, "select_pages", "cand = np.arange(n_sink, i - n_local + 1, dtype=np.int64)",
                                 "cand = np.arange(n_sink, i, dtype=np.int64)"),
    "query_mean_one_head": (OS, "query_page_means", "blk[:, g * G:(g + 1) * G, :]", "blk[:, g * G:g * G + 1, :]"),
    "key_mean_skips_first_token": (OS, "key_page_means", "k[j * page:min((j + 1) * page, n)]",
                                   "k[j * page + 1:min((j + 1) * page, n)]"),
    "depage_wrong_slot": (OA, "depage", "pool[g, table[g, j], :hi - lo]", "pool[g, j, :hi - lo]"),
    "scores_without_scale": (OA, "_rows", "S = scale * (q @ k.T)", "S = (q @ k.T)"),
    "probabilities_unnormalised": (OA, "_rows", "P = E / Z", "P = E"),
    "lse_in_base_2": (OA, "_rows", "lse = (m + np.log(Z))[:, 0]", "lse = (m + np.log2(Z))[:, 0]"),
    "D_without_O": (OA, "_rows", "D = (do * O).sum(axis=1, keepdims=True)",
                    "D = do.sum(axis=1, keepdims=True)"),
    "dP_with_keys": (OA, "_rows", "dP = do @ v.T", "dP = do @ k.T"),
    "dk_from_dO": (OA, "_chunk", 'dk[:nk, g] += scale * (res["dS"].T @ q[r0:r1, h])',
                   'dk[:nk, g] += scale * (res["dS"].T @ do[r0:r1, h])'),
    "rows_ignore_chunk_start": (OA, "_chunk", "t_abs = q_pos0 + np.arange(r0, r1)",
                                "t_abs = np.arange(r0, r1) + 0 * q_pos0"),
    "page_mask_shifted": (OA, "_mask", "m &= pages_ok[:, s // page]",
                          "m &= pages_ok[:, np.minimum(s + 1, n_keys - 1) // page]"),
    "sinks_dropped": (OS, "select_pages", "forced = set(range(0, min(n_sink, i + 1))) | ",
                      "forced = set() | "),
    "one_page_too_many": (OS, "select_pages", "keep = cand[order[:min(top_k, cand.size)]]",
                          "keep = cand[order[:min(top_k + 1, cand.size)]]"),
    "page_grads_dk_without_scale": (OA, "chunk_page_grads", 'dk[want[p], :n, g] += scale * (res["dS"]',
                                    'dk[want[p], :n, g] += (res["dS"]'),
    "page_grads_strict_causal": (OA, "chunk_page_grads", "mask = pos[None, :] <= t_abs[:, None]",
                                 "mask = pos[None, :] < t_abs[:, None]"),
    "page_grads_next_page_columns": (OA, "chunk_page_grads", "cols = np.nonzero(pos // page == p)[0]",
                                     "cols = np.nonzero(pos // page == min(p + 1, sel_pages[-1]))[0]"),
    "page_grads_dv_from_q": (OA, "chunk_page_grads", 'dv[want[p], :n, g] += res["P"][:, cols].T @ doh',
                             'dv[want[p], :n, g] += res["P"][:, cols].T @ qh'),
    "page_grads_group_mapping": (OA, "chunk_page_grads", "for h in range(g * G, (g + 1) * G):",
                                 "for h in range(g, hq, hkv):"),
}


def _rewrite(module, name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, name)))
    assert src.count(old) == 1, f"{name}: the text to replace must occur exactly once"
    ns = dict(module.__dict__)
    exec(compile(src.replace(old, new), f"<planted mistake in {module.__name__}.{name}>", "exec"), ns)
    return ns[name]


def _install(monkeypatch, module, name, fn):
    """Put fn in place of module.name and of the same name re-exported by the
    package or imported by the attention module."""
    for m in {module, oracle, OA}:
        if hasattr(m, name):
            monkeypatch.setattr(m, name, fn)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(mutant, monkeypatch):
    module, name, old, new = MUTANTS[mutant]
    _install(monkeypatch, module, name, _rewrite(module, name, old, new))
    caught = []
    for pin, fn in PINS.items():
        try:
            fn()
        except Exception as e:  # an assertion, or a shape error from a broken formula
            caught.append(f"{pin} ({type(e).__name__})")
    assert caught, f"planted mistake {mutant!r} passed every pin"
    print(f"{mutant}: caught by {', '.join(caught)}")


def test_unmutated_oracle_passes_every_pin():
    for pin, fn in PINS.items():
        fn()
