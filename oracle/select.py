"""Page-level top-K selection (oracle).

Follows the page-level sparse attention described in "Out of the Memory
Barrier" (gist.science de, section 2.D; gist.science nl, "Methodologie",
page-level sparse attention; sciencestack.ai, Figure 5): each query page keeps
the key pages whose representative vector scores highest against it, and
attends only to those.

Readings used (the pages give no formula):
  * representative of key page j, KV head g: mean of the keys of page j
    (over the tokens present);
  * representative of query page i, KV head g: mean of q over the page's
    tokens in this chunk and over the query heads of group g
    (heads g*G .. g*G+G-1);
  * score = plain dot product of the two means (no scale, no softmax);
  * forced pages: sinks {0..n_sink-1} and the n_local most recent pages
    {i-n_local+1 .. i} (the query's own page included); candidates are the
    pages strictly between them; the top_k best candidates are kept, ties
    going to the lower page index;
  * the selection is a constant for the gradient.
"""
from __future__ import annotations

import numpy as np


def key_page_means(k: np.ndarray, page: int) -> np.ndarray:
    """k [n][hkv][d] -> kbar [n_pages][hkv][d] (fp64), mean over present tokens."""
    n, hkv, d = k.shape
    npg = -(-n // page)
    out = np.zeros((npg, hkv, d))
    for j in range(npg):
        out[j] = k[j * page:min((j + 1) * page, n)].astype(np.float64).mean(axis=0)
    return out


def query_page_means(q: np.ndarray, page: int, hkv: int) -> np.ndarray:
    """q [n_q][hq][d] of one chunk (starting on a page boundary)
    -> qbar [n_qpages][hkv][d], mean over the page's tokens and the group's heads."""
    n, hq, d = q.shape
    G = hq // hkv
    nqp = -(-n // page)
    out = np.zeros((nqp, hkv, d))
    for i in range(nqp):
        blk = q[i * page:min((i + 1) * page, n)].astype(np.float64)
        for g in range(hkv):
            out[i, g] = blk[:, g * G:(g + 1) * G, :].reshape(-1, d).mean(axis=0)
    return out


def select_pages(q: np.ndarray, k_all: np.ndarray, q_pos0: int, page: int,
                 hkv: int, top_k: int, n_sink: int = 1, n_local: int = 2,
                 score_dtype=np.float64, return_scores: bool = False):
    """Selection for every query page of one chunk.

    q: [n_q][hq][d] chunk queries (q_pos0 % page == 0).
    k_all: keys [>= q_pos0+n_q][hkv][d] in logical order.
    score_dtype=np.float32 rounds both means and the dot product to fp32
    (the precision the GPU decides in); ties always go to the lower page.

    Returns sel: list over local query page i_loc of list over g of a sorted
    int64 array of absolute key-page ids; with return_scores also the fp64
    scores {(i_loc, g): (candidate ids, sigma)}.
    """
    assert q_pos0 % page == 0
    n_q = q.shape[0]
    kbar = key_page_means(k_all[:q_pos0 + n_q], page)
    qbar = query_page_means(q, page, hkv)
    first = q_pos0 // page
    sel, scores = [], {}
    for il in range(qbar.shape[0]):
        i = first + il
        row = []
        for g in range(hkv):
            cand = np.arange(n_sink, i - n_local + 1, dtype=np.int64)
            forced = set(range(0, min(n_sink, i + 1))) | set(range(max(0, i - n_local + 1), i + 1))
            if cand.size:
                # sum over e of kbar_e * qbar_e, evaluated the same way for
                # every candidate, so that pages with equal representatives
                # score equal and the tie rule decides between them (a BLAS
                # matrix-vector product may round equal rows differently)
                s64 = (kbar[cand, g, :] * qbar[il, g, :][None, :]).sum(axis=1)
                if score_dtype == np.float32:
                    kb = kbar[cand, g, :].astype(np.float32)
                    qb = qbar[il, g, :].astype(np.float32)
                    s = (kb * qb[None, :]).sum(axis=1, dtype=np.float32)
                else:
                    s = s64
                order = np.lexsort((cand, -s.astype(np.float64)))
                keep = cand[order[:min(top_k, cand.size)]]
                scores[(il, g)] = (cand, s64)
            else:
                keep = cand
            row.append(np.array(sorted(forced | set(keep.tolist())), dtype=np.int64))
        sel.append(row)
    return (sel, scores) if return_scores else sel
