"""Exact paged causal attention, forward and backward (oracle, fp64).

Definition followed ("Out of the Memory Barrier", gist.science de, sections
2.A and 2.B; sciencestack.ai, Figure 3):
  * the sequence is processed in query chunks; chunk c's keys/values are in
    the cache before its attention runs, so a query at absolute position t
    attends to every key s <= t (all earlier pages plus the causal part of
    its own chunk);
  * K/V live in fixed-size pages reached through a page table; the result is
    that of attention over the de-paged, logical-order sequence;
  * the backward recomputes the forward (activations are not kept) and the
    gradients of the cached K/V are accumulated in place, i.e. dK/dV of a
    multi-chunk run is the sum of every chunk's contribution.

Formulas (tau = softmax scale, g(h) = h // G with G = hq // hkv, A = allowed
keys of (t, h)):
  S = tau * q_t,h . k_s,g ;  LSE = log sum_{s in A} exp(S) ;  P = exp(S - LSE)
  O_t,h = sum_s P v_s,g
  D = dO_t,h . O_t,h ;  dP = dO_t,h . v_s,g ;  dS = P (dP - D)
  dQ_t,h = tau sum_s dS k_s,g
  dK_s,g = tau sum_{h in g} sum_t dS q_t,h ;  dV_s,g = sum_{h in g} sum_t P dO_t,h
This is the gradient of L = sum O * dO.  Rows are processed in blocks with a
full-row softmax; nothing is tiled over keys.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .select import select_pages


def page_in(k: np.ndarray, table: np.ndarray, slots: int, page: int) -> np.ndarray:
    """Logical k [n][hkv][d] -> pool [hkv][slots][page][d] (zeros elsewhere)."""
    n, hkv, d = k.shape
    pool = np.zeros((hkv, slots, page, d), dtype=k.dtype)
    for g in range(hkv):
        for j in range(-(-n // page)):
            lo, hi = j * page, min((j + 1) * page, n)
            pool[g, table[g, j], :hi - lo] = k[lo:hi, g]
    return pool


def depage(pool: np.ndarray, table: np.ndarray, n: int) -> np.ndarray:
    """pool [hkv][slots][page][d] + table [hkv][pages] -> logical [n][hkv][d] fp64."""
    hkv, _, page, d = pool.shape
    out = np.empty((n, hkv, d))
    for g in range(hkv):
        for j in range(-(-n // page)):
            lo, hi = j * page, min((j + 1) * page, n)
            out[lo:hi, g] = pool[g, table[g, j], :hi - lo]
    return out


def allowed_pages_matrix(sel, n_key_pages: int) -> np.ndarray:
    """sel[i_loc][g] (sorted page ids) -> bool [n_qpages][hkv][n_key_pages]."""
    nqp, hkv = len(sel), len(sel[0])
    m = np.zeros((nqp, hkv, n_key_pages), dtype=bool)
    for i in range(nqp):
        for g in range(hkv):
            m[i, g, sel[i][g]] = True
    return m


def _mask(t_abs: np.ndarray, n_keys: int, page: Optional[int], pages_ok) -> np.ndarray:
    """Allowed (t, s) for absolute query positions t_abs and keys 0..n_keys-1.
    pages_ok: None (dense) or bool [len(t_abs)][n_key_pages] for these rows."""
    s = np.arange(n_keys)
    m = s[None, :] <= t_abs[:, None]
    if pages_ok is not None:
        m &= pages_ok[:, s // page]
    return m


def _rows(q, k, v, do, t_abs, scale, mask):
    """One block of rows of one head: q/do [B][d], k/v [n_keys][d]."""
    S = scale * (q @ k.T)
    S = np.where(mask, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    Z = E.sum(axis=1, keepdims=True)
    P = E / Z
    O = P @ v
    lse = (m + np.log(Z))[:, 0]
    out = dict(P=P, O=O, lse=lse)
    if do is not None:
        D = (do * O).sum(axis=1, keepdims=True)
        dP = do @ v.T
        dS = P * (dP - D)
        out.update(dS=dS, dq=scale * (dS @ k))
    return out


def _chunk(q, k, v, do, q_pos0, scale, page, sel, block):
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    n_keys = q_pos0 + n_q
    k = k[:n_keys].astype(np.float64)
    v = v[:n_keys].astype(np.float64)
    q = q.astype(np.float64)
    do = None if do is None else do.astype(np.float64)
    pages_ok = None
    if sel is not None:
        pages_ok = allowed_pages_matrix(sel, -(-n_keys // page))
    O = np.zeros((n_q, hq, d))
    lse = np.zeros((hq, n_q))
    dq = dk = dv = None
    if do is not None:
        dq = np.zeros((n_q, hq, d))
        dk = np.zeros((n_keys, hkv, d))
        dv = np.zeros((n_keys, hkv, d))
    for h in range(hq):
        g = h // G
        for r0 in range(0, n_q, block):
            r1 = min(n_q, r0 + block)
            t_abs = q_pos0 + np.arange(r0, r1)
            nk = int(t_abs[-1]) + 1
            ok = None
            if pages_ok is not None:
                ok = pages_ok[(t_abs - q_pos0) // page, g][:, :-(-nk // page)]
            mask = _mask(t_abs, nk, page, ok)
            res = _rows(q[r0:r1, h], k[:nk, g], v[:nk, g],
                        None if do is None else do[r0:r1, h], t_abs, scale, mask)
            O[r0:r1, h] = res["O"]
            lse[h, r0:r1] = res["lse"]
            if do is not None:
                dq[r0:r1, h] = res["dq"]
                dk[:nk, g] += scale * (res["dS"].T @ q[r0:r1, h])
                dv[:nk, g] += res["P"].T @ do[r0:r1, h]
    return O, lse, dq, dk, dv


def attn_fwd(q, k, v, q_pos0: int, scale: float, page: Optional[int] = None,
             sel=None, block: int = 256):
    """Forward of one chunk.  q [n_q][hq][d]; k, v [>= q_pos0+n_q][hkv][d]
    logical order.  sel: None (dense) or the chunk's page selection.
    Returns O [n_q][hq][d], LSE [hq][n_q] (natural log)."""
    O, lse, *_ = _chunk(q, k, v, None, q_pos0, scale, page, sel, block)
    return O, lse


def attn_bwd(q, k, v, do, q_pos0: int, scale: float, page: Optional[int] = None,
             sel=None, block: int = 256):
    """Recompute-forward + backward of one chunk.
    Returns dict O, lse, dq [n_q][hq][d], dk, dv [q_pos0+n_q][hkv][d]."""
    O, lse, dq, dk, dv = _chunk(q, k, v, do, q_pos0, scale, page, sel, block)
    return dict(O=O, lse=lse, dq=dq, dk=dk, dv=dv)


def run_chunks(q, k, v, do, chunk: int, scale: float, page: int, sparse=None,
               block: int = 256, sels=None):
    """Chunk-recurrent run over the whole sequence (q_pos0 of chunk c = c*chunk).

    sparse: None or dict(top_k=, n_sink=, n_local=, score_dtype=) -> page
    top-K per chunk (selection from the chunk's queries and all keys so far).
    Returns dict O [N][hq][d], lse [hq][N], dq, dk, dv [N][hkv][d] (sums over
    chunks), sel (list per chunk, or None).  sels: fixed per-chunk selections
    to use instead of selecting (the selection is a constant for gradients)."""
    N, hq, d = q.shape
    hkv = k.shape[1]
    O = np.zeros((N, hq, d))
    lse = np.zeros((hq, N))
    dq = np.zeros((N, hq, d))
    dk = np.zeros((N, hkv, d))
    dv = np.zeros((N, hkv, d))
    fixed = sels
    sels = []
    for q_pos0 in range(0, N, chunk):
        n_q = min(chunk, N - q_pos0)
        sl = slice(q_pos0, q_pos0 + n_q)
        sel = None
        if fixed is not None:
            sel = fixed[q_pos0 // chunk]
        elif sparse is not None:
            sel = select_pages(q[sl], k, q_pos0, page, hkv, **sparse)
        sels.append(sel)
        r = attn_bwd(q[sl], k, v, do[sl], q_pos0, scale, page, sel, block)
        O[sl], lse[:, sl], dq[sl] = r["O"], r["lse"], r["dq"]
        dk[:q_pos0 + n_q] += r["dk"]
        dv[:q_pos0 + n_q] += r["dv"]
    return dict(O=O, lse=lse, dq=dq, dk=dk, dv=dv,
                sel=sels if (sparse is not None or fixed is not None) else None)


def rows_fwd_bwd(q_rows, do_rows, t_abs, h: int, k, v, scale: float, G: int,
                 page: Optional[int] = None, pages_ok=None):
    """O, LSE and dQ of individual query rows of head h (each row is
    independent of every other).  q_rows/do_rows [B][d]; t_abs [B] absolute
    positions; k, v logical [>= max(t)+1][hkv][d]; pages_ok: None or bool
    [B][n_key_pages] (the selection of each row's query page)."""
    g = h // G
    t_abs = np.asarray(t_abs)
    nk = int(t_abs.max()) + 1
    ok = None if pages_ok is None else pages_ok[:, :-(-nk // page)]
    mask = _mask(t_abs, nk, page, ok)
    res = _rows(q_rows.astype(np.float64), k[:nk, g].astype(np.float64),
                v[:nk, g].astype(np.float64),
                None if do_rows is None else do_rows.astype(np.float64),
                t_abs, scale, mask)
    return res["O"], res["lse"], res.get("dq")


def key_grads_sampled(s0: int, q_all, do_all, k, v, scale: float, chunk: int,
                      page: Optional[int] = None, sels=None, block: int = 256):
    """dK, dV (summed over every chunk) of keys s >= s0, in full.

    Only queries t >= s0 touch these keys, so the work is
    (N - s0) rows x N keys.  q_all/do_all are the rows t >= s0 only
    ([N - s0][hq][d]); k, v are logical [N][hkv][d].  sels: per chunk
    selections (sparse) or None.  Returns dk, dv [N - s0][hkv][d]."""
    n_rows, hq, d = q_all.shape
    N = s0 + n_rows
    hkv = k.shape[1]
    G = hq // hkv
    kk = k[:N].astype(np.float64)
    vv = v[:N].astype(np.float64)
    dk = np.zeros((N - s0, hkv, d))
    dv = np.zeros((N - s0, hkv, d))
    for h in range(hq):
        g = h // G
        for r0 in range(0, n_rows, block):
            r1 = min(n_rows, r0 + block)
            t_abs = s0 + np.arange(r0, r1)
            nk = int(t_abs[-1]) + 1
            ok = None
            if sels is not None:
                rowsok = []
                npg = -(-nk // page)
                for t in t_abs:
                    c = int(t) // chunk
                    il = (int(t) - c * chunk) // page
                    m = np.zeros(npg, dtype=bool)
                    pgs = sels[c][il][g]
                    m[pgs[pgs < npg]] = True
                    rowsok.append(m)
                ok = np.array(rowsok)
            mask = _mask(t_abs, nk, page, ok)
            res = _rows(q_all[r0:r1, h].astype(np.float64), kk[:nk, g], vv[:nk, g],
                        do_all[r0:r1, h].astype(np.float64), t_abs, scale, mask)
            dk[:nk - s0, g] += scale * (res["dS"][:, s0:].T @ q_all[r0:r1, h].astype(np.float64))
            dv[:nk - s0, g] += res["P"][:, s0:].T @ do_all[r0:r1, h].astype(np.float64)
    return dk, dv


def chunk_page_grads(q, do, q_pos0: int, k, v, scale: float, page: int, sel, pages):
    """dK, dV that one top-K chunk adds to the key pages listed in `pages`.

    Attention restricted to the selected pages (gist.science de, section 2.D;
    nl "Methodologie"): a row t of query page i and head h attends to the keys
    s <= t of the pages sel[i][g(h)].  Only those keys enter its softmax, so
    each (query page, head) is computed against the keys of its selection,
    gathered in page order (the same softmax as the masked form over all
    keys; the columns it masks out are simply not formed).  From each row's
    P and dS the columns of the listed pages give their contributions
    dK += tau dS^T q and dV += P^T dO.  The work is rows x selected keys,
    which makes the shared pages of a full-size chunk checkable.
    q, do [n_q][hq][d]; k, v logical [>= q_pos0 + n_q][hkv][d]; sel[i][g]
    page ids.  Returns dk, dv [len(pages)][page][hkv][d] (rows past the end
    of the keys stay zero)."""
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    G = hq // hkv
    n_keys = q_pos0 + n_q
    want = {int(p): j for j, p in enumerate(pages)}
    dk = np.zeros((len(pages), page, hkv, d))
    dv = np.zeros((len(pages), page, hkv, d))
    for il in range(-(-n_q // page)):
        r0, r1 = il * page, min(n_q, (il + 1) * page)
        t_abs = q_pos0 + np.arange(r0, r1)
        for g in range(hkv):
            sel_pages = sorted(int(x) for x in sel[il][g])
            pos = np.concatenate([np.arange(p * page, min((p + 1) * page, n_keys))
                                  for p in sel_pages])
            kk = k[pos, g].astype(np.float64)
            vv = v[pos, g].astype(np.float64)
            mask = pos[None, :] <= t_abs[:, None]
            for h in range(g * G, (g + 1) * G):
                qh = q[r0:r1, h].astype(np.float64)
                doh = do[r0:r1, h].astype(np.float64)
                res = _rows(qh, kk, vv, doh, t_abs, scale, mask)
                for p in sel_pages:
                    if p not in want:
                        continue
                    cols = np.nonzero(pos // page == p)[0]
                    n = len(cols)
                    dk[want[p], :n, g] += scale * (res["dS"][:, cols].T @ qh)
                    dv[want[p], :n, g] += res["P"][:, cols].T @ doh
    return dk, dv
