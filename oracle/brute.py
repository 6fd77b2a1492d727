"""Pure-Python loop versions of the oracle's definitions, for micro sizes.

Written independently of the vectorised oracle (explicit loops, math.exp, no
numpy linear algebra) so that the two can pin each other.  Same definitions
as oracle.attention ("Out of the Memory Barrier", gist.science de, sections
2.A, 2.B and 2.D; sciencestack.ai, Figure 3).
"""
from __future__ import annotations

import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += float(x) * float(y)
    return s


def brute_select(q, k, q_pos0, page, hkv, top_k, n_sink=1, n_local=2):
    """Selection by plain sorting of (score, page) pairs with Python's sorted()."""
    n_q, hq, d = len(q), len(q[0]), len(q[0][0])
    G = hq // hkv
    n_keys = q_pos0 + n_q
    out = []
    for il in range(-(-n_q // page)):
        i = q_pos0 // page + il
        row = []
        for g in range(hkv):
            toks = range(il * page, min((il + 1) * page, n_q))
            qbar = [0.0] * d
            cnt = 0
            for t in toks:
                for h in range(g * G, (g + 1) * G):
                    cnt += 1
                    for e in range(d):
                        qbar[e] += float(q[t][h][e])
            qbar = [x / cnt for x in qbar]
            scored = []
            for j in range(n_sink, i - n_local + 1):
                rows = range(j * page, min((j + 1) * page, n_keys))
                kbar = [sum(float(k[s][g][e]) for s in rows) / len(rows) for e in range(d)]
                scored.append((-_dot(qbar, kbar), j))
            keep = [j for _, j in sorted(scored)[:top_k]]
            forced = [j for j in range(n_sink) if j <= i] + [j for j in range(i - n_local + 1, i + 1) if j >= 0]
            row.append(sorted(set(forced) | set(keep)))
        out.append(row)
    return out


def attn_brute(q, k, v, do, chunk, scale, page=None, sels=None):
    """Chunk loop with explicit per-(t, h, s) loops.

    q, do: [N][hq][d] nested sequences; k, v: [N][hkv][d].  sels: None or a
    per-chunk list sel[i_loc][g] of allowed key pages.  Returns O, lse, dq, dk,
    dv as nested lists (dk, dv summed over chunks)."""
    N, hq, d = len(q), len(q[0]), len(q[0][0])
    hkv = len(k[0])
    G = hq // hkv
    O = [[[0.0] * d for _ in range(hq)] for _ in range(N)]
    lse = [[0.0] * N for _ in range(hq)]
    dq = [[[0.0] * d for _ in range(hq)] for _ in range(N)]
    dk = [[[0.0] * d for _ in range(hkv)] for _ in range(N)]
    dv = [[[0.0] * d for _ in range(hkv)] for _ in range(N)]
    for c0 in range(0, N, chunk):
        for t in range(c0, min(N, c0 + chunk)):
            for h in range(hq):
                g = h // G
                keys = []
                for s in range(t + 1):
                    if sels is not None:
                        il = (t - c0) // page
                        if (s // page) not in sels[c0 // chunk][il][g]:
                            continue
                    keys.append(s)
                logits = [scale * _dot(q[t][h], k[s][g]) for s in keys]
                mx = max(logits)
                z = sum(math.exp(x - mx) for x in logits)
                L = mx + math.log(z)
                lse[h][t] = L
                p = [math.exp(x - L) for x in logits]
                for e in range(d):
                    O[t][h][e] = sum(pi * float(v[s][g][e]) for pi, s in zip(p, keys))
                D = _dot(do[t][h], O[t][h])
                for pi, s in zip(p, keys):
                    ds = pi * (_dot(do[t][h], v[s][g]) - D)
                    for e in range(d):
                        dq[t][h][e] += scale * ds * float(k[s][g][e])
                        dk[s][g][e] += scale * ds * float(q[t][h][e])
                        dv[s][g][e] += pi * float(do[t][h][e])
    return O, lse, dq, dk, dv
