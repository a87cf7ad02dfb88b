"""A second, scalar-loop transcription of the segment forward (no numpy inside
the arithmetic), used only to guard the oracle against transcription slips.
It restates the same equations, so it pins nothing about their reading."""

import math


def _sig(x):
    return x + 1.0 if x > 0.0 else math.exp(x)


def run(q, k, v, beta, rule, n_seg, scale):
    """q, k: nested lists [H][L][dk]; v: [H][L][dv]; returns (A, M, z) as lists."""
    H, L, dk, dv = len(q), len(q[0]), len(q[0][0]), len(v[0][0])
    A = [[[0.0] * dv for _ in range(L)] for _ in range(H)]
    Ms, zs = [], []
    for h in range(H):
        M = [[0.0] * dv for _ in range(dk)]
        z = [0.0] * dk
        g = 1.0 / (1.0 + math.exp(-beta[h]))
        for s in range(L // n_seg):
            base = s * n_seg
            first = s == 0
            for i in range(n_seg):
                qi = q[h][base + i]
                sc = []
                for j in range(i + 1):
                    kj = k[h][base + j]
                    sc.append(scale * sum(qi[c] * kj[c] for c in range(dk)))
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                tot = sum(w)
                fq = [_sig(x) for x in qi]
                den = sum(fq[c] * z[c] for c in range(dk))
                for c in range(dv):
                    a_dot = sum(w[j] * v[h][base + j][c] for j in range(i + 1)) / tot
                    a_mem = 0.0
                    if not first and den > 0.0:
                        a_mem = sum(fq[r] * M[r][c] for r in range(dk)) / den
                    A[h][base + i][c] = g * a_mem + (1.0 - g) * a_dot
            fk = [[_sig(x) for x in k[h][base + t]] for t in range(n_seg)]
            upd = []
            for t in range(n_seg):
                row = list(v[h][base + t])
                if rule == "delta" and not first:
                    den = sum(fk[t][r] * z[r] for r in range(dk))
                    for c in range(dv):
                        row[c] -= sum(fk[t][r] * M[r][c] for r in range(dk)) / den
                upd.append(row)
            for r in range(dk):
                for c in range(dv):
                    M[r][c] += sum(fk[t][r] * upd[t][c] for t in range(n_seg))
                z[r] += sum(fk[t][r] for t in range(n_seg))
        Ms.append(M)
        zs.append(z)
    return A, Ms, zs
