"""Pure-Python brute force of the same layer, for tiny shapes only.

TEST INFRASTRUCTURE ONLY. It pins ``moe_oracle``: no numpy in the arithmetic, no sorting
helpers beyond ``sorted`` on explicit keys, one scalar at a time. Where ``moe_oracle`` uses
matrix products and vectorised gathers, this module walks every (token, expert) pair with
nested loops, so a transposed operand, a wrong index or a dropped term in either shows up as
a mismatch. It follows the same readings (see the package docstring of ``moe_oracle``).
"""
from __future__ import annotations

import math


def topk(logits_row, K):
    """K experts with the largest logits, ties to the lower id (key (-l, e) ascending)."""
    keyed = sorted(((-float(l) + 0.0, e) for e, l in enumerate(logits_row)))
    return [e for _, e in keyed[:K]]


def softmax(vals):
    m = max(vals)
    ex = [math.exp(v - m) for v in vals]
    s = sum(ex)
    return [v / s for v in ex]


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def layer(X, logits, Wg, Wu, Wd, dOut, K, e0, E_loc):
    """Forward and backward for every token, pair by pair.

    X, dOut: lists [N][H]; logits [N][E]; Wg, Wu [E_loc][I][H]; Wd [E_loc][H][I] (floats).
    Returns a dict with idx, p, out (None for untouched tokens), dX, dp, dWg, dWu, dWd,
    dlogits (only meaningful when all experts are local) and the pair lists per expert.
    """
    N = len(X); H = len(X[0]); E = len(logits[0]); I = len(Wg[0])
    idx, p = [], []
    for n in range(N):
        sel = topk(logits[n], K)
        idx.append(sel)
        p.append(softmax([float(logits[n][e]) for e in sel]))
    # Schedule: for each local expert, its pairs in ascending token id.
    pairs = {e: [] for e in range(E_loc)}
    for n in range(N):
        for k in range(K):
            e = idx[n][k] - e0
            if 0 <= e < E_loc:
                pairs[e].append((n, k))
    out = [None] * N
    dX = [None] * N
    dp = [[0.0] * K for _ in range(N)]
    dWg = [[[0.0] * H for _ in range(I)] for _ in range(E_loc)]
    dWu = [[[0.0] * H for _ in range(I)] for _ in range(E_loc)]
    dWd = [[[0.0] * I for _ in range(H)] for _ in range(E_loc)]
    y_of = {}
    for e in range(E_loc):
        for (n, k) in pairs[e]:
            x = X[n]
            g = [sum(x[c] * Wg[e][i][c] for c in range(H)) for i in range(I)]
            u = [sum(x[c] * Wu[e][i][c] for c in range(H)) for i in range(I)]
            h = [_silu(g[i]) * u[i] for i in range(I)]
            y = [sum(h[i] * Wd[e][c][i] for i in range(I)) for c in range(H)]
            y_of[(n, k)] = y
            # Backward of <dOut[n], p * y>.
            D = dOut[n]
            pk = p[n][k]
            dp[n][k] = sum(D[c] * y[c] for c in range(H))
            dh = [pk * sum(D[c] * Wd[e][c][i] for c in range(H)) for i in range(I)]
            dg = [dh[i] * u[i] * _sig(g[i]) * (1.0 + g[i] * (1.0 - _sig(g[i]))) for i in range(I)]
            du = [dh[i] * _silu(g[i]) for i in range(I)]
            dx = [sum(dg[i] * Wg[e][i][c] + du[i] * Wu[e][i][c] for i in range(I))
                  for c in range(H)]
            if dX[n] is None:
                dX[n] = [0.0] * H
            for c in range(H):
                dX[n][c] += dx[c]
            for i in range(I):
                for c in range(H):
                    dWg[e][i][c] += dg[i] * x[c]
                    dWu[e][i][c] += du[i] * x[c]
                    dWd[e][c][i] += pk * D[c] * h[i]
    for n in range(N):
        acc = None
        for k in range(K):
            if (n, k) in y_of:
                if acc is None:
                    acc = [0.0] * H
                for c in range(H):
                    acc[c] += p[n][k] * y_of[(n, k)][c]
        out[n] = acc
    # Softmax-over-top-k backward, per token: dl_j = sum_k dp_k * dp_k/dl_j with
    # dp_k/dl_j = p_k (delta_kj - p_j).
    dlogits = [[0.0] * E for _ in range(N)]
    for n in range(N):
        for j in range(K):
            acc = 0.0
            for k in range(K):
                acc += dp[n][k] * p[n][k] * ((1.0 if k == j else 0.0) - p[n][j])
            dlogits[n][idx[n][j]] = acc
    return dict(idx=idx, p=p, pairs=pairs, out=out, dX=dX, dp=dp, dWg=dWg, dWu=dWu,
                dWd=dWd, dlogits=dlogits)
