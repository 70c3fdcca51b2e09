"""Brute-force pure-Python versions of the sublayer, for tiny shapes.

These loops are an independent statement of the definitions (explicit index
sums, math.erf / math.exp), used to pin the NumPy oracle.  They are slow:
only for shapes of a few elements per side.
"""
from __future__ import annotations

import math


def _gelu(u: float) -> float:
    return 0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0)))


def _silu(u: float) -> float:
    return u / (1.0 + math.exp(-u))


def ffn_rank(x, w1, w3, w2, T_p, t, act):
    """Rank t: explicit loops over its hidden units j in [t*n, (t+1)*n)."""
    T, d = len(x), len(x[0])
    d_ff = len(w1[0])
    n = d_ff // T_p
    hid = list(range(t * n, (t + 1) * n))
    H = [[0.0] * n for _ in range(T)]
    for i in range(T):
        for jj, j in enumerate(hid):
            u = sum(x[i][k] * w1[k][j] for k in range(d))
            if act == "none":
                h = u
            elif act == "gelu":
                h = _gelu(u)
            else:
                v = sum(x[i][k] * w3[k][j] for k in range(d))
                h = _silu(u) * v if act == "swiglu" else u * v
            H[i][jj] = h
    y = [[sum(H[i][jj] * w2[j][c] for jj, j in enumerate(hid)) for c in range(d)] for i in range(T)]
    return H, y


def attention(q, k, v, causal=True):
    """One head: loops over queries and keys; softmax with the max subtracted."""
    T, dh = len(q), len(q[0])
    out = []
    for i in range(T):
        keys = range(i + 1) if causal else range(len(k))
        s = [sum(q[i][c] * k[j][c] for c in range(dh)) / math.sqrt(dh) for j in keys]
        m = max(s)
        e = [math.exp(z - m) for z in s]
        z = sum(e)
        out.append([sum(e[jj] * v[j][c] for jj, j in enumerate(keys)) / z for c in range(dh)])
    return out


def matmul(a, b):
    return [[sum(a[i][k] * b[k][j] for k in range(len(b))) for j in range(len(b[0]))]
            for i in range(len(a))]
