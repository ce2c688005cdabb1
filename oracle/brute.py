"""Pure-Python brute force for tiny attention problems (TEST INFRASTRUCTURE).

Lists of floats, math.exp and math.fsum only: no numpy, no BLAS.  It restates
Attention(Q, K, V) = softmax(s Q K^T) V ([P3] "概念揭曉") element by element,
with the softmax as e^{x_i} / sum_j e^{x_j} ([P2] section 六, classic softmax
formula), and the analytic gradient for the backward.  It is meant for
N <= 8 and d <= 8; page tags are defined in ``oracle/__init__.py``.
"""

from __future__ import annotations

import math
from typing import List, Sequence

Matrix = List[List[float]]


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    return math.fsum(x * y for x, y in zip(a, b))


def brute_forward(q: Matrix, k: Matrix, v: Matrix, scale: float):
    """Returns (O, LSE) as nested lists for one head."""
    O: Matrix = []
    L: List[float] = []
    for qi in q:
        scores = [scale * _dot(qi, kj) for kj in k]
        top = max(scores)
        w = [math.exp(x - top) for x in scores]
        z = math.fsum(w)
        O.append([math.fsum(w[j] * v[j][c] for j in range(len(k))) / z
                  for c in range(len(v[0]))])
        L.append(top + math.log(z))
    return O, L


def brute_backward(q: Matrix, k: Matrix, v: Matrix, dO: Matrix, scale: float):
    """Returns (dQ, dK, dV) as nested lists for one head.

    Uses P_ij = softmax_j(s q_i . k_j) and, per query row i,
    dS_ij = P_ij (dO_i . v_j - sum_l P_il dO_i . v_l)."""
    n, nk, d, dv = len(q), len(k), len(q[0]), len(v[0])
    P: Matrix = []
    for qi in q:
        scores = [scale * _dot(qi, kj) for kj in k]
        top = max(scores)
        w = [math.exp(x - top) for x in scores]
        z = math.fsum(w)
        P.append([x / z for x in w])
    dP = [[_dot(dO[i], v[j]) for j in range(nk)] for i in range(n)]
    dS = []
    for i in range(n):
        mean = math.fsum(P[i][j] * dP[i][j] for j in range(nk))
        dS.append([P[i][j] * (dP[i][j] - mean) for j in range(nk)])
    dQ = [[scale * math.fsum(dS[i][j] * k[j][c] for j in range(nk)) for c in range(d)]
          for i in range(n)]
    dK = [[scale * math.fsum(dS[i][j] * q[i][c] for i in range(n)) for c in range(d)]
          for j in range(nk)]
    dV = [[math.fsum(P[i][j] * dO[i][c] for i in range(n)) for c in range(dv)]
          for j in range(nk)]
    return dQ, dK, dV
