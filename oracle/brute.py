"""Pure-Python brute-force attention for tiny inputs (N <= 8).

TEST INFRASTRUCTURE ONLY: the second, independent statement of the
definition used to pin the fp64 oracle. Plain loops, ``math.exp`` and
``math.fsum`` over Python floats; no numpy, no BLAS, no vectorisation, so it
shares no arithmetic path with the numpy oracle.

Definition: for each query row i, score s_ij = scale * sum_c q_ic k_jc over
the keys j visible to i (all j < kv_len, and j <= i when causal), then
softmax over those keys and the weighted sum of value rows (marketmaker.cc
article, section "为什么注意力是受记忆限制的"). A row with no visible key gives
O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

Matrix = List[List[float]]


def _as_rows(x) -> Matrix:
    return [[float(e) for e in row] for row in x]


def brute_head_forward(q: Sequence[Sequence[float]], k: Sequence[Sequence[float]],
                       v: Sequence[Sequence[float]], scale: float, causal: bool = False,
                       kv_len: Optional[int] = None) -> Tuple[Matrix, List[float]]:
    """One head: returns (O as a list of rows, LSE per row)."""
    q, k, v = _as_rows(q), _as_rows(k), _as_rows(v)
    n = len(k)
    dv = len(v[0]) if v else 0
    lim = n if kv_len is None else max(0, min(n, int(kv_len)))
    o_rows: Matrix = []
    lse: List[float] = []
    for i, qi in enumerate(q):
        keys = [j for j in range(lim) if (not causal or j <= i)]
        if not keys:
            o_rows.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        s = [scale * math.fsum(qi[c] * k[j][c] for c in range(len(qi))) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        o_rows.append([math.fsum(e[t] * v[j][c] for t, j in enumerate(keys)) / tot
                       for c in range(dv)])
        lse.append(mx + math.log(tot))
    return o_rows, lse


def brute_loss(q, k, v, do, scale: float, causal: bool = False,
               kv_len: Optional[int] = None) -> float:
    """L = sum_ic dO_ic * O_ic for one head (the scalar whose gradient the
    backward returns)."""
    o, _ = brute_head_forward(q, k, v, scale, causal, kv_len)
    return math.fsum(do[i][c] * o[i][c] for i in range(len(o)) for c in range(len(o[i])))


def brute_head_grad_fd(q, k, v, do, scale: float, causal: bool = False,
                       kv_len: Optional[int] = None, step: float = 1e-5):
    """Central finite differences of ``brute_loss`` w.r.t. every element of
    q, k and v. Returns (dQ, dK, dV) as lists of rows."""
    base = {"q": _as_rows(q), "k": _as_rows(k), "v": _as_rows(v)}
    do = _as_rows(do)
    grads = {}
    for name in ("q", "k", "v"):
        mat = base[name]
        g = [[0.0] * len(row) for row in mat]
        for i in range(len(mat)):
            for c in range(len(mat[i])):
                orig = mat[i][c]
                mat[i][c] = orig + step
                lp = brute_loss(base["q"], base["k"], base["v"], do, scale, causal, kv_len)
                mat[i][c] = orig - step
                lm = brute_loss(base["q"], base["k"], base["v"], do, scale, causal, kv_len)
                mat[i][c] = orig
                g[i][c] = (lp - lm) / (2.0 * step)
        grads[name] = g
    return grads["q"], grads["k"], grads["v"]


def brute_head_part(q, k, v, scale: float, causal: bool = False, q_pos0: int = 0,
                    k_pos0: int = 0) -> Tuple[Matrix, List[float]]:
    """One head, queries at global positions q_pos0 + i against keys at
    global positions k_pos0 + j (causal hides later key positions); returns
    (O rows, LSE per row), O = 0 and LSE = -inf for a row with no visible key."""
    q, k, v = _as_rows(q), _as_rows(k), _as_rows(v)
    dv = len(v[0]) if v else len(q[0])
    o_rows: Matrix = []
    lse: List[float] = []
    for i, qi in enumerate(q):
        keys = [j for j in range(len(k)) if (not causal or k_pos0 + j <= q_pos0 + i)]
        if not keys:
            o_rows.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        s = [scale * math.fsum(qi[c] * k[j][c] for c in range(len(qi))) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        o_rows.append([math.fsum(e[t] * v[j][c] for t, j in enumerate(keys)) / tot
                       for c in range(dv)])
        lse.append(mx + math.log(tot))
    return o_rows, lse


def brute_head_allowed(q, k, v, scale: float, allowed) -> Tuple[Matrix, List[float]]:
    """One head with an explicit visibility table: key j is visible to query
    i iff allowed[i][j]. Returns (O rows, LSE per row); a row with no visible
    key gives O = 0 and LSE = -inf."""
    q, k, v = _as_rows(q), _as_rows(k), _as_rows(v)
    dv = len(v[0]) if v else len(q[0])
    o_rows: Matrix = []
    lse: List[float] = []
    for i, qi in enumerate(q):
        keys = [j for j in range(len(k)) if allowed[i][j]]
        if not keys:
            o_rows.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        s = [scale * math.fsum(qi[c] * k[j][c] for c in range(len(qi))) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = math.fsum(e)
        o_rows.append([math.fsum(e[t] * v[j][c] for t, j in enumerate(keys)) / tot
                       for c in range(dv)])
        lse.append(mx + math.log(tot))
    return o_rows, lse


def brute_loss_allowed(q, k, v, do, scale: float, allowed) -> float:
    """L = sum_ic dO_ic * O_ic for ``brute_head_allowed``."""
    o, _ = brute_head_allowed(q, k, v, scale, allowed)
    do = _as_rows(do)
    return math.fsum(do[i][c] * o[i][c] for i in range(len(o)) for c in range(len(o[i])))
