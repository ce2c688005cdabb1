"""Float64 numpy oracle for scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline use this module.  It shares no code with the HIP library.

What is computed (page tags are defined in ``oracle/__init__.py``):

  Attention(Q, K, V) = softmax(s * Q K^T) V,  s = 1/sqrt(d)
      [P3] "概念揭曉", the scaled dot-product attention formula;
      [P2] section 五, the three-line standard attention (S, P, O).

The pages call the tiled method exact ([P1] "为什么这个故事对应
FlashAttention" list; [P3] "精確注意力" row of the metaphor table), so the
oracle is the plain definition written out: it materialises S and P for one
(batch, head) at a time, in float64, on inputs upcast exactly from bf16/fp32.

Conventions chosen where the pages are silent:
  * ``scale`` is the same fp32 value the GPU path receives, used as a float64.
  * The saved per-row statistic is the natural-log logsumexp,
    LSE_i = m_i + ln(l_i) = ln sum_j exp(S_ij)  ([P1] technical notes say only
    that O and "statistics" go back to HBM; [P2] section 六 keeps m and l).
  * The backward is the analytic gradient of the formula above (the pages only
    say that P is recomputed, [P2] section 七):
        D  = rowsum(dO * O)
        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D 1^T)
        dQ = s dS K,   dK = s dS^T Q
  * Arrays are [..., N, d]; leading axes are looped over one head at a time.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "softmax_rows",
    "sdpa_forward_head",
    "sdpa_forward",
    "sdpa_rows",
    "sdpa_backward_head",
    "sdpa_backward_rows",
    "sdpa_backward",
    "online_forward_head",
    "online_forward_normalised_head",
    "two_pass_forward_head",
    "split_bounds",
    "sdpa_split_head",
    "merge_parts",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def softmax_rows(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row softmax of S with the max subtracted ([P2] section 六, the
    classic softmax formula; [P3] "兩大核心魔法": subtract the maximum to
    avoid overflow).  Returns (P, m, l): P = exp(S - m) / l, m the row max,
    l the row sum of exp(S - m)."""
    m = S.max(axis=-1)
    E = np.exp(S - m[..., None])
    l = E.sum(axis=-1)
    return E / l[..., None], m, l


def sdpa_forward_head(q, k, v, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One head, plain definition.  q [Nq,d], k [Nk,d], v [Nk,dv].

    Steps: S = s Q K^T ([P2] section 五, first line); P = softmax(S) (second
    line); O = P V (third line); LSE = m + ln l.  Returns (O [Nq,dv], LSE [Nq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = float(scale) * (q @ k.T)
    P, m, l = softmax_rows(S)
    O = P @ v
    lse = m + np.log(l)
    return O, lse


def _heads(x: np.ndarray) -> Tuple[Tuple[int, ...], np.ndarray]:
    lead = x.shape[:-2]
    return lead, x.reshape((-1,) + x.shape[-2:])


def sdpa_forward(q, k, v, scale: float, heads: Optional[Iterable[int]] = None):
    """Plain forward over [..., N, d] arrays, one (batch, head) at a time.

    ``heads`` optionally restricts the work to some flattened (b*H + h)
    indices; the other outputs are left as NaN.  Returns (O, LSE).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead, qf = _heads(q)
    _, kf = _heads(k)
    _, vf = _heads(v)
    O = np.full(qf.shape[:-1] + (vf.shape[-1],), np.nan)
    L = np.full(qf.shape[:-1], np.nan)
    for i in (range(qf.shape[0]) if heads is None else heads):
        O[i], L[i] = sdpa_forward_head(qf[i], kf[i], vf[i], scale)
    return O.reshape(lead + O.shape[-2:]), L.reshape(lead + L.shape[-1:])


def sdpa_rows(q_rows, k, v, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Forward for selected query rows of one head against the full K and V.

    Each output row depends only on its own query row and all keys, so a row
    subset is the plain definition restricted to those rows."""
    return sdpa_forward_head(q_rows, k, v, scale)


def sdpa_backward_head(q, k, v, dO, scale: float):
    """One head, analytic gradient of O = softmax(s Q K^T) V.

    Recomputes S and P from Q and K as the forward does ([P2] section 七:
    P is recomputed rather than stored), then applies the chain rule.
    Returns dict with dQ, dK, dV, and the intermediates O, LSE, D, P, dP, dS.
    """
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    s = float(scale)
    S = s * (q @ k.T)
    P, m, l = softmax_rows(S)
    O = P @ v
    lse = m + np.log(l)
    D = (dO * O).sum(axis=-1)              # rowsum(dO * O)
    dV = P.T @ dO                          # through O = P V, w.r.t. V
    dP = dO @ v.T                          # through O = P V, w.r.t. P
    dS = P * (dP - D[:, None])             # softmax Jacobian applied row-wise
    dQ = s * (dS @ k)                      # through S = s Q K^T, w.r.t. Q
    dK = s * (dS.T @ q)                    # through S = s Q K^T, w.r.t. K
    return dict(dQ=dQ, dK=dK, dV=dV, O=O, LSE=lse, D=D, P=P, dP=dP, dS=dS)


def sdpa_backward_rows(q_rows, k, v, dO_rows, scale: float):
    """dQ and D for selected query rows of one head against the full K and V.

    Row i of dQ needs only q_i, dO_i and all keys: P_i = softmax(s q_i K^T),
    O_i = P_i V, D_i = dO_i . O_i, dP_i = dO_i V^T, dS_i = P_i * (dP_i - D_i),
    dQ_i = s dS_i K.  So a row subset is the plain backward restricted to those
    rows (dK and dV, which sum over every query, are not formed).
    Returns (dQ_rows [R, d], D_rows [R])."""
    q, k, v, dO = _f64(q_rows), _f64(k), _f64(v), _f64(dO_rows)
    s = float(scale)
    P, _, _ = softmax_rows(s * (q @ k.T))
    O = P @ v
    D = (dO * O).sum(axis=-1)
    dS = P * ((dO @ v.T) - D[:, None])
    return s * (dS @ k), D


def sdpa_backward(q, k, v, dO, scale: float, heads: Optional[Iterable[int]] = None):
    """Analytic backward over [..., N, d] arrays.  Returns (dQ, dK, dV, D).

    Heads not in ``heads`` are left as NaN."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    lead, qf = _heads(q)
    _, kf = _heads(k)
    _, vf = _heads(v)
    _, gf = _heads(dO)
    dQ = np.full(qf.shape, np.nan)
    dK = np.full(kf.shape, np.nan)
    dV = np.full(vf.shape, np.nan)
    D = np.full(qf.shape[:-1], np.nan)
    for i in (range(qf.shape[0]) if heads is None else heads):
        r = sdpa_backward_head(qf[i], kf[i], vf[i], gf[i], scale)
        dQ[i], dK[i], dV[i], D[i] = r["dQ"], r["dK"], r["dV"], r["D"]
    return (dQ.reshape(q.shape), dK.reshape(k.shape), dV.reshape(v.shape),
            D.reshape(lead + D.shape[-1:]))


# ---------------------------------------------------------------------------
# Online-softmax forms, used to check the tiled recurrence against the plain
# definition.  They walk the key/value rows in blocks ([P2] section 六,
# "Tiling": K and V cut into T_c blocks), carrying the running max m, the
# running sum l and the output ([P2] section 六, update rule; [P1] fable
# section 三: only two running numbers are kept between stacks).
# ---------------------------------------------------------------------------

def _blocks(n: int, block: int, order: Optional[Sequence[int]]):
    spans = [(a, min(a + block, n)) for a in range(0, n, block)]
    if order is not None:
        spans = [spans[i] for i in order]
    return spans


def online_forward_head(q, k, v, scale: float, block: int = 8,
                        order: Optional[Sequence[int]] = None):
    """One pass with an unnormalised output accumulator.

    For each key block b: S_b = s Q K_b^T; m' = max(m, rowmax S_b);
    alpha = exp(m - m'); P~ = exp(S_b - m'); l = alpha l + rowsum P~;
    U = alpha U + P~ V_b; m = m'.  The rescale by exp(m_old - m_new) of the
    output accumulated so far is the identity of [P3] "兩大核心魔法"
    (e^{x-m_new} = e^{x-m_old} e^{m_old-m_new}).  At the end O = U / l and
    LSE = m + ln l.  Initial state m = -inf, l = 0, U = 0 (exp(-inf) = 0).
    ``order`` permutes the blocks ([P1] fable section 四: the merge does not
    depend on the order the stacks arrive in)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq = q.shape[0]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    U = np.zeros((nq, v.shape[1]))
    for a, b in _blocks(k.shape[0], block, order):
        Sb = float(scale) * (q @ k[a:b].T)
        m_new = np.maximum(m, Sb.max(axis=1))
        alpha = np.exp(m - m_new)
        Pt = np.exp(Sb - m_new[:, None])
        l = alpha * l + Pt.sum(axis=1)
        U = alpha[:, None] * U + Pt @ v[a:b]
        m = m_new
    return U / l[:, None], m + np.log(l)


def online_forward_normalised_head(q, k, v, scale: float, block: int = 8,
                                   order: Optional[Sequence[int]] = None):
    """One pass in which the output is, after every block, the attention
    output over the keys seen so far ([P2] section 六 keeps O normalised this
    way).

    Derivation used here: the keys seen so far carry total weight
    w_old = alpha * l_old against the new reference m' (alpha = exp(m - m')),
    and the new block carries w_b = rowsum P~ with P~ = exp(S_b - m').  The
    output over all of them is the weighted mean of the two partial outputs,
        O = (w_old O_old + w_b A_b) / (w_old + w_b),   A_b = P~ V_b / w_b,
    i.e. the merge of two partial results by their weights (the same rescale
    identity, [P3] "兩大核心魔法").  Written as theta O_old + (1 - theta) A_b
    with theta = w_old / (w_old + w_b), it needs no division by l_old, so the
    first block (l_old = 0, theta = 0) is not a special case."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq = q.shape[0]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    O = np.zeros((nq, v.shape[1]))
    for a, b in _blocks(k.shape[0], block, order):
        Sb = float(scale) * (q @ k[a:b].T)
        m_new = np.maximum(m, Sb.max(axis=1))
        w_old = np.exp(m - m_new) * l
        Pt = np.exp(Sb - m_new[:, None])
        w_b = Pt.sum(axis=1)
        A_b = (Pt @ v[a:b]) / w_b[:, None]
        theta = w_old / (w_old + w_b)
        O = theta[:, None] * O + (1.0 - theta)[:, None] * A_b
        l, m = w_old + w_b, m_new
    return O, m + np.log(l)


def two_pass_forward_head(q, k, v, scale: float, block: int = 8,
                          order: Optional[Sequence[int]] = None):
    """Two passes over the key blocks: the first keeps only the running max
    and running sum (the "two numbers" of [P1] fable section 三), the second
    forms P_b = exp(S_b - m) / l per block and accumulates O += P_b V_b."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq = q.shape[0]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    spans = _blocks(k.shape[0], block, order)
    for a, b in spans:
        Sb = float(scale) * (q @ k[a:b].T)
        m_new = np.maximum(m, Sb.max(axis=1))
        l = np.exp(m - m_new) * l + np.exp(Sb - m_new[:, None]).sum(axis=1)
        m = m_new
    O = np.zeros((nq, v.shape[1]))
    for a, b in spans:
        Sb = float(scale) * (q @ k[a:b].T)
        O += (np.exp(Sb - m[:, None]) / l[:, None]) @ v[a:b]
    return O, m + np.log(l)


# ---------------------------------------------------------------------------
# Split-KV partial results and their merge.
#
# A key range's forward is the plain definition restricted to those keys; the
# merge is the rescale identity of [P3] "兩大核心魔法" (e^{x-m_new} =
# e^{x-m_old} e^{m_old-m_new}) applied to whole ranges: with weights
# e^{LSE_p - LSE}, the ranges' normalised outputs add up to the full one.
# [P1] section 四: accounts kept separately combine without conflict, so the
# order of the parts does not matter.
# ---------------------------------------------------------------------------


def split_bounds(n: int, n_split: int, tile: int) -> list:
    """Key ranges [a, b) of a split forward: the keys are cut into whole
    tiles of ``tile`` keys (the last one may be short), T = ceil(n / tile),
    and range p holds tiles [p*T//n_split, (p+1)*T//n_split) (the rule the
    library's header states for fa_fwd_split)."""
    t = -(-n // tile)
    if not 1 <= n_split <= t:
        raise ValueError("need 1 <= n_split <= number of key tiles")
    out = []
    for p in range(n_split):
        a, b = p * t // n_split, (p + 1) * t // n_split
        out.append((a * tile, min(n, b * tile)))
    return out


def sdpa_split_head(q, k, v, scale: float, bounds) -> Tuple[np.ndarray, np.ndarray]:
    """One head: the plain forward on each key range.  Returns (O_parts
    [P, Nq, dv], LSE_parts [P, Nq])."""
    outs = [sdpa_forward_head(q, _f64(k)[a:b], _f64(v)[a:b], scale) for a, b in bounds]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def merge_parts(o_parts, lse_parts) -> Tuple[np.ndarray, np.ndarray]:
    """Merge of partial results over the leading axis.  o_parts [P, ..., dv],
    lse_parts [P, ...].  LSE = m + ln sum_p e^{LSE_p - m} (m = max_p LSE_p) and
    O = sum_p e^{LSE_p - LSE} O_p.  A part with LSE_p = -inf has weight 0 and
    is skipped (whatever its O_p); rows whose parts are all -inf get O = 0 and
    LSE = -inf."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    m = lse_parts.max(axis=0)
    has = m > -np.inf                      # rows with at least one live part
    m0 = np.where(has, m, 0.0)
    total = np.zeros(m.shape)
    for p in range(lse_parts.shape[0]):
        total += np.exp(lse_parts[p] - m0)   # exp(-inf) = 0
    lse = np.where(has, m0 + np.log(np.where(has, total, 1.0)), -np.inf)
    o = np.zeros(o_parts.shape[1:])
    for p in range(o_parts.shape[0]):
        live = lse_parts[p] > -np.inf
        w = np.where(live, np.exp(lse_parts[p] - np.where(has, lse, 0.0)), 0.0)
        o += w[..., None] * np.where(live[..., None], o_parts[p], 0.0)
    return o, lse
