"""Pins for the CPU oracle (runs without a GPU).

Each check ties the oracle to something other than itself: closed forms,
a worked example done by hand, brute force in pure Python, invariants that
follow from the softmax definition, finite differences, and torch's own
float64 CPU attention with autograd.  The planted-mistake tests at the end
show that a plausible error anywhere in the oracle (a dropped term, a wrong
sign, a transposed operand, a missing scale) fails at least one check.

Pages: [P1] 算珠楼的掌簿人; [P2] 账房先生的奔命：Flash Attention 与内存 I/O
革命; [P3] the star-observatory FlashAttention fable (概念揭曉 section).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# Check functions, written so that they can also be run against mutants of the
# oracle.  Each returns a list of failure strings (empty = pass).
# ---------------------------------------------------------------------------

def _fwd_checks(fwd_head, online_heads=()):
    """Forward pins.  fwd_head(q,k,v,scale) -> (O, LSE)."""
    fails = []
    s = 0.37
    # (1) hand-worked example ([P3] 概念揭曉 formula; [P2] section 六 softmax)
    g = json.load(open(os.path.join(GOLDEN, "hand_worked.json")))
    ln3 = math.log(3.0)
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [ln3, 0.0]])
    v = np.array(g["v"])
    O, L = fwd_head(q, k, v, 1.0)
    if not np.allclose(O, g["O"], rtol=0, atol=1e-14):
        fails.append("hand-worked O")
    if abs(L[0] - math.log(4.0)) > 1e-14:
        fails.append("hand-worked LSE")
    # (2) Q = 0: every score is 0, P uniform, O = column mean of V, LSE = ln N
    q = np.zeros((5, 6)); k = rnd((7, 6), 1); v = rnd((7, 3), 2)
    O, L = fwd_head(q, k, v, s)
    if np.abs(O - v.mean(0)).max() > 1e-13 or np.abs(L - math.log(7)).max() > 1e-13:
        fails.append("Q=0 closed form")
    # (3) dominant key: q_i = a e_0 for all i, k_j* = a e_0 large, other keys
    # orthogonal to e_0 -> O_i = V_j*, LSE_i = S_ij* up to (N-1) e^-delta
    n, d = 6, 8
    a = math.sqrt(100.0 / s)
    q = np.zeros((4, d)); q[:, 0] = a
    k = np.zeros((n, d)); k[:, 1:] = rnd((n, d - 1), 3)
    jstar = 4
    k[jstar, 0] = a
    v = rnd((n, 5), 4)
    O, L = fwd_head(q, k, v, s)
    delta = 100.0
    bound = (n - 1) * math.exp(-delta) * 2 * np.abs(v).max() + 1e-13
    if np.abs(O - v[jstar]).max() > bound:
        fails.append("dominant key O")
    if np.abs(L - s * a * a).max() > 1e-12:
        fails.append("dominant key LSE")
    # (4) N = 1: O = V_0, LSE = s q.k_0
    q = rnd((3, 4), 5); k = rnd((1, 4), 6); v = rnd((1, 2), 7)
    O, L = fwd_head(q, k, v, s)
    if np.abs(O - v[0]).max() > 1e-15 or np.abs(L - s * (q @ k[0])).max() > 1e-14:
        fails.append("N=1")
    # (5) brute force in pure Python at N <= 8, d <= 4
    for seed, (nq, nk, dd) in enumerate([(3, 5, 4), (8, 8, 4), (2, 7, 3)]):
        q = rnd((nq, dd), 10 + seed); k = rnd((nk, dd), 20 + seed); v = rnd((nk, dd), 30 + seed)
        Ob, Lb = brute.brute_forward(q.tolist(), k.tolist(), v.tolist(), s)
        O, L = fwd_head(q, k, v, s)
        if np.abs(O - np.array(Ob)).max() > 1e-13 or np.abs(L - np.array(Lb)).max() > 1e-13:
            fails.append(f"brute force {nq}x{nk}x{dd}")
    # (6) invariants on a random problem
    q = rnd((9, 5), 40); k = rnd((11, 5), 41); v = rnd((11, 4), 42)
    O, L = fwd_head(q, k, v, s)
    S = s * q @ k.T
    u = rnd(5, 43)
    O2, L2 = fwd_head(q, k + u, v, s)           # key shift
    if np.abs(O2 - O).max() > 1e-12 or np.abs(L2 - (L + s * q @ u)).max() > 1e-12:
        fails.append("key shift")
    perm = np.random.default_rng(44).permutation(11)
    O3, L3 = fwd_head(q, k[perm], v[perm], s)    # permute keys with values
    if np.abs(O3 - O).max() > 1e-12 or np.abs(L3 - L).max() > 1e-12:
        fails.append("key permutation")
    qp = np.random.default_rng(45).permutation(9)
    O4, _ = fwd_head(q[qp], k, v, s)             # permute queries
    if np.abs(O4 - O[qp]).max() > 1e-12:
        fails.append("query permutation")
    v2 = rnd((11, 4), 46)
    O5, _ = fwd_head(q, k, 2.0 * v - 3.0 * v2, s)  # linear in V
    O6, _ = fwd_head(q, k, v2, s)
    if np.abs(O5 - (2.0 * O - 3.0 * O6)).max() > 1e-12:
        fails.append("linearity in V")
    if (L < S.max(1) - 1e-12).any() or (L > S.max(1) + math.log(11) + 1e-12).any():
        fails.append("LSE bounds")
    # (7) torch float64 CPU attention (a library routine, not used by the oracle)
    for (nq, nk, d, dv) in [(16, 16, 8, 8), (5, 13, 7, 3)]:
        q = rnd((nq, d), 50); k = rnd((nk, d), 51); v = rnd((nk, dv), 52)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
            torch.from_numpy(v)[None, None], scale=s)[0, 0].numpy()
        lse_ref = torch.logsumexp(torch.from_numpy(s * q @ k.T), dim=-1).numpy()
        O, L = fwd_head(q, k, v, s)
        if np.abs(O - ref).max() > 1e-13 or np.abs(L - lse_ref).max() > 1e-13:
            fails.append(f"torch sdpa {nq}x{nk}")
    # (8) online forms agree with the one-shot definition
    for oh in online_heads:
        q = rnd((10, 6), 60); k = rnd((19, 6), 61, 2.0); v = rnd((19, 5), 62)
        O, L = fwd_head(q, k, v, s)
        for block in (1, 8, 19):
            nb = -(-19 // block)
            for order in (None, list(range(nb))[::-1],
                          list(np.random.default_rng(block).permutation(nb))):
                O1, L1 = oh(q, k, v, s, block=block, order=order)
                if np.abs(O1 - O).max() > 1e-12 or np.abs(L1 - L).max() > 1e-12:
                    fails.append(f"online {oh.__name__} block={block}")
    return fails


def _bwd_checks(bwd_head):
    """Backward pins.  bwd_head(q,k,v,dO,scale) -> dict(dQ, dK, dV, ...)."""
    fails = []
    # (1) hand-worked example
    g = json.load(open(os.path.join(GOLDEN, "hand_worked.json")))
    ln3 = math.log(3.0)
    q = np.array([[1.0, 0.0]]); k = np.array([[0.0, 0.0], [ln3, 0.0]])
    v = np.array(g["v"]); dO = np.array(g["dO"])
    r = bwd_head(q, k, v, dO, 1.0)
    if np.abs(r["dQ"] - np.array([[0.75 * ln3, 0.0]])).max() > 1e-14:
        fails.append("hand-worked dQ")
    if np.abs(r["dK"] - np.array(g["dK"])).max() > 1e-14:
        fails.append("hand-worked dK")
    if np.abs(r["dV"] - np.array(g["dV"])).max() > 1e-14:
        fails.append("hand-worked dV")
    # (2) central finite differences on L = sum(O * G) at N = 8, d in {4, 8}
    s = 0.41
    for d in (4, 8):
        q = rnd((8, d), 70 + d); k = rnd((8, d), 71 + d); v = rnd((8, d), 72 + d)
        G = rnd((8, d), 73 + d)
        r = bwd_head(q, k, v, G, s)

        def loss(qq, kk, vv):
            O, _ = A.sdpa_forward_head(qq, kk, vv, s)
            return float((O * G).sum())

        h = 1e-6
        for name, X, idx in (("dQ", q, 0), ("dK", k, 1), ("dV", v, 2)):
            num = np.zeros_like(X)
            for pos in np.ndindex(X.shape):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[idx][pos] += h
                args_m[idx][pos] -= h
                num[pos] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            rel = np.linalg.norm(r[name] - num) / np.linalg.norm(num)
            if rel > 1e-7:
                fails.append(f"finite differences {name} d={d} rel={rel:.2e}")
    # (3) brute force
    q = rnd((4, 3), 80); k = rnd((6, 3), 81); v = rnd((6, 2), 82); G = rnd((4, 2), 83)
    bq, bk, bv = brute.brute_backward(q.tolist(), k.tolist(), v.tolist(), G.tolist(), s)
    r = bwd_head(q, k, v, G, s)
    for name, ref in (("dQ", bq), ("dK", bk), ("dV", bv)):
        if np.abs(r[name] - np.array(ref)).max() > 1e-13:
            fails.append(f"brute force {name}")
    # (4) identities that follow from rows of P summing to one
    q = rnd((9, 5), 90); k = rnd((12, 5), 91); v = rnd((12, 4), 92); G = rnd((9, 4), 93)
    r = bwd_head(q, k, v, G, s)
    if np.abs(r["dK"].sum(0)).max() > 1e-12:
        fails.append("sum_j dK_j = 0")
    if np.abs(r["dV"].sum(0) - G.sum(0)).max() > 1e-12:
        fails.append("sum_j dV_j = sum_i dO_i")
    if "dS" in r and np.abs(r["dS"].sum(1)).max() > 1e-12:
        fails.append("rowsum dS = 0")
    if "D" in r and "P" in r and np.abs(r["D"] - (r["P"] * r["dP"]).sum(1)).max() > 1e-12:
        fails.append("D = rowsum(P * dP)")
    # (5) Q = 0: dK is exactly zero, dV_j = mean_i dO_i
    q = np.zeros((6, 4)); k = rnd((7, 4), 94); v = rnd((7, 3), 95); G = rnd((6, 3), 96)
    r = bwd_head(q, k, v, G, s)
    if np.any(r["dK"] != 0.0):
        fails.append("Q=0 dK exactly 0")
    if np.abs(r["dV"] - G.sum(0) / 7.0).max() > 1e-13:
        fails.append("Q=0 dV")
    # (6) torch float64 autograd through its own attention
    q = rnd((10, 6), 100); k = rnd((14, 6), 101); v = rnd((14, 5), 102); G = rnd((10, 5), 103)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None],
                                                           tv[None, None], scale=s)[0, 0]
    out.backward(torch.from_numpy(G))
    r = bwd_head(q, k, v, G, s)
    for name, t in (("dQ", tq), ("dK", tk), ("dV", tv)):
        if np.abs(r[name] - t.grad.numpy()).max() > 1e-12:
            fails.append(f"torch autograd {name}")
    return fails


# ---------------------------------------------------------------------------
# The oracle itself passes every pin.
# ---------------------------------------------------------------------------

def test_forward_pins():
    assert _fwd_checks(A.sdpa_forward_head,
                       online_heads=(A.online_forward_head,
                                     A.online_forward_normalised_head,
                                     A.two_pass_forward_head)) == []


def test_backward_pins():
    assert _bwd_checks(A.sdpa_backward_head) == []


def test_softmax_rows_sum_to_one():
    S = rnd((17, 33), 1, 20.0)
    P, m, l = A.softmax_rows(S)
    assert np.abs(P.sum(1) - 1.0).max() <= 1e-13
    assert (P >= 0).all()
    assert np.abs(m - S.max(1)).max() == 0.0


def test_online_block8_on_the_64_row_example():
    # [P1] fable section 二: 64 rows cut into 8 stacks of 8, merged stack by
    # stack; and the tiny workload is described with that block size.
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["items"][0]
    w = synth.WORKLOADS["tiny_f32_n64_d64"]
    assert w.N == g["n"] and w.block == g["block"] and w.N // w.block == g["blocks"]
    assert w.N * w.N == g["cells"] and w.block * w.block == g["tile_cells"]
    q, k, v, _ = synth.make_inputs(w)
    q, k, v = (synth.to_f64(t)[0, 0] for t in (q, k, v))
    O, L = A.sdpa_forward_head(q, k, v, w.scale)
    for fn in (A.online_forward_head, A.online_forward_normalised_head,
               A.two_pass_forward_head):
        O1, L1 = fn(q, k, v, w.scale, block=w.block)
        assert np.abs(O1 - O).max() <= 1e-12
        assert np.abs(L1 - L).max() <= 1e-12


def test_page_size_numbers():
    items = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))["items"]
    s_bytes = items[1]
    assert s_bytes["n"] ** 2 * s_bytes["bytes_per_score"] == s_bytes["bytes"]
    assert round(s_bytes["bytes"] / 1e6) == s_bytes["printed_mb"]
    trips = items[2]
    assert 2 * trips["n"] ** 2 == trips["round_trips"]
    assert abs(trips["round_trips"] - trips["printed"]) / trips["printed"] < 0.05


def test_batched_wrappers_match_per_head():
    q = rnd((2, 3, 9, 4), 1); k = rnd((2, 3, 9, 4), 2); v = rnd((2, 3, 9, 4), 3)
    G = rnd((2, 3, 9, 4), 4)
    O, L = A.sdpa_forward(q, k, v, 0.5)
    dQ, dK, dV, D = A.sdpa_backward(q, k, v, G, 0.5)
    for b in range(2):
        for h in range(3):
            Oh, Lh = A.sdpa_forward_head(q[b, h], k[b, h], v[b, h], 0.5)
            r = A.sdpa_backward_head(q[b, h], k[b, h], v[b, h], G[b, h], 0.5)
            assert np.array_equal(O[b, h], Oh) and np.array_equal(L[b, h], Lh)
            assert np.array_equal(dQ[b, h], r["dQ"]) and np.array_equal(D[b, h], r["D"])
    # a head subset leaves the rest as NaN
    O2, _ = A.sdpa_forward(q, k, v, 0.5, heads=[1])
    assert np.isnan(O2[0, 0]).all() and np.array_equal(O2[0, 1], O[0, 1])


def test_rows_subset_matches_full():
    q = rnd((50, 8), 1); k = rnd((40, 8), 2); v = rnd((40, 8), 3)
    O, L = A.sdpa_forward_head(q, k, v, 0.3)
    rows = [0, 7, 49]
    Or, Lr = A.sdpa_rows(q[rows], k, v, 0.3)
    assert np.abs(Or - O[rows]).max() <= 1e-15 and np.abs(Lr - L[rows]).max() <= 1e-15


def test_outlier_variant_and_large_scores():
    # an outlier key scaled by 8 (the long workload's variant) keeps the
    # online forms exact: the running max jumps late and everything before it
    # is rescaled
    q = rnd((12, 16), 1); k = rnd((64, 16), 2); v = rnd((64, 16), 3)
    k[45] *= 8.0
    s = 0.25
    O, L = A.sdpa_forward_head(q, k, v, s)
    O1, L1 = A.online_forward_head(q, k, v, s, block=8)
    assert np.abs(O1 - O).max() <= 1e-12 and np.abs(L1 - L).max() <= 1e-12
    # scores far beyond exp's range still give finite results (max subtracted)
    O2, L2 = A.sdpa_forward_head(q * 100, k, v, s)
    assert np.isfinite(O2).all() and np.isfinite(L2).all()


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one pin.
# ---------------------------------------------------------------------------

def _mut_no_scale(q, k, v, s):
    return A.sdpa_forward_head(q, k, v, 1.0)


def _mut_transposed_p(q, k, v, s):
    S = s * np.asarray(q) @ np.asarray(k).T
    P, m, l = A.softmax_rows(S)
    n = min(P.shape)
    P2 = P.copy(); P2[:n, :n] = P[:n, :n].T
    return P2 @ v, m + np.log(l)


def _mut_lse_without_max(q, k, v, s):
    S = s * np.asarray(q) @ np.asarray(k).T
    P, m, l = A.softmax_rows(S)
    return P @ v, np.log(l)


def _mut_sum_includes_max_twice(q, k, v, s):
    S = s * np.asarray(q) @ np.asarray(k).T
    m = S.max(1)
    E = np.exp(S - m[:, None])
    l = E.sum(1) + 1.0          # an extra term in the denominator
    return (E / l[:, None]) @ v, m + np.log(l)


def _mut_online_no_rescale(q, k, v, s, block=8, order=None):
    # forgets to rescale the accumulated output when the max moves
    q, k, v = map(np.asarray, (q, k, v))
    m = np.full(q.shape[0], -np.inf); l = np.zeros(q.shape[0]); U = np.zeros((q.shape[0], v.shape[1]))
    for a, b in A._blocks(k.shape[0], block, order):
        Sb = s * q @ k[a:b].T
        m_new = np.maximum(m, Sb.max(1))
        alpha = np.exp(m - m_new)
        Pt = np.exp(Sb - m_new[:, None])
        l = alpha * l + Pt.sum(1)
        U = U + Pt @ v[a:b]
        m = m_new
    return U / l[:, None], m + np.log(l)


FWD_MUTANTS = [_mut_no_scale, _mut_transposed_p, _mut_lse_without_max,
               _mut_sum_includes_max_twice]


@pytest.mark.parametrize("mutant", FWD_MUTANTS, ids=lambda f: f.__name__)
def test_planted_forward_mistake_is_caught(mutant):
    assert _fwd_checks(mutant) != []


def test_planted_online_mistake_is_caught():
    assert _fwd_checks(A.sdpa_forward_head, online_heads=(_mut_online_no_rescale,)) != []


def _bwd_mutant(change):
    def f(q, k, v, dO, s):
        r = A.sdpa_backward_head(q, k, v, dO, s)
        q, k, v, dO = map(np.asarray, (q, k, v, dO))
        P, dP, D = r["P"], r["dP"], r["D"]
        if change == "drop_D":
            dS = P * dP
        elif change == "sign_D":
            dS = P * (dP + D[:, None])
        else:
            dS = r["dS"]
        out = dict(r)
        out["dS"] = dS
        out["dQ"] = s * dS @ k
        out["dK"] = s * dS.T @ q
        if change == "dK_untransposed":
            n = min(dS.shape)
            out["dK"] = out["dK"].copy()
            out["dK"][:n] = s * (dS[:n, :n] @ q[:n])
        if change == "dV_no_transpose":
            n = min(P.shape)
            out["dV"] = r["dV"].copy()
            out["dV"][:n] = P[:n, :n] @ dO[:n]
        if change == "dQ_no_scale":
            out["dQ"] = dS @ k
        return out
    f.__name__ = change
    return f


@pytest.mark.parametrize("change", ["drop_D", "sign_D", "dK_untransposed",
                                    "dV_no_transpose", "dQ_no_scale"])
def test_planted_backward_mistake_is_caught(change):
    assert _bwd_checks(_bwd_mutant(change)) != []


# ---------------------------------------------------------------------------
# Split-KV parts and their merge ([P3] "兩大核心魔法" rescale identity applied
# to whole key ranges; [P1] section 四: the ranges combine in any order).
# ---------------------------------------------------------------------------

def _merge_checks(merge, split_head=A.sdpa_split_head):
    """Merge pins.  merge(o_parts, lse_parts) -> (O, LSE)."""
    bad = []
    # 1. Hand-worked: two parts with LSE ln 2 and ln 6 -> LSE ln 8, weights
    #    2/8 and 6/8.
    o, l = merge(np.array([[[1.0, 0.0]], [[0.0, 1.0]]]), np.array([[math.log(2)], [math.log(6)]]))
    if abs(l[0] - math.log(8)) > 1e-15 or np.abs(o[0] - [0.25, 0.75]).max() > 1e-15:
        bad.append("hand-worked two-part merge")
    # 2. The merge of the parts equals the plain forward on all keys, for
    #    ragged N and every split count (closed-form identity, no tolerance
    #    beyond float64 rounding).
    for n, tile in ((37, 8), (64, 8), (9, 4)):
        q, k, v = rnd((5, 6), 1), rnd((n, 6), 2, 1.5), rnd((n, 3), 3)
        O, L = A.sdpa_forward_head(q, k, v, 0.4)
        for p in range(1, -(-n // tile) + 1):
            op, lp = split_head(q, k, v, 0.4, A.split_bounds(n, p, tile))
            o, l = merge(op, lp)
            if np.abs(o - O).max() > 1e-12 or np.abs(l - L).max() > 1e-12:
                bad.append(f"merge of {p} parts != full forward (n={n})")
                break
    # 3. Order of the parts does not matter.
    op, lp = A.sdpa_split_head(rnd((4, 5), 4), rnd((40, 5), 5), rnd((40, 5), 6), 0.7,
                               A.split_bounds(40, 5, 8))
    perm = [3, 0, 4, 2, 1]
    o1, l1 = merge(op, lp)
    o2, l2 = merge(op[perm], lp[perm])
    if np.abs(o1 - o2).max() > 1e-13 or np.abs(l1 - l2).max() > 1e-13:
        bad.append("merge depends on the order of the parts")
    # 4. One part: identity.
    o, l = merge(op[:1], lp[:1])
    if np.abs(o - op[0]).max() > 0 or np.abs(l - lp[0]).max() > 0:
        bad.append("single-part merge is not the identity")
    # 5. A part with LSE = -inf contributes nothing, whatever its O holds.
    o, l = merge(np.array([[[np.nan, 7.0]], [[0.5, 1.0]]]), np.array([[-np.inf], [0.3]]))
    if not (np.isfinite(o).all() and np.abs(o[0] - [0.5, 1.0]).max() == 0 and l[0] == 0.3):
        bad.append("-inf part not skipped")
    return bad


def test_merge_pins():
    assert _merge_checks(A.merge_parts) == []


def test_split_bounds_rule():
    # Whole tiles, every range non-empty, ranges cover [0, N) in order.
    for n, tile in ((8192, 128), (1000, 64), (1, 128), (129, 128)):
        t = -(-n // tile)
        for p in range(1, t + 1):
            b = A.split_bounds(n, p, tile)
            assert b[0][0] == 0 and b[-1][1] == n
            assert all(x[1] == y[0] for x, y in zip(b, b[1:]))
            assert all(a < c for a, c in b)
            assert all(a % tile == 0 for a, _ in b)
    with pytest.raises(ValueError):
        A.split_bounds(100, 0, 64)
    with pytest.raises(ValueError):
        A.split_bounds(100, 3, 64)


def _mut_merge_plain_average(o_parts, lse_parts):
    o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
    m = lse_parts.max(axis=0)
    return o_parts.mean(axis=0), m + np.log(np.exp(lse_parts - m).sum(axis=0))


def _mut_merge_weights_unnormalised(o_parts, lse_parts):
    o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m)
    return (w[..., None] * o_parts).sum(axis=0), m + np.log(w.sum(axis=0))


def _mut_merge_lse_max_only(o_parts, lse_parts):
    o, _ = A.merge_parts(o_parts, lse_parts)
    return o, np.asarray(lse_parts, float).max(axis=0)


@pytest.mark.parametrize("mutant", [_mut_merge_plain_average, _mut_merge_weights_unnormalised,
                                    _mut_merge_lse_max_only], ids=lambda f: f.__name__)
def test_planted_merge_mistake_is_caught(mutant):
    assert _merge_checks(mutant) != []


# ---------------------------------------------------------------------------
# The backward restricted to selected query rows (dQ on sampled rows of very
# long sequences): row i of dQ depends only on q_i, dO_i and all keys.
# ---------------------------------------------------------------------------

def _rows_bwd_checks(rows_fn):
    """rows_fn(q_rows, k, v, dO_rows, scale) -> (dQ_rows, D_rows)."""
    bad = []
    # 1. Hand-worked example: dQ = [[3/4 ln 3, 0]].
    g = json.load(open(os.path.join(GOLDEN, "hand_worked.json")))
    ln3 = math.log(3.0)
    dq, _ = rows_fn(np.array([[1.0, 0.0]]), np.array([[0.0, 0.0], [ln3, 0.0]]),
                    np.array(g["v"]), np.array(g["dO"]), 1.0)
    if np.abs(dq - np.array([[0.75 * ln3, 0.0]])).max() > 1e-14:
        bad.append("hand-worked dQ")
    # 2. torch float64 autograd through its own attention, on a row subset.
    q = rnd((10, 6), 110); k = rnd((14, 6), 111); v = rnd((14, 5), 112); G = rnd((10, 5), 113)
    s = 0.41
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None],
                                                           tv[None, None], scale=s)[0, 0]
    out.backward(torch.from_numpy(G))
    rows = [0, 4, 9]
    dq, D = rows_fn(q[rows], k, v, G[rows], s)
    if np.abs(dq - tq.grad.numpy()[rows]).max() > 1e-12:
        bad.append("torch autograd dQ rows")
    O = out.detach().numpy()
    if np.abs(D - (G[rows] * O[rows]).sum(1)).max() > 1e-12:
        bad.append("D = rowsum(dO * O)")
    # 3. Q = 0 closed form: P uniform, dP_ij = dO_i . v_j, so
    #    dQ_i = s (1/N) sum_j (dO_i . (v_j - vbar)) k_j.
    k = rnd((7, 4), 114); v = rnd((7, 3), 115); G = rnd((2, 3), 116)
    dq, _ = rows_fn(np.zeros((2, 4)), k, v, G, s)
    ref = s / 7.0 * ((G @ (v - v.mean(0)).T) @ k)
    if np.abs(dq - ref).max() > 1e-13:
        bad.append("Q=0 dQ closed form")
    return bad


def test_backward_rows_pins():
    assert _rows_bwd_checks(A.sdpa_backward_rows) == []


def test_backward_rows_match_full_backward():
    q = rnd((40, 8), 1); k = rnd((33, 8), 2); v = rnd((33, 8), 3); G = rnd((40, 8), 4)
    r = A.sdpa_backward_head(q, k, v, G, 0.3)
    rows = [0, 7, 21, 39]
    dq, D = A.sdpa_backward_rows(q[rows], k, v, G[rows], 0.3)
    assert np.abs(dq - r["dQ"][rows]).max() <= 1e-14
    assert np.abs(D - r["D"][rows]).max() <= 1e-14


def _mut_rows(change):
    def f(q, k, v, dO, s):
        q, k, v, dO = map(np.asarray, (q, k, v, dO))
        P, _, _ = A.softmax_rows(s * (q @ k.T))
        D = (dO * (P @ v)).sum(1)
        dP = dO @ v.T
        if change == "drop_D":
            dS = P * dP
        elif change == "D_of_dO_only":
            D = dO.sum(1)
            dS = P * (dP - D[:, None])
        else:
            dS = P * (dP - D[:, None])
        return (dS @ k if change == "no_scale" else s * (dS @ k)), D
    f.__name__ = change
    return f


@pytest.mark.parametrize("change", ["drop_D", "D_of_dO_only", "no_scale"])
def test_planted_rows_mistake_is_caught(change):
    assert _rows_bwd_checks(_mut_rows(change)) != []


def _mut_normalised_without_rescale(q, k, v, s, block=8, order=None):
    # mixes the old output by l_old instead of exp(m - m') * l_old
    q, k, v = map(np.asarray, (q, k, v))
    m = np.full(q.shape[0], -np.inf); l = np.zeros(q.shape[0]); O = np.zeros((q.shape[0], v.shape[1]))
    for a, b in A._blocks(k.shape[0], block, order):
        Sb = s * q @ k[a:b].T
        m_new = np.maximum(m, Sb.max(1))
        Pt = np.exp(Sb - m_new[:, None])
        w_b = Pt.sum(1)
        theta = l / (l + w_b)
        O = theta[:, None] * O + (1.0 - theta)[:, None] * ((Pt @ v[a:b]) / w_b[:, None])
        l, m = l + w_b, m_new
    return O, m + np.log(l)


def test_planted_normalised_online_mistake_is_caught():
    assert _fwd_checks(A.sdpa_forward_head,
                       online_heads=(_mut_normalised_without_rescale,)) != []
