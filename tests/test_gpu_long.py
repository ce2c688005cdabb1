"""GPU parity at the sequence lengths of the N sweep (B=1, H=16, d=128, bf16,
seed N: the inputs `bench.py --sweep` times), through the C ABI.

N = 16384: forward and backward against the full fp64 oracle on two heads
(each head is independent; the GPU runs all sixteen).  N = 32768 ... 131072:
the oracle cannot form N x N per head in seconds, so O, LSE and dQ are
compared on 256 sampled query rows per head against all keys (a row of O or
dQ depends only on its own query row and every key), and dK, dV are checked
through two identities that hold at any size because every row of P sums to
one: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i.

Tolerances: the stated bf16 bounds (O max-abs 1e-2, mean-abs 1e-3, LSE
max-abs 1e-3, gradients relative Frobenius 2e-2); O also within 2e-2
relative Frobenius; for the identities, the norm of the residual at most 2e-2
of the gradient's Frobenius norm (with independent per-row errors e_j the
residual sum_j e_j has norm about ||e||_F, so this is the relative-Frobenius
bound carried over).
"""

import math

import numpy as np
import pytest
import torch

import io_aware_softmax_02_amd as fa
import oracle
import synth
from _compare import (TOL_BF16_GRAD_REL, TOL_BF16_LSE_MAX, TOL_BF16_O_MAX, TOL_BF16_O_MEAN,
                      max_abs, mean_abs, rel_frobenius)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D_HEAD = 128


def say(msg):
    print(msg, flush=True)


def f64(t):
    return synth.to_f64(t)


def run(N):
    q, k, v, dO = synth.sweep_inputs(N)
    qg, kg, vg, gg = (x.to(DEV) for x in (q, k, v, dO))
    s = synth.default_scale(D_HEAD)
    O, L = fa.fa_fwd(qg, kg, vg, s)
    dq, dk, dv = fa.fa_bwd(qg, kg, vg, O, L, gg, s)
    torch.cuda.synchronize()
    return (q, k, v, dO), (gg, O, L, dq, dk, dv), s


def test_n16384_full_oracle_two_heads():
    N = 16384
    say(f"case sweep N={N}: fwd+bwd, heads 0 and 15 against the full oracle")
    (q, k, v, dO), (_, O, L, dq, dk, dv), s = run(N)
    for h in (0, 15):
        qh, kh, vh, gh = (f64(x[0, h]) for x in (q, k, v, dO))
        Oref, Lref = oracle.sdpa_forward_head(qh, kh, vh, s)
        o, l = f64(O[0, h].cpu()), f64(L[0, h].cpu())
        ma, mn, ml = max_abs(o, Oref), mean_abs(o, Oref), max_abs(l, Lref)
        ro = rel_frobenius(o, Oref)
        say(f"  head {h}: O max-abs {ma:.3e} mean-abs {mn:.3e} rel {ro:.3e}; LSE max-abs {ml:.3e}")
        assert ma <= TOL_BF16_O_MAX and mn <= TOL_BF16_O_MEAN and ml <= TOL_BF16_LSE_MAX
        assert ro <= 2e-2
        r = oracle.sdpa_backward_head(qh, kh, vh, gh, s)
        for name, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
            e = rel_frobenius(f64(x[0, h].cpu()), r[name])
            say(f"  head {h}: {name} rel-Frobenius {e:.3e}")
            assert e <= TOL_BF16_GRAD_REL, name
        del r


@pytest.mark.parametrize("N", [32768, 65536, 131072])
def test_long_sampled_rows_and_gradient_identities(N):
    rows_per_head = 256
    say(f"case sweep N={N}: O, LSE, dQ on {rows_per_head} sampled rows per head; "
        f"dK, dV identities")
    (q, k, v, dO), (gg, O, L, dq, dk, dv), s = run(N)
    H = q.shape[1]
    rows = synth.draw_rows(N, H, rows_per_head, seed=N)
    worst = dict(o_max=0.0, o_mean=0.0, lse=0.0)
    sq = {"o": [0.0, 0.0], "dq": [0.0, 0.0]}
    for h in range(H):
        r = rows[h]
        qh, kh, vh, gh = (f64(x[0, h]) for x in (q, k, v, dO))
        Oref, Lref = oracle.sdpa_rows(qh[r], kh, vh, s)
        dQref, _ = oracle.sdpa_backward_rows(qh[r], kh, vh, gh[r], s)
        ridx = torch.from_numpy(r).to(DEV)
        o = f64(O[0, h].index_select(0, ridx).cpu())
        l = f64(L[0, h].index_select(0, ridx).cpu())
        g = f64(dq[0, h].index_select(0, ridx).cpu())
        worst["o_max"] = max(worst["o_max"], max_abs(o, Oref))
        worst["o_mean"] = max(worst["o_mean"], mean_abs(o, Oref))
        worst["lse"] = max(worst["lse"], max_abs(l, Lref))
        for key, x, ref in (("o", o, Oref), ("dq", g, dQref)):
            sq[key][0] += float(((x - ref) ** 2).sum())
            sq[key][1] += float((ref ** 2).sum())
    rel_o = math.sqrt(sq["o"][0] / sq["o"][1])
    rel_dq = math.sqrt(sq["dq"][0] / sq["dq"][1])
    say(f"  sampled rows: O max-abs {worst['o_max']:.3e} mean-abs {worst['o_mean']:.3e} "
        f"rel {rel_o:.3e}; LSE max-abs {worst['lse']:.3e}; dQ rel-Frobenius {rel_dq:.3e}")
    assert worst["o_max"] <= TOL_BF16_O_MAX and worst["o_mean"] <= TOL_BF16_O_MEAN
    assert worst["lse"] <= TOL_BF16_LSE_MAX
    assert rel_o <= 2e-2
    assert rel_dq <= TOL_BF16_GRAD_REL
    # Identities over all keys of every head (float64 on the device).
    dk64, dv64, g64 = dk.double()[0], dv.double()[0], gg.double()[0]
    for h in range(H):
        res_k = float(dk64[h].sum(0).norm() / dk64[h].norm())
        res_v = float((dv64[h].sum(0) - g64[h].sum(0)).norm() / dv64[h].norm())
        if h in (0, H - 1):
            say(f"  head {h}: |sum dK| / ||dK|| {res_k:.3e}; "
                f"|sum dV - sum dO| / ||dV|| {res_v:.3e}")
        assert res_k <= TOL_BF16_GRAD_REL, ("dK", h)
        assert res_v <= TOL_BF16_GRAD_REL, ("dV", h)


def test_heads_beyond_4gib_offsets():
    """B=2, H=136, N=65536, d=128: each tensor is 4.6 GB, so the last head's
    rows start 4.55 GB past the base pointer (64-bit per-head offsets in
    every kernel).  O, LSE and dQ of the first and the last head on 64
    sampled rows against the oracle, and the dK/dV identities on both."""
    B, H, N, d = 2, 136, 65536, 128
    print(f"case heads past 4 GiB: B={B} H={H} N={N} d={d}", flush=True)
    q, k, v, dO = synth.make_qkv(B, H, N, d, torch.bfloat16, seed=1500, backward=True,
                                 device=DEV)
    s = synth.default_scale(d)
    O, L = fa.fa_fwd(q, k, v, s)
    dq, dk, dv = fa.fa_bwd(q, k, v, O, L, dO, s)
    torch.cuda.synchronize()
    assert (B * H - 1) * N * d * 2 > (1 << 32)
    rows = synth.draw_rows(N, 2, 64, seed=1500)
    for idx, (b, h) in enumerate(((0, 0), (B - 1, H - 1))):
        r = rows[idx]
        ridx = torch.from_numpy(r).to(DEV)
        qh, kh, vh, gh = (f64(x[b, h].cpu()) for x in (q, k, v, dO))
        Oref, Lref = oracle.sdpa_rows(qh[r], kh, vh, s)
        dQref, _ = oracle.sdpa_backward_rows(qh[r], kh, vh, gh[r], s)
        o = f64(O[b, h].index_select(0, ridx).cpu())
        l = f64(L[b, h].index_select(0, ridx).cpu())
        g = f64(dq[b, h].index_select(0, ridx).cpu())
        ma, mn, ml = max_abs(o, Oref), mean_abs(o, Oref), max_abs(l, Lref)
        rel_o, rel_dq = rel_frobenius(o, Oref), rel_frobenius(g, dQref)
        say(f"  head ({b},{h}): O max-abs {ma:.3e} mean-abs {mn:.3e} rel {rel_o:.3e}; "
            f"LSE max-abs {ml:.3e}; dQ rel-Frobenius {rel_dq:.3e}")
        assert ma <= TOL_BF16_O_MAX and mn <= TOL_BF16_O_MEAN and ml <= TOL_BF16_LSE_MAX
        assert rel_o <= 2e-2 and rel_dq <= TOL_BF16_GRAD_REL
        dk64, dv64, g64 = dk[b, h].double(), dv[b, h].double(), dO[b, h].double()
        res_k = float(dk64.sum(0).norm() / dk64.norm())
        res_v = float((dv64.sum(0) - g64.sum(0)).norm() / dv64.norm())
        say(f"  head ({b},{h}): |sum dK| / ||dK|| {res_k:.3e}; |sum dV - sum dO| / ||dV|| {res_v:.3e}")
        assert res_k <= TOL_BF16_GRAD_REL and res_v <= TOL_BF16_GRAD_REL


def test_d64_long_sequence_sampled_rows():
    """The d = 64 kernels at N = 65536 (B=1, H=4, ragged by 37 keys): O, LSE
    and dQ on 128 sampled rows per head against the oracle, and the dK/dV
    identities per head."""
    B, H, N, d = 1, 4, 65536 - 37, 64
    print(f"case d=64 long sequence B={B} H={H} N={N}", flush=True)
    q, k, v, dO = synth.make_qkv(B, H, N, d, torch.bfloat16, seed=1600, backward=True,
                                 device=DEV)
    s = synth.default_scale(d)
    O, L = fa.fa_fwd(q, k, v, s)
    dq, dk, dv = fa.fa_bwd(q, k, v, O, L, dO, s)
    torch.cuda.synchronize()
    rows = synth.draw_rows(N, H, 128, seed=1600)
    for h in range(H):
        r = rows[h]
        ridx = torch.from_numpy(r).to(DEV)
        qh, kh, vh, gh = (f64(x[0, h].cpu()) for x in (q, k, v, dO))
        Oref, Lref = oracle.sdpa_rows(qh[r], kh, vh, s)
        dQref, _ = oracle.sdpa_backward_rows(qh[r], kh, vh, gh[r], s)
        o = f64(O[0, h].index_select(0, ridx).cpu())
        l = f64(L[0, h].index_select(0, ridx).cpu())
        g = f64(dq[0, h].index_select(0, ridx).cpu())
        ma, mn, ml = max_abs(o, Oref), mean_abs(o, Oref), max_abs(l, Lref)
        rel_o, rel_dq = rel_frobenius(o, Oref), rel_frobenius(g, dQref)
        dk64, dv64, g64 = dk[0, h].double(), dv[0, h].double(), dO[0, h].double()
        res_k = float(dk64.sum(0).norm() / dk64.norm())
        res_v = float((dv64.sum(0) - g64.sum(0)).norm() / dv64.norm())
        say(f"  head {h}: O max-abs {ma:.3e} rel {rel_o:.3e}; LSE max-abs {ml:.3e}; "
            f"dQ rel {rel_dq:.3e}; dK sum {res_k:.3e}; dV sum {res_v:.3e}")
        assert ma <= TOL_BF16_O_MAX and mn <= TOL_BF16_O_MEAN and ml <= TOL_BF16_LSE_MAX
        assert rel_o <= 2e-2 and rel_dq <= TOL_BF16_GRAD_REL
        assert res_k <= TOL_BF16_GRAD_REL and res_v <= TOL_BF16_GRAD_REL
