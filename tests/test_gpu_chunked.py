"""GPU checks that grids larger than one launch run in full, through the C ABI.

A kernel dispatch holds its grid as a 32-bit count of work-items, and a launch
of 2^32 or more is cut short without an error, so the launchers cut a large
grid into launches of at most 2^31 work-items, of whole heads (or of whole
blocks of rows).  Each case here crosses that line with a problem that fits
one GPU, fills the outputs with NaN first (a row no launch wrote stays NaN),
and checks every row through an identity that holds at any size, plus
sampled rows, among them the rows on both sides of the launch boundary,
against the oracle:

* one key per head: the softmax row is [1], so O = V exactly, LSE = scale
  q.k, dV = dO (exactly in bf16, where P is rounded to bf16 first; to a few
  fp32 roundings in fp32), and dQ = dK = 0 (exactly in fp32, where dP and D
  are the same sum; up to the rounding of dP - D in bf16);
* the preprocess D = rowsum(dO * O) per row;
* the merge of two identical parts: O = O_0 exactly and LSE = LSE_0 + ln 2,
  which also fails if a part were read at the wrong stride.
"""

import gc
import math

import numpy as np
import pytest
import torch

import io_aware_softmax_02_amd as fa
import oracle
import synth
from _compare import TOL_BF16_LSE_MAX, TOL_BF16_O_MAX, max_abs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LAUNCH_ITEMS = 1 << 31      # work-items per launch at most


def say(msg):
    print(msg, flush=True)


def f64(t):
    return synth.to_f64(t)


def nan_like(x):
    return torch.full_like(x, math.nan)


def free():
    gc.collect()
    torch.cuda.empty_cache()


def boundary_heads(per_launch, H, extra=(0,)):
    return sorted({*extra, per_launch - 1, per_launch, per_launch + 1, H - 1})


def test_bf16_one_key_heads_across_launches():
    # 512 work-items per head in the forward and dQ kernels (256 query rows
    # of 8 waves), 256 in dK/dV: 2^22 heads per forward launch.
    per_launch = LAUNCH_ITEMS // 512
    H, d = per_launch + 3, 64
    say(f"case bf16 B=1 H={H} N=1 d={d}: forward and backward in two launches")
    q, k, v, dO = synth.make_qkv(1, H, 1, d, torch.bfloat16, seed=31, backward=True, device=DEV)
    s = synth.default_scale(d)
    O, L = fa.fa_fwd(q, k, v, s, o=nan_like(q), lse=torch.full((1, H, 1), math.nan, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(O, v)
    lref = s * (q.double() * k.double()).sum(-1)
    err = float((L.double() - lref).abs().max())
    say(f"  O == V on every head; LSE max-abs {err:.3e}")
    assert err <= TOL_BF16_LSE_MAX
    for h in boundary_heads(per_launch, H):
        Or, Lr = oracle.sdpa_rows(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), s)
        assert max_abs(f64(O[0, h]), Or) <= TOL_BF16_O_MAX
        assert max_abs(f64(L[0, h]), Lr) <= TOL_BF16_LSE_MAX
    dq, dk, dv = fa.fa_bwd(q, k, v, O, L, dO, s, dq=nan_like(q), dk=nan_like(q), dv=nan_like(q))
    torch.cuda.synchronize()
    assert torch.equal(dv, dO)
    mq, mk = float(dq.float().abs().max()), float(dk.float().abs().max())
    say(f"  dV == dO on every head; max |dQ| {mq:.3e}, max |dK| {mk:.3e}")
    assert mq <= 1e-3 and mk <= 1e-3           # NaN fails both
    for h in boundary_heads(per_launch, H):
        r = oracle.sdpa_backward_head(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(dO[0, h]), s)
        assert max_abs(f64(dq[0, h]), r["dQ"]) <= 1e-3
        assert max_abs(f64(dk[0, h]), r["dK"]) <= 1e-3
        assert np.array_equal(f64(dv[0, h]), r["dV"])
    del q, k, v, dO, O, L, dq, dk, dv
    free()


def test_f32_one_key_heads_across_launches():
    # fp32 at d = 17 runs the 8-key-block kernels: 64 work-items per head.
    per_launch = LAUNCH_ITEMS // 64
    H, d = per_launch + 3, 17
    say(f"case f32 B=1 H={H} N=1 d={d}: forward and backward in two launches")
    assert fa.fa_f32_key_block(1, d) == 8
    q, k, v, dO = synth.make_qkv(1, H, 1, d, torch.float32, seed=32, backward=True, device=DEV)
    s = synth.default_scale(d)
    O, L = fa.fa_fwd_f32(q, k, v, s, o=nan_like(q),
                         lse=torch.full((1, H, 1), math.nan, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(O, v)
    # LSE = scale * (q . k), one fp32 dot product: within d * 2^-24 of the
    # sum of |terms| (summation bound) plus the rounding of the product.
    prod = q.double() * k.double()
    bound = s * (d * 2.0 ** -24 * prod.abs().sum(-1)) + 2.0 ** -23 * (s * prod.sum(-1)).abs()
    err = (L.double() - s * prod.sum(-1)).abs()
    say(f"  O == V on every head; LSE max-abs {float(err.max()):.3e}")
    assert bool((err <= bound + 1e-30).all())
    del prod, bound, err
    for h in boundary_heads(per_launch, H):
        Or, Lr = oracle.sdpa_rows(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), s)
        assert max_abs(f64(O[0, h]), Or) <= 1e-6
        assert max_abs(f64(L[0, h]), Lr) <= 1e-5
    dq, dk, dv = fa.fa_bwd_f32(q, k, v, O, L, dO, s, dq=nan_like(q), dk=nan_like(q),
                               dv=nan_like(q))
    torch.cuda.synchronize()
    # P = exp(s - LSE) with LSE = s; the compiler may fuse the product of the
    # scale into the subtraction (one rounding fewer), so P = 1 to within
    # 2^-24 (|s| + 2), and dV = P dO to that relative accuracy.  dP and D are
    # the same fp32 sum, so dS, dQ and dK are exactly 0.
    rel = 2.0 ** -24 * (L.double().abs() + 2.0)
    ev = (dv.double() - dO.double()).abs()
    assert bool((ev <= rel[..., None] * dO.double().abs()).all())
    assert bool((dq == 0).all()) and bool((dk == 0).all())
    say(f"  dV = dO to within 2^-24 (|s| + 2) relative (max-abs {float(ev.max()):.3e}), "
        f"dQ == 0 and dK == 0 on every head")
    del rel, ev
    del q, k, v, dO, O, L, dq, dk, dv
    free()


def test_bf16_preprocess_rows_across_launches():
    # d = 128: 16 lanes per row, 16 rows per 256-lane block, 2^27 rows per launch.
    per_launch = LAUNCH_ITEMS // 16
    B, H, N, d = 1, 128, (1 << 20) + 3, 128
    rows = B * H * N
    assert per_launch < rows < 2 * per_launch
    say(f"case bf16 preprocess B={B} H={H} N={N} d={d}: {rows} rows in two launches")
    g = torch.Generator(device=DEV).manual_seed(33)
    O = torch.empty((B, H, N, d), device=DEV, dtype=torch.bfloat16).normal_(generator=g)
    dO = torch.empty((B, H, N, d), device=DEV, dtype=torch.bfloat16).normal_(generator=g)
    delta = fa.fa_bwd_preprocess(O, dO, delta=torch.full((B, H, N), math.nan, device=DEV))
    torch.cuda.synchronize()
    Of, gf, df = O.view(rows, d), dO.view(rows, d), delta.view(rows)
    # every row, against the fp64 sum, within the summation bound d * 2^-24 * sum |terms|
    worst = 0.0
    step = 1 << 22
    for r0 in range(0, rows, step):
        t = Of[r0:r0 + step].double() * gf[r0:r0 + step].double()
        e = (df[r0:r0 + step].double() - t.sum(-1)).abs()
        assert bool((e <= d * 2.0 ** -24 * t.abs().sum(-1) + 1e-30).all()), r0
        worst = max(worst, float(e.max()))
    say(f"  every row within the fp32 summation bound; max-abs {worst:.3e}")
    idx = sorted({0, per_launch - 1, per_launch, per_launch + 1, rows - 1})
    ii = torch.tensor(idx, device=DEV)
    ref = (f64(Of.index_select(0, ii)) * f64(gf.index_select(0, ii))).sum(-1)
    assert max_abs(f64(df.index_select(0, ii)), ref) <= 1e-4
    del O, dO, delta, Of, gf, df
    free()


def test_merge_rows_across_launches():
    # d = 128: 32 lanes per row, 8 rows per 256-lane block, 2^26 rows per launch.
    per_launch = LAUNCH_ITEMS // 32
    B, H, N, d = 1, 64, (1 << 20) + 3, 128
    rows = B * H * N
    assert per_launch < rows < 2 * per_launch
    say(f"case merge P=2 B={B} H={H} N={N} d={d}: {rows} rows in two launches")
    g = torch.Generator(device=DEV).manual_seed(34)
    op = torch.empty((2, B, H, N, d), device=DEV)
    lp = torch.empty((2, B, H, N), device=DEV)
    op[0].normal_(generator=g)
    lp[0].normal_(generator=g).mul_(3.0)
    op[1].copy_(op[0])
    lp[1].copy_(lp[0])
    o, lse = fa.fa_merge(op, lp, o=torch.full((B, H, N, d), math.nan, device=DEV,
                                               dtype=torch.bfloat16),
                         lse=torch.full((B, H, N), math.nan, device=DEV))
    torch.cuda.synchronize()
    of, lf, o0, l0 = o.view(rows, d), lse.view(rows), op[0].view(rows, d), lp[0].view(rows)
    step = 1 << 24
    for r0 in range(0, rows, step):
        assert torch.equal(of[r0:r0 + step], o0[r0:r0 + step].to(torch.bfloat16)), r0
    dl = float((lf.double() - l0.double() - math.log(2.0)).abs().max())
    say(f"  O == O_0 on every row; LSE - (LSE_0 + ln 2) max-abs {dl:.3e}")
    assert dl <= 1e-5
    idx = sorted({0, per_launch - 1, per_launch, per_launch + 1, rows - 1})
    ii = torch.tensor(idx, device=DEV)
    parts_o = np.stack([f64(op[p].view(rows, d).index_select(0, ii)) for p in range(2)])
    parts_l = np.stack([f64(lp[p].view(rows).index_select(0, ii)) for p in range(2)])
    Or, Lr = oracle.merge_parts(parts_o, parts_l)
    og, lg = f64(of.index_select(0, ii)), f64(lf.index_select(0, ii))
    assert max_abs(og, Or) <= 2.0 ** -8 * np.abs(Or).max() and max_abs(lg, Lr) <= 1e-5
    del op, lp, o, lse, of, lf, o0, l0
    free()
