"""fa_bwd_noalloc (the backward for callers that cannot allocate device
memory) against fa_bwd, through the C ABI: two calls in a row, the second on
a smaller problem (the fixed scratch array then still holds the first call's
rows), each bit-identical to fa_bwd and within the bf16 gradient bound of the
fp64 oracle; the calls allocate no device memory; a problem larger than the
array is refused before anything is enqueued."""

import ctypes
import gc

import numpy as np
import pytest
import torch

import io_aware_softmax_02_amd as fa
from io_aware_softmax_02_amd._lib import LIB, FA_OK, FA_ERR_SCRATCH, FA_BWD_NOALLOC_MAX_ROWS
import oracle
import synth
from _compare import TOL_BF16_GRAD_REL, rel_frobenius

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def c_noalloc(q, k, v, o, lse, dO, dq, dk, dv, scale, stream):
    B, H, N, d = q.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return LIB.fa_bwd_noalloc(p(q), p(k), p(v), p(o), p(lse), p(dO), p(dq), p(dk), p(dv),
                              B, H, N, d, ctypes.c_float(scale), ctypes.c_void_p(stream))


def test_noalloc_matches_fa_bwd_on_two_calls_second_smaller():
    stream = torch.cuda.current_stream(DEV).cuda_stream
    # The first call on a device looks up its scratch array, which loads the
    # code object that holds it (the array's 16 MiB of static storage, once
    # per process and device); the calls checked below then allocate nothing.
    ins = [torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16, device=DEV) for _ in range(5)]
    L0 = torch.zeros(1, 1, 16, dtype=torch.float32, device=DEV)
    outs = [torch.empty_like(ins[0]) for _ in range(3)]
    torch.cuda.synchronize()
    free_a = torch.cuda.mem_get_info()[0]
    qz, kz, vz, oz, gz = ins
    assert c_noalloc(qz, kz, vz, oz, L0, gz, *outs, 0.125, stream) == FA_OK
    torch.cuda.synchronize()
    loaded = free_a - torch.cuda.mem_get_info()[0]
    print(f"first call on the device: free memory fell by {loaded} B "
          f"(scratch array {FA_BWD_NOALLOC_MAX_ROWS * 4} B)", flush=True)
    assert loaded <= FA_BWD_NOALLOC_MAX_ROWS * 4 + 8 * 1024 * 1024
    for case, (B, H, N, d) in enumerate([(2, 4, 1000, 128), (1, 3, 300, 64)]):
        print(f"case fa_bwd_noalloc call {case + 1}: B={B} H={H} N={N} d={d}", flush=True)
        q, k, v, dO = synth.make_qkv(B, H, N, d, torch.bfloat16, seed=1200 + case,
                                     backward=True)
        qg, kg, vg, gg = (x.to(DEV) for x in (q, k, v, dO))
        s = synth.default_scale(d)
        O, L = fa.fa_fwd(qg, kg, vg, s)
        ref = fa.fa_bwd(qg, kg, vg, O, L, gg, s)
        dq, dk, dv = (torch.full_like(qg, float("nan")) for _ in range(3))
        gc.collect()   # tensors left by earlier tests are freed now, not during the call
        torch.cuda.synchronize()
        used0 = torch.cuda.memory_allocated()
        free0 = torch.cuda.mem_get_info()[0]
        st = c_noalloc(qg, kg, vg, O, L, gg, dq, dk, dv, s, stream)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        assert st == FA_OK, fa.status_str(st)
        assert torch.cuda.memory_allocated() <= used0   # nothing allocated through torch
        assert free0 - free1 <= 2 * 1024 * 1024         # nor any device memory at all
        for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            assert torch.equal(x, r), name
        rq, rk, rv, _ = oracle.sdpa_backward(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v),
                                             synth.to_f64(dO), s)
        for name, x, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            e = rel_frobenius(synth.to_f64(x.cpu()), r)
            print(f"  {name} rel-Frobenius {e:.3e}", flush=True)
            assert e <= TOL_BF16_GRAD_REL, name


def test_noalloc_refuses_problems_beyond_its_scratch():
    x = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    p = ctypes.c_void_p(x.data_ptr())
    N = FA_BWD_NOALLOC_MAX_ROWS // 2 + 1
    st = LIB.fa_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, 2, N, 128, ctypes.c_float(0.1), None)
    assert st == FA_ERR_SCRATCH
    assert "FA_ERR_SCRATCH" in fa.status_str(st)
    torch.cuda.synchronize()


def test_noalloc_at_its_maximum_rows():
    """B*H*N equal to the scratch array's size (2^22 rows): bit-identical to
    fa_bwd, and the call allocates nothing."""
    B, H, N, d = 4, 64, 16384, 128
    assert B * H * N == FA_BWD_NOALLOC_MAX_ROWS
    print(f"case fa_bwd_noalloc at its maximum: B={B} H={H} N={N} d={d}", flush=True)
    q, k, v, dO = synth.make_qkv(B, H, N, d, torch.bfloat16, seed=1400, backward=True,
                                 device=DEV)
    s = synth.default_scale(d)
    O, L = fa.fa_fwd(q, k, v, s)
    ref = fa.fa_bwd(q, k, v, O, L, dO, s)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    gc.collect()
    torch.cuda.synchronize()
    used0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    st = c_noalloc(q, k, v, O, L, dO, dq, dk, dv, s, torch.cuda.current_stream(DEV).cuda_stream)
    torch.cuda.synchronize()
    assert st == FA_OK, fa.status_str(st)
    assert torch.cuda.memory_allocated() <= used0
    assert free0 - torch.cuda.mem_get_info()[0] <= 2 * 1024 * 1024
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert torch.equal(x, r), name
    print("  bit-identical to fa_bwd", flush=True)
