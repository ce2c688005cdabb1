"""The whole step (fa_fwd, then fa_bwd_noalloc) captured into a HIP graph
through torch's graph API and replayed: every replay, with eager work and
synchronisations between replays, must give bit for bit the outputs of the
same calls run eagerly.  The captured calls allocate nothing and record no
memset (their scratch is written by a kernel before it is read)."""

import pytest
import torch

import io_aware_softmax_02_amd as fa
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_step_in_a_graph_replays_bit_for_bit():
    B, H, N, d = 1, 4, 1000, 128
    print(f"case graph capture of fa_fwd + fa_bwd_noalloc B={B} H={H} N={N} d={d}", flush=True)
    s = synth.default_scale(d)
    q, k, v, dO = (x.to(DEV) for x in synth.make_qkv(B, H, N, d, torch.bfloat16, seed=1300,
                                                    backward=True))
    o, lse = torch.empty_like(q), torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def step():
        fa.fa_fwd(q, k, v, s, o=o, lse=lse)
        fa.fa_bwd_noalloc(q, k, v, o, lse, dO, s, dq=dq, dk=dk, dv=dv)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # loads the code objects and the scratch
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((o, lse, dq, dk, dv), ref)), rep
        # eager work on the same tensors between replays
        step()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((o, lse, dq, dk, dv), ref)), rep
    print("  4 replays bit-identical to the eager step", flush=True)
