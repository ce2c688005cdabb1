"""GPU test of the materialised contrast (standard attention through device
memory, 账房先生的奔命 section 五; the star-observatory fable page,
"為什麼過去的 Attention 會慢"): its O against the fp64 oracle at the bf16
bounds, and its O(N^2) device memory against the tiled forward's none.

The contrast is run by bench.py (`standard_attention`) with torch's own
kernels; it is not part of the library.
"""

import pytest
import torch

import bench
import io_aware_softmax_02_amd as fa
import oracle
import synth
from _compare import TOL_BF16_O_MAX, TOL_BF16_O_MEAN, max_abs, mean_abs, rel_frobenius

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("name,heads", [("fwd_bf16_b4h16_n2048_d64", None),
                                        ("long_bf16_b1h16_n8192_d128", 2)])
def test_standard_attention_matches_oracle_and_holds_nxn_memory(name, heads):
    w = synth.WORKLOADS[name]
    q, k, v, _ = synth.make_inputs(w, backward=False)
    if heads is not None:
        q, k, v = (x[:, :heads].contiguous() for x in (q, k, v))
    B, H, N, d = q.shape
    print(f"case contrast {name} B={B} H={H} N={N} d={d}", flush=True)
    qg, kg, vg = (x.to(DEV) for x in (q, k, v))
    # warm both paths (code objects, library handles) before measuring memory
    bench.standard_attention(qg[:, :1, :256].contiguous(), kg[:, :1, :256].contiguous(),
                             vg[:, :1, :256].contiguous(), w.scale)
    o = torch.empty_like(qg)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    fa.fa_fwd(qg, kg, vg, w.scale, o=o, lse=lse)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fa.fa_fwd(qg, kg, vg, w.scale, o=o, lse=lse)
    torch.cuda.synchronize()
    extra_fa = torch.cuda.max_memory_allocated() - base

    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    S, P, O = bench.standard_attention(qg, kg, vg, w.scale)
    torch.cuda.synchronize()
    extra_std = torch.cuda.max_memory_allocated() - base
    nxn = B * H * N * N * 2
    print(f"  extra device memory: standard {extra_std / 1e6:.1f} MB "
          f"(one bf16 N x N tensor {nxn / 1e6:.1f} MB), tiled {extra_fa} B", flush=True)
    assert extra_fa == 0
    assert extra_std >= 2 * nxn          # S and P both live at once
    del S, P

    Oref, _ = oracle.sdpa_forward(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), w.scale)
    Os = synth.to_f64(O.cpu())
    ma, mn, rel = max_abs(Os, Oref), mean_abs(Os, Oref), rel_frobenius(Os, Oref)
    print(f"  standard O: max-abs {ma:.3e} mean-abs {mn:.3e} rel-Frobenius {rel:.3e}", flush=True)
    assert ma <= TOL_BF16_O_MAX and mn <= TOL_BF16_O_MEAN and rel <= 2e-2
