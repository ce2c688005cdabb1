"""Seeded synthetic inputs for exact scaled-dot-product attention.

This module only draws random tensors and describes workload shapes.  It holds
none of the attention arithmetic, so the CPU oracle and the HIP path can both
take their inputs from here without sharing any of the method.

Shapes follow the long-context sizes the FlashAttention pages discuss
("Flash Attention 与内存 I/O 革命", section 九, memory table at N = 2k ... 128k,
and the FlashAttention fable page, "為什麼過去的 Attention 會慢", 8k/32k/128k
tokens).  Values are iid N(0, 1): no page prints activations, and no dataset is
involved.

Recipe (every workload):
  * ``g = torch.Generator().manual_seed(seed)`` on the CPU;
  * draw fp32 ``torch.randn(B, H, N, d, generator=g)`` in the order Q, K, V,
    then dO when a backward is needed;
  * round to the workload dtype with ``.to(dtype)`` (round-to-nearest-even);
  * the outlier variant multiplies one key row by 8 after rounding, which is
    exact in bf16 because 8 is a power of two.
Tensors are contiguous ``[B, H, N, d]`` with d fastest.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16"
    seed: int
    backward: bool = False
    outlier_row: Optional[int] = None
    outlier_factor: float = 8.0
    sample_rows: Optional[int] = None   # query rows per head checked one by one
    block: Optional[int] = None         # key block size the workload is described with

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def fwd_flops(self) -> float:
        """Counted forward work: two N x N x d contractions, 4*B*H*N^2*d."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d

    def bwd_flops(self) -> float:
        """Counted backward work: 2.5x the forward (five contractions)."""
        return 2.5 * self.fwd_flops()


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded once to fp32; the same float goes to every path."""
    return float(np.float32(1.0 / math.sqrt(d)))


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        # 64 rows cut into 8 blocks of 8, as in the fable of the 64 merchants.
        Workload("tiny_f32_n64_d64", 1, 1, 64, 64, "f32", seed=1, block=8),
        Workload("fwd_bf16_b4h16_n2048_d64", 4, 16, 2048, 64, "bf16", seed=2),
        Workload("long_bf16_b1h16_n8192_d128", 1, 16, 8192, 128, "bf16", seed=3),
        Workload("long_bf16_b1h16_n8192_d128_outlier", 1, 16, 8192, 128, "bf16",
                 seed=3, outlier_row=6181),
        Workload("vlong_bf16_b1h8_n131072_d128", 1, 8, 131072, 128, "bf16",
                 seed=4, sample_rows=256),
        Workload("fwdbwd_bf16_b2h16_n4096_d128", 2, 16, 4096, 128, "bf16",
                 seed=5, backward=True),
        # The shape the throughput is quoted on: B=1, H=16, N=8192, d=128,
        # forward and forward+backward.  Same Q, K, V as the long forward.
        Workload("attn_bf16_b1h16_n8192_d128_fwdbwd", 1, 16, 8192, 128, "bf16",
                 seed=3, backward=True),
    ]
}


def make_inputs(w: Workload, backward: Optional[bool] = None):
    """Return CPU tensors (q, k, v, dO or None) in the workload dtype."""
    return make_qkv(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed,
                    backward=w.backward if backward is None else backward,
                    outlier_row=w.outlier_row, outlier_factor=w.outlier_factor)


def make_qkv(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
             backward: bool = False, outlier_row: Optional[int] = None,
             outlier_factor: float = 8.0, device: Optional[torch.device] = None):
    """Seeded iid N(0,1) tensors, drawn on the CPU (the recipe above), or
    with ``device`` given, by that device's own generator seeded the same way
    (other values, same distribution; for sizes whose CPU draw would take
    long)."""
    g = torch.Generator(device=device or "cpu").manual_seed(seed)
    shape = (B, H, N, d)
    dev = {} if device is None else {"device": device}
    q = torch.randn(shape, generator=g, **dev).to(dtype)
    k = torch.randn(shape, generator=g, **dev).to(dtype)
    v = torch.randn(shape, generator=g, **dev).to(dtype)
    dO = torch.randn(shape, generator=g, **dev).to(dtype) if backward else None
    if outlier_row is not None:
        k[:, :, outlier_row, :] *= outlier_factor
    return q, k, v, dO


def make_parts(P: int, B: int, H: int, N: int, d: int, seed: int, dead_every: int = 0):
    """Seeded partial results for merge tests: o_part fp32 N(0,1)
    [P,B,H,N,d], lse_part fp32 3*N(0,1) [P,B,H,N].  With dead_every = k > 0,
    every k-th (part, row) entry gets lse = -inf and a NaN output row (a
    part with no key), and the last row of every head is dead in all parts."""
    g = torch.Generator().manual_seed(seed)
    o = torch.randn((P, B, H, N, d), generator=g)
    lse = 3.0 * torch.randn((P, B, H, N), generator=g)
    if dead_every:
        flat = lse.view(-1)
        dead = torch.arange(0, flat.numel(), dead_every)
        flat[dead] = -math.inf
        o.view(-1, d)[dead] = math.nan
        lse[..., N - 1] = -math.inf
        o[..., N - 1, :] = math.nan
    return o, lse


def sampled_rows(w: Workload) -> np.ndarray:
    """Query rows checked per head for the very long workload
    (``draw_rows`` with the workload's sizes and seed)."""
    assert w.sample_rows is not None
    return draw_rows(w.N, w.B * w.H, w.sample_rows, w.seed)


def draw_rows(N: int, heads: int, count: int, seed: int) -> np.ndarray:
    """Query rows checked one by one at sizes the oracle cannot run in full.

    Per head: rows 0 and N-1 plus (count - 2) rows drawn without replacement
    from the rest with ``np.random.default_rng(seed)``; the heads draw in
    order.  Returns an int64 array [heads, count], sorted per head.
    """
    assert count >= 2 and N >= count
    rng = np.random.default_rng(seed)
    out = np.empty((heads, count), dtype=np.int64)
    for bh in range(heads):
        rest = rng.choice(np.arange(1, N - 1), size=count - 2, replace=False)
        out[bh] = np.sort(np.concatenate([[0, N - 1], rest]))
    return out


def sweep_inputs(N: int, backward: bool = True):
    """Inputs of the sequence-length sweep: B=1, H=16, d=128, bf16, seed N."""
    return make_qkv(1, 16, N, 128, torch.bfloat16, seed=N, backward=backward)


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact upcast of a CPU tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
