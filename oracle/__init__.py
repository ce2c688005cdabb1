"""CPU oracle for exact scaled-dot-product attention (TEST INFRASTRUCTURE).

This package is the slow, plainly correct reference that the HIP path is
checked against.  It is test infrastructure only: the tests, the smoke check
and the CPU-baseline leg of the benchmark may import it; the library and its
Python binding never do, and nothing here imports them.

Pages cited (all on FlashAttention, read as the description of what is
computed):
  [P1] "算珠楼的掌簿人" - hespethorn.github.io/posts/fable-flashattention/
  [P2] "账房先生的奔命：Flash Attention 与内存 I/O 革命" -
       carrie-l.github.io/AI/2026-06-11-knowledge-20
  [P3] the star-observatory FlashAttention fable -
       ckw19810413.github.io/blog/2026-10-11-flashattention-fable/

Modules:
  attention  - float64 numpy: the plain definition (materialises S and P),
               the analytic backward, and the three online-softmax forms.
  brute      - pure Python with math.fsum, for tiny inputs.
"""

from .attention import (  # noqa: F401
    sdpa_forward,
    sdpa_forward_head,
    sdpa_backward,
    sdpa_backward_head,
    sdpa_backward_rows,
    sdpa_rows,
    online_forward_head,
    online_forward_normalised_head,
    two_pass_forward_head,
    softmax_rows,
    split_bounds,
    sdpa_split_head,
    merge_parts,
)
from .brute import brute_forward, brute_backward  # noqa: F401
