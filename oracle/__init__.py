"""FP64 CPU oracles for starting-node triangle attention and the triangle multiplication
core (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package.  The GPU product path never calls it and shares no code
with it.

What it computes is the plain definition of the method, evaluated in float64
on the exact (upcast) bf16 input values.  The method is exact attention, not an
approximation, so the oracle is the definition written out, slice by slice.

Sources:
- "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
  Optimized Triangle Attention Kernel" (arXiv 2610.05854), Abstract: triangular
  attention as in AlphaFold3-style models; a pair bias shared by all attention
  slices, whose gradient is a reduction across slices in addition to the usual
  reductions over queries and keys; the softmax backward correction computed
  from the forward output.
- The per-slice formula (the pages print none): for every batch b, slice i and
  head h, o[j] = sum_k softmax_k(alpha * q[j].k[k] + bias[j,k] + mask[k]) v[k],
  with alpha = 1/sqrt(d), the bias indexed [b,h,j,k] and shared by every slice,
  and the key mask leaving masked keys out of the softmax (the workloads' additive
  -1e9; a row with no key of finite score outputs 0, has lse = +inf and no
  gradient).

The triangle multiplication core (``tri_mul_oracle``) follows the kongchang.com
article on fast_trimul, section "什么是三角乘法更新"; its reading is stated in that
module.

Every function here is pinned by tests under ``tests/test_oracle.py`` and
``tests/test_tri_mul_oracle.py`` (closed forms, invariants, a library attention
routine with autograd, explicit loops, central finite differences); none is
"parity unpinned".
"""
from .tri_attn_oracle import (  # noqa: F401
    MASK_NEG,
    backward64,
    dbias_rows64,
    forward64,
    slice_backward64,
    slice_forward64,
)
from .tri_mul_oracle import (  # noqa: F401
    DIRECTIONS,
    gate_backward64,
    gate_forward64,
    tri_mul_backward64,
    tri_mul_forward64,
    tri_mul_loops64,
)
