"""fp64 CPU oracle of the tensor-parallel transformer block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only module both sides use is ``synth`` (seeded input draws).

What it computes: the UNSHARDED block, in float64, from the definitions on
the pages.  Tensor parallelism reaches the single-device result exactly (up
to rounding order) -- the block-matrix identities of "张量并行" (section
并行化矩阵乘法运算 / 两个矩阵相乘) and the column/row-wise equations of
"Infra: Tensor Parallel" -- so the unsharded definition IS the oracle.  The
per-shard quantities (H_i, P_i, dW_i, ...) are obtained by slicing inputs and
outputs with the shard mapping, never by a different formula.

Two implementations:
  * ``oracle.block``  -- NumPy float64 (BLAS matmul and scipy ``erf`` as
    library primitives), used for all sizes;
  * ``oracle.brute``  -- pure-Python loops with ``math.erf``/``math.exp``,
    used on tiny inputs to pin ``oracle.block``.

Every function is pinned by a ``-m "not gpu"`` test (tests/test_oracle_*.py)
against something other than itself: closed forms, printed normal-CDF values,
brute force, finite differences, torch float64 autograd / SDPA as independent
library routines, and the pages' sharding invariants.  No function here is
parity-unpinned.
"""
from .block import (  # noqa: F401
    gelu, gelu_grad, silu, silu_grad, softmax_rows,
    linear, row_partial, shard_sum,
    mlp_gelu, mlp_swiglu, mlp_gelu_backward, mlp_swiglu_backward,
    attention_heads, mha, mha_gqa, attention_head_backward, mha_backward, layernorm, reduce_scatter_layernorm,
    cross_entropy_rows, vocab_shard_stats, vocab_parallel_cross_entropy,
)
