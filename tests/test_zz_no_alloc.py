"""The allocation-free column linear (tp_col_linear_gelu_noalloc) against
tp_col_linear_gelu on the GPU.  Both compute the same sums in the same order
(the decode path's split-K partials are added in split order either way), so
their outputs must be bitwise equal.  Each case runs two calls in a row, the
second on a smaller input, and the decode cases repeat, so that partials a
call left in the library's static scratch would show up in the next one if
any were read without being rewritten."""
import pytest

from gpu_util import note, torch

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, bias, seed):
    T = torch()
    g = T.Generator(device="cuda:0")
    g.manual_seed(seed)
    X = T.randn((M, K), generator=g, device="cuda:0").to(T.bfloat16)
    W = (T.randn((K, N), generator=g, device="cuda:0") * 0.02).to(T.bfloat16)
    b = (T.randn((N,), generator=g, device="cuda:0") * 0.1).to(T.bfloat16) if bias else None
    return X, W, b


def _both(M, K, N, act, bias, seed):
    import megatron_tensor_transformer_col_amd as tp
    T = torch()
    X, W, b = _inputs(M, K, N, bias, seed)
    ref = T.empty((M, N), dtype=T.bfloat16, device="cuda:0")
    out = T.full((M, N), float("nan"), dtype=T.bfloat16, device="cuda:0")
    tp.tp_col_linear_gelu(X, W, ref, act=act, bias=b)
    tp.tp_col_linear_gelu_noalloc(X, W, out, act=act, bias=b)
    T.cuda.synchronize()
    return ref, out


# (M, K, N, act, bias): the decode workload's column shard (split K over 9
# ranges), then smaller ragged shapes (K not a multiple of the 64-row slab,
# N not a multiple of the 64-column strip), a single-split shape, and the
# GEMM path (M above the decode threshold)
@pytest.mark.parametrize("first,second", [
    ((16, 8192, 3584, "gelu", False), (5, 1000, 520, "none", True)),
    ((16, 3584, 8192, "none", False), (1, 72, 72, "gelu", True)),
    ((7, 4096, 33280, "gelu", True), (16, 8192, 3584, "gelu", True)),
    ((64, 1024, 1024, "gelu", False), (16, 2048, 1024, "gelu", True)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for rep in range(2):
        for i, (M, K, N, act, bias) in enumerate((first, second)):
            note(f"no-alloc col linear rep {rep} call {i}: M {M} K {K} N {N} act {act} bias {bias}")
            ref, out = _both(M, K, N, act, bias, seed=10 * i + rep)
            assert torch().equal(ref, out), f"M {M} K {K} N {N}: no-alloc result differs"
