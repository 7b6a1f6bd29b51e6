"""GPU parity of the vocabulary-parallel cross-entropy against the fp64
oracle: per-shard row statistics, the combined row log-sum-exp, the shard
losses (rows whose target the shard holds) and the total."""
import numpy as np
import pytest

import megatron_tensor_transformer_col_amd as tp
import oracle
import synth
from gpu_util import assert_close, dev, host, note, torch

pytestmark = pytest.mark.gpu


def _run(d, n, dtype):
    T_, V = d["logits"].shape
    w = V // n
    T = torch()
    Z = dev(d["logits"])
    tg = T.from_numpy(d["targets"]).to("cuda:0")
    stats = [T.empty((T_, 2), dtype=T.float32, device="cuda:0") for _ in range(n)]
    for i in range(n):
        tp.tp_vocab_ce_shard_stats(Z[:, i * w:(i + 1) * w], stats[i])
    lse = T.empty(T_, dtype=T.float32, device="cuda:0")
    tp.tp_vocab_ce_lse(stats, lse)
    losses = [T.empty(1, dtype=T.float32, device="cuda:0") for _ in range(n)]
    rows = [T.empty(T_, dtype=T.float32, device="cuda:0") for _ in range(n)]
    for i in range(n):
        tp.tp_vocab_ce_shard_loss(Z[:, i * w:(i + 1) * w], i * w, tg, lse, losses[i], row_loss=rows[i])
    total = T.empty(1, dtype=T.float32, device="cuda:0")
    tp.tp_vocab_ce_total(losses, total)
    T.cuda.synchronize()
    return stats, lse, losses, rows, total


def _check(d, n, res):
    stats, lse, losses, rows, total = res
    ref = oracle.vocab_parallel_cross_entropy(d["logits"].f32, d["targets"], n)
    for i, (m, s) in enumerate(ref["stats"]):
        st = host(stats[i])
        np.testing.assert_array_equal(st[:, 0], m)            # the max of stored values is exact
        assert_close(st[:, 1], s, "f32", f"sumexp shard {i}")
    assert_close(host(lse), ref["lse"], "f32", "lse")
    assert_close(np.array([host(x)[0] for x in losses]), ref["shard_loss"], "f32", "shard losses")
    assert_close(sum(host(r) for r in rows), ref["rows"], "f32", "row losses")
    assert_close(host(total), np.array([ref["total"]]), "f32", "total")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,V,n", [(200, 4000, 4), (37, 1032, 2), (45, 1030, 2), (16, 20, 4), (64, 8, 1), (129, 24576, 8)])
def test_vocab_ce_medium(dtype, T, V, n):
    note(f"vocab ce T={T} V={V} n={n} {dtype}")
    d = synth.make_ce_inputs(T, V, dtype, seed=T + V, scale=3.0)
    _check(d, n, _run(d, n, dtype))


def test_targets_outside_every_shard_contribute_nothing():
    note("vocab ce out-of-range targets")
    T, V, n = 96, 2048, 4
    d = synth.make_ce_inputs(T, V, "bf16", seed=5)
    d["targets"][::7] = -1
    d["targets"][3::11] = V
    stats, lse, losses, rows, total = _run(d, n, "bf16")
    keep = (d["targets"] >= 0) & (d["targets"] < V)
    ref = oracle.cross_entropy_rows(d["logits"].f32[keep], d["targets"][keep])
    row_sum = sum(host(r) for r in rows)
    assert np.all(row_sum[~keep] == 0)
    assert_close(row_sum[keep], ref, "f32", "row losses")
    assert_close(host(total), np.array([ref.sum()]), "f32", "total")


def test_full_vocabulary_width():
    """Llama-3 vocabulary 128256 over 4 shards of 32064 columns (the bench
    configuration's row width), 1024 token rows."""
    W = synth.WORKLOADS["vocab_ce_bf16"]
    note("vocab ce full width")
    d = synth.make_ce_inputs(1024, W.h, "bf16", seed=W.seed, row_block=256)
    _check(d, W.n_shards, _run(d, W.n_shards, "bf16"))


def test_rows_of_minus_infinity_and_repeat_is_bitwise():
    """Where one shard's slice of a row is all -inf (a masked vocabulary
    range) that shard's statistics are (-inf, 0) -- the limits of the max and
    of a sum of exp(-inf) -- and the row's log-sum-exp is the other shard's
    alone; a second run gives the same bits."""
    note("vocab ce -inf rows, determinism")
    T_, V, n = 40, 1600, 2
    w = V // n
    d = synth.make_ce_inputs(T_, V, "f32", seed=11)
    d["logits"].f32[:5, w:] = -np.inf
    d["targets"][:5] %= w
    r1 = _run(d, n, "f32")
    r2 = _run(d, n, "f32")
    st = host(r1[0][1])
    assert np.all(st[:5, 0] == -np.inf) and np.all(st[:5, 1] == 0)
    Z = d["logits"].f32
    masked = oracle.vocab_parallel_cross_entropy(Z[:5, :w], d["targets"][:5], 1)
    rest = oracle.vocab_parallel_cross_entropy(Z[5:], d["targets"][5:], n)
    lse = host(r1[1])
    assert_close(lse[:5], masked["lse"], "f32", "lse of masked rows")
    assert_close(lse[5:], rest["lse"], "f32", "lse")
    rows = host(r1[3][0]) + host(r1[3][1])
    assert_close(rows, np.concatenate([masked["rows"], rest["rows"]]), "f32", "row losses")
    for a, b in zip([r1[1], r1[4]] + r1[2] + r1[3], [r2[1], r2[4]] + r2[2] + r2[3]):
        np.testing.assert_array_equal(host(a), host(b))


def test_zero_rows():
    """No token rows: every shard loss and the total are exactly 0."""
    note("vocab ce T=0")
    d = synth.make_ce_inputs(0, 64, "bf16", seed=1)
    stats, lse, losses, rows, total = _run(d, 2, "bf16")
    assert all(host(x)[0] == 0 for x in losses) and host(total)[0] == 0
