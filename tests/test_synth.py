"""The seeded input generator: bf16 rounding and reproducible draws."""
import numpy as np
import torch

import synth


def test_bf16_round_to_nearest_even_known_patterns():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)           # bf16 spacing at 1.0
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0, 0.0,
                     1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    bits = synth.round_to_bf16_bits(vals)
    # halfway 1 + ulp/2 ties to even (1.0); 1 + 3/2 ulp ties to even (1 + 2 ulp)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000, 0x3F81]
    back = synth.bf16_bits_to_f32(bits)
    assert back[2] == one + 2 * ulp


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = synth.round_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_draws_are_reproducible_and_ordered():
    a = synth.make_mlp_inputs(32, 128, 512, "f32", seed=0)
    b = synth.make_mlp_inputs(32, 128, 512, "f32", seed=0)
    for k in ("X", "W1", "W2"):
        assert np.array_equal(a[k].f32, b[k].f32)
    # X is drawn first from the stream
    x0 = np.random.default_rng(0).standard_normal((32, 128), dtype=np.float32)
    assert np.array_equal(a["X"].f32, x0)
    # row-block drawing consumes the same stream
    c = synth.make_mlp_inputs(32, 128, 512, "f32", seed=0, row_block=7)
    for k in ("X", "W1", "W2"):
        assert np.array_equal(a[k].f32, c[k].f32)


def test_shard_slicing_is_contiguous_blocks():
    d = synth.make_mha_inputs(4, 32, "bf16", seed=0)
    q = synth.qkv_shard(d["Wq"], d["Wk"], d["Wv"], 1, 4, 8)
    assert q.shape == (32, 24)
    assert np.array_equal(q.f32[:, :8], d["Wq"].f32[:, 8:16])
    assert np.array_equal(q.bits[:, 16:], d["Wv"].bits[:, 8:16])
    assert np.array_equal(synth.out_shard(d["Wo"], 3, 4).f32, d["Wo"].f32[24:32])
