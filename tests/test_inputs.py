"""The seeded input generator (CPU only): deterministic, and its samples follow
the stated recipe (Q, V ~ N(0, 1); K = N(0, 1) noise plus one N(0, 0.5^2)
offset vector per (sequence, KV head, block))."""

import numpy as np
import torch

import moba_inputs


def test_same_seed_same_bytes_and_seeds_differ():
    w = moba_inputs.custom("gen", "bf16", 2, 300, 700, 4, 2, 64, 128, 3, 5)
    a = moba_inputs.make_inputs(w)
    b = moba_inputs.make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = moba_inputs.make_inputs(moba_inputs.custom("gen", "bf16", 2, 300, 700, 4, 2, 64, 128,
                                                   3, 6))
    assert not torch.equal(a[1], c[1])
    # shapes: batched / chunked form [S, L, heads, D]
    assert a[0].shape == (2, 300, 4, 64) and a[1].shape == (2, 700, 2, 64)


def test_samples_follow_the_recipe():
    B, L, D = 64, 8192, 128
    w = moba_inputs.custom("stats", "f32", 1, L, None, 2, 1, D, B, 3, 9)
    q, k, v = (t.double().numpy() for t in moba_inputs.make_inputs(w))
    for name, x in (("q", q), ("v", v)):
        assert abs(x.mean()) < 0.01, name
        assert abs(x.std() - 1.0) < 0.01, name
    kb = k[:, 0].reshape(L // B, B, D)
    means = kb.mean(axis=1)              # per block: offset + N(0, 1/B) noise
    noise = kb - means[:, None, :]
    # offsets ~ N(0, 0.25): the block means' spread is 0.25 + 1/B around 0
    assert abs(means.var() - (0.25 + 1.0 / B)) < 0.02, means.var()
    assert abs(noise.var() * B / (B - 1) - 1.0) < 0.01, noise.var()
    # the offset is shared by every token of a block: the block means of two
    # halves of each block agree up to the noise
    half = kb[:, : B // 2].mean(axis=1) - kb[:, B // 2:].mean(axis=1)
    assert abs(half.var() - 4.0 / B) < 0.01, half.var()


def test_bf16_is_the_rounded_float32_draw():
    """bf16 workloads are the float32 draws rounded to nearest even: the same
    seed in float32, rounded, gives the same bytes."""
    wb = moba_inputs.custom("r", "bf16", 1, 256, None, 2, 1, 64, 64, 3, 11)
    wf = moba_inputs.custom("r", "f32", 1, 256, None, 2, 1, 64, 64, 3, 11)
    for xb, xf in zip(moba_inputs.make_inputs(wb), moba_inputs.make_inputs(wf)):
        assert torch.equal(xb.view(torch.int16), xf.to(torch.bfloat16).view(torch.int16))
    assert np.isfinite(moba_inputs.make_inputs(wb)[0].float().numpy()).all()
