"""Pins of the oracle's elementary operations against library routines and
closed forms (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.numerics import rms_norm, rope, round_bf16, softmax
from oracle.sampler import philox4x64_10, uniforms


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-8, 8, 10000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125, 3.0e38]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x32), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 sits halfway between bf16 neighbours 1 and 1 + 2^-7: even is 1.
    assert round_bf16(np.float32(1.0 + 2 ** -8)) == 1.0
    # 1 + 3*2^-8 sits halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert round_bf16(np.float32(1.0 + 3 * 2 ** -8)) == 1.0 + 2 ** -6


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96))
    g = rng.uniform(0.5, 1.5, 96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(rms_norm(x, g, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_rope_complex_closed_form():
    # Rotate-half RoPE is multiplication of z_d = x_d + i x_{d+D/2} by
    # exp(i * pos * theta^(-2d/D)).
    rng = np.random.default_rng(3)
    D, theta = 16, 10000.0
    x = rng.standard_normal((5, 3, D))
    pos = np.array([0, 1, 7, 1000, 131071])
    y = rope(x, pos, theta)
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    w = theta ** (-np.arange(half) * 2.0 / D)
    zr = z * np.exp(1j * pos[:, None, None] * w[None, None, :])
    np.testing.assert_allclose(y[..., :half], zr.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., half:], zr.imag, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(y[0], x[0])                     # position 0 = identity
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_matches_transformers():
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb
    rng = np.random.default_rng(4)
    D, theta = 16, 10000.0
    pos = np.arange(0, 40, 3)
    q = rng.standard_normal((len(pos), 2, D))
    inv = 1.0 / (theta ** (torch.arange(0, D, 2, dtype=torch.float64) / D))
    freqs = torch.from_numpy(pos.astype(np.float64))[:, None] * inv[None, :]
    emb = torch.cat([freqs, freqs], dim=-1)
    cos, sin = emb.cos()[None], emb.sin()[None]
    qt = torch.from_numpy(q).transpose(0, 1)[None]            # [1, heads, seq, D]
    ref, _ = apply_rotary_pos_emb(qt, qt, cos, sin)
    ref = ref[0].transpose(0, 1).numpy()
    np.testing.assert_allclose(rope(q, pos, theta), ref, rtol=1e-12, atol=1e-12)


def test_softmax_weighted_sum_matches_sdpa():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 16))
    k = rng.standard_normal((20, 16))
    v = rng.standard_normal((20, 16))
    mask = rng.uniform(size=(6, 20)) < 0.7
    mask[:, 0] = True
    ours = np.stack([softmax(k[mask[i]] @ q[i] / 4.0) @ v[mask[i]] for i in range(6)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(mask)[None])[0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 6, 7, 8), (123, 456)),
    ((2 ** 64 - 2, 2 ** 63, 12345678901234, 2 ** 64 - 1), (2 ** 64 - 1, 987654321)),
    ((31, 3, 199, 0), (0, 63)),
])
def test_philox_matches_numpy(ctr, key):
    # numpy's Philox bit generator advances the counter by one before each
    # block of four outputs.
    whole = sum(c << (64 * i) for i, c in enumerate(ctr))
    whole = (whole - 1) % 2 ** 256
    prev = [(whole >> (64 * i)) & (2 ** 64 - 1) for i in range(4)]
    bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    ref = bg.random_raw(4)
    got = philox4x64_10(tuple(np.array([c], dtype=np.uint64) for c in ctr), key)
    assert [int(g[0]) for g in got] == [int(r) for r in ref]


def test_uniforms_are_exact_float32_in_open_interval():
    u = uniforms(7, 3, 11, 2, 4099)
    assert u.min() > 0.0 and u.max() < 1.0
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
    # 23-bit grid with a half-step offset
    k = u * 2 ** 23 - 0.5
    np.testing.assert_array_equal(k, np.round(k))
    # tokens 8..15 read the four words of counter block 1: bits 63..41 of word
    # j for token 8 + 2j, bits 40..18 for token 8 + 2j + 1
    w = philox4x64_10((np.array([1], dtype=np.uint64), np.array([2], dtype=np.uint64),
                       np.array([11], dtype=np.uint64), np.array([0], dtype=np.uint64)), (7, 3))
    for j in range(4):
        assert u[8 + 2 * j] == ((int(w[j][0]) >> 41) + 0.5) * 2.0 ** -23
        assert u[8 + 2 * j + 1] == (((int(w[j][0]) >> 18) & 0x7FFFFF) + 0.5) * 2.0 ** -23
