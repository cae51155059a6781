"""CPU checks of the synthetic-input generator (synth/)."""
import numpy as np
import torch

import synth


def test_mix64_published_values():
    """SplitMix64 with seed 0: the first outputs of the published generator (state advanced by
    the golden gamma, output = mix64(state)) are 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4."""
    g = 0x9E3779B97F4A7C15
    assert synth.mix64(g) == 0xE220A8397B1DCDAF
    assert synth.mix64((2 * g) % 2 ** 64) == 0x6E789E6AA1B965F4


def test_streams_deterministic_and_distinct():
    a = synth.matrix(0, 3, 7, synth.GATE, 64, 256, 4)
    b = synth.matrix(0, 3, 7, synth.GATE, 64, 256, 4)
    c = synth.matrix(0, 3, 8, synth.GATE, 64, 256, 4)
    d = synth.matrix(1, 3, 7, synth.GATE, 64, 256, 4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert not np.array_equal(a[0], d[0])


def test_code_bytes_are_the_hash_stream():
    codes, _, _ = synth.matrix(5, 1, 2, synth.DOWN, 32, 128, 4)
    key = synth.stream(5, synth.TAG_CODES, 1, 2, synth.DOWN)
    flat = codes.reshape(-1)
    for w in range(flat.size // 8):
        h = synth.hash_at(key, w)
        assert bytes(flat[8 * w:8 * w + 8]) == h.to_bytes(8, "little")


def test_distributions():
    codes, scale, bias = synth.matrix(0, 0, 0, synth.GATE, 1024, 4096, 4)
    lo = codes & 0x0F
    hi = codes >> 4
    counts = np.bincount(np.concatenate([lo.ravel(), hi.ravel()]), minlength=16)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()
    s = synth.bf16_to_f32(scale)
    b = synth.bf16_to_f32(bias)
    assert s.min() >= 0.000999 and s.max() <= 0.0201
    assert b.min() >= -0.1001 and b.max() <= 0.1001
    assert abs(float(s.mean()) - 0.0105) < 2e-4 and abs(float(b.mean())) < 2e-3
    r = synth.router(0, 0, 512, 4096)
    assert abs(float(r.std()) - 0.02) < 2e-4 and abs(float(r.mean())) < 2e-5
    x = synth.token(0, 0, 4096)
    assert abs(float(x.std()) - 1.0) < 0.05


def test_bf16_bits_match_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000)).astype(np.float32)
    want = torch.tensor(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(v), want)


def test_two_bit_codes_uniform():
    codes, _, _ = synth.matrix(0, 0, 0, synth.UP, 1024, 4096, 2)
    vals = np.concatenate([(codes >> (2 * t)) & 3 for t in range(4)]).ravel()
    counts = np.bincount(vals, minlength=4)
    assert counts.min() > 0.98 * counts.mean()


def test_three_bit_codes_uniform():
    """3-bit matrices take rows * cols * 3 / 8 bytes of the hash stream, so every code 0..7
    is equally likely (decoded here as a little-endian bit stream, 3 bits per column)."""
    rows, cols = 256, 512
    codes, scale, bias = synth.matrix(0, 0, 0, synth.GATE, rows, cols, 3)
    assert codes.shape == (rows, cols * 3 // 8) and scale.shape == (rows, cols // 64)
    bits = np.unpackbits(codes, axis=1, bitorder="little").reshape(rows, cols, 3).astype(np.int64)
    q = bits[:, :, 0] + 2 * bits[:, :, 1] + 4 * bits[:, :, 2]
    freq = np.bincount(q.ravel(), minlength=8) / q.size
    assert np.all(np.abs(freq - 0.125) < 0.005)
