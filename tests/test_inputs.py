"""The seeded input generator's bf16 encoder against IEEE-754 round to
nearest, ties to even, on hand-worked bit patterns, and against torch's own
float32 -> bfloat16 cast on random and special values."""
import numpy as np
import torch

import gdn_inputs as gi

# (float32 bits, expected bf16 bits): the upper 16 bits of the word, rounded
# on the lower 16 by nearest, ties to the even upper half
CASES = [
    (0x3F800000, 0x3F80),  # 1.0, exact
    (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway, 0x3F80 is even
    (0x3F818000, 0x3F82),  # 1 + 3 2^-8: halfway, 0x3F82 is even
    (0x3F808001, 0x3F81),  # just above halfway
    (0x3F807FFF, 0x3F80),  # just below halfway
    (0xBF808000, 0xBF80),  # negative tie
    (0xBF818000, 0xBF82),
    (0x7F7FFFFF, 0x7F80),  # largest float32 rounds to +inf
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
    (0x00000000, 0x0000),  # +0
    (0x80000000, 0x8000),  # -0
    (0x00008000, 0x0000),  # subnormal tie to even (0)
    (0x00018000, 0x0002),  # subnormal tie to even (2)
    (0x00017FFF, 0x0001),
    (0x7FFF8000, 0x7FC0),  # NaN (payload would carry into the sign): quiet NaN
    (0x7FC00000, 0x7FC0),  # quiet NaN
    (0xFFC00001, 0x7FC0),  # negative NaN: quiet NaN
]


def test_bf16_encoder_cases():
    bits = np.array([c[0] for c in CASES], dtype=np.uint32)
    got = gi.f32_to_bf16_bits(bits.view(np.float32))
    want = np.array([c[1] for c in CASES], dtype=np.uint16)
    for (src, exp), g in zip(CASES, got):
        assert int(g) == exp, f"{src:#010x} -> {int(g):#06x}, expected {exp:#06x}"
    assert np.array_equal(got, want)


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(1 << 20).astype(np.float32),
        (rng.standard_normal(1 << 16) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(1 << 16) * 1.5e38).clip(-3.4e38, 3.4e38).astype(np.float32),  # near overflow
        rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64).astype(np.uint32).view(np.float32),  # every pattern kind
    ])
    got = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(gi.bf16_bits_to_f32(got[nan])))


def test_bf16_round_trip_exact():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = gi.bf16_bits_to_f32(bits)
    back = gi.f32_to_bf16_bits(f)
    ok = ~np.isnan(f)
    assert np.array_equal(back[ok], bits[ok])
