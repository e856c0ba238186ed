"""Pins of the oracle's bf16 rounding (the optional gradient convert step).

The rounding is checked against a library routine (torch's CPU float32 ->
bfloat16 conversion, round to nearest even) and against values worked out by
hand from the bit patterns (ties, carries into the exponent, overflow to
infinity, subnormals, signed zeros, NaN)."""
import numpy as np
import torch

import oracle


def _bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def test_matches_torch_rounding_on_random_values():
    rng = np.random.default_rng(7)
    mags = rng.uniform(-140, 126.9, size=200_000)
    x = (rng.choice([-1.0, 1.0], size=mags.size) * np.exp2(mags) * rng.uniform(1, 2, size=mags.size)).astype(np.float32)
    # plus exact ties: a random kept pattern followed by 0x8000 in the dropped half
    ties = ((rng.integers(0, 0x7F7F, size=20_000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to_bf16_bits(x), want)


def test_hand_worked_patterns():
    cases = {
        0x3F800000: 0x3F80,   # 1.0 exactly
        0x3F808000: 0x3F80,   # 1 + 2^-8: tie, kept pattern even -> stays
        0x3F818000: 0x3F82,   # 1 + 3 * 2^-8: tie, kept pattern odd -> up to even
        0x3F808001: 0x3F81,   # just above the tie -> up
        0x3F807FFF: 0x3F80,   # just below the tie -> down
        0x3FFF8000: 0x4000,   # tie at the top of a binade: carries into the exponent
        0x7F7FFFFF: 0x7F80,   # largest float32 rounds to +inf
        0x7F800000: 0x7F80,   # +inf
        0xFF800000: 0xFF80,   # -inf
        0x00000000: 0x0000,   # +0
        0x80000000: 0x8000,   # -0
        0x00000001: 0x0000,   # smallest subnormal rounds to +0
        0x00008000: 0x0000,   # subnormal tie, even -> down
        0x00018000: 0x0002,   # subnormal tie, odd -> up
        0x807FFFFF: 0x8080,   # largest negative subnormal rounds up to the smallest normal
    }
    x = np.array(list(cases), dtype=np.uint32).view(np.float32)
    got = oracle.round_to_bf16_bits(x)
    assert [int(g) for g in got] == list(cases.values())


def test_nan_stays_nan():
    x = np.array([0x7FC00000, 0x7F800001, 0xFFC00123, 0x7FBFFFFF], dtype=np.uint32).view(np.float32)
    got = oracle.round_to_bf16_bits(x)
    assert all((g & 0x7F80) == 0x7F80 and (g & 0x007F) != 0 for g in got)
    assert [(g >> 15) for g in got] == [0, 0, 1, 0]
