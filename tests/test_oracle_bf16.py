"""Pins for the oracle's bf16 decoding (CPU only).

The oracle widens bf16 bit patterns itself.  Here every one of the 65,536
patterns is checked against PyTorch's own bfloat16 -> float64 conversion, an
independent library routine, including signed zeros, subnormals, both
infinities and every NaN payload; and against hand-worked values.
"""
import numpy as np
import torch

import oracle


def _torch_decode(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_every_bit_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits)
    want = _torch_decode(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127                      # exponent all ones, nonzero mantissa
    assert np.array_equal(got[~nan], want[~nan])
    # the sign bit survives everywhere, zeros included
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_hand_worked_values():
    cases = {
        0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3F00: 0.5,
        0x4049: 3.140625,                 # 1.1001001b x 2^1
        0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,   # largest finite
        0x0080: 2.0 ** -126,              # smallest normal
        0x0001: 2.0 ** -133,              # smallest subnormal (2^-126 x 2^-7)
        0x7F80: np.inf, 0xFF80: -np.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = oracle.decode_bf16(bits)
    assert np.array_equal(got, np.array(list(cases.values()), dtype=np.float64))
    neg0 = oracle.decode_bf16(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and np.signbit(neg0)


def test_shapes_and_as_f64():
    bits = np.array([[0x3F80, 0x4000], [0xC040, 0x0000]], dtype=np.uint16)
    got = oracle.decode_bf16(bits)
    assert got.shape == (2, 2) and got.dtype == np.float64
    assert np.array_equal(oracle.as_f64(bits), got)
    f = np.array([1.5, -2.25, 1e-30], dtype=np.float32)
    assert np.array_equal(oracle.as_f64(f), f.astype(np.float64))


def test_generator_encoding_round_trips_like_torch():
    """The generators' float32 -> bf16 rounding (nearest, ties to even) and
    the oracle's decoding, end to end, against torch's own conversion: ties
    in both directions, values that carry into the exponent, the largest
    finite values and overflow to infinity."""
    import synth
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),   # ties: to even
                  1.0 + 2.0 ** -8 + 2.0 ** -20, 2.0 - 2.0 ** -9,               # above a tie; carry
                  3.3895e38, -3.3895e38, 3.4e38, 1e-40, -0.0, 0.0],
                 dtype=np.float32),
    ])
    got = oracle.decode_bf16(synth.round_to_bf16_bits(x))
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
