"""Pins of the oracle's storage rounding (oracle/storage.py).

round_f64_to_bf16_bits defines the reference of every bf16 tensor the
serving-precision oracle materialises, so it is pinned here by values
worked out by hand from the bf16 format (1 sign bit, 8 exponent bits, 7
stored mantissa bits: 8 significant bits) and round-to-nearest-even, and by
two independent routines on float32-exact inputs.
"""
import numpy as np
import pytest

from oracle import storage

E = 2.0 ** -8        # half an ulp of bf16 at [1, 2)

# value, expected bf16 bits, what the case checks
HAND = [
    (1.0, 0x3F80, "exact"),
    (0.0, 0x0000, "zero"),
    (-0.0, 0x8000, "negative zero keeps its sign"),
    (1.0 + E, 0x3F80, "tie between 0x3F80 and 0x3F81 goes to the even mantissa"),
    (1.0 + 3 * E, 0x3F82, "tie between 0x3F81 and 0x3F82 goes to the even mantissa"),
    (1.0 + E + 2.0 ** -30, 0x3F81, "just above a tie rounds up"),
    (1.0 + E - 2.0 ** -30, 0x3F80, "just below a tie rounds down"),
    (1.0 + E + 2.0 ** -40, 0x3F81, "above a tie by less than float32 resolves: no double rounding"),
    (1.0 + 3 * E - 2.0 ** -40, 0x3F81, "below a tie by less than float32 resolves: no double rounding"),
    (2.0 - 2.0 ** -9, 0x4000, "rounding up carries into the exponent"),
    (2.0 - 2.0 ** -8, 0x4000, "tie below 2 goes to the even mantissa of 2.0"),
    (2.0 - 2.0 ** -7, 0x3FFF, "largest bf16 below 2"),
    (-(1.0 + 3 * E), 0xBF82, "negative tie"),
    (-(1.0 + E + 2.0 ** -40), 0xBF81, "negative, above a tie"),
    (3.141592653589793, 0x4049, "pi: 1.1001001|0... rounds down to 3.140625"),
    (0.1, 0x3DCD, "0.1: 1.1001100|11... rounds up"),
    (2.0 ** -126, 0x0080, "smallest normal"),
    (3.3895313892515355e38, 0x7F7F, "largest finite bf16"),
    (1.0 / 3.0, 0x3EAB, "1/3: 1.0101010|10... rounds up"),
    (-1000.0, 0xC47A, "-1000 = -1.1111010 x 2^9, exact"),
]


@pytest.mark.parametrize("value,bits,what", HAND, ids=[h[2] for h in HAND])
def test_round_to_bf16_hand_cases(value, bits, what):
    got = int(storage.round_f64_to_bf16_bits(np.array([value]))[0])
    assert got == bits, f"{what}: {value!r} -> {got:#06x}, expected {bits:#06x}"


def test_round_to_bf16_decodes_to_nearest():
    """Brute force on a grid: the decoded result is a bf16 value no farther
    from x than any other bf16 value (checked against its two neighbours),
    and on an exact tie it has an even mantissa."""
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-6, 6, 20000),
                        g.uniform(-4, 4, 20000)])
    bits = storage.round_f64_to_bf16_bits(x).astype(np.int64)
    y = storage.bf16_bits_to_f64(bits.astype(np.uint16))
    mag = bits & 0x7FFF
    sign = bits & 0x8000
    up = storage.bf16_bits_to_f64((sign | (mag + 1)).astype(np.uint16))
    down = storage.bf16_bits_to_f64((sign | np.maximum(mag - 1, 0)).astype(np.uint16))
    d = np.abs(x - y)
    assert np.all(d <= np.abs(x - up))
    assert np.all(d <= np.abs(x - down))
    tie = (d == np.abs(x - up)) | ((mag > 0) & (d == np.abs(x - down)))
    assert np.all((mag[tie] & 1) == 0)


def test_round_to_bf16_matches_float32_routines():
    """On float32-exact inputs (where no double rounding can arise) the
    direct float64 rounding agrees with torch's float32 -> bfloat16
    conversion and with the integer rounding of the stored-input encoder."""
    import torch
    g = np.random.default_rng(1)
    x32 = (g.standard_normal(100000) * 10.0 ** g.integers(-8, 8, 100000)).astype(np.float32)
    ours = storage.round_f64_to_bf16_bits(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    u = x32.view(np.uint32).astype(np.uint64)
    manual = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(ours, manual)
