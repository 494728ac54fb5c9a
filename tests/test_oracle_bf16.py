"""Pin of the oracle's bf16 widening against an independent decoder (CPU only).

Every one of the 65,536 bfloat16 bit patterns is widened by the oracle and by
torch's own bfloat16 -> float64 conversion.  They must agree bit for bit on
every non-NaN pattern (signed zeros, subnormals and infinities included), and
both must give NaN on exactly the NaN patterns (exponent all ones, mantissa
non-zero).  A third, arithmetic decoding from the IEEE fields -- sign,
biased exponent, 7-bit mantissa -- pins the same values without either
library.
"""

import math

import numpy as np
import torch

import oracle


ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _fields_decode(bits: int) -> float:
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if man == 0 else math.nan
    if exp == 0:
        return sign * man * 2.0 ** (-126 - 7)          # subnormal (and signed zero)
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


def test_every_bf16_pattern_against_torch():
    ours = oracle.bf16_bits_to_f64(ALL)
    ref = torch.from_numpy(ALL.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    np.testing.assert_array_equal(nan_ours, nan_ref)
    exp_all_ones = (ALL.astype(np.uint32) >> 7) & 0xFF == 0xFF
    man_nonzero = (ALL.astype(np.uint32) & 0x7F) != 0
    np.testing.assert_array_equal(nan_ours, exp_all_ones & man_nonzero)
    keep = ~nan_ours
    # bit-for-bit (so -0.0 stays -0.0)
    np.testing.assert_array_equal(ours[keep].view(np.uint64), ref[keep].view(np.uint64))


def test_every_bf16_pattern_against_the_ieee_fields():
    ours = oracle.bf16_bits_to_f64(ALL)
    for bits in range(1 << 16):
        want = _fields_decode(bits)
        got = float(ours[bits])
        if math.isnan(want):
            assert math.isnan(got), hex(bits)
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), hex(bits)


def test_as_f64_dispatch():
    bits = np.array([0x3F80, 0xC000, 0x0001], dtype=np.uint16)     # 1, -2, smallest subnormal
    np.testing.assert_array_equal(oracle.as_f64(bits, "bf16"), [1.0, -2.0, 2.0 ** -133])
    f = np.array([0.1, -3.5], dtype=np.float32)
    np.testing.assert_array_equal(oracle.as_f64(f, "f32"), f.astype(np.float64))
