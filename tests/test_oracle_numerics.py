"""Pins for the oracle's storage-type conversions (oracle/numerics.py).

The bf16 branch of as_f64 (uint16 bit patterns shifted into the top half of
a float32) is checked against torch's own bfloat16 -> float64 conversion on
every one of the 65,536 bit patterns: a wrong shift, sign or byte order fails
here.  NaN patterns are compared as NaN."""
import numpy as np

from oracle.numerics import as_f64, f64_to_f16_bits


def test_bf16_upcast_matches_torch_on_every_bit_pattern():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = as_f64(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert int((~nan).sum()) == 65536 - 2 * 127     # exponent all ones, mantissa != 0: NaN
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros and infinities keep their sign
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0 and not np.signbit(got[0])
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x0001] == 2.0 ** -133


def test_f16_upcast_and_rounding_are_exact_on_every_bit_pattern():
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    got = as_f64(x, "f16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # a value that is already fp16 rounds to itself
    assert np.array_equal(f64_to_f16_bits(got[~nan]), bits[~nan])
