"""CPU pin of the E4M3 decoding the FP8 parity tests rely on (marker: not gpu).

The FP8 tests give the oracle the exact values of the E4M3 inputs, decoded by
torch's float8_e4m3fn conversion.  That decoding is pinned here to the OCP
8-bit floating point definition written out: sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 gives subnormals m * 2^-9; the
all-ones pattern S.1111.111 is NaN and there is no infinity, so the largest
finite value is 1.75 * 2^8 = 448.
"""

import math

import torch


def decode_e4m3(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_every_code_decodes_as_defined():
    codes = torch.arange(256, dtype=torch.uint8)
    got = codes.view(torch.float8_e4m3fn).float().tolist()
    for c in range(256):
        want = decode_e4m3(c)
        if math.isnan(want):
            assert math.isnan(got[c]), c
        else:
            assert got[c] == want, (c, got[c], want)


def test_extremes_and_rounding():
    assert decode_e4m3(0x7E) == 448.0 and decode_e4m3(0x01) == 2.0 ** -9
    # encoding rounds to nearest, ties to even: 1 + 1/16 lies halfway between
    # 1 and 1.125 and goes to the even mantissa 1; 1 + 3/16 goes to 1.25
    x = torch.tensor([1.0 + 1 / 16, 1.0 + 3 / 16, 0.3]).to(torch.float8_e4m3fn).float().tolist()
    assert x[0] == 1.0 and x[1] == 1.25 and x[2] == 0.3125
