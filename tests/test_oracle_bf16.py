"""Pin of oracle.bf16_to_f64, the decode every GPU comparison goes through,
over all 65,536 bit patterns: against torch's bfloat16 -> float64 conversion
(a library routine) and against the IEEE-754 binary32 field definition
(bf16 is the top half of a binary32: sign, 8 exponent bits, 7 fraction bits)."""
import math

import numpy as np
import torch

import oracle


def _ieee(bits: int) -> float:
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    sign = -1.0 if s else 1.0
    if e == 0xFF:
        return math.nan if m else sign * math.inf
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)          # subnormal (and signed zero)
    return sign * math.ldexp(128 + m, e - 127 - 7)


def test_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):                                     # NaN payloads
        got = oracle.bf16_to_f64(bits)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ref_i = np.array([_ieee(int(b)) for b in bits])
    for ref in (ref_t, ref_i):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))   # -0.0 stays -0.0
    assert int(np.isnan(got).sum()) == 2 * 127                                 # 0x7F81..0x7FFF, 0xFF81..0xFFFF
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x0001] == 2.0 ** -133
