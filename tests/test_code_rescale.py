"""Host check of the device codes' binary32 rescale (no GPU).  The definition divides
the code's raw value v by D in binary64 (147.8 for 1MAD, 1.244 for 3INST; QTIP blog,
"The codebook is computed") and rounds once to binary32.  The device computes
fma(v, r_lo, v * r_hi) in binary32, with r_hi = 1/D rounded to 13 significant bits
(so v * r_hi is exact) and r_lo = fl32(1/D - r_hi).  That is exact iff it gives the same
binary32 bits on the code's whole input domain: every byte sum minus 510 (1MAD) and
every finite fp16 value below 4 in magnitude (3INST raw values are fp16 sums of two
halves in +-[0.125, 2)).  Both domains are small, so this is checked exhaustively with
exact rational arithmetic.  The split constants are the ones written in codes.hpp.
The search kernels' once-per-workgroup form multiplies by the binary64 reciprocal of
the divisor instead, checked on the same domains."""
from fractions import Fraction

import numpy as np

# (r_hi, r_lo) as binary32 bit patterns, as in codes.hpp
SPLIT_1MAD = (0x3BDDB800, 0xB4E12B4D)
SPLIT_3INST = (0x3F4DC800, 0x37D604F0)


def f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def round_f32(x: Fraction) -> np.float32:
    """Nearest binary32 to the exact rational x, ties to even."""
    c = np.float32(float(x))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        key = (abs(Fraction(float(cand)) - x), int(np.array(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def device_rescale(v: float, split) -> np.float32:
    r_hi, r_lo = (Fraction(float(f32(b))) for b in split)
    p = Fraction(v) * r_hi
    assert Fraction(float(np.float32(float(p)))) == p          # v * r_hi is exact in binary32
    if v == 0:   # signed zeros: exact zero products, IEEE sum of zeros (as the FMA does)
        z = np.float32(v)
        return np.float32(z * f32(split[1]) + z * f32(split[0]))
    return round_f32(Fraction(v) * r_lo + p)


def check(values, D, split):
    for v in values:
        v = float(v)
        want = np.float32(np.float64(v) / np.float64(D))
        got = device_rescale(v, split)
        assert np.array(got).view(np.uint32) == np.array(want).view(np.uint32), v


def test_split_constants():
    for D, split in ((147.8, SPLIT_1MAD), (1.244, SPLIT_3INST)):
        r = Fraction(1) / Fraction(D)
        r_hi = Fraction(float(f32(split[0])))
        assert r_hi.numerator.bit_length() <= 13        # odd numerator over a power of 2
        assert abs(r - r_hi) <= r * Fraction(1, 2 ** 13)
        assert f32(split[1]) == np.float32(float(r - r_hi))


def test_1mad_rescale_exact_on_all_byte_sums():
    check(np.arange(0, 1021) - 510, 147.8, SPLIT_1MAD)


def test_3inst_rescale_exact_on_all_fp16_values():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float64)
    check(h[np.abs(h) < 4], 1.244, SPLIT_3INST)


def test_1mad_binary64_reciprocal_exact_on_all_byte_sums():
    num = (np.arange(0, 1021, dtype=np.int64) - 510).astype(np.float64)
    want = (num / 147.8).astype(np.float32)
    got = (num * (1.0 / 147.8)).astype(np.float32)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))


def test_3inst_binary64_reciprocal_exact_on_all_fp16_values():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float64)
    want = (h / 1.244).astype(np.float32)
    got = (h * (1.0 / 1.244)).astype(np.float32)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))
