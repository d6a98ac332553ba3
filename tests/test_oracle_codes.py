"""Pins for the oracle's computed codes (1MAD, 3INST) against what the pages print
and what the mathematics fixes.  CPU only.

Sources: QTIP blog, section "The codebook is computed" (1MAD listing and its comment,
3INST prose, the 908-distinct-values and raw-sigma remarks); XOR-Trellis explainer,
section "The sign at each junction has to be cheap" (3INST ends in an FP16 add).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")))


@pytest.fixture(scope="module")
def c1mad16():
    return oracle.code_table("1mad", 16)


@pytest.fixture(scope="module")
def raw3inst16():
    return np.array([oracle.code_3inst_raw(x) for x in range(1 << 16)])


def test_1mad_distinct_values_printed(c1mad16):
    # the page counts the distinct 1MAD outputs over all 2^16 states
    assert len(np.unique(c1mad16)) == GOLD["code_1mad_distinct_values_L16"]["value"]


def test_1mad_values_are_rescaled_byte_sums(c1mad16):
    # every value is (S - 510) / 147.8 for an integer byte sum S in [0, 1020]
    S = c1mad16.astype(np.float64) * 147.8 + 510.0
    Si = np.rint(S)
    assert np.all(np.abs(S - Si) < 1e-3)
    assert Si.min() >= 0 and Si.max() <= 1020
    # and the rounding to binary32 is a single rounding of the binary64 quotient
    q = ((Si - 510.0) / 147.8).astype(np.float32)
    assert np.array_equal(q.view(np.uint32), c1mad16.view(np.uint32))


def test_1mad_irwin_hall_moments(c1mad16):
    # the sum of 4 uniform bytes has mean 4 * 127.5 = 510 and variance 4 (256^2 - 1) / 12,
    # so the rescaled code is close to zero mean and unit variance over the states
    mu = GOLD["code_1mad_bytesum_mean"]["value"]
    sd = GOLD["code_1mad_bytesum_sigma"]["value"]
    assert mu == 4 * 127.5
    assert abs(sd - np.sqrt(4 * (256 ** 2 - 1) / 12)) < 0.05
    assert abs(float(c1mad16.mean())) < 0.02
    assert abs(float(c1mad16.std()) - 1.0) < 0.02


def test_1mad_small_L_is_prefix(c1mad16):
    # the code is a fixed function of the state integer: smaller L takes a prefix
    for L in (6, 8, 12):
        assert np.array_equal(oracle.code_table("1mad", L), c1mad16[: 1 << L])


def test_3inst_magic_is_fp16_nearest():
    m = GOLD["code_3inst_magic"]["value"]
    assert np.float16(m).view(np.uint16) == 0x3B60


def test_3inst_raw_sigma_printed(raw3inst16):
    target = GOLD["code_3inst_raw_sigma"]["value"]
    assert round(float(raw3inst16.std()), 3) == target


def test_3inst_raw_is_fp16_sum_of_two_halves(raw3inst16):
    # each raw value is a binary16 number (the result of an FP16 add) below 4 in size
    assert np.array_equal(raw3inst16.astype(np.float16).astype(np.float64), raw3inst16)
    assert np.all(np.abs(raw3inst16) < 4.0)
    # each half lies in +-[0.125, 2): exponents 12..15 after XOR into 0x3B60's low
    # exponent bits; the sum of two such values cannot be below 2^-13 unless it is 0
    nz = raw3inst16[raw3inst16 != 0]
    assert np.abs(nz).min() >= 2.0 ** -13


def test_3inst_scaled_unit_variance():
    C3 = oracle.code_table("3inst", 16)
    assert abs(float(C3.std()) - 1.0) < 2e-3
    raw = np.array([oracle.code_3inst_raw(x) for x in range(4096)])
    q = (raw / 1.244).astype(np.float32)
    assert np.array_equal(q, C3[:4096])


def test_code_value_scalar_matches_table(c1mad16):
    for x in (0, 1, 12345, 65535):
        assert oracle.code_value("1mad", x) == c1mad16[x]
