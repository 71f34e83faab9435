"""Pins for the oracle's number formats: e4m3, e8m0 and bf16 rounding.

Independent references: torch's float8_e4m3fn / float8_e8m0fnu / bfloat16
casts (library routines), the page facts in tests/golden/, and textbook
special cases (ties, double-rounding traps, subnormal and overflow edges).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ e4m3
def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero survives
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_page_facts():
    facts = json.load(open(os.path.join(GOLD, "e4m3_facts.json")))
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = vals[~np.isnan(vals)]
    assert finite.max() == facts["max_finite"]
    assert vals[facts["max_code"]] == facts["max_finite"]
    # 254 finite codes (two NaNs, no infinities), smallest subnormal 2^-9
    assert finite.size == 254
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** -9
    # saturation above the maximum
    sat = np.array([float(v) for v in facts["saturate_inputs"]], np.float32)
    assert np.all(oracle.e4m3_encode(sat) == 0x7E)
    assert np.all(oracle.e4m3_encode(-sat) == 0xFE)
    # every e4m3 value is exactly a bf16 value
    b = oracle.bf16_round(finite)
    assert np.array_equal(oracle.bf16_value(b), finite)


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_midpoints_round_to_even_code():
    # the midpoint of two adjacent positive codes must go to the even one
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2  # exact in float32 (<= 5 significant bits)
    enc = oracle.e4m3_encode(mids.astype(np.float32))
    lo = np.arange(0, 0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, expect.astype(np.uint8))
    # one fp32 ulp either side of a midpoint goes to the nearer code
    up = np.nextafter(mids.astype(np.float32), np.float32(np.inf))
    dn = np.nextafter(mids.astype(np.float32), np.float32(0))
    assert np.array_equal(oracle.e4m3_encode(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.e4m3_encode(dn), lo.astype(np.uint8))


def test_e4m3_encode_sweep_matches_torch_below_overflow():
    # strided sweep over all fp32 bit patterns; torch's cast is RNE and agrees
    # with the page rule wherever |v| <= 464 (above 464 it returns NaN where
    # the page saturates to 448).
    bits = np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) <= 464)
    f = f[keep]
    ours = oracle.e4m3_encode(f)
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_nan_and_inf():
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F
    assert oracle.e4m3_encode(np.array([np.inf], np.float32))[0] == 0x7E
    assert oracle.e4m3_encode(np.array([-np.inf], np.float32))[0] == 0xFE
    assert oracle.e4m3_encode(np.array([-0.0], np.float32))[0] == 0x80
    assert oracle.e4m3_encode(np.array([-1e-9], np.float32))[0] == 0x80


# ------------------------------------------------------------------ e8m0
def test_e8m0_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = np.array([oracle.e8m0_decode(c) for c in range(256)])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_e8m0_page_tie_rule():
    rows = [l.split() for l in open(os.path.join(GOLD, "e8m0_ties.txt"))
            if l.strip() and not l.startswith("#")]
    v = np.array([float(r[0]) for r in rows], np.float32)
    codes = oracle.e8m0_encode(v)
    assert codes.tolist() == [int(r[2]) for r in rows]
    assert [oracle.e8m0_decode(c) for c in codes] == [float(r[1]) for r in rows]
    # one fp32 ulp either side of a tie goes to the nearer power of two
    e = np.arange(-100, 100)
    ties = (1.5 * np.exp2(e.astype(np.float64))).astype(np.float32)
    up = oracle.e8m0_encode(np.nextafter(ties, np.float32(np.inf)))
    dn = oracle.e8m0_encode(np.nextafter(ties, np.float32(0)))
    assert np.array_equal(up, (e + 1 + 127).astype(np.uint8))
    assert np.array_equal(dn, (e + 127).astype(np.uint8))
    # at a tie the result's exponent is even
    at = oracle.e8m0_encode(ties).astype(np.int64) - 127
    assert np.all(at % 2 == 0) and np.all((at == e) | (at == e + 1))


def test_e8m0_non_ties_match_torch():
    # off the ties the page rule and torch's cast agree: nearest power of two
    rng = np.random.default_rng(7)
    v = np.exp2(rng.uniform(-120, 120, 200000)).astype(np.float32)
    m, _ = np.frexp(v.astype(np.float64))
    v = v[2 * m != 1.5]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e8m0_encode(v), ref)
    # documented edges: sign dropped, zero -> 0, NaN/inf -> 255
    assert oracle.e8m0_encode(np.array([-1.0, 0.0, np.nan, np.inf], np.float32)).tolist() == [127, 0, 255, 255]


# ------------------------------------------------------------------ bf16 rounding
def test_bf16_round_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, 500000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_round_special_cases():
    r = lambda v: int(oracle.bf16_round(np.array([v]))[0])
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert r(1 + 2 ** -8) == 0x3F80
    assert r(1 + 3 * 2 ** -8) == 0x3F82
    # a value just above the tie must round up (a detour through fp32 would
    # first land exactly on the tie and then round down to even)
    assert r(1 + 2 ** -8 + 2 ** -40) == 0x3F81
    # subnormals: quantum 2^-133, ties to even
    assert r(2.0 ** -133) == 0x0001
    assert r(1.5 * 2.0 ** -133) == 0x0002
    assert r(0.5 * 2.0 ** -133) == 0x0000
    assert r(0.75 * 2.0 ** -133) == 0x0001
    # overflow: the largest bf16 is (2 - 2^-7) * 2^127; halfway to 2^128 rounds to inf
    assert r((2 - 2 ** -7) * 2.0 ** 127) == 0x7F7F
    assert r((2 - 2 ** -8) * 2.0 ** 127) == 0x7F80
    assert r(-(2 - 2 ** -8) * 2.0 ** 127 * 0.999999) == 0xFF7F
    assert r(float("nan")) == 0x7FC0
    assert r(-0.0) == 0x8000
    assert r(float("-inf")) == 0xFF80
