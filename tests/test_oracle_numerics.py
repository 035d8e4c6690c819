"""Pins for the oracle's scalar numerics: the router sigmoid and the E4M3 codec.

Nothing here compares the oracle with itself.  The sigmoid is checked against
the FP64 mathematical function, the codec against the OCP OFP8 E4M3 format's
defining values and against torch's independent float8_e4m3fn conversion.
"""
import math

import numpy as np
import pytest
import torch


def _ulp32(v: np.ndarray) -> np.ndarray:
    """Spacing of binary32 numbers at |v| (subnormal spacing below FLT_MIN)."""
    a = np.abs(v).astype(np.float32)
    return np.maximum(np.spacing(a).astype(np.float64), 2.0 ** -149)


# ------------------------------------------------------------------ sigmoid / exp
def test_exp_spec_special_values(oracle_mod):
    assert oracle_mod.exp_spec(0.0) == 1.0
    assert oracle_mod.exp_spec(-100.0) == 0.0
    assert oracle_mod.exp_spec(100.0) == math.inf
    # near multiples of ln 2 the reduced argument is ~0 and p(r) ~ 1
    for n in (-20, -1, 1, 7, 30):
        y = float(np.float32(n * math.log(2)))
        ref = math.exp(y)
        assert abs(oracle_mod.exp_spec(y) - ref) <= 2 * float(_ulp32(np.array([ref]))[0])


def test_exp_spec_accuracy_vs_fp64(oracle_mod):
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-87, 88.72, 2_000_000),
                        np.linspace(-87, 88.72, 200_001)]).astype(np.float32)
    got = oracle_mod.exp_spec_array(y).astype(np.float64)
    ref = np.exp(y.astype(np.float64))
    err_ulp = np.abs(got - ref) / _ulp32(ref)
    assert err_ulp.max() <= 2.0, err_ulp.max()


def test_sigmoid_spec_accuracy_vs_fp64(oracle_mod):
    """Within 4 binary32 ulps of the FP64 sigmoid wherever the result is a
    normal number (x >= -87); exactly 0.5 at 0; in [0, 1] everywhere."""
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.normal(0, 2, 2_000_000), rng.uniform(-87, 90, 1_000_000),
                        np.linspace(-87, 40, 300_001)]).astype(np.float32)
    got = oracle_mod.sigmoid_spec_array(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    err_ulp = np.abs(got - ref) / _ulp32(ref)
    assert err_ulp.max() <= 4.0, err_ulp.max()
    assert oracle_mod.sigmoid_spec(0.0) == 0.5
    assert np.all((got >= 0) & (got <= 1))


def test_sigmoid_spec_symmetry_and_tails(oracle_mod):
    x = np.linspace(-30, 30, 100_001).astype(np.float32)
    s = oracle_mod.sigmoid_spec_array(x).astype(np.float64)
    sm = oracle_mod.sigmoid_spec_array(-x).astype(np.float64)
    assert np.max(np.abs(s + sm - 1.0)) <= 4 * 2.0 ** -24
    assert oracle_mod.sigmoid_spec(120.0) == 1.0
    assert oracle_mod.sigmoid_spec(-120.0) == 0.0   # exp_spec saturates to +inf


def test_sigmoid_spec_monotone_on_router_range(oracle_mod):
    """Non-decreasing over a fine sweep of the logit range the router sees."""
    x = np.arange(-12.0, 12.0, 1.0 / 4096, dtype=np.float32)
    s = oracle_mod.sigmoid_spec_array(x)
    assert np.all(np.diff(s.astype(np.float64)) >= 0)


# ------------------------------------------------------------------ E4M3 codec
def test_e4m3_defining_values(oracle_mod):
    """OCP OFP8 E4M3: bias 7, 3 mantissa bits, max normal 448 (S.1111.110),
    NaN only at S.1111.111, min normal 2^-6, min subnormal 2^-9."""
    dec = oracle_mod.e4m3_decode
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert math.isnan(dec(0x7F)) and math.isnan(dec(0xFF))
    assert dec(0x38) == 1.0
    assert dec(0x08) == 2.0 ** -6
    assert dec(0x07) == 7 * 2.0 ** -9
    assert dec(0x01) == 2.0 ** -9
    assert dec(0x00) == 0.0 and math.copysign(1, dec(0x80)) == -1.0
    assert dec(0x40) == 2.0 and dec(0x3F) == 1.875
    vals = np.array([dec(c) for c in range(0x7F)])
    assert np.all(np.diff(vals) > 0), "magnitude codes must increase with value"
    finite = [c for c in range(256) if not math.isnan(dec(c))]
    assert len(finite) == 254


def test_e4m3_roundtrip_every_code(oracle_mod):
    for c in range(256):
        v = oracle_mod.e4m3_decode(c)
        if math.isnan(v):
            continue
        assert oracle_mod.e4m3_encode(v) == c


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_all_bf16(oracle_mod):
    """Round-to-nearest-even against torch's float8_e4m3fn conversion over
    every bf16 bit pattern below the overflow threshold 464."""
    x = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 464)]
    np.testing.assert_array_equal(oracle_mod.e4m3_encode_array(x), _torch_e4m3(x))


def test_e4m3_encode_matches_torch_near_midpoints(oracle_mod):
    """+-4 binary32 ulps around every midpoint between neighbouring codes
    (where a rounding mistake would show), plus a random sample."""
    vals = np.array([oracle_mod.e4m3_decode(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    pts = []
    for m in mids:
        b = np.array([m], np.float32).view(np.int32)[0]
        pts.extend(np.arange(b - 4, b + 5, dtype=np.int32).view(np.float32))
    pts = np.array(pts, np.float32)
    pts = np.concatenate([pts, -pts])
    rng = np.random.default_rng(3)
    sample = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-12, 6, 1_000_000))).astype(np.float32)
    sample = sample[np.abs(sample) < 464]
    x = np.concatenate([pts, sample])
    np.testing.assert_array_equal(oracle_mod.e4m3_encode_array(x), _torch_e4m3(x))


def test_e4m3_saturation_and_nan(oracle_mod):
    """Finite overflow saturates to +-448; NaN keeps its sign with mantissa 111."""
    x = np.array([448.0, 463.99, 464.0, 1e6, 3.4e38, np.inf, -500.0, -np.inf], np.float32)
    np.testing.assert_array_equal(oracle_mod.e4m3_encode_array(x),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert oracle_mod.e4m3_encode(float("nan")) & 0x7F == 0x7F


def test_e4m3_relative_error_bound(oracle_mod):
    """|decode(encode(x)) - x| <= 2^-4 |x| in the normal range and <= 2^-10
    (half the subnormal step) below it."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(400_000) * np.exp(rng.uniform(-9, 6, 400_000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    q = oracle_mod.e4m3_encode_array(x)
    table = oracle_mod.e4m3_table()
    err = np.abs(table[q] - x.astype(np.float64))
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10)
