"""Pins of the oracle's fp8 (E4M3) cache rows against the OCP 8-bit floating
point definition: closed forms, brute force and invariants, independent of
the oracle's own code paths (test infrastructure, CPU only)."""

import math
import random

import numpy as np
import pytest

import synth
from oracle import fp8


def spec_value(code: int) -> float:
    """E4M3 from the definition, one code at a time (Python floats)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)              # m/8 * 2^-6
    return s * math.ldexp(8 + m, e - 10)          # (1 + m/8) * 2^(e-7)


def test_decode_matches_definition_for_every_code():
    got = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        want = spec_value(c)
        if math.isnan(want):
            assert np.isnan(got[c]), c
        else:
            assert got[c] == np.float32(want) and math.copysign(1, got[c]) == math.copysign(1, want), c


def test_known_codes():
    d = fp8.e4m3_decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x7E, 0xFE], np.uint8))
    assert list(d) == [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 2.0, 448.0, -448.0]
    assert np.isnan(fp8.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_positive_codes_increase_strictly():
    v = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(v) > 0).all()


def test_encode_inverts_decode():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def brute_nearest(x: float) -> int:
    """Nearest finite code by exhaustive search; ties to the even mantissa;
    magnitudes past 448 saturate."""
    if math.isnan(x):
        return 0x7F
    a = min(abs(x), 448.0)
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(spec_value(c) - a)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_encode_is_nearest_by_brute_force():
    rnd = random.Random(5)
    xs = []
    for _ in range(1500):
        e = rnd.uniform(-12, 9.5)
        xs.append(float(np.float32(rnd.choice([-1, 1]) * 2.0 ** e)))
    xs += [0.0, -0.0, 447.9, 448.0, 449.0, 463.9, 464.0, 500.0, 1e30, -1e30, 2.0 ** -10, 2.0 ** -11]
    got = fp8.e4m3_encode(np.array(xs, np.float32))
    for x, g in zip(xs, got):
        assert g == brute_nearest(x), (x, g, brute_nearest(x))


def test_midpoints_round_to_even_mantissa():
    v = [spec_value(c) for c in range(0x7F)]
    mids = np.array([(v[c] + v[c + 1]) / 2 for c in range(0x7E)], np.float64)
    assert (mids.astype(np.float32).astype(np.float64) == mids).all()   # exact in fp32
    got = fp8.e4m3_encode(mids.astype(np.float32))
    for c in range(0x7E):
        assert got[c] == (c if c % 2 == 0 else c + 1), c


def test_saturation_and_nan():
    got = fp8.e4m3_encode(np.array([448.5, 1e6, np.inf, -np.inf, -600.0, np.nan], np.float32))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]


def test_row_quantisation_invariants():
    rng = np.random.default_rng(3)
    x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((rng.standard_normal((64, 256)) *
                                                       rng.uniform(0.01, 100, (64, 1))).astype(np.float32)))
    x[5] = 0.0
    codes, scales = fp8.quantize_rows(x)
    assert scales[5] == 1.0 and (codes[5] == 0).all()
    amax = np.abs(x).max(axis=1)
    nz = amax > 0
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(448.0)).astype(np.float32))
    # the largest magnitude of each row takes code +-448
    i = np.abs(x).argmax(axis=1)
    top = codes[np.arange(64), i]
    assert ((top & 0x7F) == 0x7E)[nz].all()
    # widened values are within e4m3's half-ulp (2^-4 relative, 2^-10 scale absolute) plus bf16's
    w = synth.bf16_bits_to_f32(fp8.dequantize_rows_bf16(codes, scales))
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scales[:, None] + 2.0 ** -8 * np.abs(w)
    assert (np.abs(w - x) <= bound).all()


def test_fp8_attention_stays_near_the_bf16_definition():
    """A consistency check that catches a misplaced scale or a transposed
    value row: with K and V moved by at most 1/16 relative, the gated
    outputs move by a small fraction of their spread."""
    import oracle
    orc = oracle.get()
    p = synth.make_problem(T=96, n_q_heads=4, n_kv_heads=2, seed=4)
    ref = synth.bf16_bits_to_f32(orc.attention(p)).astype(np.float64)
    got = synth.bf16_bits_to_f32(fp8.attention_fp8(orc, p)).astype(np.float64)
    err = np.abs(got - ref)
    assert np.median(err) < 0.02 * np.median(np.abs(ref)) + 1e-3
    assert err.max() < 0.25 * np.abs(ref).max()
    # and the cache rows really are the quantised prepared keys / raw values
    kv = fp8.fp8_cache_kv(orc, p)
    assert kv["k_codes"].shape == (2, 96, 256) and kv["v_scales"].shape == (2, 96)
    assert not np.array_equal(kv["kp"], orc.prepare_keys(p))
