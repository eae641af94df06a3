"""Pins for the oracle's INT4/INT8 encoders (CPU only).

The pages state only that the full context is calibration-free INT4 and the
protected positions INT8 (KV4-RL review, sections 1 and 3). These tests pin
the oracle to the stated reading by means other than the oracle itself:
hand-derived fixtures, an independent pure-Python encoder that rounds through
``struct`` (float32 / IEEE half packing), a brute-force nearest-code search,
closed-form error bounds and symmetry.
"""
import math
import struct

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from golden.read import cases
from oracle import quant


def r32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def r16(x):
    x = max(-65504.0, min(65504.0, x))
    return struct.unpack("<e", struct.pack("<e", x))[0]


def py_int4(group):
    """Independent INT4 encoder over one group of 32 float32-representable floats."""
    mn, mx = min(group), max(group)
    s32 = r32(r32(mx - mn) / 15.0)
    scale = r16(s32)
    mnh = r16(mn)
    inv = r32(1.0 / scale) if scale > 0 else 0.0
    codes = []
    for x in group:
        t = r32(r32(x - mnh) * inv)
        codes.append(min(15, max(0, round(t))))  # Python round(): ties to even
    return codes, scale, mnh


def py_int8(vec):
    a = max(abs(x) for x in vec)
    s = r32(a / 127.0)
    inv = r32(1.0 / s) if s >= 2.0 ** -126 else 0.0
    return [min(127, max(-127, round(r32(x * inv)))) for x in vec], s


# ------------------------------------------------------------------ fixtures
@pytest.mark.parametrize("case", cases("int4_groups.txt"), ids=lambda c: c["name"])
def test_int4_golden(case):
    x = np.array(case["x"], np.float32)[None, :]
    c, s, m = quant.int4_encode(x)
    assert float(s[0, 0]) == case["scale"][0]
    assert float(m[0, 0]) == case["min"][0]
    assert c[0].tolist() == [int(v) for v in case["codes"]]


@pytest.mark.parametrize("case", cases("int8_vectors.txt"), ids=lambda c: c["name"])
def test_int8_golden(case):
    x = np.array(case["x"], np.float32)[None, :]
    c, s = quant.int8_encode(x)
    assert float(s[0]) == np.float32(case["scale"][0])
    assert c[0].tolist() == [int(v) for v in case["codes"]]


def test_nibble_order_hand_example():
    # Byte j holds code 2j in its low nibble and code 2j+1 in its high nibble.
    codes = np.array([1, 2, 3, 4, 15, 0, 0, 15], np.uint8)
    assert quant.pack_nibbles(codes).tolist() == [0x21, 0x43, 0x0F, 0xF0]
    assert quant.unpack_nibbles(quant.pack_nibbles(codes)).tolist() == codes.tolist()


# ------------------------------------------------------ independent encoder
f32s = st.floats(min_value=-200.0, max_value=200.0, allow_nan=False, width=32)


@settings(max_examples=300, deadline=None)
@given(st.lists(f32s, min_size=32, max_size=32))
def test_int4_matches_independent_encoder(vals):
    c, s, m = quant.int4_encode(np.array(vals, np.float32)[None, :])
    pc, ps, pm = py_int4(vals)
    assert c[0].tolist() == pc
    assert float(s[0, 0]) == ps and float(m[0, 0]) == pm


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(0, 30), min_size=32, max_size=32), st.integers(-6, 6), st.integers(-40, 40))
def test_int4_lattice_ties(mants, e, off):
    # Values on a power-of-two lattice hit exact .5 ties of (x - min)/scale.
    vals = [float(m * 2.0 ** e + off) for m in mants]
    c, s, m = quant.int4_encode(np.array(vals, np.float32)[None, :])
    pc, ps, pm = py_int4([r32(v) for v in vals])
    assert c[0].tolist() == pc and float(s[0, 0]) == ps and float(m[0, 0]) == pm


@settings(max_examples=300, deadline=None)
@given(st.lists(f32s, min_size=1, max_size=64))
def test_int8_matches_independent_encoder(vals):
    c, s = quant.int8_encode(np.array(vals, np.float32)[None, :])
    pc, ps = py_int8(vals)
    assert c[0].tolist() == pc and float(s[0]) == ps


def test_int4_many_random_groups_vs_independent():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((400, 32)) * rng.choice([0.01, 1.0, 30.0], size=(400, 1))).astype(np.float32)
    c, s, m = quant.int4_encode(x)
    for i in range(x.shape[0]):
        pc, ps, pm = py_int4([float(v) for v in x[i]])
        assert c[i].tolist() == pc and float(s[i, 0]) == ps and float(m[i, 0]) == pm


# ------------------------------------------------------ brute-force / bounds
def test_int4_code_is_nearest_brute_force():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2000, 32)).astype(np.float32)
    c, s, m = quant.int4_encode(x)
    sf = s.astype(np.float64)
    mf = m.astype(np.float64)
    for i in range(0, 2000, 7):
        inv = r32(1.0 / float(sf[i, 0])) if sf[i, 0] > 0 else 0.0
        for j in range(32):
            t = r32(r32(float(x[i, j]) - float(mf[i, 0])) * inv)
            best = min(range(16), key=lambda k: (abs(t - k), k % 2))
            assert c[i, j] == best


def test_int4_error_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5000, 128)) * 3).astype(np.float32)
    c, s, m = quant.int4_encode(x)
    xh = quant.int4_decode(c, s, m)
    g = x.reshape(5000, 4, 32).astype(np.float64)
    s32 = (g.max(-1) - g.min(-1)) / 15.0
    bound = (s.astype(np.float64) / 2 + np.abs(g.min(-1) - m.astype(np.float64))
             + 15 * np.abs(s32 - s.astype(np.float64)) + 1e-5)
    err = np.abs(xh.reshape(5000, 4, 32) - g).max(-1)
    assert (err <= bound).all()


def test_int8_error_bound_and_symmetry():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3000, 128)).astype(np.float32)
    c, s = quant.int8_encode(x)
    c2, s2 = quant.int8_encode(-x)
    assert (c2 == -c).all() and (s2 == s).all()
    err = np.abs(quant.int8_decode(c, s) - x.astype(np.float64)).max(-1)
    assert (err <= s.astype(np.float64) * (0.5 + 1e-5)).all()
    assert c.min() >= -127


def test_int4_saturates_fp16():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = -1.0e6
    x[0, 1] = 1.0e6
    c, s, m = quant.int4_encode(x)
    assert float(s[0, 0]) == 65504.0 and float(m[0, 0]) == -65504.0
    assert np.isfinite(quant.int4_decode(c, s, m)).all()


def test_int8_subnormal_scale_counts_as_zero():
    x = np.array([[1.0e-38, 0.0, -5.0e-39, 0.0]], np.float32)
    c, s = quant.int8_encode(x)
    assert (c == 0).all() and 0 < float(s[0]) < 2.0 ** -126


def test_int4_constant_group_is_exact():
    x = np.full((3, 32), -1.75, np.float32)
    c, s, m = quant.int4_encode(x)
    assert (c == 0).all() and (s == 0).all()
    assert (quant.int4_decode(c, s, m) == -1.75).all()
