"""Pins for the oracle's number formats against library conversions and
exact rational arithmetic (CPU only)."""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _bf16_exact_nearest(v: float) -> int:
    """Nearest bf16 to a double by exact rational comparison of the two
    candidates around it (ties to the even code).  Finite normal range only."""
    f32 = np.float32(v)
    bits = int(np.array([f32], np.float32).view(np.uint32)[0])
    lo = bits >> 16
    cands = []
    for c in (lo - 1, lo, lo + 1, lo + 2):
        if c < 0 or (c & 0x7F80) == 0x7F80:
            continue
        val = struct.unpack("<f", struct.pack("<I", (c & 0xFFFF) << 16))[0]
        cands.append((abs(Fraction(val) - Fraction(v)), c & 1, c))
    cands.sort()
    return cands[0][2]


def test_bf16_matches_torch_cast_on_floats():
    r = np.random.default_rng(0)
    vals = np.concatenate([
        r.standard_normal(4000).astype(np.float32),
        (r.standard_normal(2000) * 1e-39).astype(np.float32),   # bf16 subnormals
        (r.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -2.5, 3.3895314e38, 65504.0], np.float32),
    ])
    # exact ties between neighbouring bf16 values: low 16 bits == 0x8000
    tie_bits = (r.integers(0x0080, 0x7F00, 1000, dtype=np.uint32) << 16) | 0x8000
    vals = np.concatenate([vals, tie_bits.view(np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_double(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_from_double_is_single_rounding():
    r = np.random.default_rng(1)
    vals = r.standard_normal(3000) * np.exp2(r.integers(-60, 60, 3000))
    for v in vals:
        assert oracle.bf16_from_double(float(v)) == _bf16_exact_nearest(float(v)), v


def test_bf16_overflow_and_decode():
    assert oracle.bf16_from_double(1e39) == 0x7F80
    assert oracle.bf16_from_double(-1e39) == 0xFF80
    for b in [0x3F80, 0xC000, 0x0001, 0x7F7F]:
        want = struct.unpack("<f", struct.pack("<I", b << 16))[0]
        assert oracle.bf16_to_double(b) == want


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.e4m3_to_double(c)
        if math.isnan(want[c]):
            assert math.isnan(got), c
        else:
            assert got == float(want[c]), c
    # exactly two NaN codes; 448 is the largest finite magnitude
    assert sum(math.isnan(oracle.e4m3_to_double(c)) for c in range(256)) == 2
    assert max(abs(oracle.e4m3_to_double(c)) for c in range(256) if not math.isnan(oracle.e4m3_to_double(c))) == 448.0


def test_e4m3_roundtrip_every_finite_code():
    for c in range(256):
        v = oracle.e4m3_to_double(c)
        if math.isnan(v):
            continue
        back = oracle.e4m3_from_double(v)
        if v == 0.0:
            assert back in (0x00, 0x80)
        else:
            assert back == c, (c, v, back)


def test_e4m3_encode_matches_torch_below_saturation():
    r = np.random.default_rng(2)
    vals = np.concatenate([
        (r.standard_normal(6000) * np.exp2(r.integers(-12, 9, 6000))).astype(np.float32),
        np.linspace(-447.9, 447.9, 3001, dtype=np.float32),
    ])
    # midpoints between consecutive finite codes (ties go to the even code)
    pos = sorted({oracle.e4m3_to_double(c) for c in range(0, 127)})
    mids = np.array([(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])], np.float32)
    vals = np.concatenate([vals, mids, -mids])
    vals = vals[np.abs(vals) < 448.0]
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_from_double(float(v)) for v in vals], np.uint8)
    # zero may come back with either sign from the library; compare values
    wz = (want & 0x7F) == 0
    assert np.array_equal(got[~wz], want[~wz])
    assert np.all((got[wz] & 0x7F) == 0)


def test_e4m3_saturates():
    assert oracle.e4m3_from_double(448.0) == 0x7E
    assert oracle.e4m3_from_double(460.0) == 0x7E
    assert oracle.e4m3_from_double(1e30) == 0x7E
    assert oracle.e4m3_from_double(-1e30) == 0xFE
    assert math.isnan(oracle.e4m3_to_double(oracle.e4m3_from_double(float("nan"))))


def test_quant_rows_matches_torch_cast():
    r = np.random.default_rng(3)
    x = (r.standard_normal((7, 512)) * np.exp2(r.integers(-8, 8, (7, 1)))).astype(np.float32)
    x[3, 128:256] = 0.0            # an all-zero block takes scale 1
    q, s = oracle.quant_rows_e4m3(x)
    xt = torch.from_numpy(x).view(7, 4, 128)
    amax = xt.abs().amax(dim=2)
    st = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    qt = (xt / st[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(7, 512).numpy()
    assert np.array_equal(s, st.numpy())
    nz = (qt & 0x7F) != 0
    assert np.array_equal(q[nz], qt[nz])
    assert np.all((q[~nz] & 0x7F) == 0)
