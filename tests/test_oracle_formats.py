"""Pins for the oracle's NVFP4 codecs and block quantiser (CPU only).

What pins what:
* the E2M1 / E4M3FN value tables against the formats' published definitions,
  typed here by hand (not recomputed from the oracle's bit arithmetic);
* the round-to-nearest-even encoders against an exact nearest-value search in
  rational arithmetic (``fractions.Fraction``) at every midpoint of both grids
  and at its neighbouring float64 values;
* the block quantiser against hand-derived vectors in
  ``tests/golden/nvfp4_blocks.txt`` and, on random blocks, against brute-force
  enumeration of every scale and every element code in rational arithmetic;
* properties: sign symmetry, power-of-two equivariance, the dequantisation
  error bound.
Format source: model card "FastWAM UR3 3-task -- 4-bit quantisations", method
table (NVFP4 = E2M1 elements, block 16, E4M3 block scales).
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_blocks.txt")

# ---------------------------------------------------------------- tables


def test_e2m1_table_matches_definition():
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.E2M1_VALUES[:8].tolist() == want
    assert F.E2M1_VALUES[8:].tolist() == [-v for v in want]
    assert np.signbit(F.E2M1_VALUES[8])  # code 0x8 is -0.0


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x28, 0.25), (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),
    (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0), (0x80, -0.0), (0xB8, -1.0),
    (0xFE, -448.0),
])
def test_e4m3_spot_values(code, value):
    got = F.E4M3_VALUES[code]
    assert got == value and np.signbit(got) == np.signbit(value)


def test_e4m3_structure():
    pos = F.E4M3_VALUES[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must be strictly increasing"
    assert np.isnan(F.E4M3_VALUES[0x7F]) and np.isnan(F.E4M3_VALUES[0xFF])
    assert np.array_equal(F.E4M3_VALUES[0x80:0xFF], -F.E4M3_VALUES[:0x7F])
    assert np.sum(np.isfinite(F.E4M3_VALUES)) == 254


def test_encode_decode_roundtrip():
    assert np.array_equal(F.e2m1_encode_magnitude(F.E2M1_VALUES[:8]), np.arange(8))
    assert np.array_equal(F.e4m3_encode(F.E4M3_VALUES[:0x7F]), np.arange(0x7F))


# ------------------------------------------------ RNE vs exact nearest search


def _nearest_even(grid, q):
    """Exact nearest grid index to q; ties go to the even index; saturating."""
    qf = Fraction(q)
    best, best_d = None, None
    for i, g in enumerate(grid):
        d = abs(qf - Fraction(g))
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def _probe_points(grid):
    pts = []
    for a, b in zip(grid[:-1], grid[1:]):
        mid = (a + b) / 2.0  # exact in float64 for both grids
        pts += [mid, np.nextafter(mid, -np.inf), np.nextafter(mid, np.inf),
                a, np.nextafter(a, np.inf), b, np.nextafter(b, -np.inf)]
    top = grid[-1]
    pts += [top, top * 1.03, top * 1.5, top * 4.0, 0.0]
    return pts


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_rne_against_exact_nearest(fmt):
    if fmt == "e2m1":
        grid = F.E2M1_VALUES[:8].tolist()
        enc = F.e2m1_encode_magnitude
    else:
        grid = F.E4M3_VALUES[:0x7F].tolist()
        enc = F.e4m3_encode
    pts = _probe_points(grid)
    got = enc(np.array(pts))
    want = [_nearest_even(grid, p) for p in pts]
    bad = [(p, g, w) for p, g, w in zip(pts, got, want) if g != w]
    assert not bad, bad[:5]


def test_e4m3_underflow_and_saturation():
    tiny = 2.0 ** -10
    assert F.e4m3_encode(np.array([tiny]))[0] == 0x00          # tie to even (zero)
    assert F.e4m3_encode(np.array([np.nextafter(tiny, 1)]))[0] == 0x01
    assert F.e4m3_encode(np.array([2.0 ** -11]))[0] == 0x00
    for q in (448.0, 460.0, 464.0, 470.0, 1e6):
        assert F.e4m3_encode(np.array([q]))[0] == 0x7E
    for q in (6.0, 6.5, 7.0, 100.0):
        assert F.e2m1_encode_magnitude(np.array([q]))[0] == 7


# ------------------------------------------------------ golden block vectors


def _load_golden():
    cases = []
    with open(GOLDEN) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            name, inputs, scale, packed, _why = [f.strip() for f in line.split("|", 4)]
            block = np.zeros(16, dtype=np.float32)
            for item in inputs.split(","):
                idx, val = item.split(":")
                block[int(idx)] = np.float32(val)
            cases.append((name, block, int(scale, 16),
                          bytes(int(b, 16) for b in packed.split())))
    return cases


@pytest.mark.parametrize("name,block,scale,packed", _load_golden(),
                         ids=[c[0] for c in _load_golden()])
def test_golden_block(name, block, scale, packed):
    codes, scales = F.quantize_nvfp4(block[None, :])
    assert scales.shape == (1, 1) and codes.shape == (1, 8)
    assert int(scales[0, 0]) == scale, name
    assert bytes(codes[0].tolist()) == packed, name


# ---------------------------------------- brute force on random tiny blocks


def _random_blocks(rng, n):
    mags = rng.choice([1e-4, 1e-2, 1.0, 30.0, 900.0], size=(n, 1))
    b = rng.standard_normal((n, 16)) * mags
    # plant exact grid ties and zeros
    b[::5, 3] = 0.0
    b[::7, 5] = -0.0
    return b.astype(np.float32)


def test_quantizer_brute_force():
    rng = np.random.default_rng(7)
    blocks = _random_blocks(rng, 60)
    codes, scales = F.quantize_nvfp4(blocks)
    unpacked = F.unpack_codes(codes)
    e4m3 = F.E4M3_VALUES[:0x7F].tolist()
    e2m1 = F.E2M1_VALUES[:8].tolist()
    for i, blk in enumerate(blocks):
        amax = max(abs(Fraction(float(v))) for v in blk)
        # scale: exact nearest E4M3 to amax / 6 (saturating)
        q = amax / 6
        want_s = _nearest_even(e4m3, q) if q <= 448 else 0x7E
        assert scales[i, 0] == want_s
        sd = Fraction(e4m3[want_s])
        for j, v in enumerate(blk):
            c = int(unpacked[i, j])
            assert (c >> 3) == int(np.signbit(v))
            if sd == 0:
                assert c & 7 == 0
                continue
            r = abs(Fraction(float(v))) / sd
            want_m = _nearest_even(e2m1, r) if r <= 6 else 7
            assert c & 7 == want_m, (i, j, float(v))


def test_sign_symmetry():
    rng = np.random.default_rng(3)
    blocks = _random_blocks(rng, 40)
    c1, s1 = F.quantize_nvfp4(blocks)
    c2, s2 = F.quantize_nvfp4(-blocks)
    assert np.array_equal(s1, s2)
    assert np.array_equal(F.unpack_codes(c1) ^ 8, F.unpack_codes(c2))


def test_power_of_two_equivariance():
    rng = np.random.default_rng(4)
    blocks = (rng.standard_normal((40, 16)) * 3.0).astype(np.float32)
    c0, s0 = F.quantize_nvfp4(blocks)
    for k in (-3, -1, 2, 4):
        ck, sk = F.quantize_nvfp4((blocks * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(c0, ck)
        # the scale's exponent field moves by k, its mantissa stays
        assert np.array_equal(sk.astype(int) - s0.astype(int), np.full(s0.shape, 8 * k))


def test_dequantization_error_bound():
    rng = np.random.default_rng(5)
    a = (rng.standard_normal((64, 256)) * 2.0).astype(np.float32)
    codes, scales = F.quantize_nvfp4(a)
    dq = F.dequantize_nvfp4(codes, scales).reshape(64, 16, 16)
    sd = F.E4M3_VALUES[scales][..., None]
    err = np.abs(dq - a.reshape(64, 16, 16))
    # with a normal scale every element is within one scale unit (half the
    # widest grid gap is 1; the clamp above 6 costs at most 6/16 of a unit)
    assert np.all(err <= sd + 0.0)


def test_shapes_and_input_checks():
    a = np.zeros((3, 32), dtype=np.float32)
    c, s = F.quantize_nvfp4(a)
    assert c.shape == (3, 16) and s.shape == (3, 2)
    assert np.all(c == 0) and np.all(s == 0)
    with pytest.raises(TypeError):
        F.quantize_nvfp4(a.astype(np.float64))
    with pytest.raises(ValueError):
        F.quantize_nvfp4(np.zeros((1, 24), dtype=np.float32))
    c, s = F.quantize_nvfp4(np.zeros((0, 32), dtype=np.float32))
    assert c.shape == (0, 16) and s.shape == (0, 2)
