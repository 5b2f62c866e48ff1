"""Pins for the oracle's number formats and scale rule (CPU only).

Each check ties the oracle to something other than itself: torch's own
float8/bfloat16 casts (library routines implementing the OCP formats), exact
rational arithmetic (fractions.Fraction) for the rceil definition, brute-force
nearest-code search, and hand-derived spot values.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch


def _torch_decode(codes, dtype):
    return torch.tensor(codes, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


def test_bf16_decode_matches_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.bf16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3_decode_matches_torch_and_spot_values(orc):
    table = orc.e4m3_decode_table()
    ref = _torch_decode(list(range(256)), torch.float8_e4m3fn)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(nan, np.isnan(table))
    assert np.array_equal(ref[~nan], table[~nan])
    # OCP E4M3 closed forms
    assert table[0x7E] == 448.0
    assert table[0x08] == 2.0 ** -6
    assert table[0x01] == 2.0 ** -9
    assert table[0x38] == 1.0
    assert table[0x80] == 0.0 and math.copysign(1.0, table[0x80]) == -1.0
    # positive codes are strictly increasing
    assert np.all(np.diff(table[:0x7F]) > 0)


def test_e8m0_decode_matches_torch(orc):
    table = orc.e8m0_decode_table()
    ref = _torch_decode(list(range(256)), torch.float8_e8m0fnu)
    assert math.isnan(table[0xFF]) and math.isnan(ref[0xFF])
    assert np.array_equal(table[:255], ref[:255])
    assert table[127] == 1.0 and table[0] == 2.0 ** -127 and table[254] == 2.0 ** 127


def _grid_values():
    """Every value with an 8-bit significand over the binades that matter for
    E4M3 rounding (2^-13 .. 2^9), both signs, plus zeros."""
    vals = [0.0, -0.0]
    for ex in range(-13, 10):
        for m in range(128, 256):
            v = m * 2.0 ** (ex - 7)
            vals += [v, -v]
    return np.array(vals)


def _brute_force_e4m3(v, table):
    """Nearest finite code, ties to the code with LSB 0, saturating at +-448."""
    finite = [c for c in range(256) if not np.isnan(table[c])]
    fv = table[finite]
    out = []
    for x in v:
        if x >= 448.0:
            out.append(0x7E)
            continue
        if x <= -448.0:
            out.append(0xFE)
            continue
        d = np.abs(fv - x)
        best = np.min(d)
        cands = [finite[i] for i in np.nonzero(d == best)[0]]
        # zero has two codes: keep the sign of x
        if best == abs(x) and any(table[c] == 0 for c in cands):
            out.append(0x80 if math.copysign(1.0, x) < 0 else 0x00)
            continue
        if len(cands) == 1:
            out.append(cands[0])
            continue
        even = [c for c in cands if c & 1 == 0]  # an exact tie: even mantissa
        assert len(cands) == 2 and len(even) == 1, (x, cands)
        out.append(even[0])
    return np.array(out, dtype=np.uint8)


def test_e4m3_round_brute_force(orc):
    table = orc.e4m3_decode_table()
    v = _grid_values()
    # add the midpoints between neighbouring positive codes (exact ties) and
    # points just off them
    pos = np.sort(table[:0x7F])
    mids = (pos[:-1] + pos[1:]) / 2
    extra = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    v = np.concatenate([v, extra, -extra])
    got = orc.e4m3_round_array(v)
    ref = _brute_force_e4m3(v, table)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(v[i], got[i], ref[i]) for i in bad[:10]]


def test_e4m3_round_matches_torch_cast(orc):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000),
                        rng.normal(0, 0.01, 20000), _grid_values()])
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_round_array(v)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("v,code", [
    (448.0, 0x7E), (256.0, 0x78), (240.0, 0x77), (224.0, 0x76),
    (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (232.0, 0x76), (248.0, 0x78),
    (3 * 2.0 ** -10, 0x02), (5 * 2.0 ** -10, 0x02), (2.0 ** -10, 0x00),
    (-2.0 ** -11, 0x80), (1.0625, 0x38), (1.1875, 0x3A), (-448.0, 0xFE),
    (1000.0, 0x7E), (float("nan"), 0x7F),
])
def test_e4m3_round_spot_values(orc, v, code):
    # derived by hand from the OCP E4M3 definition (bias 7, 3 mantissa bits)
    assert orc.e4m3_round(v) == code


def _rceil_exact(amax: Fraction) -> int:
    """Smallest integer e with amax <= 448 * 2^e, by exact rational search,
    clamped to [-127, 127]."""
    if amax == 0:
        return -127
    e = -127
    while e < 127 and amax > 448 * Fraction(2) ** e:
        e += 1
    return e


def test_rceil_exhaustive_bf16(orc):
    """All 32640 positive finite BF16 amax values against the exact rational
    definition and against the bit-level closed form
    e = E - 135 + [m > 96] (448 = 1.75 * 2^8, 1.75 = 1 + 96/128)."""
    bad = []
    for bits in range(1, 0x7F80):
        E, m = bits >> 7, bits & 0x7F
        if E == 0:
            amax = Fraction(m, 2 ** 133)
            closed = -127
        else:
            amax = Fraction(128 + m, 128) * Fraction(2) ** (E - 127)
            closed = max(-127, E - 135 + (1 if m > 96 else 0))
        want = _rceil_exact(amax)
        got = orc.rceil_exponent(float(amax))
        if not (got == want == closed):
            bad.append((hex(bits), got, want, closed))
    assert not bad, bad[:10]


@pytest.mark.parametrize("amax,byte", [
    (1.0, 0x77), (1.75, 0x77), (1.7578125, 0x78), (2.0, 0x78), (0.25, 0x75),
    (100.0, 0x7D), (448.0, 0x7F), (450.0, 0x80), (2.0 ** -126, 0x00), (0.0, 0x00),
    (2.0 ** 127, 0xF6),
])
def test_rceil_spot_values(orc, amax, byte):
    # hand-derived: byte = 127 + smallest e with amax <= 448 * 2^e
    assert orc.rceil_exponent(amax) + 127 == byte


def test_golden_page_constants(orc):
    """The few numbers the pages fix, stored with their citations."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")
    with open(path) as f:
        g = json.load(f)
    assert g["mx_block_elements"]["value"] == 32
    assert g["e4m3_max"]["value"] == 448.0 == orc.e4m3_decode_table()[0x7E]
    assert g["block_sizes"]["value"] == [[1, 1, 32], [1, 32, 32]]
    assert g["pre_all_gather_tuple_len"]["value"] == {"mxfp8": 4, "mxfp8-32x32": 3}
