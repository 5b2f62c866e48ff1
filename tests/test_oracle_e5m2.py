"""Pins for the oracle's E5M2 payload option (CPU only).

E5M2 (OCP OFP8: S.EEEEE.MM, bias 15, 0x7C infinity, 0x7D..0x7F NaN, largest
finite 57344) is decoded against torch's float8_e5m2, rounded against a
brute-force nearest-code search with exact midpoints and torch's cast, and
the E5M2 scale rule (the smallest e with amax <= 57344 * 2^e) against an
exact rational search over every positive finite BF16 value.  Quantisation
with E5M2 payloads is checked against an independent vectorised quantiser
built from torch's cast; the GEMM with E5M2 (and mixed) operands against
numpy float64 matmul of torch-dequantised operands.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from mxfp8_microscaled_precision_amd import workloads as W

E5M2 = 1


def _torch_e5m2(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e5m2).to(
        torch.float64).numpy()


def test_e5m2_decode_matches_torch(orc):
    mine = orc.e5m2_decode_table()
    ref = _torch_e5m2(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7B] == 57344.0 and mine[0x7C] == np.inf and mine[0xFC] == -np.inf
    assert mine[0x04] == 2.0 ** -14 and mine[0x01] == 2.0 ** -16 and mine[0x3C] == 1.0


def _finite_codes(orc):
    t = orc.e5m2_decode_table()
    return [(c, t[c]) for c in range(0x80) if np.isfinite(t[c])]


def _brute(v, table):
    """Nearest finite E5M2 magnitude (ties to the even code), sign kept,
    saturating at 57344."""
    a = abs(v)
    best = None
    for c, val in table:
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    code = best[1]
    if a >= 57344.0:
        code = 0x7B
    return code | (0x80 if np.signbit(v) else 0)


def test_e5m2_round_brute_force(orc):
    table = _finite_codes(orc)
    vals = [v for _, v in table]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(len(vals) - 1)]   # exact ties
    rng = np.random.default_rng(3)
    rand = list(np.exp2(rng.uniform(-19, 16.5, 3000)))
    probe = vals + mids + rand + [70000.0, 2.0 ** -17, 2.0 ** -18, 3 * 2.0 ** -18]
    for v in probe:
        for sv in (v, -v):
            assert orc.e5m2_round(sv) == _brute(sv, table), sv


@pytest.mark.parametrize("v,code", [
    (57344.0, 0x7B), (49152.0, 0x7A), (1.0, 0x3C), (1.25, 0x3D), (1.125, 0x3C),
    (1.375, 0x3E), (2.0 ** -14, 0x04), (2.0 ** -16, 0x01), (2.0 ** -17, 0x00),
    (3 * 2.0 ** -17, 0x02), (-2.0 ** -18, 0x80), (61440.0, 0x7B),
])
def test_e5m2_spot_values(orc, v, code):
    """Hand-derived: 57344 = 1.75 * 2^15 is the largest finite value; 1.125
    and 1.375 are ties that go to the even mantissa; 2^-17 ties to 0 (even);
    3 * 2^-17 ties up to 2 * 2^-16; tiny negatives keep their sign."""
    assert orc.e5m2_round(v) == code


def test_e5m2_round_matches_torch_cast(orc):
    rng = np.random.default_rng(5)
    v = np.concatenate([np.exp2(rng.uniform(-17, 15.7, 20000)) * rng.choice([-1, 1], 20000)])
    want = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([orc.e5m2_round(x) for x in v], np.uint8)
    assert np.array_equal(got, want)


def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    return bits, W.bits_to_bf16(bits.reshape(1, -1)).double().numpy().ravel()


def test_e5m2_rceil_exhaustive(orc):
    """The smallest e with amax <= 57344 * 2^e, found by exact rational
    search, and the bit closed form E - 142 + [m > 96], over all 32,639
    positive finite BF16 values."""
    bits, vals = _all_positive_bf16()
    for b, v in zip(bits, vals):
        e = orc.rceil_exponent_e5m2(float(v))
        a = Fraction(float(v))
        lim = Fraction(57344)
        want = -127
        while want < 127 and a > lim * Fraction(2) ** want:
            want += 1
        assert e == want, (hex(b), v, e, want)
        E, m = int(b) >> 7, int(b) & 0x7F
        closed = (E - 142 + (1 if m > 96 else 0)) if E > 0 else -127
        assert e == max(-127, min(127, closed)), hex(b)


def _vectorised_row_e5m2(xbits):
    """Independent row quantiser: exponent from the BF16 bits of each block's
    amax by the closed form, elements by torch's cast."""
    x = W.bits_to_bf16(xbits).double()
    R, C = x.shape
    blocks = x.reshape(R, C // 32, 32)
    amax_bits = torch.from_numpy(xbits.reshape(R, C // 32, 32) & 0x7FFF).int().amax(dim=2)
    E, m = amax_bits >> 7, amax_bits & 0x7F
    e = torch.where(E > 0, E - 142 + (m > 96).int(), torch.full_like(E, -127)).clamp(-127, 127)
    scaled = blocks * torch.pow(2.0, -e.double()).unsqueeze(2)
    q = scaled.to(torch.float8_e5m2).view(torch.uint8).reshape(R, C).numpy()
    return q, (e + 127).to(torch.uint8).numpy()


@pytest.mark.parametrize("gen", ["normal", "outliers", "student"])
def test_row_quant_e5m2_matches_vectorised(orc, gen):
    shape = (64, 256)
    x = {"normal": W.normal_bf16(shape, 1.0, 1),
         "outliers": W.normal_with_outliers_bf16(shape, 1.0, 0.01, 100.0, 2),
         "student": W.student_t_bf16(shape, 3, 3)}[gen]
    xb = W.bf16_bits(x)
    q, s = orc.quant_row(xb, E5M2)
    wq, ws = _vectorised_row_e5m2(xb)
    assert np.array_equal(s, ws)
    assert np.array_equal(q, wq)


def test_e5m2_block_max_lands_in_top_binade(orc):
    """Under the rceil rule every non-clamped, non-zero block's largest code
    decodes into [28672, 57344]."""
    xb = W.bf16_bits(W.student_t_bf16((128, 512), 3, 9))
    q, s = orc.quant_row(xb, E5M2)
    dec = np.abs(orc.e5m2_decode_table()[q]).reshape(128, 16, 32).max(axis=2)
    live = s > 0
    assert np.all((dec[live] >= 28672.0) & (dec[live] <= 57344.0))


def test_e5m2_layouts(orc):
    xb = W.bf16_bits(W.normal_bf16((96, 64), 1.0, 4))
    qt, st = orc.quant_col(xb, E5M2)
    qr, sr = orc.quant_row(np.ascontiguousarray(xb.T), E5M2)
    assert np.array_equal(qt, qr) and np.array_equal(st, sr)
    q32, s32 = orc.quant_block32(xb, E5M2)
    q32t, s32t = orc.quant_block32(np.ascontiguousarray(xb.T), E5M2)
    assert np.array_equal(q32.T, q32t) and np.array_equal(s32.T, s32t)
    # E4M3 and E5M2 blocks see the same amax: scale bytes differ by exactly 7
    # (57344 / 448 = 2^7)
    _, s4 = orc.quant_row(xb)
    _, s5 = orc.quant_row(xb, E5M2)
    assert np.array_equal(s4.astype(int) - 7, s5.astype(int))


def _deq(q, s_exp, elem):
    t = torch.float8_e5m2 if elem == E5M2 else torch.float8_e4m3fn
    v = torch.from_numpy(np.ascontiguousarray(q)).view(t).to(torch.float64).numpy()
    sc = torch.from_numpy(np.ascontiguousarray(s_exp)).view(torch.float8_e8m0fnu).to(
        torch.float64).numpy()
    return v * sc


@pytest.mark.parametrize("a_elem,b_elem", [(1, 1), (1, 0), (0, 1)])
def test_gemm_e5m2_operands_match_numpy(orc, a_elem, b_elem):
    rng = np.random.default_rng(10 + 2 * a_elem + b_elem)
    M, N, K = 24, 40, 128

    def operand(rows, elem):
        q = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        bad = (q & 0x7C) == 0x7C if elem == E5M2 else (q & 0x7F) == 0x7F
        q[bad] = 0x38
        return q, rng.integers(115, 135, size=(rows, K // 32), dtype=np.uint8)

    qa, sa = operand(M, a_elem)
    qb, sb = operand(N, b_elem)
    ref, bound = orc.gemm(qa, sa, qb, sb, a_elem=a_elem, b_elem=b_elem)
    A = _deq(qa, np.repeat(sa, 32, axis=1), a_elem)
    B = _deq(qb, np.repeat(sb, 32, axis=1), b_elem)
    assert np.all(np.abs(ref - A @ B.T) <= 2.0 * K * 2.0 ** -53 * bound + 1e-300)
