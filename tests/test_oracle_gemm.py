"""Pins for the oracle's MXFP8 GEMM and grouped GEMM (CPU only).

The reference product is the binary64 sum of dequantised products.  It is
checked against numpy's float64 matmul of operands dequantised through torch's
float8_e4m3fn / float8_e8m0fnu casts (library routines, independent of the
oracle's decoders), against one-hot and scale-shift special cases whose
results are exact, and the 32x32-tile layouts against the 1x32 layout with
expanded scales.
"""
import numpy as np
import pytest
import torch

B_ROW, B_TILE, B_TILE_T = 0, 1, 2


def _deq(q, s_expanded):
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    sc = torch.from_numpy(np.ascontiguousarray(s_expanded)).view(torch.float8_e8m0fnu).to(
        torch.float64).numpy()
    return v * sc


def _rand_operand(rng, rows, K, scale_lo=110, scale_hi=140):
    q = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x3C                  # no NaN payloads
    s = rng.integers(scale_lo, scale_hi, size=(rows, K // 32), dtype=np.uint8)
    return q, s


def _fp64_slack(bound, K):
    # two binary64 summations of the same exact products differ by at most
    # 2 * K * 2^-53 * sum|ab|
    return 2.0 * K * 2.0 ** -53 * bound + 1e-300


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 5, 64), (17, 9, 256), (64, 48, 96),
                                   (33, 64, 32)])
def test_gemm_matches_numpy_float64(orc, M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    qa, sa = _rand_operand(rng, M, K)
    qb, sb = _rand_operand(rng, N, K)
    ref, bound = orc.gemm(qa, sa, qb, sb, B_ROW)
    A = _deq(qa, np.repeat(sa, 32, axis=1))
    B = _deq(qb, np.repeat(sb, 32, axis=1))
    want = A @ B.T
    assert np.all(np.abs(ref - want) <= _fp64_slack(bound, K))
    assert np.allclose(bound, np.abs(A) @ np.abs(B).T, rtol=1e-12, atol=0)


def test_gemm_one_hot_rows_select_b(orc):
    """K = 32, A rows one-hot (1.0 at k, scale 2^0): C[m, n] = B[n, k] exactly."""
    rng = np.random.default_rng(5)
    N, K = 40, 32
    qb, sb = _rand_operand(rng, N, K)
    qa = np.zeros((K, K), np.uint8)
    for k in range(K):
        qa[k, k] = 0x38                              # 1.0
    sa = np.full((K, 1), 127, np.uint8)
    ref, _ = orc.gemm(qa, sa, qb, sb, B_ROW)
    B = _deq(qb, np.repeat(sb, 32, axis=1))
    assert np.array_equal(ref, B.T)


def test_gemm_scale_shift_is_exact_power_of_two(orc):
    rng = np.random.default_rng(6)
    qa, sa = _rand_operand(rng, 8, 128)
    qb, sb = _rand_operand(rng, 8, 128)
    r0, _ = orc.gemm(qa, sa, qb, sb, B_ROW)
    r1, _ = orc.gemm(qa, (sa.astype(int) + 3).astype(np.uint8), qb, sb, B_ROW)
    assert np.array_equal(r1, r0 * 8.0)


def test_gemm_zero(orc):
    qa = np.zeros((4, 64), np.uint8)
    sa = np.full((4, 2), 127, np.uint8)
    rng = np.random.default_rng(7)
    qb, sb = _rand_operand(rng, 5, 64)
    ref, bound = orc.gemm(qa, sa, qb, sb, B_ROW)
    assert (ref == 0).all() and (bound == 0).all()


def test_gemm_tile_scales_equal_expanded_row_scales(orc):
    rng = np.random.default_rng(8)
    M, N, K = 12, 64, 96
    qa, sa = _rand_operand(rng, M, K)
    qb = rng.integers(0, 0x7E, size=(N, K), dtype=np.uint8)
    tiles = rng.integers(100, 150, size=(N // 32, K // 32), dtype=np.uint8)
    r_tile, b_tile = orc.gemm(qa, sa, qb, tiles, B_TILE)
    expanded = np.repeat(tiles, 32, axis=0)            # [N, K/32]
    r_row, b_row = orc.gemm(qa, sa, qb, expanded, B_ROW)
    assert np.array_equal(r_tile, r_row) and np.array_equal(b_tile, b_row)


def test_gemm_transposed_tile_weight(orc):
    """B stored [K][N] (weight [out][in]) contracted over rows equals the
    forward layout applied to its transpose with transposed tile scales."""
    rng = np.random.default_rng(9)
    M, N, K = 10, 64, 128
    qa, sa = _rand_operand(rng, M, K)
    w = rng.integers(0, 0x7E, size=(K, N), dtype=np.uint8)
    tiles = rng.integers(100, 150, size=(K // 32, N // 32), dtype=np.uint8)
    r_t, _ = orc.gemm(qa, sa, w, tiles, B_TILE_T)
    r_f, _ = orc.gemm(qa, sa, np.ascontiguousarray(w.T), np.ascontiguousarray(tiles.T), B_TILE)
    assert np.array_equal(r_t, r_f)
    # and against numpy on the dequantised weight
    Wd = _deq(w, np.repeat(np.repeat(tiles, 32, axis=0), 32, axis=1))
    A = _deq(qa, np.repeat(sa, 32, axis=1))
    _, bound = orc.gemm(qa, sa, w, tiles, B_TILE_T)
    assert np.all(np.abs(r_t - A @ Wd) <= _fp64_slack(bound, K))


def test_gemm_rejects_bad_k(orc):
    with pytest.raises(ValueError):
        orc.gemm(np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8),
                 np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8))


def _offsets(sizes):
    o = np.zeros(len(sizes) + 1, np.int64)
    np.cumsum(sizes, out=o[1:])
    return o


def test_grouped_is_per_group_matmul(orc):
    rng = np.random.default_rng(10)
    sizes = [5, 0, 33, 1, 0, 17]
    G, N, K = len(sizes), 24, 64
    off = _offsets(sizes)
    T = int(off[-1])
    qa, sa = _rand_operand(rng, T, K)
    qb = rng.integers(0, 0x7E, size=(G, N, K), dtype=np.uint8)
    sb = rng.integers(110, 140, size=(G, N, K // 32), dtype=np.uint8)
    ref, bound = orc.grouped_gemm(off, qa, sa, qb, sb)
    A = _deq(qa, np.repeat(sa, 32, axis=1))
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        Bg = _deq(qb[g], np.repeat(sb[g], 32, axis=1))
        want = A[r0:r1] @ Bg.T
        assert np.all(np.abs(ref[r0:r1] - want) <= _fp64_slack(bound[r0:r1], K))
    assert not np.isnan(ref).any()


def test_grouped_permutation_of_groups(orc):
    """Reordering experts (and their token blocks) reorders the output blocks."""
    rng = np.random.default_rng(11)
    sizes = [7, 3, 0, 12]
    G, N, K = 4, 16, 32
    off = _offsets(sizes)
    qa, sa = _rand_operand(rng, int(off[-1]), K)
    qb = rng.integers(0, 0x7E, size=(G, N, K), dtype=np.uint8)
    sb = rng.integers(110, 140, size=(G, N, K // 32), dtype=np.uint8)
    ref, _ = orc.grouped_gemm(off, qa, sa, qb, sb)
    perm = [2, 3, 0, 1]
    sizes_p = [sizes[g] for g in perm]
    off_p = _offsets(sizes_p)
    rows = np.concatenate([np.arange(off[g], off[g + 1]) for g in perm]).astype(int)
    ref_p, _ = orc.grouped_gemm(off_p, qa[rows], sa[rows], qb[perm], sb[perm])
    assert np.array_equal(ref_p, ref[rows])


def test_grouped_rejects_bad_offsets(orc):
    qa = np.zeros((4, 32), np.uint8)
    sa = np.zeros((4, 1), np.uint8)
    qb = np.zeros((2, 8, 32), np.uint8)
    sb = np.zeros((2, 8, 1), np.uint8)
    for off in ([0, 3, 2], [0, 1, 5], [1, 2, 4]):
        with pytest.raises(ValueError):
            orc.grouped_gemm(np.array(off), qa, sa, qb, sb)


def test_tolerance_rule(orc):
    ref = np.array([1.0, 1.0, 0.0])
    bound = np.array([128.0, 128.0, 0.0])
    ok = orc.within_tolerance(np.array([2.0, 2.01, 5e-7]), ref, bound)
    assert ok.tolist() == [True, False, True]
