"""Tolerance-free GEMM parity at the workloads' contraction lengths.

The GEMM tolerance (2^-7 sum|ab|) cannot see one dropped or mis-scaled
32-element K block once K runs to thousands.  These cases make every output
exact instead: each A row is one-hot (a single E4M3 code at position k_m, a
different K block per row, with a different A scale on every block), so
C[m][n] = E4M3(a) E4M3(b[n][k_m]) 2^(sa + sb - 254) is one product of two
4-bit significands times a power of two, exact in FP32 and in BF16.  The
GPU result must then equal the oracle's binary64 reference bit for bit, and
a wrong K position, a wrong A or B scale index, a skipped or repeated K step
or a mis-mapped tile changes the value.

Every pipeline of the dense kernel is run at the linear-stack K values
(7168, 18432, 32768; K a multiple of 512), at K = 18048 / 18176 / 18304
(a partial last group of 1, 2 and 3 of four K steps), at a K that is not a
multiple of 128 (the general variant), through the 32x32-weight forward
(tile scales) and backward-data (the shared weight read transposed) forms,
the grouped MoE GEMM, the per-expert weight gradient, and the fused
producer, whose expected bytes are the oracle's row quantisation of the
oracle's exact product.  The persistent GEMM (more output tiles than compute
units, the next tile's first stage loading under the current tile's
stores) is run at the stack's K values and, with 32x32 weights, at
K = 4096; the grouped GEMM walks two or three tiles per workgroup at the
MoE K values."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_microscaled_precision_amd as mx
from mxfp8_microscaled_precision_amd import workloads as W
from parity import assert_bytes, bits, dev, host, say

pytestmark = pytest.mark.gpu

# E4M3 codes with a nonzero finite value (no +-0, no NaN), so every output is
# a nonzero product and the sign of zero never decides a fused byte
_NONZERO = np.array([c for c in range(256) if c not in (0x00, 0x80, 0x7F, 0xFF)], np.uint8)


def one_hot_a(M, K, seed):
    """A [M, K] with one nonzero code per row at k_m = 32 kb_m + j_m (kb_m
    runs through the K blocks, so rows cover every block when M >= K/32),
    and A scales that differ between neighbouring blocks of a row."""
    rng = np.random.default_rng(seed)
    nkb = K // 32
    kb = (np.arange(M) * 7919) % nkb if M > nkb else rng.permutation(nkb)[:M]
    k = 32 * kb + rng.integers(0, 32, M)
    qa = np.zeros((M, K), np.uint8)
    qa[np.arange(M), k] = rng.choice(_NONZERO, M)
    blocks = np.arange(nkb)[None, :]
    sa = (121 + (5 * blocks + 3 * np.arange(M)[:, None]) % 13).astype(np.uint8)   # 121 .. 133
    return qa, sa


def random_b(N, K, seed, scale_rows=None):
    """B codes uniform over the nonzero finite E4M3 codes and scale bytes in
    120 .. 134 (scale_rows rows of K/32 scales; default N)."""
    rng = np.random.default_rng(seed)
    qb = rng.choice(_NONZERO, (N, K)).astype(np.uint8)
    sb = rng.integers(120, 135, (scale_rows if scale_rows is not None else N, K // 32)).astype(np.uint8)
    return qb, sb


def assert_exact(got_t, ref, what):
    got = got_t.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(ref).all() and (ref != 0).all(), what
    bad = got != ref
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs differ; first {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r}")


def bf16_bits_exact(ref):
    """BF16 bit patterns of binary64 values that BF16 holds exactly."""
    u = ref.astype(np.float32).view(np.uint32)
    assert (ref.astype(np.float32).astype(np.float64) == ref).all()
    assert ((u & 0xFFFF) == 0).all(), "not exact in BF16"
    return (u >> 16).astype(np.uint16)


# K = 7168, 18432, 32768: the stack's contractions (pipeline 1: K a multiple
# of 512); 18048 / 18176 / 18304: pipeline 2 with 1, 2, 3 steps of a partial
# last group; 7200: the general variant (K not a multiple of 128)
ROW_K = [7168, 18432, 32768, 18048, 18176, 18304, 7200]


@pytest.mark.parametrize("K", ROW_K)
def test_row_scales_exact(K):
    M, N = min(K // 32, 1024), 288            # every K block in one row or more; ragged N
    say(f"[exact] 1x32 M={M} N={N} K={K}")
    qa, sa = one_hot_a(M, K, K)
    qb, sb = random_b(N, K, K + 1)
    c = mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb), "fprop", "1x32")
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(qa, sa, qb, sb, oracle.BKIND_ROW, want_bound=False)
    assert_exact(c, ref, f"1x32 K={K}")


@pytest.mark.parametrize("K", [7168, 18432, 18048, 18304, 7200])
def test_tile_scales_fprop_exact(K):
    """The 32x32 weight's forward product: B [N, K] with one scale per 32x32
    tile, tiles [N/32, K/32]."""
    M, N = min(K // 32, 1024), 320
    say(f"[exact] 32x32 fprop M={M} N={N} K={K}")
    qa, sa = one_hot_a(M, K, K + 2)
    qb, sb = random_b(N, K, K + 3, scale_rows=N // 32)
    c = mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb), "fprop", "32x32")
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(qa, sa, qb, sb, oracle.BKIND_TILE, want_bound=False)
    assert_exact(c, ref, f"32x32 fprop K={K}")


@pytest.mark.parametrize("K,N", [(7168, 384), (18432, 384), (18048, 512), (18304, 384), (7168, 352)])
def test_tile_scales_dgrad_exact(K, N):
    """The 32x32 weight's backward-data product: the same FP8 weight W
    [out = K, in = N] contracted over its rows (read transposed), tiles
    [K/32, N/32].  N = 352 takes the general variant (N not a multiple of
    128)."""
    M = min(K // 32, 1024)
    say(f"[exact] 32x32 dgrad M={M} N={N} K={K}")
    qa, sa = one_hot_a(M, K, K + 4)
    rng = np.random.default_rng(K + 5)
    qw = rng.choice(_NONZERO, (K, N)).astype(np.uint8)
    sw = rng.integers(120, 135, (K // 32, N // 32)).astype(np.uint8)
    c = mx.gemm(dev(qa), dev(sa), dev(qw), dev(sw), "dgrad", "32x32")
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(qa, sa, qw, sw, oracle.BKIND_TILE_T, want_bound=False)
    assert_exact(c, ref, f"32x32 dgrad K={K} N={N}")


def _persistent_rows(qa, M, K, rng):
    """Rows checked in the persistent cases: 24 seeded rows of every 256-row
    tile plus, in every tile, the rows whose nonzero lies in the first or
    the last K step (the split prologue and the last stage)."""
    k = np.argmax(qa != 0, axis=1)
    step = k // 128
    nks = K // 128
    rows = []
    for m0 in range(0, M, 256):
        tile = np.arange(m0, min(m0 + 256, M))
        rows.append(rng.choice(tile, min(24, len(tile)), replace=False))
        rows.append(tile[(step[tile] == 0) | (step[tile] == nks - 1)])
    return np.unique(np.concatenate(rows)).astype(np.int64)


@pytest.mark.parametrize("K,bscale,layout,M,N", [
    (7168, "1x32", "fprop", 4352, 4096), (18432, "1x32", "fprop", 4352, 4096),
    (32768, "1x32", "fprop", 4352, 4096), (4096, "32x32", "fprop", 4352, 4096),
    (4096, "32x32", "dgrad", 4352, 4096),
    (18432, "1x32", "fprop", 4096, 10240),   # 16 x 40 = 640 tiles: a contiguous eighth per XCD
])
def test_persistent_exact(K, bscale, layout, M, N):
    """More output tiles than compute units (17 x 16 = 272, runs of 32 dealt to
    the XCDs in turn; 16 x 40 = 640, a contiguous eighth per XCD): the
    persistent GEMM, whose tiles after the first load their first stages
    while the previous result is stored.  All rows one-hot; the checked rows
    cover every tile row and, across the tiles, the first and last K steps;
    each equals the oracle bit for bit over all N."""
    say(f"[exact] persistent {bscale} {layout} M={M} N={N} K={K}")
    qa, sa = one_hot_a(M, K, K + 11)
    rng = np.random.default_rng(K + 12)
    if bscale == "1x32":
        qb, sb = random_b(N, K, K + 13)
        bk = oracle.BKIND_ROW
    elif layout == "fprop":
        qb, sb = random_b(N, K, K + 13, scale_rows=N // 32)
        bk = oracle.BKIND_TILE
    else:
        qb = rng.choice(_NONZERO, (K, N)).astype(np.uint8)
        sb = rng.integers(120, 135, (K // 32, N // 32)).astype(np.uint8)
        bk = oracle.BKIND_TILE_T
    c = mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb), layout, bscale)
    torch.cuda.synchronize()
    rows = _persistent_rows(qa, M, K, rng)
    ref, _ = oracle.gemm(qa[rows], sa[rows], qb, sb, bk, want_bound=False)
    assert_exact(c.index_select(0, torch.from_numpy(rows).cuda()), ref,
                 f"persistent {bscale} {layout} K={K} ({len(rows)} rows)")


def _offsets(sizes):
    off = np.zeros(len(sizes) + 1, np.int64)
    np.cumsum(sizes, out=off[1:])
    return off


@pytest.mark.parametrize("K", [4096, 2048, 7168, 18048])
def test_grouped_exact(K):
    """The MoE grouped GEMM at the expert shapes' K (and longer): each
    group's rows one-hot against that expert's own weight rows and scales;
    group sizes ragged, one group empty."""
    sizes = [300, 0, 517, 33, 700, 1]
    off = _offsets(sizes)
    T, N, G = int(off[-1]), 288, len(sizes)
    say(f"[exact] grouped T={T} N={N} K={K} G={G}")
    qa, sa = one_hot_a(T, K, K + 6)
    qb, sb = random_b(G * N, K, K + 7)
    qb, sb = qb.reshape(G, N, K), sb.reshape(G, N, K // 32)
    c = mx.grouped_gemm(dev(off), dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_gemm(off, qa, sa, qb, sb, want_bound=False)
    assert_exact(c, ref, f"grouped K={K}")


@pytest.mark.parametrize("K", [4096, 2048])
def test_grouped_persistent_exact(K):
    """The grouped GEMM with 40 x 14 = 560 tiles: every workgroup walks two or
    three, each tile after the first loading its first stage while the
    previous result is stored; ragged and empty groups; every output equals
    the oracle bit for bit."""
    sizes = [1500, 700, 0, 2100, 900, 1300, 33, 2600]
    off = _offsets(sizes)
    T, N, G = int(off[-1]), 3584, len(sizes)
    say(f"[exact] grouped persistent T={T} N={N} K={K} G={G}")
    qa, sa = one_hot_a(T, K, K + 8)
    qb, sb = random_b(G * N, K, K + 9)
    qb, sb = qb.reshape(G, N, K), sb.reshape(G, N, K // 32)
    c = mx.grouped_gemm(dev(off), dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_gemm(off, qa, sa, qb, sb, want_bound=False)
    assert_exact(c, ref, f"grouped persistent K={K}")


@pytest.mark.parametrize("sizes", [[18000, 0, 9001, 13000], [4097, 2049, 130, 31]])
def test_grouped_wgrad_exact(sizes):
    """The per-expert weight gradient over long expert groups (up to 141 K
    steps per expert): the gradient dY [T, M] holds one nonzero per feature m
    (at token t_m), so each expert's dW[g][m][n] is one product (or 0 when
    t_m lies in another group).  Both operands are quantised by the oracle
    (per-group column blocks) and uploaded."""
    off = _offsets(sizes)
    T, G, M, N = int(off[-1]), len(sizes), 256, 320
    say(f"[exact] wgrad T={T} sizes={sizes} M={M} N={N}")
    rng = np.random.default_rng(T)
    t_m = rng.integers(0, T, M)
    dy = np.zeros((T, M), np.float32)
    dy[t_m, np.arange(M)] = rng.choice([-2.0, -0.75, 0.5, 1.0, 1.5, 3.0], M)
    dyb = bits(torch.from_numpy(dy).to(torch.bfloat16))
    xb = bits(W.normal_bf16((T, N), 1.0, T + 1))
    qa, sa = oracle.quant_col_grouped(dyb, off)
    qb, sb = oracle.quant_col_grouped(xb, off)
    c = mx.grouped_gemm_wgrad(dev(off), T, dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_gemm_wgrad(off, qa, sa, qb, sb, want_bound=False)
    got = c.float().cpu().numpy().astype(np.float64)
    owner = np.searchsorted(off, t_m, side="right") - 1            # expert of each m's token
    for g in range(G):
        live = owner == g
        assert (ref[g][~live] == 0).all()
        bad = got[g] != ref[g]
        assert not bad.any(), (g, int(bad.sum()), np.argwhere(bad)[:4])
        if live.any():
            assert np.count_nonzero(ref[g][live]) > 0, g


FUSED_CASES = [  # (M, N, K, layout, bscale)
    (128, 128, 256, "fprop", "1x32"),
    (300, 224, 160, "dgrad", "1x32"),
    (257, 544, 1056, "wgrad", "1x32"),
    (512, 384, 7168, "fprop", "1x32"),
    (300, 256, 18048, "fprop", "1x32"),
    (384, 256, 2048, "fprop", "32x32"),
    (320, 384, 18432, "dgrad", "32x32"),
    (256, 384, 1408, "dgrad", "32x32"),
]


def _fused_operands(M, N, K, layout, bscale, seed):
    qa, sa = one_hot_a(M, K, seed)
    rng = np.random.default_rng(seed + 1)
    if bscale == "1x32":
        qb, sb = random_b(N, K, seed + 1)
        bk = oracle.BKIND_ROW
    elif layout == "fprop":
        qb, sb = random_b(N, K, seed + 1, scale_rows=N // 32)
        bk = oracle.BKIND_TILE
    else:
        qb = rng.choice(_NONZERO, (K, N)).astype(np.uint8)
        sb = rng.integers(120, 135, (K // 32, N // 32)).astype(np.uint8)
        bk = oracle.BKIND_TILE_T
    return qa, sa, qb, sb, bk


@pytest.mark.parametrize("out_elem", ["e4m3", "e5m2"])
@pytest.mark.parametrize("M,N,K,layout,bscale", FUSED_CASES)
def test_fused_producer_bytes_equal_oracle(M, N, K, layout, bscale, out_elem):
    """The fused producer's payload and scale bytes equal the oracle's row
    quantisation of the oracle's own product: every output is exact in BF16
    here, so the BF16 result the epilogue quantises is fixed by the oracle
    alone, and nothing the GPU computed feeds the expected bytes."""
    say(f"[exact] fused {layout} {bscale} {M}x{N}x{K} -> {out_elem}")
    qa, sa, qb, sb, bk = _fused_operands(M, N, K, layout, bscale, M + N + K)
    q, s = mx.gemm_quant(dev(qa), dev(sa), dev(qb), dev(sb), layout, bscale, out_elem)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(qa, sa, qb, sb, bk, want_bound=False)
    wq, ws = oracle.quant_row(bf16_bits_exact(ref), oracle.ELEMS[out_elem])
    assert_bytes(q, wq, f"fused payload {layout} {bscale} K={K}")
    assert_bytes(s, ws, f"fused scales {layout} {bscale} K={K}")


@pytest.mark.parametrize("out_elem", ["e4m3", "e5m2"])
@pytest.mark.parametrize("M,N,K,bscale", [
    (4200, 4096, 1024, "1x32"),    # 17 x 16 = 272 tiles, the last row of tiles ragged
    (4200, 4096, 2048, "32x32"),   # the 32x32 weight's persistent walk
    (2100, 9216, 512, "1x32"),     # 9 x 36 = 324 tiles: a contiguous eighth per XCD
])
def test_fused_producer_persistent_sampled_rows(M, N, K, bscale, out_elem):
    """More tiles than compute units with N a multiple of 256: the fused
    producer walks its tiles persistently and quantises each result on its
    way out of LDS.  The first and last row of every row of tiles and a few
    seeded rows (all N columns) equal the oracle's row quantisation of its
    exact product; rows past M are never written (a sentinel stays)."""
    say(f"[exact] fused persistent {bscale} {M}x{N}x{K} -> {out_elem}")
    qa, sa, qb, sb, bk = _fused_operands(M, N, K, "fprop", bscale, M + N + K + 11)
    Mp = M + 32                    # sentinel rows below the result
    q = torch.full((Mp, N), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((Mp, N // 32), 0xA5, dtype=torch.uint8, device="cuda")
    A, SA, B, SB = dev(qa), dev(sa), dev(qb), dev(sb)
    rc = mx.mx_gemm_quant(mx.GEMM_LAYOUTS["fprop"], mx.BSCALE_KINDS[bscale], mx.ELEM_TYPES[out_elem],
                          M, N, K, A.data_ptr(), SA.data_ptr(), B.data_ptr(), SB.data_ptr(),
                          q.data_ptr(), s.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mx.mx_last_error()
    torch.cuda.synchronize()
    edges = np.concatenate([np.arange(0, M, 256), np.minimum(np.arange(255, M + 255, 256), M - 1)])
    extra = np.random.default_rng(M + K).choice(M, 8, replace=False)
    rows = np.unique(np.concatenate([edges, extra])).astype(np.int64)
    ref, _ = oracle.gemm(qa[rows], sa[rows], qb, sb, bk, want_bound=False)
    wq, ws = oracle.quant_row(bf16_bits_exact(ref), oracle.ELEMS[out_elem])
    ri = torch.from_numpy(rows).cuda()
    assert_bytes(q.index_select(0, ri), wq, "fused persistent payload rows")
    assert_bytes(s.index_select(0, ri), ws, "fused persistent scale rows")
    assert torch.all(q[M:] == 0xA5) and torch.all(s[M:] == 0xA5), "rows past M were written"


def test_fused_producer_full_size_sampled_rows():
    """The up projection's shape (32768 x 18432 x 7168) through the fused
    producer with one-hot token rows against the oracle-quantised stack
    weight: 32 seeded full rows of payload and scale bytes (all 18432
    columns) equal the oracle's row quantisation of its exact product."""
    T, F, H = 32768, 18432, 7168
    Wt = W.normal_bf16((F, H), 0.02, 96, "cuda")          # the stack weights' N(0, 0.02)
    say(f"[exact] fused full size T={T} F={F} H={H}")
    qw, sw = oracle.quant_row(bits(Wt))
    qa, sa = one_hot_a(T, H, 97)
    q, s = mx.gemm_quant(dev(qa), dev(sa), dev(qw), dev(sw))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(98).choice(T, 32, replace=False))
    rows[0], rows[-1] = 0, T - 1
    ref, _ = oracle.gemm(qa[rows], sa[rows], qw, sw, want_bound=False)
    wq, ws = oracle.quant_row(bf16_bits_exact(ref))
    ri = torch.from_numpy(rows).cuda()
    assert_bytes(q.index_select(0, ri), wq, "fused full-size payload rows")
    assert_bytes(s.index_select(0, ri), ws, "fused full-size scale rows")
