"""GPU parity of mx_gemm against the oracle: every element of C within
|gpu - ref| <= 2^-7 * sum_k |a_k b_k| + 1e-6, ref and the bound computed in
binary64 by the oracle from the same quantised bytes.  Small cases quantise
with the oracle and upload its bytes; full-size cases check seeded samples of
C end to end (GPU quant + GEMM against oracle quant + GEMM of the same BF16
rows and columns)."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_microscaled_precision_amd as mx
from mxfp8_microscaled_precision_amd import workloads as W
from parity import assert_gemm, bits, dev, say

pytestmark = pytest.mark.gpu


def _run(a, sa, b, sb, layout, bscale, bkind, what):
    say(f"[gemm] {what} layout={layout} bscale={bscale} A={a.shape} B={b.shape}")
    c = mx.gemm(dev(a), dev(sa), dev(b), dev(sb), layout, bscale)
    torch.cuda.synchronize()
    ref, bound = oracle.gemm(a, sa, b, sb, bkind)
    assert_gemm(c, ref, bound, what)


def test_tiny_config_fprop():
    d = W.tiny("cpu")
    qa, sa = oracle.quant_row(bits(d["A"]))
    qw, sw = oracle.quant_row(bits(d["W"]))
    _run(qa, sa, qw, sw, "fprop", "1x32", oracle.BKIND_ROW, "tiny")


def test_largest_k():
    """The longest contraction the boundary accepts (K = 2^23 - 32, so a
    256-row tile of an operand spans just under 2^31 bytes), with ragged M
    and N: every element against the oracle."""
    M, N, K = 3, 40, (1 << 23) - 32
    qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, 71)))
    qb, sb = oracle.quant_row(bits(W.normal_bf16((N, K), 1.0, 72)))
    _run(qa, sa, qb, sb, "fprop", "1x32", oracle.BKIND_ROW, "largest K")


SHAPES = [(1, 1, 32), (64, 64, 32), (300, 200, 160), (257, 513, 96), (512, 256, 4096),
          (33, 290, 1056), (256, 256, 128),
          # K a multiple of 128 but not of 512: the pipelined kernel with a partial last
          # group of four K steps (1, 2 and 3 steps of it real)
          (300, 520, 1152), (257, 384, 1280), (512, 256, 1408)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("layout", ["fprop", "dgrad", "wgrad"])
def test_row_scales_all_layouts(M, N, K, layout):
    # the three products of a linear layer are all "TN" on 1x32 operands;
    # build them the way the layer does (row / column quantisation)
    seed = M * 7 + N * 3 + K
    if layout == "fprop":      # Y = X W^T: a = X_row [M,K], b = W_row [N,K]
        qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, seed)))
        qb, sb = oracle.quant_row(bits(W.normal_bf16((N, K), 0.02, seed + 1)))
    elif layout == "dgrad":    # dX = dY W: a = dY_row [M,K=out], b = W_col_T [N=in, K=out]
        qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1e-3, seed)))
        qb, sb = oracle.quant_col(bits(W.normal_bf16((K, N), 0.02, seed + 1)))
    else:                      # dW = dY^T X: a = dY_col_T [M=out, K=tok], b = X_col_T [N=in, K=tok]
        qa, sa = oracle.quant_col(bits(W.normal_bf16((K, M), 1e-3, seed)))
        qb, sb = oracle.quant_col(bits(W.normal_bf16((K, N), 1.0, seed + 1)))
    _run(qa, sa, qb, sb, layout, "1x32", oracle.BKIND_ROW, f"{layout} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 224, 160), (257, 544, 1056), (512, 256, 4096),
                                   (384, 384, 2048), (640, 896, 1536),
                                   (300, 512, 1152), (257, 384, 1408)])
def test_block32_weight_fprop_and_dgrad(M, N, K):
    # fprop: Y[M, out=N] = X[M, in=K] W[out=N, in=K]^T with W in 32x32 tiles
    qx, sx = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, M + K)))
    qw, sw = oracle.quant_block32(bits(W.normal_bf16((N, K), 0.02, N + K)))
    _run(qx, sx, qw, sw, "fprop", "32x32", oracle.BKIND_TILE, f"fprop32 {M}x{N}x{K}")
    # dgrad: dX[M, in=N] = dY[M, out=K] W[out=K, in=N], the same FP8 weight
    qd, sd = oracle.quant_row(bits(W.normal_bf16((M, K), 1e-3, M + 2 * K)))
    qw2, sw2 = oracle.quant_block32(bits(W.normal_bf16((K, N), 0.02, 3 * N + K)))
    _run(qd, sd, qw2, sw2, "dgrad", "32x32", oracle.BKIND_TILE_T, f"dgrad32 {M}x{N}x{K}")


def test_one_hot_rows_select_b():
    """K = 32, A rows one-hot 1.0: C rows are B's rows (exact in BF16)."""
    N = 96
    qb, sb = oracle.quant_row(bits(W.normal_bf16((N, 32), 1.0, 3)))
    qa = np.zeros((32, 32), np.uint8)
    qa[np.arange(32), np.arange(32)] = 0x38
    sa = np.full((32, 1), 127, np.uint8)
    c = mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb))
    ref, _ = oracle.gemm(qa, sa, qb, sb)
    assert np.array_equal(c.float().cpu().numpy().astype(np.float64), ref)


def test_k_zero_writes_zeros():
    def e(r):
        return torch.empty((r, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    mx.gemm(e(5), e(5), e(7), e(7), out=out)
    torch.cuda.synchronize()
    assert (out.float() == 0).all()


def test_nan_scale_propagates():
    M, N, K = 40, 48, 64
    qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, 5)))
    qb, sb = oracle.quant_row(bits(W.normal_bf16((N, K), 1.0, 6)))
    sa[3, 1] = 0xFF
    _run(qa, sa, qb, sb, "fprop", "1x32", oracle.BKIND_ROW, "nan scale")


def test_deterministic():
    qa, sa = oracle.quant_row(bits(W.normal_bf16((512, 1024), 1.0, 8)))
    qb, sb = oracle.quant_row(bits(W.normal_bf16((384, 1024), 1.0, 9)))
    A, SA, B, SB = dev(qa), dev(sa), dev(qb), dev(sb)
    assert torch.equal(mx.gemm(A, SA, B, SB), mx.gemm(A, SA, B, SB))


# --------------------------------------------------------------------------
# Full-size products, sampled
# --------------------------------------------------------------------------

def _sample(n, k, rng, extra=()):
    idx = np.unique(np.concatenate([[0, n - 1], list(extra), rng.integers(0, n, k)]))
    return idx.astype(np.int64)


def _end_to_end(what, c_gpu, a_src, a_mode, b_src, b_mode, bkind, rows, cols):
    """Compare c_gpu[rows][:, cols] with the oracle's quantise-then-multiply
    of the same BF16 sources.  a_src/b_src: BF16 device tensors; *_mode says
    how the operand is quantised: 'row' (rows of the source are the operand
    rows) or 'col' (columns of the source are the operand rows, blocks run
    down the column), 'tile' / 'tile_t' for the 32x32 weight."""
    ri = torch.from_numpy(rows).cuda()
    ci = torch.from_numpy(cols).cuda()
    if a_mode == "row":
        qa, sa = oracle.quant_row(bits(a_src.index_select(0, ri)))
    else:
        qa, sa = oracle.quant_col(bits(a_src.index_select(1, ri)))
    if b_mode == "row":
        qb, sb = oracle.quant_row(bits(b_src.index_select(0, ci)))
    elif b_mode == "col":
        qb, sb = oracle.quant_col(bits(b_src.index_select(1, ci)))
    elif b_mode == "tile":       # cols are whole 32-row groups of the weight [N, K]
        qb, sb = oracle.quant_block32(bits(b_src.index_select(0, ci)))
    else:                        # tile_t: cols are whole 32-column groups of weight [K, N]
        qb, sb = oracle.quant_block32(bits(b_src.index_select(1, ci)))
    ref, bound = oracle.gemm(qa, sa, qb, sb, bkind)
    got = c_gpu.index_select(0, ri).index_select(1, ci)
    assert_gemm(got, ref, bound, what)


def _groups32(n, k, rng):
    g = np.unique(np.concatenate([[0, n // 32 - 1], rng.integers(0, n // 32, k)]))
    return (g[:, None] * 32 + np.arange(32)[None, :]).ravel().astype(np.int64)


def test_dense_full_three_products():
    d = W.dense("cuda")
    X, Wt, dY = d["X"], d["W"], d["dY"]
    M, K = X.shape
    N = Wt.shape[0]
    say(f"[gemm] dense full M={M} N={N} K={K}")
    qx, sx, qxt, sxt = mx.quant(X, "dual")
    qw, sw, qwt, swt = mx.quant(Wt, "dual")
    qd, sd, qdt, sdt = mx.quant(dY, "dual")
    Y = mx.gemm(qx, sx, qw, sw, "fprop")
    dX = mx.gemm(qd, sd, qwt, swt, "dgrad")
    dW = mx.gemm(qdt, sdt, qxt, sxt, "wgrad")
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    _end_to_end("dense fprop", Y, X, "row", Wt, "row", oracle.BKIND_ROW,
                _sample(M, 48, rng), _sample(N, 48, rng))
    _end_to_end("dense dgrad", dX, dY, "row", Wt, "col", oracle.BKIND_ROW,
                _sample(M, 48, rng), _sample(K, 48, rng))
    _end_to_end("dense wgrad", dW, dY, "col", X, "col", oracle.BKIND_ROW,
                _sample(N, 32, rng), _sample(K, 32, rng))


def test_block32_full_four_products():
    d = W.block32("cuda")
    W1, W2, X1, X2 = d["W1"], d["W2"], d["X1"], d["X2"]
    say(f"[gemm] block32 full W1={tuple(W1.shape)} W2={tuple(W2.shape)} X1={tuple(X1.shape)}")
    q1, s1 = mx.quant(W1, "32x32")
    q2, s2 = mx.quant(W2, "32x32")
    qx1, sx1 = mx.quant(X1, "row")
    qx2, sx2 = mx.quant(X2, "row")
    Y1 = mx.gemm(qx1, sx1, q1, s1, "fprop", "32x32")      # [T, 2048]
    Y2 = mx.gemm(qx2, sx2, q2, s2, "fprop", "32x32")      # [T, 7168]
    dX1 = mx.gemm(qx2, sx2, q1, s1, "dgrad", "32x32")     # dY1 = X2 [T, 2048] -> [T, 7168]
    dX2 = mx.gemm(qx1, sx1, q2, s2, "dgrad", "32x32")     # dY2 = X1 [T, 7168] -> [T, 2048]
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    T = X1.shape[0]
    _end_to_end("block32 fprop1", Y1, X1, "row", W1, "tile", oracle.BKIND_TILE,
                _sample(T, 40, rng), _groups32(W1.shape[0], 2, rng))
    _end_to_end("block32 fprop2", Y2, X2, "row", W2, "tile", oracle.BKIND_TILE,
                _sample(T, 40, rng), _groups32(W2.shape[0], 2, rng))
    _end_to_end("block32 dgrad1", dX1, X2, "row", W1, "tile_t", oracle.BKIND_TILE_T,
                _sample(T, 40, rng), _groups32(W1.shape[1], 2, rng))
    _end_to_end("block32 dgrad2", dX2, X1, "row", W2, "tile_t", oracle.BKIND_TILE_T,
                _sample(T, 40, rng), _groups32(W2.shape[1], 2, rng))


def _nan_filled(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")


def _assert_every_tile_written(c, what):
    """The output started as NaN: none left means every tile of the grid
    was written (the workgroup-to-tile map covers the whole output)."""
    torch.cuda.synchronize()
    assert not torch.isnan(c).any().item(), f"{what}: an output tile was never written"


def _contract_sample(what, c, qa, sa, qb, sb, bkind, qbr, sbr, rng):
    """The stack products' sample: 32 seeded rows of C over all N, 32 seeded
    columns of C over all M, and the four corner 32x32 tiles, each against
    the oracle's binary64 product of the oracle's own quantisation of the
    same BF16 sources.  (qa, sa) is A; (qb, sb, bkind) is B as the GEMM takes
    it; (qbr, sbr) is the same B in row form ([N, K] with per-row scales),
    which selects any set of columns: for 32x32 weights the tile scale
    expanded over its 32 rows (and the weight transposed for the dgrad), a
    relayout of the oracle's bytes that the oracle's own pins show equal."""
    M, N = c.shape
    rows = np.sort(rng.choice(M, 32, replace=False)).astype(np.int64)
    cols = np.sort(rng.choice(N, 32, replace=False)).astype(np.int64)
    say(f"[gemm] {what}: 32 full rows, 32 full columns, 4 corner tiles of {M}x{N}")
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ref, bound = oracle.gemm(qa[rows], sa[rows], qb, sb, bkind)
    assert_gemm(c.index_select(0, ri), ref, bound, f"{what}: rows {rows.tolist()}")
    ref, bound = oracle.gemm(qa, sa, qbr[cols], sbr[cols], oracle.BKIND_ROW)
    assert_gemm(c.index_select(1, ci), ref, bound, f"{what}: columns {cols.tolist()}")
    for r0 in (0, M - 32):
        for c0 in (0, N - 32):
            ref, bound = oracle.gemm(qa[r0:r0 + 32], sa[r0:r0 + 32], qbr[c0:c0 + 32],
                                     sbr[c0:c0 + 32], oracle.BKIND_ROW)
            assert_gemm(c[r0:r0 + 32, c0:c0 + 32], ref, bound, f"{what}: corner tile ({r0}, {c0})")


def _linear_layer_products(name, X, Wt, dY, rng):
    """fprop, dgrad and wgrad of one linear layer at full size, each checked
    on the contract sample against the oracle's dual-axis quantisation of
    the same BF16 sources and its binary64 product."""
    qx, sx, qxt, sxt = mx.quant(X, "dual")
    qw, sw, qwt, swt = mx.quant(Wt, "dual")
    qd, sd, qdt, sdt = mx.quant(dY, "dual")
    T, H = X.shape
    F = Wt.shape[0]
    ox, osx, oxt, osxt = oracle.quant_dual(bits(X))
    ow, osw, owt, oswt = oracle.quant_dual(bits(Wt))
    od, osd, odt, osdt = oracle.quant_dual(bits(dY))
    row = oracle.BKIND_ROW
    Y = mx.gemm(qx, sx, qw, sw, "fprop", out=_nan_filled(T, F))
    _assert_every_tile_written(Y, f"stack {name} fprop")
    _contract_sample(f"stack {name} fprop", Y, ox, osx, ow, osw, row, ow, osw, rng)
    del Y
    dX = mx.gemm(qd, sd, qwt, swt, "dgrad", out=_nan_filled(T, H))
    _assert_every_tile_written(dX, f"stack {name} dgrad")
    _contract_sample(f"stack {name} dgrad", dX, od, osd, owt, oswt, row, owt, oswt, rng)
    del dX
    dW = mx.gemm(qdt, sdt, qxt, sxt, "wgrad", out=_nan_filled(F, H))
    _assert_every_tile_written(dW, f"stack {name} wgrad")
    _contract_sample(f"stack {name} wgrad", dW, odt, osdt, oxt, osxt, row, oxt, osxt, rng)
    del dW


def test_stack_layer_full_six_products():
    """Both linear layers of one stack layer (7168 -> 18432 -> 7168 at 32768
    tokens): the up projection's and the down projection's three products."""
    d = W.stack_layer(0, "cuda")
    Xu, Xd, dYu, dYd, Wu, Wd = (d[k] for k in ("X_up", "X_dn", "dY_up", "dY_dn", "W_up", "W_dn"))
    say(f"[gemm] stack layer T={Xu.shape[0]} H={Xu.shape[1]} F={Wu.shape[0]}")
    rng = np.random.default_rng(41)
    _linear_layer_products("up", Xu, Wu, dYu, rng)
    _linear_layer_products("down", Xd, Wd, dYd, rng)


def test_stack_layer_full_32x32_variant():
    """The 32x32-weight variant of the same stack layer: each weight
    quantised once in 32x32 tiles, fprop with the tile scales and dgrad
    reading the same FP8 weight transposed, for both projections (N up to
    18432, i.e. more than 32 n-tiles: the other workgroup-to-tile map than
    the 16384-token weight configuration uses), on the contract sample."""
    d = W.stack_layer(0, "cuda")
    rng = np.random.default_rng(43)
    for name, X, Wt, dY in (("up", d["X_up"], d["W_up"], d["dY_up"]),
                            ("down", d["X_dn"], d["W_dn"], d["dY_dn"])):
        F, H = Wt.shape
        say(f"[gemm] stack 32x32 {name}: W {F}x{H}")
        q32, s32 = mx.quant(Wt, "32x32")
        o32, os32 = oracle.quant_block32(bits(Wt))
        qx, sx = mx.quant(X, "row")
        ox, osx = oracle.quant_row(bits(X))
        T = X.shape[0]
        Y = mx.gemm(qx, sx, q32, s32, "fprop", "32x32", out=_nan_filled(T, F))
        _assert_every_tile_written(Y, f"stack 32x32 {name} fprop")
        # forward: B = W [F, H], tile row n/32 scales output column n
        _contract_sample(f"stack 32x32 {name} fprop", Y, ox, osx, o32, os32, oracle.BKIND_TILE,
                         o32, np.repeat(os32, 32, axis=0), rng)
        del Y, qx, sx, ox, osx
        qd, sd = mx.quant(dY, "row")
        od, osd = oracle.quant_row(bits(dY))
        dX = mx.gemm(qd, sd, q32, s32, "dgrad", "32x32", out=_nan_filled(T, H))
        _assert_every_tile_written(dX, f"stack 32x32 {name} dgrad")
        # backward: output column n is input feature n of W [F, H]; in row
        # form B = W^T [H, F] with tile column n/32's scales along F
        _contract_sample(f"stack 32x32 {name} dgrad", dX, od, osd, o32, os32, oracle.BKIND_TILE_T,
                         np.ascontiguousarray(o32.T), np.repeat(np.ascontiguousarray(os32.T), 32, axis=0),
                         rng)
        del dX, qd, sd, od, osd


# --------------------------------------------------------------------------
# Tile order: every tile written once, in both workgroup-to-tile maps
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [
    (2088, 7264, 512),   # 9 x 29 = 261 tiles, at most 32 n-tiles: runs of 32 dealt to the XCDs
                         # in turn over the first 256, the last 5 in place; partial edge tiles
    (2100, 8400, 512),   # 9 x 33 = 297 tiles: more than 32 n-tiles, eighths not whole
                         # groups of 8 tiles, so runs of 32 round-robin again
    (1948, 10216, 512),  # 8 x 40 = 320 tiles: a contiguous eighth of 40 tiles per XCD
])
def test_every_tile_written(M, N, K):
    say(f"[gemm] tile coverage M={M} N={N} K={K}")
    qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, 51)))
    qb, sb = oracle.quant_row(bits(W.normal_bf16((N, K), 1.0, 52)))
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb), "fprop", out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "an output tile was never written"
    ref, bound = oracle.gemm(qa, sa, qb, sb, oracle.BKIND_ROW)
    assert_gemm(out, ref, bound, f"tile coverage {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [
    (10168, 5096, 512),   # 40 x 20 = 800 tiles (at most 32 n-tiles): 3 or 4 per workgroup
    (1180, 28144, 1024),  # 5 x 110 = 550 tiles, eighths not whole groups: runs of 32, 2 or 3 each
    (3032, 7672, 512),    # 12 x 30 = 360: the tiles past the first 256 keep their place
    (4056, 10232, 512),   # 16 x 40 = 640 tiles: a contiguous eighth of 80 per XCD, 2 or 3 each
])
def test_persistent_walk(M, N, K):
    """The 1x32 GEMM with more tiles than compute units runs one workgroup
    per unit walking several tiles, each tile's first loads overlapping the
    previous tile's stores.  Every tile is written, and one full row of every
    row of tiles and one full column of every column of tiles (so a row and
    a column of every tile, edge tiles included) equal the oracle's product."""
    say(f"[gemm] persistent walk M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, 53)))
    qb, sb = oracle.quant_row(bits(W.normal_bf16((N, K), 1.0, 54)))
    out = _nan_filled(M, N)
    mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb), "fprop", out=out)
    _assert_every_tile_written(out, f"persistent {M}x{N}x{K}")
    rows = np.minimum(np.arange(0, M, 256) + rng.integers(0, 256, (M + 255) // 256), M - 1)
    cols = np.minimum(np.arange(0, N, 256) + rng.integers(0, 256, (N + 255) // 256), N - 1)
    rows = np.unique(np.concatenate([rows, [M - 1]])).astype(np.int64)
    cols = np.unique(np.concatenate([cols, [N - 1]])).astype(np.int64)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ref, bound = oracle.gemm(qa[rows], sa[rows], qb, sb, oracle.BKIND_ROW)
    assert_gemm(out.index_select(0, ri), ref, bound, f"persistent {M}x{N}x{K}: rows")
    ref, bound = oracle.gemm(qa, sa, qb[cols], sb[cols], oracle.BKIND_ROW)
    assert_gemm(out.index_select(1, ci), ref, bound, f"persistent {M}x{N}x{K}: columns")


@pytest.mark.parametrize("layout,M,N,K", [
    ("fprop", 10168, 5088, 512),   # 40 x 20 = 800 tiles; the last n-tile 224 columns wide
    ("fprop", 1180, 28160, 512),   # 5 x 110 = 550 tiles: runs of 32 (eighths not whole groups)
    ("fprop", 4056, 10240, 512),   # 16 x 40 = 640 tiles: a contiguous eighth per XCD
    ("dgrad", 3032, 7552, 1024),   # 12 x 30 = 360 tiles; the last n-tile 128 columns wide
    ("dgrad", 10168, 5120, 512),   # 40 x 20 = 800 tiles
])
def test_persistent_walk_block32(layout, M, N, K):
    """The persistent GEMM with a 32x32-tile weight: fprop takes W [N, K] in
    tiles, dgrad the transposed weight W [K, N].  Every tile is written, and
    one full row of every row of tiles and one full column of every column of
    tiles equal the oracle's product; the columns use W's bytes in row form
    (the tile scale repeated over its 32 rows, transposed for dgrad), a
    relayout of the oracle's own quantisation."""
    say(f"[gemm] persistent walk, 32x32 weight, {layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K + 1)
    qa, sa = oracle.quant_row(bits(W.normal_bf16((M, K), 1.0, 55)))
    if layout == "fprop":
        qb, sb = oracle.quant_block32(bits(W.normal_bf16((N, K), 0.02, 56)))
        bkind = oracle.BKIND_TILE
        qbr, sbr = qb, np.repeat(sb, 32, axis=0)
    else:
        qb, sb = oracle.quant_block32(bits(W.normal_bf16((K, N), 0.02, 57)))
        bkind = oracle.BKIND_TILE_T
        qbr = np.ascontiguousarray(qb.T)
        sbr = np.repeat(np.ascontiguousarray(sb.T), 32, axis=0)
    out = _nan_filled(M, N)
    mx.gemm(dev(qa), dev(sa), dev(qb), dev(sb), layout, "32x32", out=out)
    _assert_every_tile_written(out, f"persistent 32x32 {layout} {M}x{N}x{K}")
    rows = np.minimum(np.arange(0, M, 256) + rng.integers(0, 256, (M + 255) // 256), M - 1)
    cols = np.minimum(np.arange(0, N, 256) + rng.integers(0, 256, (N + 255) // 256), N - 1)
    rows = np.unique(np.concatenate([rows, [M - 1]])).astype(np.int64)
    cols = np.unique(np.concatenate([cols, [N - 1]])).astype(np.int64)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    ref, bound = oracle.gemm(qa[rows], sa[rows], qb, sb, bkind)
    assert_gemm(out.index_select(0, ri), ref, bound, f"persistent 32x32 {layout}: rows")
    ref, bound = oracle.gemm(qa, sa, qbr[cols], sbr[cols], oracle.BKIND_ROW)
    assert_gemm(out.index_select(1, ci), ref, bound, f"persistent 32x32 {layout}: columns")


@pytest.mark.parametrize("product", ["fprop", "dgrad", "wgrad"])
def test_dense_config_every_element(product):
    """The dense configuration (8192 x 4096 x 4096): every output element of
    one product against the oracle's own dual-axis quantisation and binary64
    product of the same BF16 inputs."""
    d = W.dense("cuda")
    X, Wt, dY = d["X"], d["W"], d["dY"]
    M, K = X.shape
    N = Wt.shape[0]
    say(f"[gemm] dense config {product}, every element: M={M} N={N} K={K}")
    qx, sx, qxt, sxt = mx.quant(X, "dual")
    qw, sw, qwt, swt = mx.quant(Wt, "dual")
    qd, sd, qdt, sdt = mx.quant(dY, "dual")
    if product == "fprop":
        got = mx.gemm(qx, sx, qw, sw, "fprop")
    elif product == "dgrad":
        got = mx.gemm(qd, sd, qwt, swt, "dgrad")
    else:
        got = mx.gemm(qdt, sdt, qxt, sxt, "wgrad")
    torch.cuda.synchronize()
    ox, osx, oxt, osxt = oracle.quant_dual(bits(X))
    ow, osw, owt, oswt = oracle.quant_dual(bits(Wt))
    od, osd, odt, osdt = oracle.quant_dual(bits(dY))
    a, sa, b, sb = {"fprop": (ox, osx, ow, osw), "dgrad": (od, osd, owt, oswt),
                    "wgrad": (odt, osdt, oxt, osxt)}[product]
    ref, bound = oracle.gemm(a, sa, b, sb, oracle.BKIND_ROW)
    assert_gemm(got, ref, bound, f"dense {product}, every element")


@pytest.mark.parametrize("product", ["fprop1", "fprop2", "dgrad1", "dgrad2"])
def test_block32_config_every_element(product):
    """The 32x32-weight configuration (16384 tokens, 7168 <-> 2048): every
    output element of one product against the oracle's own quantisation
    (32x32 tiles for the weights, 1x32 rows for the activations) and binary64
    product of the same BF16 inputs."""
    d = W.block32("cuda")
    W1, W2, X1, X2 = d["W1"], d["W2"], d["X1"], d["X2"]
    say(f"[gemm] block32 config {product}, every element")
    x, w, layout, bk, wsel = {
        "fprop1": (X1, W1, "fprop", oracle.BKIND_TILE, 0),
        "fprop2": (X2, W2, "fprop", oracle.BKIND_TILE, 0),
        "dgrad1": (X2, W1, "dgrad", oracle.BKIND_TILE_T, 1),
        "dgrad2": (X1, W2, "dgrad", oracle.BKIND_TILE_T, 1),
    }[product]
    qx, sx = mx.quant(x, "row")
    qw, sw = mx.quant(w, "32x32")[:2]
    got = mx.gemm(qx, sx, qw, sw, layout, "32x32")
    torch.cuda.synchronize()
    ox, osx = oracle.quant_row(bits(x))
    ow, osw = oracle.quant_block32(bits(w))
    ref, bound = oracle.gemm(ox, osx, ow, osw, bk)
    assert_gemm(got, ref, bound, f"block32 {product}, every element")


def test_binding_rejects_mismatched_operands():
    """The binding derives the sizes from the tensors, and the library reads
    exactly the bytes those sizes describe: operands whose shapes disagree
    (a short B, wrong scale shapes, a wrong output) raise before any launch."""
    u8 = dict(dtype=torch.uint8, device="cuda")
    a, sa = torch.zeros((64, 256), **u8), torch.zeros((64, 8), **u8)
    b, sb = torch.zeros((96, 256), **u8), torch.zeros((96, 8), **u8)
    mx.gemm(a, sa, b, sb)                                               # consistent: fine
    bad = [
        (a, sa, torch.zeros((96, 128), **u8), torch.zeros((96, 4), **u8), "fprop", "1x32"),  # short K
        (a, torch.zeros((64, 4), **u8), b, sb, "fprop", "1x32"),            # sa for another K
        (a, sa, b, torch.zeros((96, 4), **u8), "wgrad", "1x32"),            # sb for another K
        (a, sa, b, sb, "fprop", "32x32"),                                   # row scales, not tiles [N/32, K/32]
        (a, sa, torch.zeros((128, 96), **u8), torch.zeros((4, 2), **u8), "dgrad", "32x32"),  # weight [K, N]
    ]
    for args in bad:
        with pytest.raises(ValueError):
            mx.gemm(*args[:4], layout=args[4], bscale=args[5])
        with pytest.raises(ValueError):
            mx.gemm_quant(*args[:4], layout=args[4], bscale=args[5])
    with pytest.raises(ValueError):
        mx.gemm(a, sa, b, sb, out=torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda"))
    off = torch.tensor([0, 30, 64], dtype=torch.int64, device="cuda")
    be, sbe = torch.zeros((2, 96, 256), **u8), torch.zeros((2, 96, 8), **u8)
    mx.grouped_gemm(off, a, sa, be, sbe)                                # consistent: fine
    for bb, ss in ((torch.zeros((3, 96, 256), **u8), torch.zeros((3, 96, 8), **u8)),  # 3 experts, 2 groups
                   (torch.zeros((2, 96, 128), **u8), torch.zeros((2, 96, 4), **u8)),  # short K
                   (be, torch.zeros((2, 96, 4), **u8))):                              # scales
        with pytest.raises(ValueError):
            mx.grouped_gemm(off, a, sa, bb, ss)
    with pytest.raises(ValueError):
        mx.grouped_gemm(off, a, sa, be, sbe, out=torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
