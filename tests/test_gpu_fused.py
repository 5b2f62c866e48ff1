"""GPU parity of the fused producer (mx_gemm_quant): the GEMM's BF16 result
quantised in 1x32 blocks along N inside the epilogue.

Two checks.  (1) Its bytes equal the row quantiser applied to the BF16 result
of the unfused GEMM, for every layout and scale kind and both payload types
(the same BF16 values go through the same rule).  (2) Against the oracle:
the dequantised output lies within the GEMM tolerance plus the payload's
rounding of the binary64 product: |deq - ref| <= tol + u (|ref| + tol) + q_e,
tol = 2^-7 sum|ab| + 1e-6, u = 2^-4 (E4M3) or 2^-3 (E5M2) the half-ulp of
the payload's 3 or 2 mantissa bits, q_e = half the smallest subnormal step
at the block's scale (2^(e-10) for E4M3, 2^(e-17) for E5M2)."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_microscaled_precision_amd as mx
from mxfp8_microscaled_precision_amd import workloads as W
from parity import assert_bytes, bits, dev, host, say

pytestmark = pytest.mark.gpu

CASES = [  # (M, N, K, layout, bscale)
    (128, 128, 256, "fprop", "1x32"),
    (300, 224, 160, "dgrad", "1x32"),
    (257, 544, 1056, "wgrad", "1x32"),
    (512, 384, 2048, "fprop", "1x32"),
    (384, 256, 2048, "fprop", "32x32"),
    (320, 384, 1536, "dgrad", "32x32"),
    (300, 256, 1152, "fprop", "1x32"),   # partial last group of four K steps
    (256, 384, 1408, "dgrad", "32x32"),
]


def _operands(M, N, K, layout, bscale, seed):
    qa, sa = oracle.quant_row(bits(W.student_t_bf16((M, K), 3, seed)))
    if bscale == "1x32":
        qb, sb = oracle.quant_row(bits(W.normal_bf16((N, K), 0.02, seed + 1)))
        bk = oracle.BKIND_ROW
    elif layout == "fprop":
        qb, sb = oracle.quant_block32(bits(W.normal_bf16((N, K), 0.02, seed + 1)))
        bk = oracle.BKIND_TILE
    else:
        qb, sb = oracle.quant_block32(bits(W.normal_bf16((K, N), 0.02, seed + 1)))
        bk = oracle.BKIND_TILE_T
    return qa, sa, qb, sb, bk


@pytest.mark.parametrize("out_elem", ["e4m3", "e5m2"])
@pytest.mark.parametrize("M,N,K,layout,bscale", CASES)
def test_fused_equals_quantised_gemm_and_oracle_bound(M, N, K, layout, bscale, out_elem):
    say(f"[fused] {layout} {bscale} {M}x{N}x{K} -> {out_elem}")
    qa, sa, qb, sb, bk = _operands(M, N, K, layout, bscale, M + N + K)
    A, SA, B, SB = dev(qa), dev(sa), dev(qb), dev(sb)
    q, s = mx.gemm_quant(A, SA, B, SB, layout, bscale, out_elem)
    c = mx.gemm(A, SA, B, SB, layout, bscale)
    q2, s2 = mx.quant(c, "row", out_elem)
    torch.cuda.synchronize()
    assert_bytes(q, host(q2), "fused payload vs quantised GEMM")
    assert_bytes(s, host(s2), "fused scales vs quantised GEMM")
    ref, bound = oracle.gemm(qa, sa, qb, sb, bk)
    _assert_within_bound(host(q), host(s), ref, bound, out_elem)


def _assert_within_bound(q, s, ref, bound, out_elem, what=""):
    """Dequantised fused output within the GEMM tolerance plus the payload's
    rounding of the binary64 product (the bound in the module docstring)."""
    elem = oracle.ELEMS[out_elem]
    table = oracle.e5m2_decode_table() if elem == oracle.ELEM_E5M2 else oracle.e4m3_decode_table()
    e = s.astype(np.int64) - 127
    deq = table[q] * np.exp2(np.repeat(e, 32, axis=1))
    tol = 2.0 ** -7 * bound + 1e-6
    u, sub = (2.0 ** -3, 17) if elem == oracle.ELEM_E5M2 else (2.0 ** -4, 10)
    lim = tol + u * (np.abs(ref) + tol) + np.exp2(np.repeat(e, 32, axis=1) - sub)
    bad = ~(np.abs(deq - ref) <= lim)
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:4])


@pytest.mark.parametrize("out_elem", ["e4m3", "e5m2"])
@pytest.mark.parametrize("M,N,K", [
    (10168, 5088, 512),   # 40 x 20 = 800 tiles (at most 32 n-tiles: runs of 32 per XCD)
    (1180, 28160, 512),   # 5 x 110 = 550 tiles: runs of 32 (eighths not whole groups)
    (4056, 10240, 512),   # 16 x 40 = 640 tiles: a contiguous eighth per XCD
    (3032, 7648, 1024),   # 12 x 30 = 360 tiles; the last n-tile 224 columns wide
])
def test_fused_many_tiles(M, N, K, out_elem):
    """The fused producer over hundreds of tiles with ragged edges, in both
    workgroup-to-tile maps.  Outputs start as a sentinel byte: every byte
    equals the row quantiser applied to the unfused GEMM's result (so every
    tile was written), and one full row of every row of tiles lies within
    the oracle bound."""
    say(f"[fused] many tiles {M}x{N}x{K} -> {out_elem}")
    qa, sa, qb, sb, bk = _operands(M, N, K, "fprop", "1x32", M + N + K + 7)
    A, SA, B, SB = dev(qa), dev(sa), dev(qb), dev(sb)
    q = torch.full((M, N), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((M, N // 32), 0xA5, dtype=torch.uint8, device="cuda")
    rc = mx.mx_gemm_quant(mx.GEMM_LAYOUTS["fprop"], mx.BSCALE_KINDS["1x32"], mx.ELEM_TYPES[out_elem],
                          M, N, K, A.data_ptr(), SA.data_ptr(), B.data_ptr(), SB.data_ptr(),
                          q.data_ptr(), s.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mx.mx_last_error()
    q2, s2 = mx.quant(mx.gemm(A, SA, B, SB), "row", out_elem)
    torch.cuda.synchronize()
    assert_bytes(q, host(q2), "fused payload vs quantised GEMM")
    assert_bytes(s, host(s2), "fused scales vs quantised GEMM")
    rng = np.random.default_rng(M + N)
    rows = np.minimum(np.arange(0, M, 256) + rng.integers(0, 256, (M + 255) // 256), M - 1)
    rows = np.unique(np.concatenate([rows, [M - 1]])).astype(np.int64)
    ref, bound = oracle.gemm(qa[rows], sa[rows], qb, sb, bk)
    _assert_within_bound(host(q)[rows], host(s)[rows], ref, bound, out_elem, "sampled rows")


@pytest.mark.parametrize("layout,bscale,N", [("dgrad", "32x32", 512), ("fprop", "32x32", 544),
                                             ("wgrad", "1x32", 320)])
def test_fused_k_zero_every_layout(layout, bscale, N):
    """An empty contraction through every operand layout: zero payload and
    scale bytes (all-zero blocks), written without a GEMM launch, so the
    transposed 32x32 weight (N > 256, several n-tiles) is never addressed."""
    u8 = dict(dtype=torch.uint8, device="cuda")
    M = 96
    a, sa = torch.empty((M, 0), **u8), torch.empty((M, 0), **u8)
    if bscale == "32x32" and layout == "dgrad":
        b, sb = torch.empty((0, N), **u8), torch.empty((0, N // 32), **u8)
    elif bscale == "32x32":
        b, sb = torch.empty((N, 0), **u8), torch.empty((N // 32, 0), **u8)
    else:
        b, sb = torch.empty((N, 0), **u8), torch.empty((N, 0), **u8)
    say(f"[fused] K=0 {layout} {bscale} N={N}")
    q, s = mx.gemm_quant(a, sa, b, sb, layout, bscale)
    torch.cuda.synchronize()
    assert tuple(q.shape) == (M, N) and tuple(s.shape) == (M, N // 32)
    assert torch.count_nonzero(q) == 0 and torch.count_nonzero(s) == 0


def test_fused_k_zero_gives_zero_blocks():
    q, s = mx.gemm_quant(torch.empty((64, 0), dtype=torch.uint8, device="cuda"),
                         torch.empty((64, 0), dtype=torch.uint8, device="cuda"),
                         torch.empty((96, 0), dtype=torch.uint8, device="cuda"),
                         torch.empty((96, 0), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(q) == 0 and torch.count_nonzero(s) == 0


def test_fused_stack_fprop_full_size():
    """The up projection of the linear stack, [32768 x 7168] x [18432 x 7168]:
    fused bytes equal the row-quantised unfused result everywhere."""
    t = W.stack_layer(0, "cuda")
    qx, sx = mx.quant(t["X_up"], "row")
    qw, sw = mx.quant(t["W_up"], "row")
    say("[fused] full up projection")
    q, s = mx.gemm_quant(qx, sx, qw, sw)
    q2, s2 = mx.quant(mx.gemm(qx, sx, qw, sw), "row")
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
