"""GPU parity of mx_grouped_gemm (MoE experts) against the oracle: every
element within the GEMM tolerance; empty groups, ragged group sizes, single
rows, all tokens in one expert; the full MoE workload on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_microscaled_precision_amd as mx
from mxfp8_microscaled_precision_amd import workloads as W
from parity import assert_gemm, bits, dev, say

pytestmark = pytest.mark.gpu


def _offsets(sizes):
    o = np.zeros(len(sizes) + 1, np.int64)
    np.cumsum(sizes, out=o[1:])
    return o


def _case(sizes, N, K, seed, what):
    off = _offsets(sizes)
    T, G = int(off[-1]), len(sizes)
    say(f"[grouped] {what} G={G} T={T} N={N} K={K}")
    qa, sa = oracle.quant_row(bits(W.normal_bf16((T, K), 1.0, seed)))
    wb = bits(W.normal_bf16((G * N, K), 0.02, seed + 1))
    qb, sb = oracle.quant_row(wb)
    qb = qb.reshape(G, N, K)
    sb = sb.reshape(G, N, K // 32)
    c = mx.grouped_gemm(dev(off), dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm(off, qa, sa, qb, sb)
    assert_gemm(c, ref, bound, what)


@pytest.mark.parametrize("sizes,N,K", [
    ([5, 0, 33, 1, 0, 17], 64, 64),
    ([300, 0, 0, 257, 1, 511, 96], 288, 160),
    ([0, 0, 700, 0], 256, 256),          # everything in one expert, empties around it
    ([1] * 40, 96, 96),                  # single-row groups
    ([513], 512, 1056),                  # one group, ragged against the 256-row tile
    ([300, 0, 257, 700], 256, 1152),     # K steps not a multiple of four
])
def test_small_cases(sizes, N, K):
    _case(sizes, N, K, sum(sizes) + N + K, f"sizes={sizes[:6]}")


def test_largest_k():
    """The longest contraction the boundary accepts (K = 2^23 - 32), two
    experts of 2 and 3 tokens, 40 features: every element."""
    _case([2, 3], 40, (1 << 23) - 32, 91, "largest K")


def test_scaled_moe_zipf():
    """MoE workload with tokens / 64 and features / 16: Zipf(1.1) sizes with
    forced-empty experts and sizes not multiples of 32."""
    d = W.moe("cpu", scale=64, fscale=16)
    off = d["offsets"]
    sizes = np.diff(off)
    assert (sizes == 0).sum() >= 1 and (sizes % 32 != 0).any()
    T = int(off[-1])
    for name, wname in (("X", "W_gu"), ("H", "W_dn")):
        x, w = d[name], d[wname]
        G, N, K = w.shape
        say(f"[grouped] scaled moe {name} T={T} G={G} N={N} K={K}")
        qa, sa = oracle.quant_row(bits(x))
        qb, sb = oracle.quant_row(bits(w.reshape(G * N, K)))
        qb, sb = qb.reshape(G, N, K), sb.reshape(G, N, K // 32)
        c = mx.grouped_gemm(dev(off), dev(qa), dev(sa), dev(qb), dev(sb))
        torch.cuda.synchronize()
        ref, bound = oracle.grouped_gemm(off, qa, sa, qb, sb)
        assert_gemm(c, ref, bound, f"scaled moe {name}")


def test_equals_dense_per_group():
    """The grouped result of each group equals the dense GEMM of that group."""
    sizes = [130, 0, 64, 257]
    off = _offsets(sizes)
    T, G, N, K = int(off[-1]), len(sizes), 192, 128
    qa, sa = oracle.quant_row(bits(W.normal_bf16((T, K), 1.0, 5)))
    qb, sb = oracle.quant_row(bits(W.normal_bf16((G * N, K), 0.02, 6)))
    A, SA = dev(qa), dev(sa)
    B, SB = dev(qb.reshape(G, N, K)), dev(sb.reshape(G, N, K // 32))
    c = mx.grouped_gemm(dev(off), A, SA, B, SB)
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        dense = mx.gemm(A[r0:r1].contiguous(), SA[r0:r1].contiguous(), B[g].contiguous(),
                        SB[g].contiguous())
        assert torch.equal(c[r0:r1], dense), g


def test_moe_full_sampled():
    """gate_up and down at full size: the first and last row of every
    non-empty expert group plus 32 seeded rows, every column, against the
    oracle quantising and multiplying the same BF16 sources."""
    d = W.moe("cuda")
    off = d["offsets"]
    offd = torch.from_numpy(off).cuda()
    T = int(off[-1])
    rng = np.random.default_rng(51)
    nonempty = [g for g in range(len(off) - 1) if off[g + 1] > off[g]]
    rows = np.unique(np.concatenate([[off[g] for g in nonempty], [off[g + 1] - 1 for g in nonempty],
                                     rng.integers(0, T, 32)])).astype(np.int64)
    for name, wname in (("X", "W_gu"), ("H", "W_dn")):
        x, w = d[name], d[wname]
        G, N, K = w.shape
        say(f"[grouped] full moe {name} T={T} G={G} N={N} K={K}")
        qa, sa = mx.quant(x, "row")
        qb, sb = mx.quant(w.reshape(G * N, K), "row")
        c = mx.grouped_gemm(offd, qa, sa, qb.reshape(G, N, K), sb.reshape(G, N, K // 32))
        torch.cuda.synchronize()
        ri = torch.from_numpy(rows).cuda()
        cols = np.arange(N, dtype=np.int64)   # every column of the sampled rows
        ci = torch.from_numpy(cols).cuda()
        # oracle: each sampled row times its expert's sampled weight rows,
        # quantised by the oracle from the BF16 sources
        ra, rsa = oracle.quant_row(bits(x.index_select(0, ri)))
        grp = np.searchsorted(off, rows, side="right") - 1
        got = c.index_select(0, ri).index_select(1, ci).float().cpu().numpy().astype(np.float64)
        for g in np.unique(grp):
            sel = np.nonzero(grp == g)[0]
            qw, sw = oracle.quant_row(bits(w[int(g)].index_select(0, ci)))
            ref, bound = oracle.gemm(ra[sel], rsa[sel], qw, sw)
            assert_gemm(got[sel], ref, bound, f"moe {name} expert {g}")
        del c, qa, sa, qb, sb
