"""GPU parity of the MoE backward pieces against the oracle: batched
quantisation of per-expert weights (bytes exact), per-group column
quantisation along the token axis (bytes exact, ragged and empty groups,
partial last blocks, whole MoE workload on sampled features) and the
per-expert weight-gradient GEMM (every element within the GEMM tolerance;
empty experts give zeros; equal to the dense GEMM over each expert's padded
column range; the full MoE workload on sampled experts and elements)."""
import numpy as np
import pytest
import torch

import oracle
import mxfp8_microscaled_precision_amd as mx
from mxfp8_microscaled_precision_amd import workloads as W
from parity import assert_bytes, assert_gemm, bits, dev, host, say

pytestmark = pytest.mark.gpu


def _offsets(sizes):
    o = np.zeros(len(sizes) + 1, np.int64)
    np.cumsum(sizes, out=o[1:])
    return o


@pytest.mark.parametrize("mode", ["row", "col", "dual", "32x32"])
def test_quant_batched_equals_per_matrix(mode):
    B, R, C = 3, 96, 160
    say(f"[moe-bwd] quant_batched {mode} [{B},{R},{C}]")
    x = W.normal_with_outliers_bf16((B * R, C), 0.02, 0.01, 100.0, 77).reshape(B, R, C)
    got = mx.quant_batched(x.cuda(), mode)
    torch.cuda.synchronize()
    for i in range(B):
        want = {"row": oracle.quant_row, "col": oracle.quant_col, "dual": oracle.quant_dual,
                "32x32": oracle.quant_block32}[mode](bits(x[i]))
        for k, (g, w) in enumerate(zip(got, want)):
            assert_bytes(g[i], w, f"batched {mode} matrix {i} output {k}")


@pytest.mark.parametrize("sizes,C", [
    ([5, 0, 33, 1, 31, 32, 64, 0, 70], 64),
    ([0, 0, 7], 32),
    ([300, 0, 0, 257, 1, 511, 96], 160),     # C not a multiple of the 128-column tile
    ([128, 256, 129], 96),
    ([0], 32),                               # no tokens at all: all zero blocks
    ([(5 * g) % 37 for g in range(512)], 32),  # the most groups: the last group's end is offsets[512]
    ([(3 * g) % 29 for g in range(65)], 64),   # a group boundary across two words of 64 offsets
])
def test_quant_grouped_col_exact(sizes, C):
    off = _offsets(sizes)
    T = int(off[-1])
    say(f"[moe-bwd] grouped col sizes={sizes} C={C}")
    x = W.normal_with_outliers_bf16((max(T, 1), C), 1.0, 0.01, 100.0, T + C)[:T]
    q, s = mx.quant_grouped_col(x.cuda(), dev(off))
    torch.cuda.synchronize()
    wq, ws = oracle.quant_col_grouped(bits(x) if T else np.zeros((0, C), np.uint16), off)
    assert_bytes(q, wq, "grouped q_t")
    assert_bytes(s, ws, "grouped s_t")


@pytest.mark.parametrize("sizes,C", [
    # 266 row tiles of 128 (more than one column tile's worth of scale
    # lines); scale rows of 1064 bytes, not a whole number of 16-byte words
    ([4000, 0, 12345, 1, 7000, 33, 0, 9000, 622], 4096),
    # 4067 row tiles, a 32-column last column tile
    ([100000, 200001, 0, 120000, 100000], 160),
])
def test_quant_grouped_col_many_tiles(sizes, C):
    """Shapes with many row tiles in the column-tiles-first dispatch order
    and partial edge tiles: every byte against the oracle."""
    off = _offsets(sizes)
    T = int(off[-1])
    say(f"[moe-bwd] grouped col many tiles T={T} G={len(sizes)} C={C}")
    x = W.normal_with_outliers_bf16((T, C), 1.0, 0.01, 100.0, T + 3 * C)
    q, s = mx.quant_grouped_col(x.cuda(), dev(off))
    torch.cuda.synchronize()
    wq, ws = oracle.quant_col_grouped(bits(x), off)
    assert_bytes(q, wq, "grouped many tiles q_t")
    assert_bytes(s, ws, "grouped many tiles s_t")


def test_quant_grouped_col_special_values():
    """NaN / Inf blocks, zeros and subnormals in ragged groups: the oracle's
    bytes exactly (a NaN block's padding rows stay 0x00)."""
    sizes = [3, 40, 0, 29]
    off = _offsets(sizes)
    T, C = int(off[-1]), 64
    rng = np.random.default_rng(4)
    xb = W.bf16_bits(W.normal_bf16((T, C), 1.0, 5))
    xb[1, 3] = 0x7FC0           # NaN in group 0
    xb[20, 7] = 0x7F80          # +Inf in group 1
    xb[44:46, :] = 0x0001       # subnormals in group 1's partial block
    xb[50:, 10] = 0x8000        # -0 column piece in group 3
    xb[rng.integers(0, T, 20), rng.integers(0, C, 20)] = 0
    q, s = mx.quant_grouped_col(W.bits_to_bf16(xb, "cuda"), dev(off))
    torch.cuda.synchronize()
    wq, ws = oracle.quant_col_grouped(xb, off)
    assert_bytes(q, wq, "special q_t")
    assert_bytes(s, ws, "special s_t")


def test_quant_grouped_col_full_moe():
    """The MoE backward's per-group column quantisation at full size: the
    tokens [131072, 4096] and the down-projection input [131072, 2048] over
    64 Zipf-sized experts, every byte against the oracle."""
    d = W.moe("cuda")
    off = d["offsets"]
    for name in ("X", "H"):
        x = d[name]
        say(f"[moe-bwd] grouped col full {name} {tuple(x.shape)}")
        q, s = mx.quant_grouped_col(x, dev(off))
        torch.cuda.synchronize()
        wq, ws = oracle.quant_col_grouped(bits(x), off)
        assert_bytes(q, wq, f"full grouped {name} q_t")
        assert_bytes(s, ws, f"full grouped {name} s_t")
        del q, s, wq, ws


def test_quant_batched_col_full_moe_weights():
    """The expert weights in column blocks, batched over the 64 experts (the
    backward-data operand of the MoE), at full size: every byte against the
    oracle's per-matrix column quantisation."""
    d = W.moe("cuda")
    for name in ("W_gu", "W_dn"):
        w = d[name]
        say(f"[moe-bwd] batched col full {name} {tuple(w.shape)}")
        qt, st = mx.quant_batched(w, "col")
        torch.cuda.synchronize()
        wq, ws = oracle.quant_col_batched(bits(w))
        assert_bytes(qt, wq, f"batched col {name} q_t")
        assert_bytes(st, ws, f"batched col {name} s_t")
        del qt, st, wq, ws


def _wgrad_case(sizes, M, N, seed):
    off = _offsets(sizes)
    T = int(off[-1])
    dy = W.normal_bf16((T, M), 0.01, seed)
    xx = W.normal_bf16((T, N), 1.0, seed + 1)
    qa, sa = oracle.quant_col_grouped(bits(dy), off)
    qb, sb = oracle.quant_col_grouped(bits(xx), off)
    c = mx.grouped_gemm_wgrad(dev(off), T, dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    return off, T, qa, sa, qb, sb, c


@pytest.mark.parametrize("sizes,M,N", [
    ([5, 0, 33, 64, 1], 64, 96),
    ([300, 0, 0, 257, 1, 511, 96], 288, 160),   # M, N not multiples of the 256 tile
    ([0, 0], 64, 64),                            # all experts empty
    ([1000], 256, 512),
    ([130, 128, 129, 127], 256, 256),            # odd and even step counts
    ([600, 700, 850, 1100], 96, 96),             # 5, 6, 7, 9 steps: partial groups of four steps
    ([128, 1000, 128, 1000, 0, 5, 1000], 64, 64),  # equal step counts: longest-first order ties
    ([(7 * g) % 45 for g in range(130)], 64, 32),  # 130 groups dealt to 64 groups of workgroups
])
def test_wgrad_small_cases(sizes, M, N):
    say(f"[moe-bwd] wgrad sizes={sizes} M={M} N={N}")
    off, T, qa, sa, qb, sb, c = _wgrad_case(sizes, M, N, sum(sizes) + M + N)
    ref, bound = oracle.grouped_gemm_wgrad(off, qa, sa, qb, sb)
    assert_gemm(c, ref, bound, f"wgrad sizes={sizes}")
    for g, m in enumerate(sizes):
        if m == 0:
            assert torch.count_nonzero(c[g]) == 0, g


def test_largest_token_capacity():
    """The most tokens the boundary accepts for the MoE backward (a padded
    capacity of 8388352 columns, just under 2^23): both operands' per-group
    column quantisation byte-exact, then the per-expert weight gradient on
    those bytes within the GEMM tolerance."""
    sizes = [4194311, 4193908]
    off = _offsets(sizes)
    T, M, N = int(off[-1]), 32, 32
    cap = mx.grouped_col_capacity(T, len(sizes))
    assert cap == 8388352 and 256 * cap < 2 ** 31
    say(f"[moe-bwd] largest capacity T={T} cap={cap}")
    dy = W.normal_bf16((T, M), 0.01, 501)
    xx = W.normal_bf16((T, N), 1.0, 502)
    qa, sa = mx.quant_grouped_col(dy.cuda(), dev(off))
    qb, sb = mx.quant_grouped_col(xx.cuda(), dev(off))
    torch.cuda.synchronize()
    wqa, wsa = oracle.quant_col_grouped(bits(dy), off)
    wqb, wsb = oracle.quant_col_grouped(bits(xx), off)
    assert_bytes(qa, wqa, "largest capacity q_t (gradients)")
    assert_bytes(sa, wsa, "largest capacity s_t (gradients)")
    assert_bytes(qb, wqb, "largest capacity q_t (inputs)")
    assert_bytes(sb, wsb, "largest capacity s_t (inputs)")
    c = mx.grouped_gemm_wgrad(dev(off), T, qa, sa, qb, sb)
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm_wgrad(off, wqa, wsa, wqb, wsb)
    assert_gemm(c, ref, bound, "wgrad at the largest capacity")


@pytest.mark.parametrize("sizes,M,N", [
    ([5, 0, 33, 64, 1], 64, 100),       # N % 8 != 0: the result leaves through both stage buffers
    ([300, 257, 1, 511], 288, 36),
])
def test_wgrad_ragged_n(sizes, M, N):
    """Output columns N that are not whole 8-column chunks (the C ABI takes
    any N; the rows of b are independent, so the first N rows of a grouped
    column quantisation are a valid b)."""
    say(f"[moe-bwd] wgrad ragged N sizes={sizes} M={M} N={N}")
    off = _offsets(sizes)
    T = int(off[-1])
    dy = W.normal_bf16((T, M), 0.01, 7 + N)
    xx = W.normal_bf16((T, 128), 1.0, 8 + N)
    qa, sa = oracle.quant_col_grouped(bits(dy), off)
    qb, sb = oracle.quant_col_grouped(bits(xx), off)
    qb, sb = np.ascontiguousarray(qb[:N]), np.ascontiguousarray(sb[:N])
    c = mx.grouped_gemm_wgrad(dev(off), T, dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm_wgrad(off, qa, sa, qb, sb)
    assert_gemm(c, ref, bound, f"wgrad ragged N={N}")


def test_wgrad_neighbour_nan_scales_stay_out():
    """Scale words past a group's last step are not read: with every scale
    byte of the next group set to NaN (0xFF), an expert whose step count is
    not a multiple of four still matches the oracle (finite), and the NaN
    group is NaN where the oracle says so."""
    sizes = [600, 700]                      # 5 and 6 steps
    M, N = 64, 96
    off = _offsets(sizes)
    T = int(off[-1])
    qa, sa = oracle.quant_col_grouped(bits(W.normal_bf16((T, M), 0.01, 61)), off)
    qb, sb = oracle.quant_col_grouped(bits(W.normal_bf16((T, N), 1.0, 62)), off)
    P1 = oracle.group_col(1, off[1])
    sa[:, P1 // 32:] = 0xFF
    sb[:, P1 // 32:] = 0xFF
    c = mx.grouped_gemm_wgrad(dev(off), T, dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    ref, bound = oracle.grouped_gemm_wgrad(off, qa, sa, qb, sb)
    assert np.isfinite(ref[0]).all() and np.isnan(ref[1]).all()
    assert_gemm(c, ref, bound, "wgrad with NaN scales in the next group")


def test_wgrad_equals_dense_gemm_per_expert():
    """Each expert's gradient equals the dense GEMM over its padded column
    range (same K-step order, so the same bits)."""
    sizes = [200, 0, 384, 45]
    M, N = 160, 192
    off, T, qa, sa, qb, sb, c = _wgrad_case(sizes, M, N, 31)
    for g, m in enumerate(sizes):
        if m == 0:
            continue
        P = oracle.group_col(g, off[g])
        Kg = 128 * ((m + 127) // 128)
        dense = mx.gemm(dev(qa[:, P:P + Kg]), dev(sa[:, P // 32:(P + Kg) // 32]),
                        dev(qb[:, P:P + Kg]), dev(sb[:, P // 32:(P + Kg) // 32]), "wgrad")
        torch.cuda.synchronize()
        assert torch.equal(c[g], dense), g


@pytest.mark.parametrize("sizes,M,N", [
    # 16 output tiles per expert: 16 groups of 16 workgroups, several
    # experts dealt to each (longest first), empty and one-token experts
    ([1900, 0, 7, 640, 1, 1200, 333, 2048, 129, 0, 900, 77, 1500, 260, 31, 1024, 555, 12, 2100, 400],
     1024, 1024),
    ([3000, 129, 2500, 600, 0, 1800, 64, 1100, 4000], 2048, 2048),   # 64 per expert: 4 groups
    ([5000, 300, 2600, 1, 700], 4096, 2048),                          # 128 per expert: 2 groups
    ([900, 0, 2000, 130, 1], 4096, 4096),                             # 256 per expert: one group
    ([700, 260], 4608, 4608),        # 324 tiles per expert, more than the grid: a strided walk
    ([(37 * g) % 300 for g in range(100)], 768, 256),                # 3 per expert: a strided walk
    # every step count from 1 to 24: a workgroup's consecutive tiles have odd
    # and even counts (an odd count starts in the other stage buffer, and
    # the previous result then leaves through the first)
    ([125 * s for s in range(1, 25)], 1024, 1024),
])
def test_wgrad_schedules_equal_dense_gemm(sizes, M, N):
    """The persistent weight gradient's tile walk, in each of its forms (the
    experts dealt to groups of workgroups, or a strided walk over all
    tiles), against the dense GEMM of every expert over its padded column
    range: the same K-step order, so the same bits; every output tile of
    every expert is compared."""
    say(f"[moe-bwd] wgrad schedule G={len(sizes)} M={M} N={N}")
    off = _offsets(sizes)
    T = int(off[-1])
    offd = dev(off)
    dy = W.normal_bf16((T, M), 0.01, 900 + M, "cuda")
    xx = W.normal_bf16((T, N), 1.0, 901 + N, "cuda")
    qa, sa = mx.quant_grouped_col(dy, offd)
    qb, sb = mx.quant_grouped_col(xx, offd)
    c = mx.grouped_gemm_wgrad(offd, T, qa, sa, qb, sb)
    torch.cuda.synchronize()
    for g, m in enumerate(sizes):
        if m == 0:
            assert torch.count_nonzero(c[g]) == 0, g
            continue
        P = oracle.group_col(g, off[g])
        Kg = 128 * ((m + 127) // 128)
        dense = mx.gemm(qa[:, P:P + Kg].contiguous(), sa[:, P // 32:(P + Kg) // 32].contiguous(),
                        qb[:, P:P + Kg].contiguous(), sb[:, P // 32:(P + Kg) // 32].contiguous(), "wgrad")
        torch.cuda.synchronize()
        assert torch.equal(c[g], dense), f"expert {g} of {len(sizes)}"


def test_moe_backward_full_sampled():
    """The whole MoE backward at the workload's size: gate_up and down,
    dgrad through the batched column quantisation of the expert weights and
    the grouped GEMM, wgrad through the per-group column quantisation and the
    grouped weight-gradient GEMM; sampled rows / experts / elements against
    the oracle quantising the same BF16 sources."""
    d = W.moe("cuda")
    gr = W.moe_grads("cuda")
    off = d["offsets"]
    offd = dev(off)
    T = int(off[-1])
    sizes = np.diff(off)
    rng = np.random.default_rng(61)
    nonempty = [g for g in range(len(sizes)) if sizes[g] > 0]
    big, small = int(np.argmax(sizes)), int(min(nonempty, key=lambda g: sizes[g]))
    empty = [g for g in range(len(sizes)) if sizes[g] == 0]
    for name, xname, wname, dyname in (("gate_up", "X", "W_gu", "dY_gu"), ("down", "H", "W_dn", "dY_dn")):
        x, w, dy = d[xname], d[wname], gr[dyname]
        G, Nout, Kin = w.shape
        say(f"[moe-bwd] full {name}: T={T} G={G} out={Nout} in={Kin}")
        # dgrad: dX = dY W_g per expert
        qd, sd = mx.quant(dy, "row")
        qwt, swt = mx.quant_batched(w, "col")                 # [G, Kin, Nout]
        dx = mx.grouped_gemm(offd, qd, sd, qwt, swt)
        torch.cuda.synchronize()
        # the first and last row of every expert group plus 32 seeded rows,
        # each over all Kin columns
        rows = np.unique(np.concatenate([[off[g] for g in nonempty], [off[g + 1] - 1 for g in nonempty],
                                         rng.integers(0, T, 32)])).astype(np.int64)
        ri = torch.from_numpy(rows).cuda()
        got = dx.index_select(0, ri).float().cpu().numpy().astype(np.float64)
        ra, rsa = oracle.quant_row(bits(dy.index_select(0, ri)))
        grp = np.searchsorted(off, rows, side="right") - 1
        for g in np.unique(grp):
            sel = np.nonzero(grp == g)[0]
            wt, swt_o = oracle.quant_col(bits(w[int(g)]))                     # [Kin, Nout]
            ref, bound = oracle.gemm(ra[sel], rsa[sel], wt, swt_o)
            assert_gemm(got[sel], ref, bound, f"{name} dgrad expert {g}, all {Kin} columns")
        del dx, qd, sd, qwt, swt
        # wgrad: dW_g = dY_g^T X_g per expert
        qa, sa = mx.quant_grouped_col(dy, offd)
        qb, sb = mx.quant_grouped_col(x, offd)
        dw = mx.grouped_gemm_wgrad(offd, T, qa, sa, qb, sb)
        torch.cuda.synchronize()
        # 32 sampled features on each side (the oracle's column blocks need
        # a multiple of 32 columns)
        mi = np.unique(np.concatenate([[0, Nout - 1], rng.choice(np.arange(1, Nout - 1), 30,
                                                                 replace=False)])).astype(np.int64)
        ni = np.unique(np.concatenate([[0, Kin - 1], rng.choice(np.arange(1, Kin - 1), 30,
                                                                replace=False)])).astype(np.int64)
        mt, nt = torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()
        oa, osa = oracle.quant_col_grouped(bits(dy.index_select(1, mt)), off)
        ob, osb = oracle.quant_col_grouped(bits(x.index_select(1, nt)), off)
        ref, bound = oracle.grouped_gemm_wgrad(off, oa, osa, ob, osb)
        for g in sorted({big, small, *empty[:1], *rng.integers(0, G, 3).tolist()}):
            got = dw[g].index_select(0, mt).index_select(1, nt)
            assert_gemm(got, ref[g], bound[g], f"{name} wgrad expert {g} ({sizes[g]} tokens)")
        del dw, qa, sa, qb, sb
