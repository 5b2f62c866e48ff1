"""Every entry point can be captured in a HIP graph: the library enqueues only
kernel launches on the caller's stream (no allocation, memset or sync).  One
captured step (dual-axis quantisation and the three products of a linear
layer, the MoE grouped GEMM and the MoE backward's grouped column
quantisation and weight gradient) is replayed several times, with the
outputs overwritten and other eager work run between replays, and every
replay must reproduce the eager results bit for bit (the kernels are
deterministic)."""
import numpy as np
import pytest
import torch

import mxfp8_microscaled_precision_amd as mx
from mxfp8_microscaled_precision_amd import workloads as W
from parity import dev, say

pytestmark = pytest.mark.gpu


def _step(d):
    qx = mx.quant(d["X"], "dual")
    qw = mx.quant(d["W"], "dual")
    qd = mx.quant(d["dY"], "dual")
    y = mx.gemm(qx[0], qx[1], qw[0], qw[1], "fprop")
    dx = mx.gemm(qd[0], qd[1], qw[2], qw[3], "dgrad")
    dw = mx.gemm(qd[2], qd[3], qx[2], qx[3], "wgrad")
    q32, s32 = mx.quant(d["W"], "32x32")
    y32 = mx.gemm(qx[0], qx[1], q32, s32, "fprop", "32x32")
    qt, st = mx.quant(d["tok"], "row")
    gy = mx.grouped_gemm(d["off"], qt, st, d["qe"], d["se"])
    ga, gsa = mx.quant_grouped_col(d["gdy"], d["off"], "e5m2")
    gb, gsb = mx.quant_grouped_col(d["gx"], d["off"])
    gw = mx.grouped_gemm_wgrad(d["off"], d["T"], ga, gsa, gb, gsb, a_elem="e5m2")
    return [*qx, *qw, *qd, y, dx, dw, q32, s32, y32, qt, st, gy, ga, gsa, gb, gsb, gw]


def _poison(outs):
    for t in outs:
        if t.dtype == torch.uint8:
            t.fill_(0xA5)
        else:
            t.fill_(float("nan"))


def test_captured_step_replays_match_eager():
    torch.cuda.synchronize()
    sizes = [300, 0, 129, 271]
    off = np.zeros(len(sizes) + 1, np.int64)
    np.cumsum(sizes, out=off[1:])
    T, G, K, N = int(off[-1]), len(sizes), 512, 256
    d = {
        "X": W.normal_bf16((512, 640), 1.0, 1, "cuda"),
        "W": W.normal_bf16((384, 640), 0.02, 2, "cuda"),
        "dY": W.normal_bf16((512, 384), 1e-3, 3, "cuda"),
        "tok": W.normal_bf16((T, K), 1.0, 4, "cuda"),
        "gdy": W.normal_bf16((T, 160), 0.01, 5, "cuda"),
        "gx": W.normal_bf16((T, 96), 1.0, 6, "cuda"),
        "off": dev(off),
        "T": T,
    }
    qe, se = mx.quant_batched(W.normal_bf16((G, N, K), 0.02, 7, "cuda"), "row")[:2]
    d["qe"], d["se"] = qe, se
    eager = [t.clone() for t in _step(d)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _step(d)
    torch.cuda.synchronize()
    assert len(outs) == len(eager)
    for r in range(3):
        _poison(outs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(outs, eager)):
            assert o.shape == e.shape and torch.equal(o, e), f"replay {r}: output {k} differs"
        say(f"[graph] replay {r}: {len(outs)} outputs equal the eager run")
        # other eager work between replays, on other inputs
        other = dict(d)
        other["X"] = W.normal_bf16((512, 640), 1.0, 11 + r, "cuda")
        _step(other)
        torch.cuda.synchronize()
