#!/usr/bin/env python3
"""Throughput of the MXFP8 hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:

  linear stack, 4 layers of hidden 7168 -> 18432 -> 7168 at 32768 tokens,
    1x32 variant:  per layer dual-axis quantisation of X, W, dY for both
                   projections, then fprop, dgrad and wgrad MXFP8 GEMMs;
    32x32 variant: the same with the weights quantised in 32x32 tiles (one
                   shared FP8 weight; fprop and the transposed-read dgrad use
                   tile scales), same seeds;
  MoE experts, 131072 routed tokens over 64 experts (Zipf(1.1) sizes):
    forward: 1x32 quantisation of tokens and expert weights, then the grouped
    gate_up (4096 -> 4096) and down (2048 -> 4096) MXFP8 GEMMs;
    backward: 1x32 quantisation of the output gradients, column quantisation
    of every expert weight (batched) for the grouped dgrad GEMMs, and
    per-group column quantisation of gradients and inputs along the token
    axis for the per-expert weight-gradient GEMMs.

Inputs are generated on the GPU and resident in HBM before timing; outputs
are preallocated.  `value` = GEMM FLOP of the step / step time (TFLOP/s).
Per-kernel times come from HIP events on the launch stream.  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM TFLOP/s (% FP8 MFMA peak) + quant GB/s (% HBM peak), 1 GPU"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--layers", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="rough budget for the oracle sample")
    p.add_argument("--no-other-configs", action="store_true",
                   help="skip the dense and 32x32-weight configuration timings")
    p.add_argument("--calibration-copy", action="store_true",
                   help="run one plain 1 GiB device-to-device copy before warm-up (untimed), the "
                        "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    return p.parse_args()


class Launcher:
    """Runs C-ABI calls on torch's current stream, optionally bracketing each
    with HIP events (torch.cuda.Event records on the same stream)."""

    def __init__(self, torch, mx):
        self.torch, self.mx = torch, mx
        self.stream = torch.cuda.current_stream().cuda_stream
        self.record = False
        self.events = []   # (kind, work, unit, start, end)

    def _wrap(self, kind, work, unit, fn):
        if self.record:
            s = self.torch.cuda.Event(enable_timing=True)
            e = self.torch.cuda.Event(enable_timing=True)
            s.record()
            st = fn()
            e.record()
            self.events.append((kind, work, unit, s, e))
        else:
            st = fn()
        if st != 0:
            raise RuntimeError(f"{kind}: status {st}: {self.mx.mx_last_error()}")

    def quant(self, kind, mode, x, outs):
        mx = self.mx
        R, C = x.shape
        q, s, qt, st = outs
        nbytes = {0: 2 + 1 + 1 / 32, 1: 2 + 1 + 1 / 32, 2: 2 + 2 + 2 / 32,
                  3: 2 + 1 + 1 / 1024}[mode] * R * C
        self._wrap(kind, nbytes, "B", lambda: mx.mx_quant(
            mode, x.data_ptr(), R, C, _p(q), _p(s), _p(qt), _p(st), self.stream))

    def gemm(self, kind, layout, bkind, M, N, K, a, sa, b, sb, c):
        mx = self.mx
        self._wrap(kind, 2.0 * M * N * K, "FLOP", lambda: mx.mx_gemm(
            layout, bkind, M, N, K, a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
            c.data_ptr(), self.stream))

    def grouped(self, kind, G, offs, T, N, K, a, sa, b, sb, c, flops):
        mx = self.mx
        # the grouped kernel needs no workspace (its size query returns 0)
        self._wrap(kind, flops, "FLOP", lambda: mx.mx_grouped_gemm(
            G, offs.data_ptr(), T, N, K, a.data_ptr(), sa.data_ptr(), b.data_ptr(),
            sb.data_ptr(), c.data_ptr(), 0, 0, self.stream))

    def quant_batched(self, kind, mode, x, outs):
        mx = self.mx
        B, R, C = x.shape
        q, s, qt, st = outs
        nbytes = 3.03125 * B * R * C
        self._wrap(kind, nbytes, "B", lambda: mx.mx_quant_batched(
            mode, x.data_ptr(), B, R, C, _p(q), _p(s), _p(qt), _p(st), self.stream))

    def quant_grouped_col(self, kind, G, offs, x, outs):
        mx = self.mx
        T, C = x.shape
        qt, st = outs
        nbytes = 3.03125 * T * C          # the tokens' own bytes; zero padding not counted
        self._wrap(kind, nbytes, "B", lambda: mx.mx_quant_grouped_col(
            x.data_ptr(), T, C, G, offs.data_ptr(), qt.data_ptr(), st.data_ptr(), self.stream))

    def grouped_wgrad(self, kind, G, offs, T, M, N, a, sa, b, sb, c):
        mx = self.mx
        self._wrap(kind, 2.0 * T * M * N, "FLOP", lambda: mx.mx_grouped_gemm_wgrad(
            G, offs.data_ptr(), T, M, N, a.data_ptr(), sa.data_ptr(), b.data_ptr(),
            sb.data_ptr(), c.data_ptr(), self.stream))


def _p(t):
    return 0 if t is None else t.data_ptr()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_row_hbm_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "mxfp8_microscaled_precision_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_common.h")]


def gemm_traffic():
    """HBM bytes per launch of the 1x32 GEMM kernel from the committed
    FETCH_SIZE / WRITE_SIZE counter summary, or (None, None) when that summary
    is missing or was taken from a different kernel source (gemm.hip and
    gemm_common.h, hashed together)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = b"".join(open(f, "rb").read() for f in GEMM_SOURCES)
    except OSError:
        return None, None
    fields = dict(re.findall(r"^(\w+): (\S+)$", text, re.M))
    if fields.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None, None
    return int(fields["traffic_bytes_per_launch"]), int(fields["algorithmic_bytes_per_launch"])


CLOCK_PROFILE = os.path.join(ROOT, "profiles", "bench_step_clock_mfma_busy.md")


def gemm_clock():
    """Engine clock (GHz) and MFMA busy fraction of the 1x32 GEMM kernel under
    the step from the committed counter summary, or (None, None) when it is
    missing or was taken from a different kernel source."""
    import hashlib
    try:
        text = open(CLOCK_PROFILE).read()
        src = b"".join(open(f, "rb").read() for f in GEMM_SOURCES)
    except OSError:
        return None, None
    fields = dict(re.findall(r"^(\w+): (\S+)$", text, re.M))
    if fields.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None, None
    return float(fields["gemm_row_clock_ghz"]), float(fields["gemm_row_mfma_busy"])


def build_workload(torch, W, layers):
    dev = "cuda"
    u8, bf = torch.uint8, torch.bfloat16
    stack = [W.stack_layer(l, dev) for l in range(layers)]
    T, H = stack[0]["X_up"].shape
    F = stack[0]["W_up"].shape[0]

    def dual_out(R, C):
        return (torch.empty((R, C), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev),
                torch.empty((C, R), dtype=u8, device=dev), torch.empty((C, R // 32), dtype=u8, device=dev))

    def tile_out(R, C):
        return (torch.empty((R, C), dtype=u8, device=dev),
                torch.empty((R // 32, C // 32), dtype=u8, device=dev), None, None)

    bufs = {
        "X_up": dual_out(T, H), "X_dn": dual_out(T, F), "dY_up": dual_out(T, F),
        "dY_dn": dual_out(T, H), "W_up": dual_out(F, H), "W_dn": dual_out(H, F),
        "W_up32": tile_out(F, H), "W_dn32": tile_out(H, F),
        "Y_up": torch.empty((T, F), dtype=bf, device=dev),
        "dX_up": torch.empty((T, H), dtype=bf, device=dev),
        "dW_up": torch.empty((F, H), dtype=bf, device=dev),
        "Y_dn": torch.empty((T, H), dtype=bf, device=dev),
        "dX_dn": torch.empty((T, F), dtype=bf, device=dev),
        "dW_dn": torch.empty((H, F), dtype=bf, device=dev),
    }
    moe = W.moe(dev)
    moe.update(W.moe_grads(dev))
    off = moe["offsets"]
    Tm = int(off[-1])
    G, Ngu, Hm = moe["W_gu"].shape
    _, Ndn, Fm = moe["W_dn"].shape
    cap = 128 * (Tm // 128 + G)
    row = lambda R, C: (torch.empty((R, C), dtype=u8, device=dev),
                        torch.empty((R, C // 32), dtype=u8, device=dev), None, None)
    colb = lambda B, R, C: (None, None, torch.empty((B, C, R), dtype=u8, device=dev),
                            torch.empty((B, C, R // 32), dtype=u8, device=dev))
    gcol = lambda C: (torch.empty((C, cap), dtype=u8, device=dev),
                      torch.empty((C, cap // 32), dtype=u8, device=dev))
    moe_bufs = {
        "offs": torch.from_numpy(off).to(dev),
        "X": row(Tm, Hm), "H": row(Tm, Fm), "W_gu": row(G * Ngu, Hm), "W_dn": row(G * Ndn, Fm),
        "Y_gu": torch.empty((Tm, Ngu), dtype=bf, device=dev),
        "Y_dn": torch.empty((Tm, Ndn), dtype=bf, device=dev),
        # backward
        "dY_gu": row(Tm, Ngu), "dY_dn": row(Tm, Ndn),
        "W_gu_t": colb(G, Ngu, Hm), "W_dn_t": colb(G, Ndn, Fm),
        "dX": torch.empty((Tm, Hm), dtype=bf, device=dev),
        "dH": torch.empty((Tm, Fm), dtype=bf, device=dev),
        "gX": gcol(Hm), "gH": gcol(Fm), "gdY_gu": gcol(Ngu), "gdY_dn": gcol(Ndn),
        "dW_gu": torch.empty((G, Ngu, Hm), dtype=bf, device=dev),
        "dW_dn": torch.empty((G, Ndn, Fm), dtype=bf, device=dev),
    }
    dims = dict(T=T, H=H, F=F, Tm=Tm, G=G, Ngu=Ngu, Hm=Hm, Ndn=Ndn, Fm=Fm)
    return stack, bufs, moe, moe_bufs, dims


def run_step(L, stack, b, moe, mb, d):
    T, H, F = d["T"], d["H"], d["F"]
    FP, DG, WG = 0, 1, 2
    B1, B32 = 0, 1
    for variant in ("1x32", "32x32"):
        for t in stack:
            # activations and gradients: dual-axis (forward row + backward column copies)
            L.quant("quant_dual", 2, t["X_up"], b["X_up"])
            L.quant("quant_dual", 2, t["dY_up"], b["dY_up"])
            L.quant("quant_dual", 2, t["X_dn"], b["X_dn"])
            L.quant("quant_dual", 2, t["dY_dn"], b["dY_dn"])
            qx, sx, qxt, sxt = b["X_up"]
            qd, sd, qdt, sdt = b["dY_up"]
            qx2, sx2, qxt2, sxt2 = b["X_dn"]
            qd2, sd2, qdt2, sdt2 = b["dY_dn"]
            if variant == "1x32":
                L.quant("quant_dual", 2, t["W_up"], b["W_up"])
                L.quant("quant_dual", 2, t["W_dn"], b["W_dn"])
                qw, sw, qwt, swt = b["W_up"]
                qw2, sw2, qwt2, swt2 = b["W_dn"]
                L.gemm("gemm", FP, B1, T, F, H, qx, sx, qw, sw, b["Y_up"])
                L.gemm("gemm", DG, B1, T, H, F, qd, sd, qwt, swt, b["dX_up"])
                L.gemm("gemm", FP, B1, T, H, F, qx2, sx2, qw2, sw2, b["Y_dn"])
                L.gemm("gemm", DG, B1, T, F, H, qd2, sd2, qwt2, swt2, b["dX_dn"])
            else:
                L.quant("quant_32x32", 3, t["W_up"], b["W_up32"])
                L.quant("quant_32x32", 3, t["W_dn"], b["W_dn32"])
                qw, sw = b["W_up32"][:2]
                qw2, sw2 = b["W_dn32"][:2]
                L.gemm("gemm_32x32", FP, B32, T, F, H, qx, sx, qw, sw, b["Y_up"])
                L.gemm("gemm_32x32_dgrad", DG, B32, T, H, F, qd, sd, qw, sw, b["dX_up"])
                L.gemm("gemm_32x32", FP, B32, T, H, F, qx2, sx2, qw2, sw2, b["Y_dn"])
                L.gemm("gemm_32x32_dgrad", DG, B32, T, F, H, qd2, sd2, qw2, sw2, b["dX_dn"])
            L.gemm("gemm", WG, B1, F, H, T, qdt, sdt, qxt, sxt, b["dW_up"])
            L.gemm("gemm", WG, B1, H, F, T, qdt2, sdt2, qxt2, sxt2, b["dW_dn"])
    # MoE experts
    G, Tm = d["G"], d["Tm"]
    L.quant("quant_row", 0, moe["X"], mb["X"])
    L.quant("quant_row", 0, moe["H"], mb["H"])
    L.quant("quant_row", 0, moe["W_gu"].reshape(-1, d["Hm"]), mb["W_gu"])
    L.quant("quant_row", 0, moe["W_dn"].reshape(-1, d["Fm"]), mb["W_dn"])
    qa, sa = mb["X"][:2]
    qw, sw = mb["W_gu"][:2]
    L.grouped("grouped_gemm", G, mb["offs"], Tm, d["Ngu"], d["Hm"], qa, sa, qw, sw, mb["Y_gu"],
              2.0 * Tm * d["Ngu"] * d["Hm"])
    qa, sa = mb["H"][:2]
    qw, sw = mb["W_dn"][:2]
    L.grouped("grouped_gemm", G, mb["offs"], Tm, d["Ndn"], d["Fm"], qa, sa, qw, sw, mb["Y_dn"],
              2.0 * Tm * d["Ndn"] * d["Fm"])
    # MoE backward: dgrad through the column-quantised expert weights, wgrad
    # over each expert's tokens
    offs = mb["offs"]
    for dyn, wn, wtn, xn, dxn, gxn, gdyn, dwn, N, K in (
            ("dY_gu", "W_gu", "W_gu_t", "X", "dX", "gX", "gdY_gu", "dW_gu", d["Ngu"], d["Hm"]),
            ("dY_dn", "W_dn", "W_dn_t", "H", "dH", "gH", "gdY_dn", "dW_dn", d["Ndn"], d["Fm"])):
        L.quant("quant_row", 0, moe[dyn], mb[dyn])
        L.quant_batched("quant_col_batched", 1, moe[wn], mb[wtn])
        qd, sd = mb[dyn][:2]
        qwt, swt = mb[wtn][2:]
        L.grouped("grouped_gemm_dgrad", G, offs, Tm, K, N, qd, sd, qwt, swt, mb[dxn],
                  2.0 * Tm * N * K)
        L.quant_grouped_col("quant_grouped_col", G, offs, moe[dyn], mb[gdyn])
        L.quant_grouped_col("quant_grouped_col", G, offs, moe[xn], mb[gxn])
        qa, sa = mb[gdyn]
        qb, sb = mb[gxn]
        L.grouped_wgrad("grouped_wgrad", G, offs, Tm, N, K, qa, sa, qb, sb, mb[dwn])


def per_kernel_medians(events, steps):
    """Per kernel kind: the work of one step and the sum over its launches of
    each launch's median duration across the timed steps.  Every step issues
    the same launches in the same order, so launch i of step j is event
    i + j * (launches per step)."""
    import statistics
    n = len(events) // steps
    assert n * steps == len(events), "every step must issue the same launches"
    per = {}
    for i in range(n):
        kind, work, unit = events[i][:3]
        ms = statistics.median(events[i + j * n][3].elapsed_time(events[i + j * n][4])
                               for j in range(steps))
        k = per.setdefault(kind, {"ms": 0.0, "work": 0.0, "unit": unit, "launches": 0})
        k["ms"] += ms
        k["work"] += work
        k["launches"] += 1
    return per


def copy_rate(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy rate (read + written bytes per second) of torch's
    copy kernel on `nbytes`, the practical ceiling the quantisers are compared
    with beside the 8 TB/s nominal peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def quantisation_error(torch, mx, t, seed=11):
    """Relative error of the MXFP8 products against the binary64 product of
    the unquantised BF16 inputs, ||C_mx - C|| / ||C||, for the 1x32 and 32x32
    weight variants of the up projection (fprop X_up.W_up^T and dgrad
    dY_up.W_up), on 32 seeded rows x all columns plus 32 seeded columns x all
    rows of each product.  Reported, not a pass/fail criterion."""
    X, dY, Wt = t["X_up"], t["dY_up"], t["W_up"]
    T, H = X.shape
    F = Wt.shape[0]
    g = torch.Generator().manual_seed(seed)
    out = {}
    qx, sx = mx.quant(X, "row")[:2]
    qd, sd = mx.quant(dY, "row")[:2]
    qw, sw, qwt, swt = mx.quant(Wt, "dual")
    q32, s32 = mx.quant(Wt, "32x32")[:2]
    Wd = Wt.double()
    prods = {
        "fprop": (X, lambda A: A @ Wd.t(), lambda idx: Wd[idx].t(), F,
                  {"1x32": (qx, sx, qw, sw, "fprop", "1x32"), "32x32": (qx, sx, q32, s32, "fprop", "32x32")}),
        "dgrad": (dY, lambda A: A @ Wd, lambda idx: Wd[:, idx], H,
                  {"1x32": (qd, sd, qwt, swt, "dgrad", "1x32"), "32x32": (qd, sd, q32, s32, "dgrad", "32x32")}),
    }
    for name, (A, row_ref, col_op, N, variants) in prods.items():
        rows = torch.randperm(T, generator=g)[:32].cuda()
        cols = torch.randperm(N, generator=g)[:32].cuda()
        ref_r = row_ref(A.index_select(0, rows).double())             # [32, N]
        ref_c = A.double() @ col_op(cols)                               # [T, 32]
        for var, (a, sa, b, sb, layout, bk) in variants.items():
            C = mx.gemm(a, sa, b, sb, layout, bk)
            got_r = C.index_select(0, rows).double()
            got_c = C.index_select(1, cols).double()
            num = (got_r - ref_r).pow(2).sum() + (got_c - ref_c).pow(2).sum()
            den = ref_r.pow(2).sum() + ref_c.pow(2).sum()
            out[f"{name}_{var}"] = float((num / den).sqrt())
            del C
        del ref_r, ref_c
    torch.cuda.synchronize()
    return out


def fused_producer(torch, mx, t, reps=5):
    """The up projection with its output quantised for a following layer
    (1x32 along N), as one fused GEMM (mx_gemm_quant) and as the GEMM's BF16
    output followed by the row quantiser; median HIP-event time of each."""
    qx, sx = mx.quant(t["X_up"], "row")
    qw, sw = mx.quant(t["W_up"], "row")
    M, N, K = qx.shape[0], qw.shape[0], qx.shape[1]
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    s = torch.empty((M, N // 32), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    P = lambda x: x.data_ptr()

    def fused():
        return mx.mx_gemm_quant(0, 0, 0, M, N, K, P(qx), P(sx), P(qw), P(sw), P(q), P(s), st)

    def unfused():
        r = mx.mx_gemm(0, 0, M, N, K, P(qx), P(sx), P(qw), P(sw), P(c), st)
        return r or mx.mx_quant(0, P(c), M, N, P(q), P(s), 0, 0, st)

    out = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        times = []
        for _ in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            if fn() != 0:
                raise RuntimeError(mx.mx_last_error())
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        out[name + "_ms"] = round(sorted(times[1:])[reps // 2], 4)
    out["gemm_shape"] = [M, N, K]
    out["saving"] = round(1.0 - out["fused_ms"] / out["unfused_ms"], 4)
    return out


def other_configs(torch, mx, W, warm=5, reps=20, queue=8):
    """The dense (8192 x 4096 x 4096, dual-axis) and 32x32-weight (16384
    tokens, 7168 <-> 2048) configurations, outside the timed step.  Every
    kernel is launched warm + reps times with a 1 GiB buffer fill before each
    launch, so no operand stays in L2 or the Infinity Cache; the median
    launch (HIP events on the launch stream) is reported.  Beside it,
    `ms_queued` / `frac_peak_queued`: `queue` launches back to back on as
    many distinct copies of the operands (all cold after the fill) between
    two events, per launch, median over the reps -- the rate when launches
    follow one another as in a step, without the fixed cost of bracketing
    one launch with events (an empty launch measures several microseconds
    that way, a large share of these short kernels)."""
    import statistics
    u8, bf = torch.uint8, torch.bfloat16
    dev = "cuda"
    flush = torch.empty(1 << 30, dtype=u8, device=dev)
    L = Launcher(torch, mx)
    L.record = True

    def med(call, calls=None):
        L.events.clear()
        for i in range(warm + reps):
            flush.fill_(i & 255)
            call()
        torch.cuda.synchronize()
        ev = L.events[warm:]
        ms = statistics.median(s.elapsed_time(e) for _, _, _, s, e in ev)
        work, unit = ev[0][1], ev[0][2]
        big = unit == "FLOP"
        scale, peak, key = (1e12, PEAK_FP8_TFLOPS, "tflops") if big else (1e9, PEAK_HBM_GBPS, "gbps")
        rate = work / (ms * 1e-3) / scale
        r = {key: round(rate, 1), "frac_peak": round(rate / peak, 4), "ms": round(ms, 4)}
        if calls:
            L.record = False
            marks = []
            for i in range(warm + reps):
                flush.fill_(i & 255)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for c in calls:
                    c()
                e1.record()
                marks.append((e0, e1))
            torch.cuda.synchronize()
            L.record = True
            msq = statistics.median(a.elapsed_time(b) for a, b in marks[warm:]) / len(calls)
            rq = work / (msq * 1e-3) / scale
            r.update({"ms_queued": round(msq, 4), "frac_peak_queued": round(rq / peak, 4)})
        return r

    def copies(*ts):
        """queue sets of the tensors ts: the originals, then clones."""
        return [ts] + [tuple(t.clone() for t in ts) for _ in range(queue - 1)]

    def dual(R, C):
        return (torch.empty((R, C), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev),
                torch.empty((C, R), dtype=u8, device=dev), torch.empty((C, R // 32), dtype=u8, device=dev))

    def row(R, C):
        return (torch.empty((R, C), dtype=u8, device=dev), torch.empty((R, C // 32), dtype=u8, device=dev),
                None, None)

    def tile(R, C):
        return (torch.empty((R, C), dtype=u8, device=dev),
                torch.empty((R // 32, C // 32), dtype=u8, device=dev), None, None)

    def quant_op(mode, x, shape_out):
        """Median of one launch, and of `queue` launches on distinct copies."""
        R, C = x.shape
        xs = copies(x)
        outs = [shape_out(R, C) for _ in range(queue)]
        one = lambda: L.quant("q", mode, x, outs[0])
        many = [(lambda i=i: L.quant("q", mode, xs[i][0], outs[i])) for i in range(queue)]
        r = med(one, many)
        del xs, outs
        return r

    def gemm_op(layout, bkind, M, N, K, a, sa, b, sb, c_shape):
        ops = copies(a, sa, b, sb)
        cs = [torch.empty(c_shape, dtype=bf, device=dev) for _ in range(queue)]
        one = lambda: L.gemm("g", layout, bkind, M, N, K, a, sa, b, sb, cs[0])
        many = [(lambda i=i: L.gemm("g", layout, bkind, M, N, K, *ops[i], cs[i])) for i in range(queue)]
        r = med(one, many)
        del ops, cs
        return r

    out = {}
    # the tiny linear: launch-latency-bound, so microseconds are the figure
    d = W.tiny(dev)
    A, Wq = d["A"], d["W"]
    ba, bw1 = row(*A.shape), row(*Wq.shape)
    C1 = torch.empty((A.shape[0], Wq.shape[0]), dtype=bf, device=dev)
    r = {
        "quant_row_A": med(lambda: L.quant("q", 0, A, ba)),
        "quant_row_W": med(lambda: L.quant("q", 0, Wq, bw1)),
        "fprop": med(lambda: L.gemm("g", 0, 0, A.shape[0], Wq.shape[0], A.shape[1], ba[0], ba[1],
                                    bw1[0], bw1[1], C1)),
    }
    out[f"tiny {A.shape[0]}x{A.shape[1]} -> {Wq.shape[0]} (launch-bound; see ms)"] = r
    d = W.dense(dev)
    X, Wt, dY = d["X"], d["W"], d["dY"]
    M, K = X.shape
    N = Wt.shape[0]
    bx, bw, bd = dual(M, K), dual(N, K), dual(M, N)
    # operands of the GEMMs (the dual quantisations of X, W and dY)
    L.record = False
    L.quant("q", 2, X, bx)
    L.quant("q", 2, Wt, bw)
    L.quant("q", 2, dY, bd)
    L.record = True
    r = {
        "quant_dual_X": quant_op(2, X, dual),
        "quant_dual_W": quant_op(2, Wt, dual),
        "quant_dual_dY": quant_op(2, dY, dual),
        "fprop": gemm_op(0, 0, M, N, K, bx[0], bx[1], bw[0], bw[1], (M, N)),
        "dgrad": gemm_op(1, 0, M, K, N, bd[0], bd[1], bw[2], bw[3], (M, K)),
        "wgrad": gemm_op(2, 0, N, K, M, bd[2], bd[3], bx[2], bx[3], (N, K)),
    }
    out[f"dense {M}x{K} -> {N}"] = r
    del d, X, Wt, dY, bx, bw, bd
    torch.cuda.empty_cache()
    d = W.block32(dev)
    W1, W2, X1, X2 = d["W1"], d["W2"], d["X1"], d["X2"]
    T, H = X1.shape
    F = W1.shape[0]
    b1, b2, bx1, bx2 = tile(F, H), tile(H, F), row(T, H), row(T, F)
    L.record = False
    L.quant("q", 3, W1, b1)
    L.quant("q", 3, W2, b2)
    L.quant("q", 0, X1, bx1)
    L.quant("q", 0, X2, bx2)
    L.record = True
    r = {
        "quant_32x32_W1": quant_op(3, W1, tile),
        "quant_32x32_W2": quant_op(3, W2, tile),
        "quant_row_X1": quant_op(0, X1, row),
        "quant_row_X2": quant_op(0, X2, row),
        "fprop1": gemm_op(0, 1, T, F, H, bx1[0], bx1[1], b1[0], b1[1], (T, F)),
        "fprop2": gemm_op(0, 1, T, H, F, bx2[0], bx2[1], b2[0], b2[1], (T, H)),
        "dgrad1": gemm_op(1, 1, T, H, F, bx2[0], bx2[1], b1[0], b1[1], (T, H)),
        "dgrad2": gemm_op(1, 1, T, F, H, bx1[0], bx1[1], b2[0], b2[1], (T, F)),
    }
    out[f"32x32 weights, {T} tokens, {H} <-> {F}"] = r
    del flush
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def cpu_baseline(W, x_dev, w_dev, budget_s):
    """The oracle (untuned) on a bounded sample of the step: dual-axis
    quantisation of leading token rows of the up-projection input and of
    leading rows of its weight (the same bytes the GPU step uses), then the
    binary64 GEMM of those rows (the up-projection fprop, K = hidden).  The
    sample is sized from a short calibration run to about `budget_s`."""
    import numpy as np
    import oracle
    oracle.lib()
    nthreads = oracle.num_threads()
    H = x_dev.shape[1]
    # calibration: 256 x 1024 outputs (large enough that thread start-up
    # does not dominate)
    xb = W.bf16_bits(x_dev[:256])
    wb = W.bf16_bits(w_dev[:1024])
    t0 = time.perf_counter()
    qa, sa = oracle.quant_row(xb)
    qb, sb = oracle.quant_row(wb)
    oracle.gemm(qa, sa, qb, sb)
    rate = 256 * 1024 / max(time.perf_counter() - t0, 1e-3)    # outputs per second
    want = rate * budget_s
    n = int(min(w_dev.shape[0], max(512, want / 256)))
    n -= n % 32
    m = int(min(x_dev.shape[0], 4096, max(64, want / n)))
    m -= m % 32
    xb = np.ascontiguousarray(W.bf16_bits(x_dev[:m]))
    wb = np.ascontiguousarray(W.bf16_bits(w_dev[:n]))
    t0 = time.perf_counter()
    qa, sa, _, _ = oracle.quant_dual(xb)
    qb, sb, _, _ = oracle.quant_dual(wb)
    t1 = time.perf_counter()
    oracle.gemm(qa, sa, qb, sb)
    t2 = time.perf_counter()
    dt = t2 - t0
    flops = 2.0 * m * n * H
    quant_bytes = 4.0625 * (m + n) * H          # dual-axis: 2 B read, 2 + 2/32 B written
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"dual-axis quantisation of {m} token rows and {n} weight rows (K={H}) of "
                      f"the up projection, then the binary64 GEMM of the {m}x{n} fprop outputs; "
                      f"{dt:.1f} s",
            # the two parts of the same sample, each in its own unit
            "quant_gbps": round(quant_bytes / max(t1 - t0, 1e-9) / 1e9, 3),
            "gemm_tflops": round(flops / max(t2 - t1, 1e-9) / 1e12, 6)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp8_microscaled_precision_amd as mx
    from mxfp8_microscaled_precision_amd import workloads as W
    torch.cuda.set_device(0)
    st = mx.mx_device_check(0)
    if st != 0:
        raise SystemExit(f"device check failed: {mx.mx_last_error()}")
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    stack, bufs, moe, mbufs, d = build_workload(torch, W, args.layers)
    torch.cuda.synchronize()
    if args.calibration_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    L = Launcher(torch, mx)
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run_step(L, stack, bufs, moe, mbufs, d)
    torch.cuda.synchronize()
    # timed region: K steps, HIP events around every launch on the launch
    # stream (the same stream as torch's current stream)
    print("[bench] timing", file=sys.stderr, flush=True)
    L.record = True
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run_step(L, stack, bufs, moe, mbufs, d)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    per = per_kernel_medians(L.events, args.steps)
    kernels = {}
    for kind, k in per.items():
        rate = k["work"] / (k["ms"] * 1e-3)
        if k["unit"] == "FLOP":
            kernels[kind] = {"tflops": rate / 1e12, "frac_peak": rate / 1e12 / PEAK_FP8_TFLOPS,
                             "ms_per_step": k["ms"], "launches_per_step": k["launches"]}
        else:
            kernels[kind] = {"gbps": rate / 1e9, "frac_peak": rate / 1e9 / PEAK_HBM_GBPS,
                             "ms_per_step": k["ms"], "launches_per_step": k["launches"]}
    gemm_flop = sum(k["work"] for k in per.values() if k["unit"] == "FLOP")
    quant_bytes = sum(k["work"] for k in per.values() if k["unit"] == "B")
    quant_ms = sum(k["ms"] for k in per.values() if k["unit"] == "B")
    value = gemm_flop / (ms_step * 1e-3) / 1e12
    g = per["gemm"]
    g_rate = g["work"] / (g["ms"] * 1e-3) / 1e12
    traffic, alg_bytes = gemm_traffic()
    clock_ghz, mfma_busy = gemm_clock()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": (f"MXFP8 linear stack, {args.layers} layers {d['H']}->{d['F']}->{d['H']} at "
                         f"{d['T']} tokens, 1x32 dual-axis and 32x32-weight variants "
                         f"(quantise + fprop/dgrad/wgrad) + MoE grouped gate_up/down forward and "
                         f"backward (dgrad, per-expert wgrad) over {d['Tm']} routed tokens, "
                         f"{d['G']} experts"),
            "tokens": d["T"], "hidden": d["H"], "ffn": d["F"], "layers": args.layers,
            "moe_tokens": d["Tm"], "experts": d["G"],
            "gemm_tflop_per_step": round(gemm_flop / 1e12, 3),
            "quant_gb_per_step": round(quant_bytes / 1e9, 3),
        },
        "roofline": {
            "bound": "mfma", "achieved": round(g_rate, 2), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(g_rate / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes read + written per launch (mean over the step's launches)",
            "timing": "per launch, the median over the timed steps; rate = work / sum of medians",
            "algorithmic_bytes_per_launch": alg_bytes,
            "kernel": "gemm_persistent_kernel<B_ROW> (1x32 fprop/dgrad/wgrad)",
        },
        "quant": {"gbps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                  "ms_per_step": round(quant_ms, 3)},
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "wall_s_timed": round(wall, 3),
    }
    if clock_ghz is not None:
        # the dense FP8 MFMA rate at the clock the chip holds under this
        # kernel (from the committed counter run): 256 CUs x 4 SIMDs x 2048
        # FLOP per cycle
        at_clock = 256 * 4 * 2048 * clock_ghz * 1e9 / 1e12
        out["roofline"]["clock_ghz_measured"] = clock_ghz
        out["roofline"]["peak_at_measured_clock"] = round(at_clock, 1)
        out["roofline"]["frac_at_measured_clock"] = round(g_rate / at_clock, 4)
        out["roofline"]["mfma_busy_measured"] = mfma_busy
    print("[bench] copy rate, quantisation error", file=sys.stderr, flush=True)
    cg = copy_rate(torch)
    out["quant"]["d2d_copy_gbps"] = round(cg, 1)
    out["quant"]["frac_of_copy"] = round(out["quant"]["gbps"] / cg, 4)
    out["quantisation_error"] = {k: float(f"{v:.6g}") for k, v in
                                 quantisation_error(torch, mx, stack[0]).items()}
    out["fused_producer"] = fused_producer(torch, mx, stack[0])
    if not args.no_other_configs:
        print("[bench] other configurations", file=sys.stderr, flush=True)
        out["other_configs"] = other_configs(torch, mx, W)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(W, stack[0]["X_up"], stack[0]["W_up"], args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
