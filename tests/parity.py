"""Helpers for the GPU parity tests: host/device byte movement and the
element-by-element comparisons against the oracle.  Oracle inputs are only
seeded BF16 tensors from the workload generators or oracle outputs."""
import sys

import numpy as np
import torch

import oracle
from mxfp8_microscaled_precision_amd import workloads as W


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return W.bf16_bits(t)


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def assert_bytes(got_t, want: np.ndarray, what: str):
    got = host(got_t) if isinstance(got_t, torch.Tensor) else got_t
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        ex = [(tuple(int(v) for v in i), int(got[tuple(i)]), int(want[tuple(i)])) for i in bad[:8]]
        raise AssertionError(f"{what}: {len(bad)} byte mismatches, first (index, gpu, oracle): {ex}")


def assert_gemm(got_t, ref: np.ndarray, bound: np.ndarray, what: str):
    got = got_t.float().cpu().numpy().astype(np.float64) if isinstance(got_t, torch.Tensor) \
        else np.asarray(got_t, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ok = np.isnan(got) & np.isnan(ref)
    ok = oracle.within_tolerance(got, ref, bound) | nan_ok
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)} of {ok.size} outside |gpu-ref| <= 2^-7 sum|ab| + 1e-6; "
            f"first {i}: gpu {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")


def oracle_quant(x_bits: np.ndarray, mode: str):
    if mode == "row":
        return oracle.quant_row(x_bits)
    if mode == "col":
        return oracle.quant_col(x_bits)
    if mode == "dual":
        return oracle.quant_dual(x_bits)
    return oracle.quant_block32(x_bits)
