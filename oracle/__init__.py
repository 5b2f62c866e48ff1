"""CPU oracle for the MXFP8 microscaled hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.  The arithmetic lives in ``mx_oracle.cpp`` (plain
C++ functions over arrays, binary64, built with g++); this module only
compiles it and marshals numpy arrays through ctypes.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, exhaustive brute force and library routines (torch's
float8 casts, numpy float64 matmul); see those files.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "mx_oracle.cpp")
# MX_ORACLE_LIB points the wrappers at another build of the oracle (the
# mutation tests load deliberately broken copies this way); it is never
# rebuilt from here.
_ALT = os.environ.get("MX_ORACLE_LIB")
_LIB = _ALT or os.path.join(_DIR, "liboracle.so")

# g++ flags: no fast-math and no FMA contraction, so every binary64 operation
# is the plain IEEE operation written in the source.
CXX = "g++"
CFLAGS = ["-O2", "-std=c++17", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-shared", "-fPIC"]

BKIND_ROW = 0        # B [N][K], scales [N][K/32]
BKIND_TILE = 1       # B [N][K], 32x32 tile scales [N/32][K/32]
BKIND_TILE_T = 2     # B [K][N] contracted over rows, tile scales [K/32][N/32]

ELEM_E4M3 = 0        # payload element types
ELEM_E5M2 = 1
ELEMS = {"e4m3": ELEM_E4M3, "e5m2": ELEM_E5M2}


def build(force: bool = True) -> str:
    """Compile mx_oracle.cpp into liboracle.so (always, when force)."""
    if _ALT:
        return _LIB
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([CXX, *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _ALT and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        L = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_round.restype = ctypes.c_uint8
        L.orc_e4m3_round.argtypes = [ctypes.c_double]
        L.orc_e5m2_value.restype = ctypes.c_double
        L.orc_e5m2_value.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_round.restype = ctypes.c_uint8
        L.orc_e5m2_round.argtypes = [ctypes.c_double]
        L.orc_rceil_exponent_e5m2.restype = ctypes.c_int
        L.orc_rceil_exponent_e5m2.argtypes = [ctypes.c_double]
        for name in ("orc_quant_row_elem", "orc_quant_col_elem", "orc_quant_block32_elem"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                          ctypes.c_void_p, ctypes.c_void_p]
        L.orc_gemm_elem.restype = ctypes.c_int
        L.orc_gemm_elem.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
        L.orc_rceil_exponent.restype = ctypes.c_int
        L.orc_rceil_exponent.argtypes = [ctypes.c_double]
        for name in ("orc_quant_row", "orc_quant_col", "orc_quant_block32"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                          ctypes.c_void_p]
        L.orc_gemm.restype = ctypes.c_int
        L.orc_gemm.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_grouped_gemm.restype = ctypes.c_int
        L.orc_grouped_gemm.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
        L.orc_grouped_col_capacity.restype = ctypes.c_int64
        L.orc_grouped_col_capacity.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.orc_quant_col_grouped.restype = ctypes.c_int
        L.orc_quant_col_grouped.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]
        L.orc_quant_col_grouped_elem.restype = ctypes.c_int
        L.orc_quant_col_grouped_elem.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        L.orc_grouped_gemm_wgrad_elem.restype = ctypes.c_int
        L.orc_grouped_gemm_wgrad_elem.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p]
        L.orc_grouped_gemm_wgrad.restype = ctypes.c_int
        L.orc_grouped_gemm_wgrad.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]
        L.orc_num_threads.restype = ctypes.c_int
        del u8p
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


# --- scalar formats ---------------------------------------------------------

def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e8m0_value(b: int) -> float:
    return lib().orc_e8m0_value(int(b))


def e4m3_round(v: float) -> int:
    return int(lib().orc_e4m3_round(float(v)))


def rceil_exponent(amax: float) -> int:
    return int(lib().orc_rceil_exponent(float(amax)))


def e5m2_value(code: int) -> float:
    return lib().orc_e5m2_value(int(code))


def e5m2_round(v: float) -> int:
    return int(lib().orc_e5m2_round(float(v)))


def rceil_exponent_e5m2(amax: float) -> int:
    return int(lib().orc_rceil_exponent_e5m2(float(amax)))


def e5m2_decode_table() -> np.ndarray:
    """binary64 value of each of the 256 E5M2 codes (+-inf, NaN included)."""
    f = lib().orc_e5m2_value
    return np.array([f(c) for c in range(256)], dtype=np.float64)


def e4m3_round_array(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64).ravel()
    f = lib().orc_e4m3_round
    return np.fromiter((f(float(x)) for x in v), dtype=np.uint8, count=v.size)


def e4m3_decode_table() -> np.ndarray:
    """binary64 value of each of the 256 E4M3 codes (NaN for 0x7F, 0xFF)."""
    f = lib().orc_e4m3_value
    return np.array([f(c) for c in range(256)], dtype=np.float64)


def e8m0_decode_table() -> np.ndarray:
    f = lib().orc_e8m0_value
    return np.array([f(c) for c in range(256)], dtype=np.float64)


# --- quantisation -------------------------------------------------------------

def _bits(x) -> np.ndarray:
    """BF16 payload as uint16 bits [R, C] (accepts uint16/int16 arrays)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.int16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("x must be a 2-D uint16 array of BF16 bit patterns")
    return x


def _elem(elem) -> int:
    if isinstance(elem, str):
        elem = ELEMS[elem]
    if elem not in (ELEM_E4M3, ELEM_E5M2):
        raise ValueError(f"unknown element type {elem!r}")
    return int(elem)


def quant_row(x, elem=ELEM_E4M3):
    """1x32 quantisation along rows: returns (q [R,C] u8, s [R,C/32] u8)."""
    x = _bits(x)
    R, C = x.shape
    if C % 32:
        raise ValueError("cols must be a multiple of 32")
    q = np.empty((R, C), np.uint8)
    s = np.empty((R, C // 32), np.uint8)
    lib().orc_quant_row_elem(_ptr(x), R, C, _elem(elem), _ptr(q), _ptr(s))
    return q, s


def quant_col(x, elem=ELEM_E4M3):
    """32x1 quantisation down columns, written transposed:
    returns (q_t [C,R] u8, s_t [C,R/32] u8)."""
    x = _bits(x)
    R, C = x.shape
    if R % 32:
        raise ValueError("rows must be a multiple of 32")
    q = np.empty((C, R), np.uint8)
    s = np.empty((C, R // 32), np.uint8)
    lib().orc_quant_col_elem(_ptr(x), R, C, _elem(elem), _ptr(q), _ptr(s))
    return q, s


def quant_dual(x, elem=ELEM_E4M3):
    """Dual-axis: (q, s, q_t, s_t) = quant_row(x) + quant_col(x)."""
    q, s = quant_row(x, elem)
    qt, st = quant_col(x, elem)
    return q, s, qt, st


def quant_col_batched(x):
    """Column quantisation of each matrix of a stack x [B,R,C]:
    returns (q_t [B,C,R], s_t [B,C,R/32])."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.int16:
        x = x.view(np.uint16)
    outs = [quant_col(x[i]) for i in range(x.shape[0])]
    return (np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]))


def grouped_col_capacity(T: int, G: int) -> int:
    """Columns of the per-group column-quantised output (reading R20)."""
    return int(lib().orc_grouped_col_capacity(int(T), int(G)))


def group_col(g: int, o_g: int) -> int:
    """First column of group g (reading R20): 128 * (o_g // 128 + g)."""
    return 128 * (int(o_g) // 128 + int(g))


def quant_col_grouped(x, offsets, elem=ELEM_E4M3):
    """MoE backward column blocks restarting at each group offset (R20).

    x [T,C] BF16 bits, offsets int64 [G+1] -> (q_t [C,cap] u8, s_t [C,cap/32] u8)
    with cap = grouped_col_capacity(T, G); elem is the payload element type."""
    x = _bits(x)
    offsets = _c(np.asarray(offsets, dtype=np.int64), np.int64)
    T, C = x.shape
    G = offsets.size - 1
    cap = grouped_col_capacity(T, G)
    q = np.empty((C, cap), np.uint8)
    s = np.empty((C, cap // 32), np.uint8)
    rc = lib().orc_quant_col_grouped_elem(_ptr(x), T, C, G, _ptr(offsets), _elem(elem), _ptr(q),
                                          _ptr(s))
    if rc:
        raise ValueError(f"oracle grouped column quantisation rejected the arguments (rc={rc})")
    return q, s


def quant_block32(x, elem=ELEM_E4M3):
    """32x32 tiles: returns (q [R,C] u8, s [R/32,C/32] u8)."""
    x = _bits(x)
    R, C = x.shape
    if R % 32 or C % 32:
        raise ValueError("rows and cols must be multiples of 32")
    q = np.empty((R, C), np.uint8)
    s = np.empty((R // 32, C // 32), np.uint8)
    lib().orc_quant_block32_elem(_ptr(x), R, C, _elem(elem), _ptr(q), _ptr(s))
    return q, s


# --- GEMM ---------------------------------------------------------------------

def gemm(a, sa, b, sb, bkind: int = BKIND_ROW, want_bound: bool = True, a_elem=ELEM_E4M3,
         b_elem=ELEM_E4M3):
    """binary64 reference C = A * B^T of the dequantised operands.

    a [M,K] u8 + sa [M,K/32]; b/sb as described by ``bkind``; a_elem / b_elem
    the payload element types.
    Returns (ref [M,N] f64, bound [M,N] f64 or None) where bound = sum_k |a*b|.
    """
    a = _c(a, np.uint8)
    sa = _c(sa, np.uint8)
    b = _c(b, np.uint8)
    sb = _c(sb, np.uint8)
    M, K = a.shape
    N = b.shape[1] if bkind == BKIND_TILE_T else b.shape[0]
    ref = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64) if want_bound else None
    rc = lib().orc_gemm_elem(bkind, _elem(a_elem), _elem(b_elem), M, N, K, _ptr(a), _ptr(sa),
                             _ptr(b), _ptr(sb), _ptr(ref),
                             _ptr(bound) if bound is not None else None)
    if rc:
        raise ValueError(f"oracle gemm rejected the shapes (rc={rc})")
    return ref, bound


def grouped_gemm(offsets, a, sa, b, sb, want_bound: bool = True):
    """Per-expert reference: rows offsets[g]:offsets[g+1] of a times b[g]^T.

    offsets int64 [G+1]; a [T,K] u8 + sa [T,K/32]; b [G,N,K] u8 + sb [G,N,K/32].
    """
    offsets = _c(np.asarray(offsets, dtype=np.int64), np.int64)
    a = _c(a, np.uint8)
    sa = _c(sa, np.uint8)
    b = _c(b, np.uint8)
    sb = _c(sb, np.uint8)
    G = offsets.size - 1
    T, K = a.shape
    N = b.shape[1]
    ref = np.full((T, N), np.nan, np.float64)
    bound = np.full((T, N), np.nan, np.float64) if want_bound else None
    rc = lib().orc_grouped_gemm(G, _ptr(offsets), T, N, K, _ptr(a), _ptr(sa), _ptr(b),
                                _ptr(sb), _ptr(ref), _ptr(bound) if bound is not None else None)
    if rc:
        raise ValueError(f"oracle grouped gemm rejected the arguments (rc={rc})")
    return ref, bound


def grouped_gemm_wgrad(offsets, a, sa, b, sb, want_bound: bool = True, a_elem=ELEM_E4M3,
                       b_elem=ELEM_E4M3):
    """Per-expert weight gradient over each group's tokens (R20 layout).

    offsets int64 [G+1] with offsets[G] = T; a [M,cap] u8 + sa [M,cap/32];
    b [N,cap] u8 + sb [N,cap/32]; returns ref/bound [G,M,N].  a_elem / b_elem:
    the payload element types."""
    offsets = _c(np.asarray(offsets, dtype=np.int64), np.int64)
    a = _c(a, np.uint8)
    sa = _c(sa, np.uint8)
    b = _c(b, np.uint8)
    sb = _c(sb, np.uint8)
    G = offsets.size - 1
    T = int(offsets[-1])
    M, N = a.shape[0], b.shape[0]
    ref = np.empty((G, M, N), np.float64)
    bound = np.empty((G, M, N), np.float64) if want_bound else None
    rc = lib().orc_grouped_gemm_wgrad_elem(G, _ptr(offsets), T, M, N, _elem(a_elem), _elem(b_elem),
                                           _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(ref),
                                           _ptr(bound) if bound is not None else None)
    if rc:
        raise ValueError(f"oracle grouped wgrad rejected the arguments (rc={rc})")
    return ref, bound


def num_threads() -> int:
    return int(lib().orc_num_threads())


# --- tolerance ----------------------------------------------------------------

def within_tolerance(gpu, ref, bound):
    """Per-element GEMM bar: |gpu - ref| <= 2^-7 * sum_k|a_k b_k| + 1e-6.

    Returns a boolean array.  The budget: BF16 output rounding contributes at
    most 2^-8 |ref| and FP32 accumulation at most K * 2^-24 * sum|ab|
    (<= 2^-9 sum|ab| for K <= 32768).
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    return np.abs(gpu - ref) <= 2.0 ** -7 * bound + 1e-6
