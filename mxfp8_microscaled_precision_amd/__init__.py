"""MXFP8 microscaled-precision hot path for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/mxfp8.h`` (``libmxfp8.so``,
built in-tree by ``python -m mxfp8_microscaled_precision_amd.build``).  The
functions named ``mx_*`` take raw device pointers and sizes exactly like the C
entry points; ``quant``, ``quant_batched``, ``quant_grouped_col``, ``gemm``,
``grouped_gemm``, ``grouped_gemm_wgrad`` and ``process_quant_result`` marshal
torch CUDA tensors (device memory and the current stream only) into those
calls.  Every step of the computation runs in
the HIP kernels; there is no CPU fallback: without the built library, or on a
device other than gfx950, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MXError", "lib", "mx_device_check", "mx_arch_supported", "mx_status_string",
    "mx_last_error", "mx_quant", "mx_gemm", "mx_grouped_gemm", "mx_grouped_gemm_workspace_size",
    "mx_quant_elem", "mx_gemm_elem",
    "mx_grouped_gemm_elem", "mx_quant_grouped_col_elem", "mx_grouped_gemm_wgrad_elem",
    "mx_gemm_quant", "gemm_quant",
    "mx_quant_batched", "mx_quant_batched_elem",
    "mx_grouped_col_capacity", "mx_quant_grouped_col", "mx_grouped_gemm_wgrad", "quant", "gemm",
    "grouped_gemm", "quant_batched", "quant_grouped_col", "grouped_gemm_wgrad",
    "grouped_col_capacity", "process_quant_result", "QUANT_MODES", "GEMM_LAYOUTS",
    "BSCALE_KINDS", "ELEM_TYPES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp8.so")

MX_OK = 0
QUANT_MODES = {"row": 0, "col": 1, "dual": 2, "32x32": 3}
GEMM_LAYOUTS = {"fprop": 0, "dgrad": 1, "wgrad": 2}
BSCALE_KINDS = {"1x32": 0, "32x32": 1}
ELEM_TYPES = {"e4m3": 0, "e5m2": 1}


class MXError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{mx_status_string(status)} (status {status}): {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmxfp8.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mxfp8_microscaled_precision_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, c_int, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.mx_device_check.restype = c_int
        L.mx_device_check.argtypes = [c_int]
        L.mx_arch_supported.restype = c_int
        L.mx_arch_supported.argtypes = [ctypes.c_char_p]
        L.mx_status_string.restype = ctypes.c_char_p
        L.mx_status_string.argtypes = [c_int]
        L.mx_last_error.restype = ctypes.c_char_p
        L.mx_last_error.argtypes = []
        L.mx_quant.restype = c_int
        L.mx_quant.argtypes = [c_int, vp, i64, i64, vp, vp, vp, vp, vp]
        L.mx_gemm.restype = c_int
        L.mx_gemm.argtypes = [c_int, c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.mx_grouped_gemm.restype = c_int
        L.mx_grouped_gemm.argtypes = [i64, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.mx_grouped_gemm_workspace_size.restype = sz
        L.mx_grouped_gemm_workspace_size.argtypes = [i64, i64, i64]
        L.mx_quant_elem.restype = c_int
        L.mx_quant_elem.argtypes = [c_int, c_int, vp, i64, i64, vp, vp, vp, vp, vp]
        L.mx_gemm_elem.restype = c_int
        L.mx_gemm_elem.argtypes = [c_int, c_int, c_int, c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.mx_grouped_gemm_elem.restype = c_int
        L.mx_grouped_gemm_elem.argtypes = [c_int, c_int, i64, vp, i64, i64, i64, vp, vp, vp, vp, vp,
                                           vp, sz, vp]
        L.mx_gemm_quant.restype = c_int
        L.mx_gemm_quant.argtypes = [c_int, c_int, c_int, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.mx_quant_batched.restype = c_int
        L.mx_quant_batched.argtypes = [c_int, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.mx_quant_batched_elem.restype = c_int
        L.mx_quant_batched_elem.argtypes = [c_int, c_int, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.mx_grouped_col_capacity.restype = i64
        L.mx_grouped_col_capacity.argtypes = [i64, i64]
        L.mx_quant_grouped_col.restype = c_int
        L.mx_quant_grouped_col.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
        L.mx_grouped_gemm_wgrad.restype = c_int
        L.mx_grouped_gemm_wgrad.argtypes = [i64, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.mx_quant_grouped_col_elem.restype = c_int
        L.mx_quant_grouped_col_elem.argtypes = [c_int, vp, i64, i64, i64, vp, vp, vp, vp]
        L.mx_grouped_gemm_wgrad_elem.restype = c_int
        L.mx_grouped_gemm_wgrad_elem.argtypes = [c_int, c_int, i64, vp, i64, i64, i64, vp, vp, vp, vp,
                                                 vp, vp]
        _lib = L
    return _lib


# ---------------------------------------------------------------------------
# The C entry points, same names and arguments (raw pointers as ints)
# ---------------------------------------------------------------------------

def mx_device_check(device: int) -> int:
    return lib().mx_device_check(device)


def mx_arch_supported(name: str) -> int:
    return lib().mx_arch_supported(name.encode() if name is not None else None)


def mx_status_string(status: int) -> str:
    return lib().mx_status_string(status).decode()


def mx_last_error() -> str:
    return lib().mx_last_error().decode()


def mx_quant(mode, x, rows, cols, q, s, q_t, s_t, stream) -> int:
    return lib().mx_quant(mode, x, rows, cols, q, s, q_t, s_t, stream)


def mx_gemm(layout, bkind, M, N, K, a, sa, b, sb, c, stream) -> int:
    return lib().mx_gemm(layout, bkind, M, N, K, a, sa, b, sb, c, stream)


def mx_grouped_gemm(G, offsets, T, N, K, a, sa, b, sb, c, workspace, workspace_bytes, stream) -> int:
    return lib().mx_grouped_gemm(G, offsets, T, N, K, a, sa, b, sb, c, workspace, workspace_bytes,
                                 stream)


def mx_grouped_gemm_workspace_size(G, T, N) -> int:
    return lib().mx_grouped_gemm_workspace_size(G, T, N)


def mx_grouped_gemm_elem(a_elem, b_elem, G, offsets, T, N, K, a, sa, b, sb, c, workspace,
                         workspace_bytes, stream) -> int:
    return lib().mx_grouped_gemm_elem(a_elem, b_elem, G, offsets, T, N, K, a, sa, b, sb, c,
                                      workspace, workspace_bytes, stream)


def mx_quant_elem(mode, elem, x, rows, cols, q, s, q_t, s_t, stream) -> int:
    return lib().mx_quant_elem(mode, elem, x, rows, cols, q, s, q_t, s_t, stream)


def mx_gemm_elem(layout, bkind, a_elem, b_elem, M, N, K, a, sa, b, sb, c, stream) -> int:
    return lib().mx_gemm_elem(layout, bkind, a_elem, b_elem, M, N, K, a, sa, b, sb, c, stream)


def mx_gemm_quant(layout, bkind, out_elem, M, N, K, a, sa, b, sb, q, s, stream) -> int:
    return lib().mx_gemm_quant(layout, bkind, out_elem, M, N, K, a, sa, b, sb, q, s, stream)


def mx_quant_batched(mode, x, batch, rows, cols, q, s, q_t, s_t, stream) -> int:
    return lib().mx_quant_batched(mode, x, batch, rows, cols, q, s, q_t, s_t, stream)


def mx_quant_batched_elem(mode, elem, x, batch, rows, cols, q, s, q_t, s_t, stream) -> int:
    return lib().mx_quant_batched_elem(mode, elem, x, batch, rows, cols, q, s, q_t, s_t, stream)


def mx_grouped_col_capacity(T, G) -> int:
    return lib().mx_grouped_col_capacity(T, G)


def mx_quant_grouped_col(x, T, C, G, offsets, q_t, s_t, stream) -> int:
    return lib().mx_quant_grouped_col(x, T, C, G, offsets, q_t, s_t, stream)


def mx_grouped_gemm_wgrad(G, offsets, T, M, N, a, sa, b, sb, c, stream) -> int:
    return lib().mx_grouped_gemm_wgrad(G, offsets, T, M, N, a, sa, b, sb, c, stream)


def mx_quant_grouped_col_elem(elem, x, T, C, G, offsets, q_t, s_t, stream) -> int:
    return lib().mx_quant_grouped_col_elem(elem, x, T, C, G, offsets, q_t, s_t, stream)


def mx_grouped_gemm_wgrad_elem(a_elem, b_elem, G, offsets, T, M, N, a, sa, b, sb, c, stream) -> int:
    return lib().mx_grouped_gemm_wgrad_elem(a_elem, b_elem, G, offsets, T, M, N, a, sa, b, sb, c,
                                            stream)


def _check(status: int):
    if status != MX_OK:
        raise MXError(status, mx_last_error())


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    # the library launches on the current device
    if t.get_device() != torch.cuda.current_device():
        raise ValueError(f"{name} is on cuda:{t.get_device()}, not on the current device "
                         f"cuda:{torch.cuda.current_device()}")


def _shape(t, shape, name):
    """The library reads exactly the bytes the sizes describe, so every
    operand must have them (a short tensor would be read past its end)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _gemm_operands(a, sa, b, sb, layout, bscale):
    """(M, N, K) of a dense GEMM call, after checking every operand's shape
    against them (K % 32 and N % 32 for 32x32 tiles are left to the library,
    which reports them as unsupported shapes)."""
    M, K = a.shape
    tiles = bscale == "32x32"
    N = b.shape[1] if (tiles and layout == "dgrad") else b.shape[0]
    if K % 32 == 0:
        _shape(sa, (M, K // 32), "sa")
        if not tiles:
            _shape(b, (N, K), "b")
            _shape(sb, (N, K // 32), "sb")
        elif N % 32 == 0:
            if layout == "dgrad":      # the shared weight [K, N], tiles along both
                _shape(b, (K, N), "b")
                _shape(sb, (K // 32, N // 32), "sb")
            else:
                _shape(b, (N, K), "b")
                _shape(sb, (N // 32, K // 32), "sb")
    return M, N, K


def quant(x, mode: str = "row", elem: str = "e4m3"):
    """Dynamic MX quantisation of a BF16 [rows, cols] tensor.

    mode "row"   -> (q [rows,cols], s [rows,cols/32])
         "col"   -> (q_t [cols,rows], s_t [cols,rows/32])
         "dual"  -> (q, s, q_t, s_t)
         "32x32" -> (q [rows,cols], s [rows/32,cols/32])
    Payloads are uint8 E4M3 (or, with elem="e5m2", E5M2) bytes, scales
    uint8 E8M0 bytes.
    """
    torch = _torch()
    if mode not in QUANT_MODES:
        raise ValueError(f"unknown quantisation mode {mode!r}; expected one of {list(QUANT_MODES)}")
    if elem not in ELEM_TYPES:
        raise ValueError(f"unknown element type {elem!r}; expected one of {list(ELEM_TYPES)}")
    _need(x, torch.bfloat16, "x", 2)
    R, C = x.shape
    dev, u8 = x.device, torch.uint8
    q = s = qt = st = None
    if mode in ("row", "dual", "32x32"):
        q = torch.empty((R, C), dtype=u8, device=dev)
        s = torch.empty((R // 32, C // 32) if mode == "32x32" else (R, C // 32), dtype=u8, device=dev)
    if mode in ("col", "dual"):
        qt = torch.empty((C, R), dtype=u8, device=dev)
        st = torch.empty((C, R // 32), dtype=u8, device=dev)
    _check(mx_quant_elem(QUANT_MODES[mode], ELEM_TYPES[elem], _ptr(x), R, C, _ptr(q), _ptr(s),
                         _ptr(qt), _ptr(st), _stream(dev)))
    if mode == "row" or mode == "32x32":
        return q, s
    if mode == "col":
        return qt, st
    return q, s, qt, st


def gemm(a, sa, b, sb, layout: str = "fprop", bscale: str = "1x32", out=None,
         a_elem: str = "e4m3", b_elem: str = "e4m3"):
    """MXFP8 GEMM C = A * B^T (FP32 accumulation, BF16 result).

    a [M,K] u8 + sa [M,K/32]; b [N,K] u8 + sb [N,K/32] for 1x32 scales;
    with bscale "32x32": fprop b [N,K] + tiles [N/32,K/32], dgrad b [K,N]
    (the shared weight, contracted over rows) + tiles [K/32,N/32].
    a_elem / b_elem: payload element types ("e4m3" or "e5m2").
    """
    torch = _torch()
    if layout not in GEMM_LAYOUTS or bscale not in BSCALE_KINDS:
        raise ValueError(f"unknown layout {layout!r} or B scale kind {bscale!r}")
    if a_elem not in ELEM_TYPES or b_elem not in ELEM_TYPES:
        raise ValueError(f"unknown element types {a_elem!r}, {b_elem!r}")
    for t, n in ((a, "a"), (sa, "sa"), (b, "b"), (sb, "sb")):
        _need(t, torch.uint8, n, 2)
    M, N, K = _gemm_operands(a, sa, b, sb, layout, bscale)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, torch.bfloat16, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}]")
    _check(mx_gemm_elem(GEMM_LAYOUTS[layout], BSCALE_KINDS[bscale], ELEM_TYPES[a_elem],
                        ELEM_TYPES[b_elem], M, N, K, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb),
                        _ptr(out), _stream(a.device)))
    return out


def gemm_quant(a, sa, b, sb, layout: str = "fprop", bscale: str = "1x32", out_elem: str = "e4m3"):
    """Fused producer: the GEMM's BF16 result quantised in 1x32 blocks along N
    in the epilogue -> (q [M,N] u8, s [M,N/32] u8), equal to
    quant(gemm(...), "row", out_elem)."""
    torch = _torch()
    if layout not in GEMM_LAYOUTS or bscale not in BSCALE_KINDS or out_elem not in ELEM_TYPES:
        raise ValueError(f"unknown layout {layout!r}, B scale kind {bscale!r} or element {out_elem!r}")
    for t, n in ((a, "a"), (sa, "sa"), (b, "b"), (sb, "sb")):
        _need(t, torch.uint8, n, 2)
    M, N, K = _gemm_operands(a, sa, b, sb, layout, bscale)
    q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    s = torch.empty((M, N // 32), dtype=torch.uint8, device=a.device)
    _check(mx_gemm_quant(GEMM_LAYOUTS[layout], BSCALE_KINDS[bscale], ELEM_TYPES[out_elem], M, N, K,
                         _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(q), _ptr(s), _stream(a.device)))
    return q, s


def grouped_gemm(offsets, a, sa, b, sb, out=None, a_elem: str = "e4m3", b_elem: str = "e4m3"):
    """MoE grouped MXFP8 GEMM: rows offsets[g]:offsets[g+1] of a times b[g]^T.

    offsets int64 [G+1] on the device; a [T,K] u8 + sa [T,K/32];
    b [G,N,K] u8 + sb [G,N,K/32]; returns BF16 [T,N].  a_elem / b_elem:
    payload element types ("e4m3" or "e5m2").
    """
    torch = _torch()
    if a_elem not in ELEM_TYPES or b_elem not in ELEM_TYPES:
        raise ValueError(f"unknown element types {a_elem!r}, {b_elem!r}")
    _need(offsets, torch.int64, "offsets", 1)
    for t, n in ((a, "a"), (sa, "sa")):
        _need(t, torch.uint8, n, 2)
    for t, n in ((b, "b"), (sb, "sb")):
        _need(t, torch.uint8, n, 3)
    G = offsets.numel() - 1
    T, K = a.shape
    N = b.shape[1]
    if G < 1:
        raise ValueError("offsets must hold at least two entries (one group)")
    if K % 32 == 0:
        _shape(sa, (T, K // 32), "sa")
        _shape(b, (G, N, K), "b")
        _shape(sb, (G, N, K // 32), "sb")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=a.device)
    _need(out, torch.bfloat16, "out", 2)
    _shape(out, (T, N), "out")
    nws = mx_grouped_gemm_workspace_size(G, T, N)
    ws = torch.empty(nws, dtype=torch.uint8, device=a.device) if nws else None
    _check(mx_grouped_gemm_elem(ELEM_TYPES[a_elem], ELEM_TYPES[b_elem], G, _ptr(offsets), T, N, K,
                                _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out), _ptr(ws), nws,
                                _stream(a.device)))
    return out


def quant_batched(x, mode: str = "row", elem: str = "e4m3"):
    """mx_quant on every matrix of a BF16 stack x [B, rows, cols] (e.g. the
    per-expert weights of an MoE layer); outputs are the stacked per-matrix
    outputs of ``quant`` in the same mode and element type."""
    torch = _torch()
    if mode not in QUANT_MODES:
        raise ValueError(f"unknown quantisation mode {mode!r}; expected one of {list(QUANT_MODES)}")
    if elem not in ELEM_TYPES:
        raise ValueError(f"unknown element type {elem!r}; expected one of {list(ELEM_TYPES)}")
    _need(x, torch.bfloat16, "x", 3)
    B, R, C = x.shape
    dev, u8 = x.device, torch.uint8
    q = s = qt = st = None
    if mode in ("row", "dual", "32x32"):
        q = torch.empty((B, R, C), dtype=u8, device=dev)
        s = torch.empty((B, R // 32, C // 32) if mode == "32x32" else (B, R, C // 32), dtype=u8,
                        device=dev)
    if mode in ("col", "dual"):
        qt = torch.empty((B, C, R), dtype=u8, device=dev)
        st = torch.empty((B, C, R // 32), dtype=u8, device=dev)
    _check(mx_quant_batched_elem(QUANT_MODES[mode], ELEM_TYPES[elem], _ptr(x), B, R, C, _ptr(q),
                                 _ptr(s), _ptr(qt), _ptr(st), _stream(dev)))
    if mode == "row" or mode == "32x32":
        return q, s
    if mode == "col":
        return qt, st
    return q, s, qt, st


def grouped_col_capacity(T: int, G: int) -> int:
    """Columns of the per-group column-quantised token matrix."""
    cap = mx_grouped_col_capacity(int(T), int(G))
    if cap < 0:
        raise ValueError(f"no capacity for T={T}, G={G}")
    return cap


def quant_grouped_col(x, offsets, elem: str = "e4m3"):
    """Per-expert column quantisation along the token axis (MoE backward):
    x BF16 [T, C], offsets int64 [G+1] on the device ->
    (q_t [C, cap] u8, s_t [C, cap/32] u8), cap = grouped_col_capacity(T, G);
    group g's tokens at columns 128 (offsets[g] // 128 + g) on.  elem: the
    payload element type ("e4m3" or "e5m2")."""
    torch = _torch()
    if elem not in ELEM_TYPES:
        raise ValueError(f"unknown element type {elem!r}")
    _need(x, torch.bfloat16, "x", 2)
    _need(offsets, torch.int64, "offsets", 1)
    T, C = x.shape
    G = offsets.numel() - 1
    cap = grouped_col_capacity(T, G)
    qt = torch.empty((C, cap), dtype=torch.uint8, device=x.device)
    st = torch.empty((C, cap // 32), dtype=torch.uint8, device=x.device)
    _check(mx_quant_grouped_col_elem(ELEM_TYPES[elem], _ptr(x), T, C, G, _ptr(offsets), _ptr(qt),
                                     _ptr(st), _stream(x.device)))
    return qt, st


def grouped_gemm_wgrad(offsets, T: int, a, sa, b, sb, out=None, a_elem: str = "e4m3",
                       b_elem: str = "e4m3"):
    """Per-expert weight gradient: out[g] = A_g * B_g^T over group g's token
    columns of a [M, cap] and b [N, cap] (both from ``quant_grouped_col`` with
    the same offsets); returns BF16 [G, M, N].  a_elem / b_elem: the payload
    element types of a and b."""
    torch = _torch()
    if a_elem not in ELEM_TYPES or b_elem not in ELEM_TYPES:
        raise ValueError(f"unknown element types {a_elem!r}, {b_elem!r}")
    _need(offsets, torch.int64, "offsets", 1)
    for t, n in ((a, "a"), (sa, "sa"), (b, "b"), (sb, "sb")):
        _need(t, torch.uint8, n, 2)
    G = offsets.numel() - 1
    M, N = a.shape[0], b.shape[0]
    cap = grouped_col_capacity(T, G)
    if a.shape[1] != cap or b.shape[1] != cap or sa.shape != (M, cap // 32) or sb.shape != (N, cap // 32):
        raise ValueError(f"operands must be [rows, {cap}] with scales [rows, {cap // 32}]")
    if out is None:
        out = torch.empty((G, M, N), dtype=torch.bfloat16, device=a.device)
    _need(out, torch.bfloat16, "out", 3)
    if tuple(out.shape) != (G, M, N):
        raise ValueError(f"out must be [{G}, {M}, {N}]")
    _check(mx_grouped_gemm_wgrad_elem(ELEM_TYPES[a_elem], ELEM_TYPES[b_elem], G, _ptr(offsets), T, M,
                                      N, _ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(out),
                                      _stream(a.device)))
    return out


def _dst_type_name(dst_type) -> str:
    """'e4m3' / 'e5m2' from a name or a torch FP8 dtype (the RFC passes the
    target dtype itself)."""
    if isinstance(dst_type, str):
        name = dst_type.lower()
    else:
        name = {"torch.float8_e4m3fn": "e4m3", "torch.float8_e5m2": "e5m2"}.get(str(dst_type), "")
    if name not in ELEM_TYPES:
        raise ValueError(f"unsupported dst_type {dst_type!r}: expected 'e4m3' (torch.float8_e4m3fn) "
                         f"or 'e5m2' (torch.float8_e5m2)")
    return name


def process_quant_result(weight, recipe: str = "mxfp8", dst_type="e4m3"):
    """Quantise a weight for both passes, in the RFC's tuple order
    (weight_fwd, scale_fwd, weight_bwd, scale_bwd).

    recipe   "mxfp8"       -> dual-axis 1x32: two FP8 copies, row and column
                              scales.
             "mxfp8-32x32" -> 32x32 tiles: weight_bwd IS weight_fwd and the
                              one tile scale array serves both passes (forward
                              blocks K along the columns, backward along the
                              rows).
    dst_type the FP8 payload type: "e4m3" / torch.float8_e4m3fn or "e5m2" /
             torch.float8_e5m2 (the scale rule follows the type's largest
             finite value).
    (MindSpeed RFC "add MXFP8-32x32 quantisation support to FSDP", sections
    3.3.3 and 3.5.2.3: process_quant_result_fn(weight, dst_type, config); an
    unsupported recipe or dst_type raises ValueError.)
    """
    if recipe not in ("mxfp8", "mxfp8-32x32"):
        raise ValueError(f"unsupported recipe {recipe!r}: expected 'mxfp8' or 'mxfp8-32x32'")
    elem = _dst_type_name(dst_type)
    if recipe == "mxfp8":
        q, s, qt, st = quant(weight, "dual", elem)
        return q, s, qt, st
    q, s = quant(weight, "32x32", elem)
    return q, s, q, s
