"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no MX arithmetic: it only draws random numbers, rounds them
to BF16 and lays out bit patterns.  Tests, the bench and the smoke check use it
to feed the same bytes to the HIP library and to the CPU oracle.

Recipe (all draws float32 from ``torch.Generator`` seeded per tensor, rounded
to BF16 with round-to-nearest-even by ``Tensor.to(torch.bfloat16)``):

  seed(config k, tensor i) = (20261200 + k) * 1000 + i

  tiny       A [128,256], W [128,256] ~ N(0,1)
  dense      X [8192,4096] ~ N(0,1) with exactly round(0.001*numel) distinct
             seeded entries multiplied by 100; W [4096,4096] ~ N(0,0.02);
             dY [8192,4096] ~ N(0,1e-3)                      ("N(0,s)": s = std)
  block32    W1 [2048,7168], W2 [7168,2048] ~ N(0,0.02);
             X1 [16384,7168], X2 [16384,2048] ~ N(0,1); X2 doubles as dY of
             layer 1 and X1 as dY of layer 2 in the backward-data products
  moe        16384 tokens x top-8 = 131072 assignments over 64 experts,
             expert popularity Zipf(1.1) over seeded ranks with the 4 least
             popular ranks forced empty; X [131072,4096], H [131072,2048]
             ~ N(0,1); W_gu [64,4096,4096], W_dn [64,4096,2048] ~ N(0,0.02)
  stack      per layer l=0..3: X_up [32768,7168], X_dn [32768,18432] ~
             Student-t(3); dY_up [32768,18432], dY_dn [32768,7168] ~
             N(0,0.01); W_up [18432,7168], W_dn [7168,18432] ~ N(0,0.02)

Every shape can be scaled down (``scale`` divides the token/row counts and,
where noted, the feature sizes) for tests that the oracle must finish in
seconds.
"""
from __future__ import annotations

import numpy as np
import torch

BASE_SEED = 20261200


def seed_of(config: int, tensor: int) -> int:
    return (BASE_SEED + config) * 1000 + tensor


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def normal_with_outliers_bf16(shape, std: float, frac: float, factor: float, seed: int,
                              device="cpu") -> torch.Tensor:
    """N(0,std) with exactly round(frac*numel) distinct entries times factor."""
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    n = x.numel()
    k = int(round(frac * n))
    if k:
        idx = torch.randperm(n, generator=g, device=device)[:k]
        x.view(-1)[idx] *= factor
    return x.to(torch.bfloat16)


def student_t_bf16(shape, nu: int, seed: int, device="cpu") -> torch.Tensor:
    """Student-t(nu) as Z / sqrt(chi2_nu / nu), chi2 from nu squared normals."""
    g = _gen(seed, device)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(nu):
        w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi.addcmul_(w, w)
    z.div_(torch.sqrt(chi.div_(nu)))
    return z.to(torch.bfloat16)


def zipf_group_offsets(tokens: int, experts: int, alpha: float, n_empty: int,
                       seed: int) -> np.ndarray:
    """Expert group offsets int64 [experts+1] for `tokens` routed assignments.

    Rank i (1-based) has popularity i^-alpha; the n_empty least popular ranks
    are forced to zero; ranks map to experts through a seeded permutation and
    sizes are one multinomial draw.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    p = np.arange(1, experts + 1, dtype=np.float64) ** (-alpha)
    if n_empty:
        p[experts - n_empty:] = 0.0
    p /= p.sum()
    perm = rng.permutation(experts)
    by_rank = rng.multinomial(tokens, p)
    sizes = np.zeros(experts, np.int64)
    sizes[perm] = by_rank
    offsets = np.zeros(experts + 1, np.int64)
    np.cumsum(sizes, out=offsets[1:])
    return offsets


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def tiny(device="cpu"):
    return {
        "A": normal_bf16((128, 256), 1.0, seed_of(1, 0), device),
        "W": normal_bf16((128, 256), 1.0, seed_of(1, 1), device),
    }


def dense(device="cpu", scale: int = 1):
    M, K, N = 8192 // scale, 4096 // scale, 4096 // scale
    return {
        "X": normal_with_outliers_bf16((M, K), 1.0, 0.001, 100.0, seed_of(2, 0), device),
        "W": normal_bf16((N, K), 0.02, seed_of(2, 1), device),
        "dY": normal_bf16((M, N), 1e-3, seed_of(2, 2), device),
    }


def block32(device="cpu", scale: int = 1):
    T, H, F = 16384 // scale, 7168 // scale, 2048 // scale
    return {
        "W1": normal_bf16((F, H), 0.02, seed_of(3, 0), device),
        "W2": normal_bf16((H, F), 0.02, seed_of(3, 1), device),
        "X1": normal_bf16((T, H), 1.0, seed_of(3, 2), device),
        "X2": normal_bf16((T, F), 1.0, seed_of(3, 3), device),
    }


def moe_offsets(scale: int = 1, experts: int = 64) -> np.ndarray:
    return zipf_group_offsets(131072 // scale, experts, 1.1, 4, seed_of(4, 9))


def moe(device="cpu", scale: int = 1, fscale: int = 1, experts: int = 64):
    """scale divides the token count; fscale divides hidden and ffn sizes."""
    T = 131072 // scale
    H, F = 4096 // fscale, 2048 // fscale
    return {
        "offsets": moe_offsets(scale, experts),
        "X": normal_bf16((T, H), 1.0, seed_of(4, 0), device),
        "H": normal_bf16((T, F), 1.0, seed_of(4, 1), device),
        "W_gu": normal_bf16((experts, 2 * F, H), 0.02, seed_of(4, 2), device),
        "W_dn": normal_bf16((experts, H, F), 0.02, seed_of(4, 3), device),
    }


def moe_grads(device="cpu", scale: int = 1, fscale: int = 1):
    """Output gradients of the MoE expert GEMMs for the backward pass: dY of
    gate_up [T, 2F] and of down [T, H], N(0, 0.01) like the linear stack's
    gradients (the MoE workload itself gives no backward tensors)."""
    T = 131072 // scale
    H, F = 4096 // fscale, 2048 // fscale
    return {
        "dY_gu": normal_bf16((T, 2 * F), 0.01, seed_of(4, 4), device),
        "dY_dn": normal_bf16((T, H), 0.01, seed_of(4, 5), device),
    }


def stack_layer(layer: int, device="cpu", scale: int = 1, fscale: int = 1):
    T = 32768 // scale
    H, F = 7168 // fscale, 18432 // fscale
    b = 10 * layer
    return {
        "X_up": student_t_bf16((T, H), 3, seed_of(5, b + 0), device),
        "X_dn": student_t_bf16((T, F), 3, seed_of(5, b + 1), device),
        "dY_up": normal_bf16((T, F), 0.01, seed_of(5, b + 2), device),
        "dY_dn": normal_bf16((T, H), 0.01, seed_of(5, b + 3), device),
        "W_up": normal_bf16((F, H), 0.02, seed_of(5, b + 4), device),
        "W_dn": normal_bf16((H, F), 0.02, seed_of(5, b + 5), device),
    }


# --------------------------------------------------------------------------
# Bit-pattern inputs for edge cases
# --------------------------------------------------------------------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a BF16 tensor's bits."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(bits: np.ndarray, device="cpu") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to(device)


def sweep_blocks_bits(seed: int = 7) -> np.ndarray:
    """Blocks of 32 that sweep every BF16 magnitude under every anchor.

    For each biased BF16 exponent A of an anchor element (A = 0..254) and
    anchor mantissa 0x60 or 0x61 (1.75 * 2^(A-127), an exact 448 * 2^e, and
    the next value up; A = 0 gives subnormal anchors), the other 31 slots of
    each block walk through every BF16 magnitude not above the anchor, with
    seeded signs.  Returns uint16 [rows, 32] bits.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = []
    for A, mant in [(a, m) for a in range(0, 255) for m in (0x60, 0x61)]:
        anchor = (A << 7) | mant
        mags = np.arange(0, anchor + 1, dtype=np.uint32)
        pad = (-mags.size) % 31
        mags = np.concatenate([mags, np.zeros(pad, np.uint32)]).reshape(-1, 31)
        signs = rng.integers(0, 2, size=mags.shape, dtype=np.uint32) << 15
        body = (mags | signs).astype(np.uint16)
        head = np.full((body.shape[0], 1), anchor, np.uint16)
        head |= (rng.integers(0, 2, size=head.shape, dtype=np.uint16) << 15).astype(np.uint16)
        blk = np.concatenate([head, body], axis=1)
        # move the anchor to a seeded slot so every lane position holds it sometimes
        pos = rng.integers(0, 32, size=blk.shape[0])
        idx = np.arange(blk.shape[0])
        tmp = blk[idx, pos].copy()
        blk[idx, pos] = blk[idx, 0]
        blk[idx, 0] = tmp
        blocks.append(blk)
    return np.concatenate(blocks, axis=0)
