"""Seeded synthetic inputs for one MoE layer (router logits, biases, activations,
expert weights).

This module serves both the oracle tests and the HIP path and therefore holds
none of the layer's own arithmetic: no top-k, no counting, no planning, no
GEMM. It only draws numbers.

Recipes (the same for every caller):
  * router logits: N(0, 1) float32 from numpy's PCG64 stream of the given seed;
  * Zipf-shaped expert bias: bias_e = -s * ln(1 + pi(e)), pi a seeded
    permutation of the experts (s = 0 gives no bias);
  * fixed-count modes: the 16-token hotspot fixture's expert pairs, and an
    exactly even mode where token t prefers experts (t*k + j) mod E;
  * activations and weights on the device: N(0, 1) * std drawn with torch's
    device generator seeded per tensor (std = 1/sqrt(fan_in) for weights),
    rounded to the requested dtype. Host copies for checking come from these.
"""
from __future__ import annotations

import math

import numpy as np

# Expert pairs of the 16-token hotspot fixture ("MoE Load Balancing: Find
# Expert Hotspots", section "Work the 16-token hotspot fixture"): tokens t00..t15,
# first expert then second expert, origin rank t mod 4, E = 8, k = 2.
FIXTURE_PAIRS = ((0, 1), (0, 2), (0, 3), (0, 4), (0, 5), (0, 6), (0, 7), (0, 1),
                 (0, 2), (1, 2), (1, 2), (1, 2), (1, 3), (3, 4), (3, 4), (5, 6))


def router_logits(T: int, E: int, seed: int) -> np.ndarray:
    """N(0,1) float32 logits [T, E] from a PCG64 stream seeded with `seed`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((T, E), dtype=np.float32)


def expert_permutation(E: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    return rng.permutation(E).astype(np.int64)


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Per-expert bias -s * ln(1 + rank), rank a seeded permutation of 0..E-1."""
    pi = expert_permutation(E, seed)
    return (-float(s) * np.log1p(pi.astype(np.float64))).astype(np.float32)


def fixture_logits() -> np.ndarray:
    """Logits [16, 8] whose top-2 are the fixture's pairs, first expert first:
    2 for the first expert, 1 for the second, 0 elsewhere."""
    lg = np.zeros((len(FIXTURE_PAIRS), 8), np.float32)
    for t, (a, b) in enumerate(FIXTURE_PAIRS):
        lg[t, a] = 2.0
        lg[t, b] = 1.0
    return lg


def even_logits(T: int, E: int, k: int, seed: int) -> np.ndarray:
    """Exactly even demand: token t strongly prefers experts (t*k + j) mod E,
    j < k, with a 0.1 step between them; all logits carry 0.01 * N(0,1)."""
    z = router_logits(T, E, seed) * np.float32(0.01)
    t = np.arange(T)[:, None]
    j = np.arange(k)[None, :]
    cols = (t * k + j) % E
    z[np.broadcast_to(t, cols.shape), cols] += (8.0 - 0.1 * j).astype(np.float32)
    return z


def host_normal(shape, std: float, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def device_normal(shape, std: float, seed: int, dtype, device, chunk_rows: int | None = None):
    """N(0,1)*std tensor on `device`, drawn by torch's generator for that device
    seeded with `seed`, in fp32 and rounded to `dtype`. Large tensors are drawn
    in chunks along dim 0 (each chunk seeded seed*65537 + chunk) to bound the
    fp32 staging memory."""
    import torch

    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    if chunk_rows is None:
        chunk_rows = max(1, (1 << 26) // max(per_row, 1))
    g = torch.Generator(device=device)
    for c, r0 in enumerate(range(0, rows, chunk_rows)):
        r1 = min(rows, r0 + chunk_rows)
        g.manual_seed(int(seed) * 65537 + c)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        out[r0:r1].copy_(tmp)
        del tmp
    return out


def weight_std(fan_in: int) -> float:
    return 1.0 / math.sqrt(fan_in)
