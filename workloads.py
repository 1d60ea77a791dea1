"""Seeded synthetic workloads for block-sparse video attention.

This module only draws inputs.  It holds none of the method's arithmetic (no
tile ordering, no window rule, no routing, no attention): both the CPU oracle
and the HIP path consume what it returns, and neither is imported here.

Shapes follow the video-DiT attention calls that the sparse-attention pages
measure on (Wan2.1-1.3B / Wan2.1-14B / Wan2.2-5B / HunyuanVideo latent grids;
"Token Radius Attention for Efficient Video Generation", results paragraph).
No dataset, prompt or trained weight is involved; these arrays stand in for
the Q/K/V activations of those models.

Recipe (per config ``c`` and head ``h``; every stream is its own
``numpy.random.default_rng([19, c, stream, h])`` so heads can be drawn in any
order or in chunks):

* stream 0: ``g`` ~ N(0, 1) of shape [nTt, nTh, nTw, D], one vector per 4x4x4
  cell of the latent grid, repeated over the cell's tokens and cropped to the
  T x H x W grid (so tokens of one cell share it);
* stream 1 / 2: independent N(0, 1) noise for Q / K;  Q = g + 0.5 n_q,
  K = g + 0.5 n_k  (the shared ``g`` gives keys near a query in the grid a
  larger dot product, i.e. local attention mass);
* stream 3: V ~ N(0, 1);
* stream 4: one radius per cell, discrete-uniform over the config's set;
* stream 5: one routing score per cell, U[0, 1) drawn in float64, stored float32;
* streams 6 / 7: per-token key budgets and routing scores (``token_inputs``);
* streams 8 / 9: skim tiers, per kept pair or per key tile (``tiers``,
  ``tiers_by_key_tile``).

Q/K/V are drawn in float32 and rounded to bfloat16 (round to nearest even);
they are returned as uint16 bit patterns, token-raster order
``n = (t*H + h)*W + w``, layout [B=1, N, heads, D].
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, Optional, Tuple

import numpy as np

SEED = 19
CELL = 4  # edge of the cubic cell that ``g``, radii and scores are drawn per


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    T: int
    H: int
    W: int
    heads: int
    D: int
    radius_set: Tuple[int, ...]
    dense_counts: Tuple[int, ...]  # routing sweep; first entry is the headline point
    batch: int = 1

    @property
    def grid_cells(self) -> Tuple[int, int, int]:
        return (-(-self.T // CELL), -(-self.H // CELL), -(-self.W // CELL))

    @property
    def n_cells(self) -> int:
        a, b, c = self.grid_cells
        return a * b * c

    @property
    def tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


def count_from_fraction(frac: float, n_cells: int) -> int:
    """Number of routed cells for a routed fraction: nearest integer, halves up."""
    return int(math.floor(frac * n_cells + 0.5))


# Routed count for the HunyuanVideo-shaped call, chosen so that about 10% of
# all tile pairs are retained with the radii this generator draws.  It is
# written by ``oracle/fit_dense_count.py`` (which uses only the oracle) and
# re-checked by a CPU test.
HUNYUAN_FITTED_DENSE_COUNT = 144


def _mk() -> Dict[int, Workload]:
    out = {}
    out[0] = Workload(0, "tiny-8x16x16", 8, 16, 16, 2, 64, (1, 2, 3),
                      (count_from_fraction(0.2, 2 * 4 * 4),))
    out[1] = Workload(1, "wan2.1-1.3b-480p", 21, 30, 52, 12, 128, (1, 2, 3),
                      (count_from_fraction(0.2, 6 * 8 * 13),))
    nt2 = 8 * 6 * 10
    out[2] = Workload(2, "wan2.2-5b-720p", 31, 22, 40, 24, 128, (1, 2, 3, 4),
                      tuple(count_from_fraction(f, nt2) for f in (0.2, 0.0, 0.1, 0.4, 1.0)))
    out[3] = Workload(3, "wan2.1-14b-720p", 21, 45, 80, 40, 128, (1, 2, 3),
                      (count_from_fraction(0.2, 6 * 12 * 20),))
    out[4] = Workload(4, "hunyuanvideo-720p-129f", 33, 45, 80, 24, 128, (1, 2, 3, 4),
                      (HUNYUAN_FITTED_DENSE_COUNT, 9 * 12 * 20))
    return out


WORKLOADS: Dict[int, Workload] = _mk()


def custom(T: int, H: int, W: int, heads: int, D: int, radius_set=(1, 2, 3),
           dense_counts=(0,), cid: int = 100, name: str = "custom") -> Workload:
    """A workload of any grid, for edge cases (ragged grids, tiny grids)."""
    return Workload(cid, name, T, H, W, heads, D, tuple(radius_set), tuple(dense_counts))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (((b >> 16) & 1) + np.uint32(0x7FFF))
    return (b >> 16).astype(np.uint16)


def _rng(w: Workload, stream: int, head: int) -> np.random.Generator:
    return np.random.default_rng([SEED, w.cid, stream, head])


def head_qkv(w: Workload, head: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V of one head as bf16 bit patterns, each [N, D], token-raster order."""
    a, b, c = w.grid_cells
    D = w.D
    g = _rng(w, 0, head).standard_normal((a, b, c, D), dtype=np.float32)
    g = np.repeat(np.repeat(np.repeat(g, CELL, 0), CELL, 1), CELL, 2)[: w.T, : w.H, : w.W]
    g = g.reshape(-1, D)
    nq = _rng(w, 1, head).standard_normal(g.shape, dtype=np.float32)
    q = f32_to_bf16_bits(g + np.float32(0.5) * nq)
    del nq
    nk = _rng(w, 2, head).standard_normal(g.shape, dtype=np.float32)
    k = f32_to_bf16_bits(g + np.float32(0.5) * nk)
    del nk
    v = f32_to_bf16_bits(_rng(w, 3, head).standard_normal(g.shape, dtype=np.float32))
    return q, k, v


def head_radii(w: Workload, head: int) -> np.ndarray:
    lo, hi = min(w.radius_set), max(w.radius_set)
    assert tuple(range(lo, hi + 1)) == tuple(sorted(w.radius_set))
    return _rng(w, 4, head).integers(lo, hi + 1, size=w.n_cells).astype(np.uint8)


def head_scores(w: Workload, head: int) -> np.ndarray:
    return _rng(w, 5, head).random(w.n_cells).astype(np.float32)


def radii_scores(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Radii uint8 [B, heads, nT] and routing scores float32 [B, heads, nT]."""
    r = np.stack([head_radii(w, h) for h in range(w.heads)])[None]
    s = np.stack([head_scores(w, h) for h in range(w.heads)])[None]
    return np.ascontiguousarray(r), np.ascontiguousarray(s)


# Per-token inputs of the token-level calls (budget -> radius, token radii /
# scores -> tile radii / scores): stream 6 draws key budgets discrete-uniform
# over [TOKEN_BUDGET_LO, TOKEN_BUDGET_HI] (roughly the key tokens of windows up
# to radius 3 of an interior tile), stream 7 draws routing scores U[0, 1) in
# float64, stored float32.  Layout [B=1, heads, N], raster token order.
TOKEN_BUDGET_LO = 1
TOKEN_BUDGET_HI = 8192


def token_inputs(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Key budgets int32 [1, heads, N] and routing scores float32 [1, heads, N]."""
    b = np.stack([_rng(w, 6, h).integers(TOKEN_BUDGET_LO, TOKEN_BUDGET_HI + 1, size=w.tokens)
                  for h in range(w.heads)])[None].astype(np.int32)
    s = np.stack([_rng(w, 7, h).random(w.tokens).astype(np.float32) for h in range(w.heads)])[None]
    return np.ascontiguousarray(b), np.ascontiguousarray(s)


# Tiers of the low-precision "skim" path: one byte per kept (query tile, key
# tile) pair in CSR order, 1 (skim) with probability p_skim, drawn i.i.d. by
# stream 8.  The pages' router (estimated error per tile) has no formulas, so
# a fixed skim fraction stands in for it.
def tiers(w: Workload, nnz: int, p_skim: float = 0.5) -> np.ndarray:
    """uint8 [nnz]: 1 = skim, 0 = refine."""
    return (_rng(w, 8, 0).random(nnz) < p_skim).astype(np.uint8)


# A second recipe: the router's decision for a pair taken from statistics of
# its key tile alone (say, the error of that tile's 4-bit K), so every query
# tile of a head gives one key tile the same tier.  Stream 9 draws one U[0, 1)
# per (batch-head, key tile); a pair skims if its key tile's draw is below
# p_skim.  I.i.d. tiers are the other extreme: two query tiles agree on a key
# tile only by chance.
def tiers_by_key_tile(w: Workload, row_ptr: np.ndarray, col_idx: np.ndarray,
                      p_skim: float = 0.5) -> np.ndarray:
    """uint8 [nnz] in CSR order (rows are batch-head-major query tiles)."""
    nT = w.n_cells
    rp = np.asarray(row_ptr, dtype=np.int64)
    nnz = int(rp[-1])
    u = _rng(w, 9, 0).random((rp.size - 1) // nT * nT)
    bh = np.repeat(np.arange(rp.size - 1) // nT, np.diff(rp))
    return (u[bh * nT + np.asarray(col_idx[:nnz], dtype=np.int64)] < p_skim).astype(np.uint8)


def qkv(w: Workload, heads: Optional[range] = None):
    """Q, K, V as bf16 bit patterns, each [B=1, N, heads, D] (uint16)."""
    hs = range(w.heads) if heads is None else heads
    N, D = w.tokens, w.D
    q = np.empty((1, N, len(hs), D), np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def one(j_h):
        j, h = j_h
        q[0, :, j], k[0, :, j], v[0, :, j] = head_qkv(w, h)

    # heads are independent streams: draw them on a few threads (numpy's
    # generators release the GIL while filling arrays)
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(hs)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, enumerate(hs)))
    return q, k, v
