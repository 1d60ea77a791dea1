"""Fit the routed-tile count of the HunyuanVideo-shaped call (test infrastructure).

The HunyuanVideo 720p 129-frame call is run at a routed count chosen so that
about 10% of all (query tile, key tile) pairs are retained -- the low end of
the retained density that "Token Radius Attention for Efficient Video
Generation" reports (results paragraph: 9-19% of interactions).  One count k
serves every head; it is the integer in [0, nT] whose mean-over-heads retained
density is closest to 0.10 (the smaller k on a tie), with the radii and scores
that ``workloads`` draws for that call.  Only the oracle's arithmetic is used.

Run ``python -m oracle.fit_dense_count`` to print the count; the value is kept
as ``workloads.HUNYUAN_FITTED_DENSE_COUNT`` and re-checked by a CPU test.
"""
from __future__ import annotations

import numpy as np

from oracle import vsa_oracle as vo


def density_by_count(radii: np.ndarray, scores: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """Mean-over-heads retained tile-pair density for every k in [0, nT]."""
    B, Hh, n = radii.shape
    total = np.zeros(n + 1)
    for b in range(B):
        for h in range(Hh):
            local = vo.tile_keep(radii[b, h], np.zeros(n, bool), T, H, W).sum(axis=1)
            # the k-th routed tile is the k-th in routing order
            order = vo.routing_order(scores[b, h])
            gain = np.concatenate([[0], np.cumsum(n - local[order])])
            total += (local.sum() + gain) / float(n * n)
    return total / (B * Hh)


def fit(radii, scores, T, H, W, target: float = 0.10) -> int:
    d = density_by_count(radii, scores, T, H, W)
    return int(np.argmin(np.abs(d - target)))


def main():
    import workloads as wl
    w = wl.WORKLOADS[4]
    r, s = wl.radii_scores(w)
    d = density_by_count(r, s, w.T, w.H, w.W)
    k = int(np.argmin(np.abs(d - 0.10)))
    print(f"{w.name}: fitted routed count k={k} density={d[k]:.5f} (k=0: {d[0]:.5f})")


if __name__ == "__main__":
    main()
