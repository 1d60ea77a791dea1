"""Pure-Python brute force of block-sparse video attention, for tiny grids.

A second, independent writing of the same definition as ``vsa_oracle`` (which
it must not import): every quantity is derived token by token from the grid
coordinates with plain loops and ``math``, no numpy.  Used by the CPU tests to
pin ``vsa_oracle``.  Test infrastructure only.

Definition (see ``vsa_oracle`` for the sources): 4x4x4 tiles, tiles numbered
in raster order over the tile grid; query tile a with radius r keeps key tile
b iff |dt| <= r and max(|dh|, |dw|) <= r - |dt| (tile units), or a is one of
the k routed tiles (highest score in IEEE total order, lower index on ties);
attention is softmax(scale * q.k) over kept keys.
"""
from __future__ import annotations

import math
import struct


def _tiles_along(x: int) -> int:
    n = 0
    while 4 * n < x:
        n += 1
    return n


def _order_key(f: float) -> int:
    (u,) = struct.unpack("<I", struct.pack("<f", f))
    if u & 0x80000000:
        return (~u) & 0xFFFFFFFF
    return u | 0x80000000


def routed(scores, k):
    """List of bools: tile i is routed iff fewer than k tiles rank before it."""
    n = len(scores)
    keys = [_order_key(s) for s in scores]
    out = []
    for i in range(n):
        ahead = 0
        for j in range(n):
            if keys[j] > keys[i] or (keys[j] == keys[i] and j < i):
                ahead += 1
        out.append(ahead < k)
    return out


def tile_of(t, h, w, T, H, W):
    nh, nw = _tiles_along(H), _tiles_along(W)
    return ((t // 4) * nh + (h // 4)) * nw + (w // 4)


def keeps(ta, tb, radius, is_routed, T, H, W):
    """Does query tile ta keep key tile tb."""
    if is_routed:
        return True
    nh, nw = _tiles_along(H), _tiles_along(W)
    at, ah, aw = ta // (nh * nw), (ta // nw) % nh, ta % nw
    bt, bh, bw = tb // (nh * nw), (tb // nw) % nh, tb % nw
    dt = abs(at - bt)
    ds = max(abs(ah - bh), abs(aw - bw))
    return dt <= radius and ds <= radius - dt


def csr(radii, scores, k, T, H, W):
    """radii / scores: [heads][nT] lists.  Returns (row_ptr, col_idx) lists, rows
    ordered (head, query tile), columns ascending."""
    n = _tiles_along(T) * _tiles_along(H) * _tiles_along(W)
    row_ptr, cols = [0], []
    for h in range(len(radii)):
        rt = routed(scores[h], k)
        for a in range(n):
            for b in range(n):
                if keeps(a, b, radii[h][a], rt[a], T, H, W):
                    cols.append(b)
            row_ptr.append(len(cols))
    return row_ptr, cols


def attention(q, kk, v, radii, scores, k, T, H, W, scale):
    """q, kk, v: [N][heads][D] nested lists of floats (token raster order).
    Returns (O [N][heads][D], LSE [heads][N])."""
    N = T * H * W
    heads = len(radii)
    D = len(q[0][0])
    coords = []
    for t in range(T):
        for h in range(H):
            for w in range(W):
                coords.append((t, h, w))
    tiles = [tile_of(t, h, w, T, H, W) for (t, h, w) in coords]
    O = [[[0.0] * D for _ in range(heads)] for _ in range(N)]
    LSE = [[0.0] * N for _ in range(heads)]
    for hd in range(heads):
        rt = routed(scores[hd], k)
        for i in range(N):
            ti = tiles[i]
            s = []
            for j in range(N):
                if keeps(ti, tiles[j], radii[hd][ti], rt[ti], T, H, W):
                    dot = 0.0
                    for d in range(D):
                        dot += q[i][hd][d] * kk[j][hd][d]
                    s.append((j, scale * dot))
            m = max(x for _, x in s)
            den = 0.0
            acc = [0.0] * D
            for j, x in s:
                e = math.exp(x - m)
                den += e
                for d in range(D):
                    acc[d] += e * v[j][hd][d]
            O[i][hd] = [a / den for a in acc]
            LSE[hd][i] = m + math.log(den)
    return O, LSE


def permute_slots(T, H, W):
    """Tile-major slot -> raster token index (or -1 for a padded slot), by
    walking tiles and the 64 positions inside each tile."""
    nt, nh, nw = _tiles_along(T), _tiles_along(H), _tiles_along(W)
    out = []
    for tt in range(nt):
        for th in range(nh):
            for tw in range(nw):
                for lt in range(4):
                    for lh in range(4):
                        for lw in range(4):
                            t, h, w = 4 * tt + lt, 4 * th + lh, 4 * tw + lw
                            if t < T and h < H and w < W:
                                out.append((t * H + h) * W + w)
                            else:
                                out.append(-1)
    return out
