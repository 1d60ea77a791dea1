"""Pins of the oracle's exact per-token window attention (each query token
attends the key tiles of its own radius's window): reduction to the block
mask when every token of a tile carries the tile's radius, a pure-Python brute
force on a tiny grid written from the window rule itself, and the subset
relation with the block mask of the tiles' largest token radii."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import vsa_oracle as vo


def _draw(T, H, W, heads, D, seed):
    rng = np.random.default_rng(seed)
    N = T * H * W
    n = vo.num_tiles(T, H, W)
    q, k, v = (wl.f32_to_bf16_bits(rng.standard_normal((1, N, heads, D)).astype(np.float32))
               for _ in range(3))
    scores = rng.standard_normal((1, heads, n)).astype(np.float32)
    return q, k, v, scores


def test_reduces_to_block_mask_when_tiles_share_radius():
    T, H, W, heads, D = 6, 7, 9, 2, 16
    q, k, v, scores = _draw(T, H, W, heads, D, 1)
    n = vo.num_tiles(T, H, W)
    rng = np.random.default_rng(2)
    tile_r = rng.integers(0, 4, size=(1, heads, n)).astype(np.uint8)
    tok_r = tile_r[:, :, vo.token_tile(T, H, W)]          # every token: its tile's radius
    for kcount in (0, 3):
        o1, l1 = vo.token_window_attention(q, k, v, tok_r, scores, kcount, 3, T, H, W, 0.25)
        o2, l2 = vo.attention(q, k, v, tile_r, scores, kcount, T, H, W, 0.25)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_brute_force_tiny_grid():
    """Explicit loops over query and key tokens: key j is attended by query i
    iff i's tile is routed, or |dt| <= r and max(|dh|, |dw|) <= r - |dt| for
    the tile offsets and r = min(r_i, r_max)."""
    T, H, W, D, r_max, kcount = 5, 5, 6, 8, 2, 1
    q, k, v, scores = _draw(T, H, W, 1, D, 3)
    rng = np.random.default_rng(4)
    tok_r = rng.integers(0, 4, size=(1, 1, T * H * W)).astype(np.uint8)
    o_ref, l_ref = vo.token_window_attention(q, k, v, tok_r, scores, kcount, r_max, T, H, W, 0.3)
    qf, kf, vf = (vo.bf16_to_f64(x[0, :, 0]) for x in (q, k, v))
    nh, nw = -(-H // 4), -(-W // 4)
    # routed tile by sorting (score desc, index asc), NaN-free scores
    order = sorted(range(len(scores[0, 0])), key=lambda a: (-float(scores[0, 0, a]), a))
    routed = set(order[:kcount])
    coords = [(t, h, w) for t in range(T) for h in range(H) for w in range(W)]
    for i, (t, h, w) in enumerate(coords):
        a = ((t // 4) * nh + h // 4) * nw + w // 4
        r = min(int(tok_r[0, 0, i]), r_max)
        logits = []
        for j, (t2, h2, w2) in enumerate(coords):
            dt, dh, dw = abs(t2 // 4 - t // 4), abs(h2 // 4 - h // 4), abs(w2 // 4 - w // 4)
            if a in routed or (dt <= r and max(dh, dw) <= r - dt):
                logits.append((j, 0.3 * float(np.dot(qf[i], kf[j]))))
        m = max(s for _, s in logits)
        ps = [(j, math.exp(s - m)) for j, s in logits]
        z = sum(p for _, p in ps)
        o = sum(p * vf[j] for j, p in ps) / z
        assert np.allclose(o, o_ref[0, i, 0], rtol=0, atol=1e-12)
        assert abs((m + math.log(z)) - l_ref[0, 0, i]) < 1e-12


@pytest.mark.parametrize("T,H,W", [(9, 10, 11), (4, 4, 4), (13, 6, 5)])
def test_subset_of_the_tile_block_mask(T, H, W):
    """R21: the block mask built from each tile's largest token radius keeps a
    superset of every token's window, equal for the tokens holding that
    largest radius."""
    rng = np.random.default_rng(T * H * W)
    N, n = T * H * W, vo.num_tiles(T, H, W)
    tok_r = rng.integers(0, 5, size=N).astype(np.uint8)
    routed = rng.random(n) < 0.2
    r_max = 3
    keep_tok = vo.token_window_keep(tok_r, routed, r_max, T, H, W)
    tile_r = np.minimum(vo.tile_radius_from_tokens(tok_r, T, H, W), r_max)
    keep_tile = vo.tile_keep(tile_r, routed, T, H, W)
    tt = vo.token_tile(T, H, W)
    assert not np.any(keep_tok & ~keep_tile[tt])
    at_max = np.minimum(tok_r, r_max) == tile_r[tt]
    assert np.array_equal(keep_tok[at_max], keep_tile[tt[at_max]])
    assert np.all(keep_tok[routed[tt]])                     # routed: every key tile
    assert np.all(keep_tok[np.arange(N), tt])               # own tile always kept
