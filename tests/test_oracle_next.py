"""Pins of the oracle's token-level input functions: budget -> radius per
query token, token radii -> tile radius, token scores -> tile score.  All on
the CPU: hand-worked fixtures, an independent closed form of the window's
token count, pure-Python tile assignment, and invariants."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import vsa_oracle as vo


def _tile_of(t, h, w, H, W):
    """Tile index by integer division, written independently of token_tile."""
    nh, nw = -(-H // 4), -(-W // 4)
    return ((t // 4) * nh + h // 4) * nw + w // 4


def _window_tokens_closed(r, T, H, W):
    """Real key tokens in each query tile's window: the sum over dt of the
    clipped token extents along t, h and w (no tile_keep matrix)."""
    a, b, c = vo.tile_grid(T, H, W)

    def span(X, lo, hi):
        n = -(-X // 4)
        lo, hi = max(lo, 0), min(hi, n - 1)
        return max(0, min(X, 4 * (hi + 1)) - 4 * lo)

    out = []
    for tt in range(a):
        for th in range(b):
            for tw in range(c):
                tot = 0
                for dt in range(-r, r + 1):
                    if 0 <= tt + dt < a:
                        s = r - abs(dt)
                        tot += span(T, tt + dt, tt + dt) * span(H, th - s, th + s) * span(W, tw - s, tw + s)
                out.append(tot)
    return out


@pytest.mark.parametrize("T,H,W", [(8, 16, 16), (21, 30, 52), (5, 4, 6), (1, 1, 1), (9, 5, 3)])
def test_tile_valid_tokens_by_extent(T, H, W):
    a, b, c = vo.tile_grid(T, H, W)
    ext = lambda X, i: min(4, X - 4 * i)
    expect = [ext(T, i) * ext(H, j) * ext(W, k) for i in range(a) for j in range(b) for k in range(c)]
    got = vo.tile_valid_tokens(T, H, W)
    assert got.tolist() == expect
    assert got.sum() == T * H * W


@pytest.mark.parametrize("T,H,W", [(8, 16, 16), (21, 30, 52), (5, 4, 6), (9, 5, 3), (13, 6, 10)])
def test_window_tokens_brute_force_vs_closed_form(T, H, W):
    for r in range(5):
        assert vo.window_tokens(r, T, H, W).tolist() == _window_tokens_closed(r, T, H, W)


def test_window_tokens_interior_tile():
    T = H = W = 28                      # 7^3 full tiles, centre unclipped up to r = 3
    centre = (3 * 7 + 3) * 7 + 3
    for r, tiles in enumerate((1, 11, 45, 119)):  # hand-worked, see window_counts.txt
        assert vo.window_tokens(r, T, H, W)[centre] == 64 * tiles


def test_budget_to_radius_golden():
    _, rows = read_golden("budget_radius.txt")
    grid = None
    for row in rows:
        if row[0] in ("gridA", "gridB"):
            grid = tuple(int(x) for x in row[1:])
            continue
        T, H, W, r_max = grid
        N = T * H * W
        if row[0] == "a":
            budget, want = int(row[1]), int(row[2])
            got = vo.budget_to_radius(np.full(N, budget), r_max, T, H, W)
            assert (got == want).all(), (row, np.unique(got))
        else:
            t, h, w, budget, want = (int(x) for x in row[1:])
            b = np.zeros(N, dtype=np.int64)
            n = (t * H + h) * W + w
            b[n] = budget
            assert vo.budget_to_radius(b, r_max, T, H, W)[n] == want, row


@pytest.mark.parametrize("T,H,W,r_max", [(9, 5, 3, 4), (13, 6, 10, 3), (5, 4, 6, 6)])
def test_budget_to_radius_is_the_smallest_sufficient(T, H, W, r_max):
    rng = np.random.default_rng(7)
    N = T * H * W
    budget = rng.integers(0, N + 2, size=N)
    r = vo.budget_to_radius(budget, r_max, T, H, W).astype(int)
    counts = np.array([_window_tokens_closed(k, T, H, W) for k in range(r_max + 1)])
    tile = np.array([_tile_of(t, h, w, H, W) for t in range(T) for h in range(H) for w in range(W)])
    for n in range(N):
        c = counts[:, tile[n]]
        if c[r_max] < budget[n]:
            assert r[n] == r_max
        else:
            assert c[r[n]] >= budget[n]
            assert r[n] == 0 or c[r[n] - 1] < budget[n]
    # monotone in the budget within a tile
    order = np.lexsort((budget, tile))
    for a_, b_ in zip(order[:-1], order[1:]):
        if tile[a_] == tile[b_]:
            assert r[a_] <= r[b_]


@pytest.mark.parametrize("T,H,W", [(5, 4, 6), (9, 5, 3), (8, 8, 8), (1, 1, 1)])
def test_tile_radius_is_max_over_real_tokens(T, H, W):
    rng = np.random.default_rng(11)
    N = T * H * W
    x = rng.integers(0, 256, size=N).astype(np.uint8)
    want = [0] * vo.num_tiles(T, H, W)
    n = 0
    for t in range(T):
        for h in range(H):
            for w in range(W):
                a = _tile_of(t, h, w, H, W)
                want[a] = max(want[a], int(x[n]))
                n += 1
    assert vo.tile_radius_from_tokens(x, T, H, W).tolist() == want


def test_tile_score_total_order_golden():
    # grid T=5, H=4, W=6: tiles 0:(0,0,0) 64 tokens, 1:(0,0,1) 32, 2:(1,0,0) 16, 3:(1,0,1) 8
    T, H, W = 5, 4, 6
    N = T * H * W
    s = np.full(N, -1.0, dtype=np.float32)

    def at(t, h, w, v):
        s[(t * H + h) * W + w] = v

    at(0, 0, 0, 0.25); at(3, 3, 3, 0.75)            # tile 0 -> 0.75
    at(1, 1, 5, -0.0)                                # tile 1: -0 vs -1 -> -0
    at(4, 0, 0, np.inf); at(4, 3, 3, 1e30)          # tile 2 -> +inf
    at(4, 2, 4, np.float32("nan"))                  # tile 3: +NaN above +inf
    got = vo.tile_score_from_tokens(s, T, H, W)
    assert got[0] == np.float32(0.75)
    assert got[1] == 0.0 and np.signbit(got[1])
    assert got[2] == np.inf
    assert np.isnan(got[3]) and not np.signbit(got[3])
    # +0 beats -0 in the total order
    at(0, 2, 4, 0.0)
    assert not np.signbit(vo.tile_score_from_tokens(s, T, H, W)[1])


@pytest.mark.parametrize("T,H,W", [(5, 4, 6), (9, 5, 3), (8, 8, 8)])
def test_tile_score_is_max_over_real_tokens(T, H, W):
    rng = np.random.default_rng(13)
    N = T * H * W
    x = rng.standard_normal(N).astype(np.float32)
    want = [-np.inf] * vo.num_tiles(T, H, W)
    n = 0
    for t in range(T):
        for h in range(H):
            for w in range(W):
                a = _tile_of(t, h, w, H, W)
                want[a] = max(want[a], float(x[n]))
                n += 1
    assert np.array_equal(vo.tile_score_from_tokens(x, T, H, W), np.array(want, dtype=np.float32))
