"""Pins of the CPU oracle against things other than itself: hand-worked golden
fixtures, brute force, closed forms, textbook attention and invariants.

Every test here runs on the CPU (no GPU marker)."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from conftest import read_golden
from oracle import brute
from oracle import vsa_oracle as vo


def _inputs(T, H, W, heads, D, radius_set=(0, 1, 2), cid=200):
    w = wl.custom(T, H, W, heads, D, radius_set=radius_set, cid=cid)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    return w, q, k, v, r, s


def _nested(bits):  # [1, N, Hh, D] bf16 bits -> nested python floats [N][Hh][D]
    return vo.bf16_to_f64(bits[0]).tolist()


# ------------------------------------------------------------ golden fixtures

def test_window_counts_golden():
    _, rows = read_golden("window_counts.txt")
    T = H = W = 4 * 11                     # 11^3 tiles, centre (5,5,5) unclipped
    n = vo.num_tiles(T, H, W)
    centre = (5 * 11 + 5) * 11 + 5
    for r, cnt in rows:
        keep = vo.tile_keep(np.full(n, int(r)), np.zeros(n, bool), T, H, W)
        assert keep[centre].sum() == int(cnt)
        assert vo.window_count_closed_form(int(r)) == int(cnt)


def test_csr_small_golden():
    g, _ = read_golden("csr_small.txt")
    T, H, W = int(g["T"][0]), int(g["H"][0]), int(g["W"][0])
    radii = np.array([int(x) for x in g["radii"]])[None, None]
    scores = np.array([float(x) for x in g["scores"]], np.float32)[None, None]
    keep, routed = vo.block_mask(radii, scores, int(g["k"][0]), T, H, W)
    rp, ci = vo.csr(keep)
    assert rp.tolist() == [int(x) for x in g["row_ptr"]]
    assert ci.tolist() == [int(x) for x in g["col_idx"]]
    assert routed[0, 0].tolist() == [False, True, False, False, False, False]


def test_topk_golden():
    g, _ = read_golden("topk_order.txt")
    scores = np.array([float(x) for x in g["scores"]], np.float32)
    order = [int(x) for x in g["order"]]
    assert vo.routing_order(scores).tolist() == order
    for k in range(len(order) + 1):
        assert set(np.flatnonzero(vo.routed_tiles(scores, k)).tolist()) == set(order[:k])
    with pytest.raises(ValueError):
        vo.routed_tiles(scores, len(order) + 1)


def test_permute_golden():
    g, _ = read_golden("permute_head.txt")
    T, H, W = int(g["T"][0]), int(g["H"][0]), int(g["W"][0])
    slots = [int(x) for x in g["slots"]]
    N = T * H * W
    x = (np.arange(N, dtype=np.int64) + 1).reshape(1, N, 1, 1)   # token n -> n+1; pad -> 0
    xt = vo.permute(x, T, H, W)[0, 0, :, 0]
    assert (xt[: len(slots)] - 1).tolist() == slots


# --------------------------------------------------------------- routing

@pytest.mark.parametrize("seed", range(6))
def test_topk_vs_brute(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    pool = np.array([0.25, 0.5, 0.5, -0.0, 0.0, np.inf, -np.inf, np.nan, 1.0, -1.0], np.float32)
    scores = rng.choice(pool, size=n).astype(np.float32)
    if seed % 2:
        scores = rng.random(n).astype(np.float32)
        scores[rng.integers(0, n, size=n // 3)] = scores[0]      # forced ties
    for k in range(n + 1):
        assert vo.routed_tiles(scores, k).tolist() == brute.routed(scores.tolist(), k)


def test_total_order_key_monotone():
    vals = np.array([-np.inf, -3.0, -1e-40, -0.0, 0.0, 1e-40, 2.0, np.inf], np.float32)
    keys = vo.total_order_key(vals)
    assert np.all(np.diff(keys.astype(np.int64)) > 0)
    nan = np.array([np.nan], np.float32)
    assert vo.total_order_key(nan)[0] > keys[-1]
    assert vo.total_order_key(-nan)[0] < keys[0]


# -------------------------------------------------------------- CSR / window

GRIDS = [(5, 6, 7), (4, 4, 4), (9, 5, 3), (1, 1, 1), (13, 9, 17)]


@pytest.mark.parametrize("T,H,W", GRIDS)
def test_csr_vs_brute(T, H, W):
    w, q, k, v, r, s = _inputs(T, H, W, 2, 8, radius_set=(0, 1, 2, 3))
    n = vo.num_tiles(T, H, W)
    for kk in sorted({0, 1, n // 2, n}):
        keep, _ = vo.block_mask(r, s, kk, T, H, W)
        rp, ci = vo.csr(keep)
        brp, bci = brute.csr(r[0].tolist(), s[0].tolist(), kk, T, H, W)
        assert rp.tolist() == brp and ci.tolist() == bci


def _clipped_len(coord, r, grid):
    """Row length by the product-of-clipped-ranges rule, dt by dt."""
    tt, th, tw = coord
    a, b, c = grid
    total = 0
    for dt in range(-r, r + 1):
        if not 0 <= tt + dt < a:
            continue
        s = r - abs(dt)
        nh = min(th + s, b - 1) - max(th - s, 0) + 1
        nw = min(tw + s, c - 1) - max(tw - s, 0) + 1
        total += nh * nw
    return total


@pytest.mark.parametrize("cid", [0, 1, 2])
def test_csr_invariants_workloads(cid):
    w = wl.WORKLOADS[cid]
    r, s = wl.radii_scores(w)
    r, s = r[:, :3], s[:, :3]
    n = w.n_cells
    grid = vo.tile_grid(w.T, w.H, w.W)
    coords = vo.tile_coords(w.T, w.H, w.W)
    k = w.dense_counts[0]
    keep, routed = vo.block_mask(r, s, k, w.T, w.H, w.W)
    rp, ci = vo.csr(keep)
    for h in range(r.shape[1]):
        assert routed[0, h].sum() == k
        for a in range(n):
            row = ci[rp[h * n + a]: rp[h * n + a + 1]]
            assert np.all(np.diff(row) > 0)
            assert a in row
            if routed[0, h, a]:
                assert len(row) == n
            else:
                assert len(row) == _clipped_len(coords[a], int(r[0, h, a]), grid)


def test_csr_symmetric_uniform_radius():
    T, H, W = 17, 13, 22
    n = vo.num_tiles(T, H, W)
    for rad in range(4):
        keep = vo.tile_keep(np.full(n, rad), np.zeros(n, bool), T, H, W)
        assert np.array_equal(keep, keep.T)
        assert keep.diagonal().all()


def test_fitted_dense_count():
    from oracle import fit_dense_count
    w = wl.WORKLOADS[4]
    r, s = wl.radii_scores(w)
    assert fit_dense_count.fit(r, s, w.T, w.H, w.W) == wl.HUNYUAN_FITTED_DENSE_COUNT


@pytest.mark.parametrize("T,H,W,rset", [(9, 10, 11, (1, 2, 3, 4)), (13, 9, 17, (0, 1, 2, 3))])
def test_density_by_count_vs_block_mask(T, H, W, rset):
    """The incremental density of fit_dense_count (each further routed tile adds
    its missing key tiles) equals the density of the mask built from scratch,
    for every routed count."""
    from oracle import fit_dense_count
    w = wl.custom(T, H, W, 3, 64, radius_set=rset, cid=310 + T)
    r, s = wl.radii_scores(w)
    d = fit_dense_count.density_by_count(r, s, T, H, W)
    n = vo.num_tiles(T, H, W)
    assert d.shape == (n + 1,)
    for k in range(n + 1):
        keep, _ = vo.block_mask(r, s, k, T, H, W)
        assert d[k] == pytest.approx(keep.mean(), abs=1e-13), k
    assert np.all(np.diff(d) >= 0)


def test_density_by_count_vs_brute():
    """The same against the pure-Python CSR on a tiny ragged grid, every k."""
    from oracle import fit_dense_count
    T, H, W = 5, 9, 6
    w = wl.custom(T, H, W, 2, 64, radius_set=(0, 1, 2), cid=320)
    r, s = wl.radii_scores(w)
    d = fit_dense_count.density_by_count(r, s, T, H, W)
    n = vo.num_tiles(T, H, W)
    for k in range(n + 1):
        rp, _ = brute.csr(r[0].tolist(), s[0].tolist(), k, T, H, W)
        assert d[k] == pytest.approx(rp[-1] / (2 * n * n), abs=1e-13), k


def test_fitted_dense_count_direct():
    """HunyuanVideo-shaped call: the retained density of the masks built at
    k = 143, 144, 145 routed tiles (straight from the keep rule), and 144 the
    count closest to 10% (density grows with k, so the closest count is one of
    the two around the crossing)."""
    w = wl.WORKLOADS[4]
    r, s = wl.radii_scores(w)
    dens = {}
    for k in (143, 144, 145):
        keep, _ = vo.block_mask(r, s, k, w.T, w.H, w.W)
        dens[k] = keep.mean()
    assert round(dens[143], 5) == 0.09968
    assert round(dens[144], 5) == 0.10012
    assert round(dens[145], 5) == 0.10057
    assert dens[143] < 0.10 <= dens[144]
    assert min(dens, key=lambda k: abs(dens[k] - 0.10)) == wl.HUNYUAN_FITTED_DENSE_COUNT


# ---------------------------------------------------------------- permute

@pytest.mark.parametrize("T,H,W", GRIDS + [(8, 16, 16), (21, 30, 52)])
def test_permute_vs_brute_slots(T, H, W):
    N = T * H * W
    x = (np.arange(N, dtype=np.int64) + 1).reshape(1, N, 1, 1)
    xt = vo.permute(x, T, H, W)[0, 0, :, 0] - 1
    assert xt.tolist() == brute.permute_slots(T, H, W)
    # transposed-tile variant carries the same slots, feature-major per tile
    x2 = np.stack([x, -x], axis=-1)[..., 0, :]                # D = 2
    xv = vo.permute(x2, T, H, W, transposed=True)[0, 0]       # [nT, 2, 64]
    assert np.array_equal(xv[:, 0, :].ravel() - 1, xt)
    assert np.array_equal(-xv[:, 1, :].ravel() - 1, xt)


@pytest.mark.parametrize("T,H,W", GRIDS)
def test_permute_roundtrip(T, H, W):
    rng = np.random.default_rng(T * 100 + H * 10 + W)
    x = rng.integers(1, 2 ** 15, size=(2, T * H * W, 3, 5)).astype(np.uint16)
    xt = vo.permute(x, T, H, W)
    assert xt.shape == (2, 3, vo.num_tiles(T, H, W) * 64, 5)
    assert np.array_equal(vo.unpermute(xt, T, H, W), x)
    # padded slots are zero and every token appears exactly once
    nz = (xt[0, 0, :, 0] != 0).sum()
    assert nz == T * H * W


# -------------------------------------------------------------- attention

@pytest.mark.parametrize("T,H,W,heads,D", [(5, 6, 7, 2, 8), (4, 4, 4, 1, 16), (9, 5, 3, 2, 8),
                                            (1, 1, 1, 1, 8)])
def test_attention_vs_brute(T, H, W, heads, D):
    w, q, k, v, r, s = _inputs(T, H, W, heads, D, radius_set=(0, 1, 2))
    n = vo.num_tiles(T, H, W)
    for kk in sorted({0, 1, n}):
        O, L = vo.attention(q, k, v, r, s, kk, T, H, W, 1 / math.sqrt(D))
        bO, bL = brute.attention(_nested(q), _nested(k), _nested(v), r[0].tolist(),
                                 s[0].tolist(), kk, T, H, W, 1 / math.sqrt(D))
        np.testing.assert_allclose(O[0], np.array(bO), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0], np.array(bL), rtol=1e-13, atol=1e-12)


def test_dense_equivalence_sdpa():
    """All tiles routed (or radii covering the grid) == textbook attention."""
    T, H, W, heads, D = 6, 7, 9, 2, 16
    w, q, k, v, r, s = _inputs(T, H, W, heads, D)
    n = vo.num_tiles(T, H, W)
    qf, kf, vf = (torch.from_numpy(vo.bf16_to_f64(x[0])).permute(1, 0, 2) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, scale=1 / math.sqrt(D))
    ref = ref.permute(1, 0, 2).numpy()
    O, L = vo.attention(q, k, v, r, s, n, T, H, W, 1 / math.sqrt(D))
    np.testing.assert_allclose(O[0], ref, rtol=0, atol=1e-12)
    big = np.full_like(r, 255)
    O2, _ = vo.attention(q, k, v, big, s, 0, T, H, W, 1 / math.sqrt(D))
    np.testing.assert_allclose(O2[0], ref, rtol=0, atol=1e-12)
    lse = torch.logsumexp(qf @ kf.transpose(1, 2) / math.sqrt(D), dim=-1).numpy()
    np.testing.assert_allclose(L[0], lse, rtol=1e-13, atol=1e-12)


def test_block_diagonal_is_per_tile_attention():
    """Radius 0 and nothing routed: attention inside each tile only.  Tokens
    are grouped into 4x4x4 cells by their coordinates, independently of the
    oracle's tile numbering, and each group runs textbook attention."""
    T, H, W, heads, D = 7, 6, 9, 2, 8
    w, q, k, v, r, s = _inputs(T, H, W, heads, D)
    zero = np.zeros_like(r)
    O, _ = vo.attention(q, k, v, zero, s, 0, T, H, W, 1 / math.sqrt(D))
    groups = {}
    for t in range(T):
        for h in range(H):
            for x in range(W):
                groups.setdefault((t // 4, h // 4, x // 4), []).append((t * H + h) * W + x)
    qf, kf, vf = (torch.from_numpy(vo.bf16_to_f64(a[0])) for a in (q, k, v))
    for idx in groups.values():
        ix = torch.tensor(idx)
        for hd in range(heads):
            ref = torch.nn.functional.scaled_dot_product_attention(
                qf[ix, hd][None], kf[ix, hd][None], vf[ix, hd][None], scale=1 / math.sqrt(D))[0]
            np.testing.assert_allclose(O[0, idx, hd], ref.numpy(), rtol=0, atol=1e-12)


def test_rows_sum_to_one_and_mask():
    """With V = identity (D = N), O is the probability matrix itself: rows sum
    to 1 and masked keys get exactly zero."""
    T, H, W = 5, 4, 6
    N = T * H * W
    w, q, k, _, r, s = _inputs(T, H, W, 1, 8)
    eye = wl.f32_to_bf16_bits(np.eye(N, dtype=np.float32)).reshape(N, 1, N)[None]
    q = q[..., :8]
    k = k[..., :8]
    P, _ = vo.attention(q, k, eye, r, s, 1, T, H, W, 0.3)
    P = P[0, :, 0, :]
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    keep, _ = vo.block_mask(r, s, 1, T, H, W)
    tok = [brute.tile_of(t, h, x, T, H, W) for t in range(T) for h in range(H) for x in range(W)]
    mask = np.array([[keep[0, 0, tok[i], tok[j]] for j in range(N)] for i in range(N)])
    assert np.all(P[~mask] == 0.0)
    assert np.all(P[mask] > 0.0)


def test_constant_v_gives_constant_o():
    T, H, W, heads, D = 6, 5, 7, 2, 8
    w, q, k, v, r, s = _inputs(T, H, W, heads, D)
    c = wl.f32_to_bf16_bits(np.full(v.shape, 1.375, np.float32))
    O, _ = vo.attention(q, k, c, r, s, 2, T, H, W, 1 / math.sqrt(D))
    np.testing.assert_allclose(O, 1.375, rtol=0, atol=1e-13)


def test_zero_q_gives_mean_of_kept_v():
    T, H, W, heads, D = 6, 5, 7, 2, 8
    w, q, k, v, r, s = _inputs(T, H, W, heads, D)
    z = np.zeros_like(q)
    O, L = vo.attention(z, k, v, r, s, 2, T, H, W, 1 / math.sqrt(D))
    vf = vo.bf16_to_f64(v[0])
    N = T * H * W
    coords = [(t, h, x) for t in range(T) for h in range(H) for x in range(W)]
    for hd in range(heads):
        rt = brute.routed(s[0, hd].tolist(), 2)
        for i in (0, N // 3, N - 1):
            ti = brute.tile_of(*coords[i], T, H, W)
            kept = [j for j in range(N)
                    if brute.keeps(ti, brute.tile_of(*coords[j], T, H, W), int(r[0, hd, ti]),
                                   rt[ti], T, H, W)]
            np.testing.assert_allclose(O[0, i, hd], vf[kept, hd].mean(axis=0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(L[0, hd, i], math.log(len(kept)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("parts", [1, 2, 3, 5])
def test_merge_partials_equals_unsplit(parts):
    rng = np.random.default_rng(parts)
    q = rng.standard_normal((7, 16)) * 2
    k = rng.standard_normal((50, 16)) * 2
    v = rng.standard_normal((50, 16))
    O, L = vo.masked_attention_rows(q, k, v, np.ones((7, 50), bool), 0.25)
    cuts = np.sort(rng.choice(np.arange(1, 50), size=parts - 1, replace=False))
    pieces = np.split(np.arange(50), cuts)
    merged = vo.merge_partials([vo.partial_attention(q, k[p], v[p], 0.25) for p in pieces])
    np.testing.assert_allclose(merged[0], O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(merged[1], L, rtol=0, atol=1e-13)


# -------------------------------------------------------------- generator

def test_generator_deterministic_and_chunkable():
    w = wl.custom(9, 10, 11, 3, 16, cid=7)
    q1, k1, v1 = wl.qkv(w)
    q2, k2, v2 = wl.qkv(w, heads=range(1, 3))
    assert np.array_equal(q1[:, :, 1:], q2) and np.array_equal(v1[:, :, 1:], v2)
    q3, _, _ = wl.qkv(w)
    assert np.array_equal(q1, q3)
    r, s = wl.radii_scores(w)
    assert r.dtype == np.uint8 and s.dtype == np.float32
    assert set(np.unique(r).tolist()) <= {1, 2, 3}


def test_generator_bf16_rounding_matches_torch():
    x = np.random.default_rng(3).standard_normal(10000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.f32_to_bf16_bits(x), ref)
