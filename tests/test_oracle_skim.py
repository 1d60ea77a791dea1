"""Pins of the oracle's low-precision "skim" tier (Triage: skip, skim or
refine each tile): the MXFP4 quantiser and attention with per-pair tiers.
All on the CPU: hand-worked blocks, an independent rounding formula, exact
round trips of representable blocks, the quantisation error bound, the
reduction of skim to the bf16 attention on representable inputs, and a
scalar brute-force row."""
import math

import numpy as np
import pytest

from conftest import read_golden
from oracle import vsa_oracle as vo


def _golden_blocks():
    _, rows = read_golden("mxfp4_blocks.txt")
    vals = {r[1]: np.array([float(x) for x in r[2:]]) for r in rows if r[0] == "vals"}
    codes = {r[1]: (int(r[2]), np.array([int(x) for x in r[3:]])) for r in rows if r[0] == "codes"}
    return vals, codes


def test_mxfp4_golden_blocks():
    vals, codes = _golden_blocks()
    assert set(vals) == set(codes) and len(vals) == 6
    for name, v in vals.items():
        assert v.shape == (32,)
        c, e = vo.mxfp4_quantize(v[None, :])
        exp_e, exp_c = codes[name]
        assert int(e[0, 0]) == exp_e, name
        np.testing.assert_array_equal(c[0], exp_c, err_msg=name)


def _round_ieee_e2m1(y: np.ndarray) -> np.ndarray:
    """E2M1 rounding written as IEEE-style rounding to a format with one
    mantissa bit: quantum 0.5 below 2 (including the subnormal 0.5), then the
    binade's quantum 2^(e-1); np.round rounds halves to even quotients, which
    are exactly the even codes; results above 6 saturate."""
    a = np.abs(y)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    quantum = np.where(a < 2.0, 0.5, np.ldexp(1.0, (e - 1).astype(np.int64)))
    r = np.minimum(np.round(a / quantum) * quantum, 6.0)
    return np.copysign(r, y)


def test_mxfp4_matches_ieee_style_rounding():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((400, 128)) * np.exp(rng.uniform(-20, 20, (400, 1)))
    x[::7, 5] = 0.0
    c, e = vo.mxfp4_quantize(x)
    got = vo.mxfp4_dequantize(c, e)
    blocks = x.reshape(400, 4, 32)
    amax = np.abs(blocks).max(axis=-1)
    expo = np.floor(np.log2(amax)) - 2
    X = np.ldexp(1.0, expo.astype(np.int64))[..., None]
    want = (_round_ieee_e2m1(blocks / X) * X).reshape(400, 128)
    np.testing.assert_array_equal(got, want)


def test_mxfp4_round_trip_of_representable_blocks():
    rng = np.random.default_rng(3)
    n = 300
    codes = rng.integers(0, 16, (n, 32)).astype(np.uint8)
    codes[codes == 8] = 0                     # -0 decodes to +0 (same value)
    # the block maximum must sit in the top binade (4 or 6) for the scale rule
    top = rng.integers(6, 8, n).astype(np.uint8) | (rng.integers(0, 2, n).astype(np.uint8) << 3)
    codes[np.arange(n), rng.integers(0, 32, n)] = top
    expo = rng.integers(-120, 120, (n, 1)).astype(np.int32)
    x = vo.mxfp4_dequantize(codes, expo)
    c2, e2 = vo.mxfp4_quantize(x)
    np.testing.assert_array_equal(e2, expo)
    np.testing.assert_array_equal(c2, codes)


def test_mxfp4_error_bound_and_scale_range():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 64)) * 3.0
    c, e = vo.mxfp4_quantize(x)
    xb = x.reshape(200, 2, 32)
    X = np.ldexp(1.0, e.astype(np.int64))[..., None]
    ratio = np.abs(xb).max(axis=-1) / X[..., 0]
    assert np.all((ratio >= 4.0) & (ratio < 8.0))
    y = np.abs(xb / X)
    err = np.abs(vo.mxfp4_dequantize(c, e).reshape(200, 2, 32) - xb) / X
    half_q = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    sat = y > 6.0
    assert np.all(err[~sat] <= half_q[~sat] + 1e-15)
    assert np.allclose(err[sat], y[sat] - 6.0)


def _representable(rng, shape):
    """Vectors whose MXFP4 round trip is exact (per 32-block: E2M1 codes with
    a top-binade maximum, one exponent)."""
    n = int(np.prod(shape[:-1])) * (shape[-1] // 32)
    codes = rng.integers(0, 8, (n, 32)).astype(np.uint8) | (rng.integers(0, 2, (n, 32)).astype(np.uint8) << 3)
    codes[codes == 8] = 0
    codes[:, 0] = 7 | (codes[:, 0] & 8)
    expo = rng.integers(-4, 0, (n, 1)).astype(np.int32)
    return vo.mxfp4_dequantize(codes, expo).reshape(shape)


def test_skim_reduces_to_bf16_attention_on_representable_inputs():
    rng = np.random.default_rng(7)
    T, H, W, D = 8, 8, 8, 64
    N = T * H * W
    q = _representable(rng, (N, D))
    k = _representable(rng, (N, D))
    v = rng.standard_normal((N, D))
    nT = vo.num_tiles(T, H, W)
    keep = rng.random((nT, nT)) < 0.6
    keep[np.arange(nT), np.arange(nT)] = True
    skim = rng.random((nT, nT)) < 0.5
    tt = vo.token_tile(T, H, W)
    rows = np.arange(N)
    o1, l1 = vo.tiered_attention_head(q, k, v, keep, skim, tt, rows, 0.125)
    o0, l0 = vo.attention_head_rows(q, k, v, keep, tt, rows, 0.125)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)
    # and all-refine equals the bf16 attention on any inputs
    qa, ka = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    o2, l2 = vo.tiered_attention_head(qa, ka, v, keep, np.zeros_like(skim), tt, rows, 0.125)
    o3, l3 = vo.attention_head_rows(qa, ka, v, keep, tt, rows, 0.125)
    np.testing.assert_array_equal(o2, o3)
    np.testing.assert_array_equal(l2, l3)


def _brute_quantize(vec):
    """Scalar MXFP4 round trip of one vector: per block, the scale from the
    exponent of the largest magnitude, then the nearest grid value by search
    (ties to the even code)."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = []
    for b0 in range(0, len(vec), 32):
        blk = vec[b0:b0 + 32]
        amax = max(abs(x) for x in blk)
        e = -127 if amax == 0 else max(-127, min(127, math.floor(math.log2(amax)) - 2))
        X = 2.0 ** e
        for x in blk:
            y = abs(x) / X
            best_i = 0
            for i in range(8):
                d, db = abs(y - grid[i]), abs(y - grid[best_i])
                if d < db or (d == db and i % 2 == 0 and best_i % 2 == 1):
                    best_i = i
            out.append(math.copysign(grid[best_i] * X, x))
    return out


def test_tiered_row_brute_force():
    rng = np.random.default_rng(13)
    T, H, W, D = 8, 4, 8, 64
    N = T * H * W
    q = rng.standard_normal((N, D))
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    nT = vo.num_tiles(T, H, W)
    keep = rng.random((nT, nT)) < 0.7
    skim = rng.random((nT, nT)) < 0.5
    tt = vo.token_tile(T, H, W)
    scale = 0.1
    for row in (0, 37, N - 1):
        keep[tt[row], tt[row]] = True
        o, lse = vo.tiered_attention_head(q, k, v, keep, skim, tt, np.array([row]), scale)
        qh = _brute_quantize(list(q[row]))
        s = []
        for j in range(N):
            if not keep[tt[row], tt[j]]:
                continue
            if skim[tt[row], tt[j]]:
                kh = _brute_quantize(list(k[j]))
                dot = sum(a * b for a, b in zip(qh, kh))
            else:
                dot = sum(a * b for a, b in zip(q[row], k[j]))
            s.append((scale * dot, j))
        m = max(x for x, _ in s)
        l = sum(math.exp(x - m) for x, _ in s)
        ob = [sum(math.exp(x - m) * v[j, d] for x, j in s) / l for d in range(D)]
        np.testing.assert_allclose(o[0], ob, rtol=1e-12, atol=1e-12)
        assert abs(lse[0] - (m + math.log(l))) < 1e-12


def test_csr_tiers_to_tiles():
    row_ptr = np.array([0, 2, 2, 5])
    col = np.array([1, 3, 0, 2, 3])
    tier = np.array([1, 0, 0, 1, 1], dtype=np.uint8)
    got = vo.csr_tiers_to_tiles(row_ptr, col, tier, 3, 4)
    want = np.array([[0, 1, 0, 0], [0, 0, 0, 0], [0, 0, 1, 1]], dtype=bool)
    np.testing.assert_array_equal(got, want)


def test_tier_recipes():
    """Both tier recipes give one byte per CSR entry at about the asked
    fraction; the per-key-tile one gives every pair of a (batch-head, key
    tile) the same tier, the i.i.d. one does not."""
    import workloads as wl
    w = wl.custom(6, 8, 8, 3, 64, radius_set=(1, 2), cid=430)
    nT = w.n_cells
    rng = np.random.default_rng(3)
    counts = rng.integers(1, nT + 1, size=w.heads * nT)
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ci = np.concatenate([np.sort(rng.choice(nT, c, replace=False)) for c in counts]).astype(np.int32)
    nnz = int(rp[-1])
    bh = np.repeat(np.arange(w.heads * nT) // nT, counts)
    for p in (0.0, 0.25, 0.5, 1.0):
        by_key = wl.tiers_by_key_tile(w, rp, ci, p)
        iid = wl.tiers(w, nnz, p)
        assert by_key.dtype == np.uint8 and by_key.shape == (nnz,) and iid.shape == (nnz,)
        assert set(np.unique(by_key)) <= {0, 1} and set(np.unique(iid)) <= {0, 1}
        key = bh * nT + ci
        for kk in np.unique(key):
            assert np.unique(by_key[key == kk]).size == 1
        if p in (0.0, 1.0):
            assert np.all(by_key == int(p)) and np.all(iid == int(p))
        else:
            assert abs(iid.mean() - p) < 0.03
            # the key tiles' draws: heads * nT of them
            u_mean = np.mean([by_key[key == kk][0] for kk in np.unique(key)])
            assert abs(u_mean - p) < 0.1
            assert any(np.unique(iid[key == kk]).size == 2 for kk in np.unique(key))
