"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Bit-exact: tile permute / unpermute (both layouts) and the CSR mask.
Tolerance (max-abs 2e-2, mean-rel 3e-3): attention outputs, full rows on small
grids and sampled query tiles at the full workload sizes."""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import LSE_ABS, assert_close, bf16_to_dev, bits_of, dev, f64_of, rising_scores, say
from oracle import vsa_oracle as vo

pytestmark = pytest.mark.gpu

vsa = pytest.importorskip("block_sparse_attention_19_amd")

if not torch.cuda.is_available():  # collected on CPU hosts only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)


def _shape(w):
    return vsa.shape(w.batch, w.heads, w.D, w.T, w.H, w.W)


def _run_all(w, q, k, v, r, s, kcount, kv_chunk=0, r_max=None, nan_out=False):
    """nan_out: the tiled output starts as NaN, so a row the call never writes shows."""
    sh = _shape(w)
    qd, kd, vd = bf16_to_dev(q), bf16_to_dev(k), bf16_to_dev(v)
    q_t = vsa.tile_permute(qd, sh, vsa.LAYOUT_TOKEN_MAJOR)
    k_t = vsa.tile_permute(kd, sh, vsa.LAYOUT_TOKEN_MAJOR)
    v_t = vsa.tile_permute(vd, sh, vsa.LAYOUT_FEATURE_MAJOR)
    rp, ci, routed = vsa.build_mask(torch.from_numpy(r).to(dev()), torch.from_numpy(s).to(dev()),
                                    sh, kcount, r_max if r_max is not None else max(w.radius_set))
    o_init = torch.full_like(q_t, float("nan")) if nan_out else None
    o_t, lse = vsa.attn_fwd(q_t, k_t, v_t, rp, ci, sh, w.scale, kv_chunk, out=o_init)
    o = vsa.tile_unpermute(o_t, sh)
    torch.cuda.synchronize()
    return dict(q_t=q_t, k_t=k_t, v_t=v_t, rp=rp, ci=ci, routed=routed, o_t=o_t, lse=lse, o=o)


# ------------------------------------------------------------------ permute

PERMUTE_CASES = [(8, 16, 16, 2, 64), (5, 6, 7, 3, 128), (9, 5, 3, 2, 64), (1, 1, 1, 1, 128),
                 (21, 30, 52, 12, 128)]


@pytest.mark.parametrize("T,H,W,heads,D", PERMUTE_CASES)
def test_permute_bitexact(T, H, W, heads, D):
    say(f"permute T={T} H={H} W={W} heads={heads} D={D}")
    w = wl.custom(T, H, W, heads, D, cid=400)
    q, _, _ = wl.qkv(w)
    sh = _shape(w)
    xd = bf16_to_dev(q)
    tok = vsa.tile_permute(xd, sh, vsa.LAYOUT_TOKEN_MAJOR)
    fea = vsa.tile_permute(xd, sh, vsa.LAYOUT_FEATURE_MAJOR)
    back = vsa.tile_unpermute(tok, sh)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(tok), vo.permute(q, T, H, W))
    assert np.array_equal(bits_of(fea), vo.permute(q, T, H, W, transposed=True))
    assert np.array_equal(bits_of(back), q)
    # unpermute of arbitrary tile contents (padded rows hold garbage)
    rnd = np.random.default_rng(T + H + W).integers(0, 2 ** 16, size=bits_of(tok).shape,
                                                    dtype=np.uint16)
    out = vsa.tile_unpermute(bf16_to_dev(rnd), sh)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out), vo.unpermute(rnd, T, H, W))


# --------------------------------------------------------------------- mask

MASK_CASES = [(0, 0), (1, 0), (2, 0), (2, 1), (2, 2), (2, 3), (2, 4), (3, 0), (4, 0), (4, 1)]


@pytest.mark.parametrize("cid,ki", MASK_CASES)
def test_mask_bitexact_workloads(cid, ki):
    w = wl.WORKLOADS[cid]
    kcount = w.dense_counts[ki]
    say(f"mask {w.name} k={kcount}")
    r, s = wl.radii_scores(w)
    rp, ci, routed = vsa.build_mask(torch.from_numpy(r).to(dev()), torch.from_numpy(s).to(dev()),
                                    _shape(w), kcount, max(w.radius_set))
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    nnz = int(rp[-1])
    ci = ci[:nnz].cpu().numpy().astype(np.int64)
    routed = routed.cpu().numpy()
    n = w.n_cells
    off = 0
    for h in range(w.heads):  # per head to bound the oracle's memory
        keep, rt = vo.block_mask(r[:, h:h + 1], s[:, h:h + 1], kcount, w.T, w.H, w.W)
        orp, oci = vo.csr(keep)
        assert np.array_equal(routed[0, h].astype(bool), rt[0, 0]), f"routed head {h}"
        assert np.array_equal(rp[h * n:(h + 1) * n + 1] - rp[h * n], orp), f"row_ptr head {h}"
        assert np.array_equal(ci[off:off + len(oci)], oci), f"col_idx head {h}"
        off += len(oci)
    assert off == nnz


def test_mask_ties_nan_inf_and_clamp():
    """Crafted scores with ties, signed zeros, infinities and NaN; radii above
    r_max are clamped to r_max."""
    T, H, W = 13, 9, 17
    w = wl.custom(T, H, W, 3, 64, radius_set=(0, 1, 2, 3, 4, 5, 6), cid=401)
    r, s = wl.radii_scores(w)
    pool = np.array([0.25, 0.5, 0.5, -0.0, 0.0, np.inf, -np.inf, np.nan, -np.nan, 1.0], np.float32)
    s = np.random.default_rng(5).choice(pool, size=s.shape).astype(np.float32)
    for kcount in (0, 1, 7, 20, w.n_cells):
        rp, ci, routed = vsa.build_mask(torch.from_numpy(r).to(dev()), torch.from_numpy(s).to(dev()),
                                        _shape(w), kcount, 4)
        torch.cuda.synchronize()
        keep, rt = vo.block_mask(np.minimum(r, 4), s, kcount, T, H, W)
        orp, oci = vo.csr(keep)
        rp = rp.cpu().numpy()
        assert np.array_equal(rp, orp)
        assert np.array_equal(ci[: rp[-1]].cpu().numpy(), oci)
        assert np.array_equal(routed.cpu().numpy().astype(bool), rt)


# ------------------------------------------------------------- attention

SMALL = [  # T, H, W, heads, D, radius set, routed counts
    (8, 16, 16, 2, 64, (1, 2, 3), (6, 0, 32)),
    (5, 6, 7, 2, 128, (0, 1, 2), (0, 1, 4)),
    (9, 5, 3, 3, 64, (0, 1), (1,)),
    (13, 9, 17, 2, 128, (1, 2, 3, 4), (0, 5, 60)),
    (1, 1, 1, 1, 64, (0,), (0, 1)),
    (12, 8, 8, 2, 128, (0,), (0,)),
    # tile grids cut unevenly into the plan's spatial blocks (10 x 9 and 6 x 8 tiles)
    (4, 40, 36, 1, 64, (1, 2, 3), (0, 9)),
    (8, 24, 32, 1, 64, (1, 2), (0, 5)),
]


@pytest.mark.parametrize("T,H,W,heads,D,rset,kset", SMALL)
def test_attention_full_small(T, H, W, heads, D, rset, kset):
    w = wl.custom(T, H, W, heads, D, radius_set=rset, cid=402)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    for kcount in kset:
        say(f"attention T={T} H={H} W={W} heads={heads} D={D} k={kcount}")
        out = _run_all(w, q, k, v, r, s, kcount)
        ref, lse = vo.attention(q, k, v, r, s, kcount, T, H, W, w.scale)
        assert_close(f64_of(out["o"]), ref, "O")
        # LSE of valid rows, read through the token-major permute of the oracle
        lse_t = out["lse"].cpu().numpy().astype(np.float64)          # [B, Hh, Npad]
        lse_ref_t = vo.permute(lse.transpose(0, 2, 1)[..., None], T, H, W)[..., 0]
        valid = vo.permute(np.ones((1, T * H * W, heads, 1)), T, H, W)[..., 0] > 0
        d = np.abs(lse_t - lse_ref_t)[valid]
        say(f"  LSE max_abs={d.max():.3e}")
        assert d.max() <= LSE_ABS


def test_attention_split_invariance_and_determinism():
    w = wl.WORKLOADS[0]
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    kcount = w.dense_counts[0]
    ref, _ = vo.attention(q, k, v, r, s, kcount, w.T, w.H, w.W, w.scale)
    base = None
    for chunk in (0, 1, 2, 5, 13):
        say(f"attention {w.name} kv_chunk={chunk}")
        out = _run_all(w, q, k, v, r, s, kcount, kv_chunk=chunk)
        got = f64_of(out["o"])
        assert_close(got, ref, f"O kv_chunk={chunk}")
        again = _run_all(w, q, k, v, r, s, kcount, kv_chunk=chunk)
        assert np.array_equal(bits_of(again["o"]), bits_of(out["o"])), "not deterministic"
        if base is None:
            base = got
        else:
            assert np.abs(got - base).max() <= 2e-2


def _sample_tiles(w, r, s, kcount, h, rng, n_routed=4, n_edge=4, n_rand=8):
    """Query tiles to check for head h: routed ones, edge (padded) ones, random."""
    n = w.n_cells
    routed = np.flatnonzero(vo.routed_tiles(s[0, h], kcount))
    c = vo.tile_coords(w.T, w.H, w.W)
    a, b, cc = vo.tile_grid(w.T, w.H, w.W)
    edge = np.flatnonzero((4 * (c[:, 0] + 1) > w.T) | (4 * (c[:, 1] + 1) > w.H) |
                          (4 * (c[:, 2] + 1) > w.W))
    pick = []
    for pool, m in ((routed, n_routed), (edge, n_edge), (np.arange(n), n_rand)):
        if len(pool):
            pick.extend(rng.choice(pool, size=min(m, len(pool)), replace=False).tolist())
    return sorted(set(pick))


def _token_slots(w):
    """Tile-major slot of every raster token (the permute's mapping)."""
    ids = vo.permute((np.arange(w.tokens, dtype=np.float64) + 1)[None, :, None, None],
                     w.T, w.H, w.W)[0, 0, :, 0]
    pos = np.empty(w.tokens, np.int64)
    filled = np.flatnonzero(ids > 0)
    pos[ids[filled].astype(np.int64) - 1] = filled
    return pos


def _check_sampled(w, q, k, v, r, s, kcount, out, heads, seed=0, light=()):
    """Sampled query tiles against the oracle, O and LSE: 16 tiles (routed,
    edge, random) of each head in `heads`, and one routed, one edge and one
    random tile of each head in `light`."""
    rng = np.random.default_rng(seed)
    tt = vo.token_tile(w.T, w.H, w.W)
    o = f64_of(out["o"])
    lse_t = out["lse"].cpu().numpy().astype(np.float64)[0]
    pos = _token_slots(w)
    got_all, ref_all, lse_err = [], [], 0.0
    for h in sorted(set(heads) | set(light)):
        keep = vo.tile_keep(r[0, h], vo.routed_tiles(s[0, h], kcount), w.T, w.H, w.W)
        qf, kf, vf = (vo.bf16_to_f64(x[0, :, h]) for x in (q, k, v))
        if h in heads:
            tiles = _sample_tiles(w, r, s, kcount, h, rng)
        else:
            tiles = _sample_tiles(w, r, s, kcount, h, rng, n_routed=1, n_edge=1, n_rand=1)
        rows = np.flatnonzero(np.isin(tt, tiles))
        ref, lref = vo.attention_head_rows(qf, kf, vf, keep, tt, rows, w.scale)
        got_all.append(o[0, rows, h])
        ref_all.append(ref)
        lse_err = max(lse_err, float(np.abs(lse_t[h, pos[rows]] - lref).max()))
    assert_close(np.concatenate(got_all), np.concatenate(ref_all), f"{w.name} k={kcount} sampled")
    say(f"  LSE max_abs={lse_err:.3e}")
    assert lse_err <= LSE_ABS


def test_attention_wan13b_sampled():
    w = wl.WORKLOADS[1]
    kcount = w.dense_counts[0]
    say(f"attention {w.name} k={kcount} (generating inputs)")
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    out = _run_all(w, q, k, v, r, s, kcount)
    _check_sampled(w, q, k, v, r, s, kcount, out, heads=[0, 5, 11], light=range(w.heads))
    # the CSR of the full-size call is exact too
    keep, _ = vo.block_mask(r[:, :1], s[:, :1], kcount, w.T, w.H, w.W)
    orp, oci = vo.csr(keep)
    assert np.array_equal(out["rp"][: w.n_cells + 1].cpu().numpy(), orp)


@pytest.mark.parametrize("cid,ki", [(2, 0), (2, 1), (2, 2), (2, 3), (2, 4), (3, 0), (4, 0),
                                    (4, 1)])
def test_attention_large_sampled(cid, ki):
    """Every workload and routing point at full size: sampled tiles of every
    head (16 on the first and last head, three on the others), O and LSE."""
    w = wl.WORKLOADS[cid]
    kcount = w.dense_counts[ki]
    say(f"attention {w.name} k={kcount} (generating inputs)")
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    out = _run_all(w, q, k, v, r, s, kcount)
    _check_sampled(w, q, k, v, r, s, kcount, out, heads=[0, w.heads - 1], seed=cid * 10 + ki,
                   light=range(w.heads))
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("heads,kv_chunk", [(32, 0), (33, 0), (33, 64)])
def test_attention_plan_block_boundary(heads, kv_chunk):
    """The work plan takes rows in blocks of 8192: exactly one full block
    (32 heads x 256 tiles), and one row of tiles past it (33 heads), with
    every row cut into key chunks in the last case.  51 routed tiles per head
    (an odd count: one complete row is left over from the pairing)."""
    T, H, W, D = 32, 32, 16, 64
    w = wl.custom(T, H, W, heads, D, radius_set=(1, 2, 3), cid=413)
    kcount = 51
    say(f"attention plan blocks T={T} H={H} W={W} heads={heads} k={kcount} kv_chunk={kv_chunk}")
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    out = _run_all(w, q, k, v, r, s, kcount, kv_chunk=kv_chunk)
    _check_sampled(w, q, k, v, r, s, kcount, out, heads=sorted({0, 31, heads - 1}), seed=heads)
    del out
    torch.cuda.empty_cache()


def test_attention_plan_order_without_lds_table():
    """The plan keeps its spatial-block row order as an LDS table for grids of
    up to 8192 tiles; this grid has 1 x 1 x 8200 tiles, so the order is
    evaluated per row.  Every valid output row is written (the output starts as
    NaN), and sampled rows match the oracle."""
    T, H, W, D = 4, 4, 4 * 8200, 64
    w = wl.custom(T, H, W, 1, D, radius_set=(1, 2, 3), cid=414)
    kcount = 3
    say(f"attention plan order T={T} H={H} W={W} k={kcount}")
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    out = _run_all(w, q, k, v, r, s, kcount, nan_out=True)
    assert torch.isfinite(out["o"].float()).all().item(), "an output row was not written"
    _check_sampled(w, q, k, v, r, s, kcount, out, heads=[0], seed=414)
    del out
    torch.cuda.empty_cache()


RASTER_CASES = [  # T, H, W, heads, D, radius set, routed count, kv_chunk
    (8, 16, 16, 2, 64, (1, 2, 3), 6, 0),
    (5, 6, 7, 2, 128, (0, 1, 2), 1, 0),
    (13, 9, 17, 2, 128, (1, 2, 3, 4), 5, 3),
    (4, 40, 36, 1, 64, (1, 2, 3), 9, 0),
    (1, 1, 1, 1, 64, (0,), 0, 0),
]


def _raster(w, q, out, kv_chunk):
    """The raster call on the caller's Q, with K/V/CSR of `out`; O starts as NaN."""
    sh = _shape(w)
    o = torch.full((w.batch, w.T * w.H * w.W, w.heads, w.D), float("nan"), dtype=torch.bfloat16,
                   device=dev())
    qd = bf16_to_dev(q)
    o, lse = vsa.attn_fwd_raster(qd, out["k_t"], out["v_t"], out["rp"], out["ci"], sh, w.scale,
                                 kv_chunk, out=o)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("T,H,W,heads,D,rset,kcount,kv_chunk", RASTER_CASES)
def test_attention_raster_matches_tiled(T, H, W, heads, D, rset, kcount, kv_chunk):
    """vsa_attn_fwd_raster gathers Q from and scatters O (and LSE) to the raster
    layout inside the call: bitwise the tile-major call followed by the
    unpermute, every element written (the output starts as NaN), and within
    tolerance of the oracle."""
    w = wl.custom(T, H, W, heads, D, radius_set=rset, cid=415)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    say(f"attention raster T={T} H={H} W={W} heads={heads} D={D} k={kcount} kv_chunk={kv_chunk}")
    out = _run_all(w, q, k, v, r, s, kcount, kv_chunk=kv_chunk)
    o, lse = _raster(w, q, out, kv_chunk)
    assert np.array_equal(bits_of(o), bits_of(out["o"])), "raster O differs from unpermuted O"
    lse_t = out["lse"].cpu().numpy()
    lse_from_t = vo.unpermute(lse_t.reshape(1, heads, -1)[..., None], T, H, W)[..., 0]
    lse_from_t = lse_from_t.transpose(0, 2, 1)
    assert np.array_equal(lse.cpu().numpy(), lse_from_t), "raster LSE differs"
    ref, _ = vo.attention(q, k, v, r, s, kcount, T, H, W, w.scale)
    assert_close(f64_of(o), ref, "O raster")


def test_attention_raster_wan13b_full_size():
    """The raster call at the Wan2.1-1.3B shape: bitwise the tile-major call
    followed by the unpermute (whose sampled rows the oracle checks above)."""
    w = wl.WORKLOADS[1]
    kcount = w.dense_counts[0]
    say(f"attention raster {w.name} k={kcount} (generating inputs)")
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    out = _run_all(w, q, k, v, r, s, kcount)
    o, lse = _raster(w, q, out, 0)
    assert np.array_equal(bits_of(o), bits_of(out["o"]))
    assert torch.isfinite(lse).all().item()
    # run to run at full size (the persistent kernel claims its units through
    # atomics, so the claim order changes; the result must not)
    for _ in range(2):
        o2, lse2 = _raster(w, q, out, 0)
        assert np.array_equal(bits_of(o2), bits_of(o)), "raster O not deterministic"
        assert torch.equal(lse2, lse), "raster LSE not deterministic"
    del out, o, lse, o2, lse2
    torch.cuda.empty_cache()


def test_attention_batch2_full():
    """Two batch entries with different inputs, radii and scores (the
    workloads draw B = 1; the batch axis stacks two draws)."""
    T, H, W, heads, D = 9, 10, 11, 2, 64
    ws = [wl.custom(T, H, W, heads, D, radius_set=(0, 1, 2), cid=c) for c in (410, 411)]
    draws = [wl.qkv(w) + wl.radii_scores(w) for w in ws]
    q, k, v, r, s = (np.concatenate([d[i] for d in draws], axis=0) for i in range(5))
    w2 = ws[0].__class__(**{**ws[0].__dict__, "batch": 2})
    for kcount in (0, 3):
        say(f"attention batch=2 T={T} H={H} W={W} heads={heads} D={D} k={kcount}")
        out = _run_all(w2, q, k, v, r, s, kcount)
        keep, _ = vo.block_mask(r, s, kcount, T, H, W)
        orp, oci = vo.csr(keep)
        assert np.array_equal(out["rp"].cpu().numpy().astype(np.int64), orp)
        assert np.array_equal(out["ci"][: int(orp[-1])].cpu().numpy().astype(np.int64), oci)
        ref, _ = vo.attention(q, k, v, r, s, kcount, T, H, W, ws[0].scale)
        assert_close(f64_of(out["o"]), ref, f"O batch=2 k={kcount}")
        # the raster call on the same batch: the same bits, every element written
        o_r, lse_r = _raster(w2, q, out, 0)
        assert np.array_equal(bits_of(o_r), bits_of(out["o"])), "raster O differs (batch 2)"
        assert torch.isfinite(lse_r).all().item()


@pytest.mark.parametrize("kv_chunk", [0, 4])
def test_attention_d64_medium_split(kv_chunk):
    """D = 64 with enough routed rows for G units and (kv_chunk 0) their
    automatic key split, or a forced chunking of every row."""
    T, H, W, heads, D = 21, 16, 16, 3, 64
    w = wl.custom(T, H, W, heads, D, radius_set=(1, 2, 3), cid=412)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    kcount = 10
    say(f"attention D=64 T={T} H={H} W={W} heads={heads} k={kcount} kv_chunk={kv_chunk}")
    out = _run_all(w, q, k, v, r, s, kcount, kv_chunk=kv_chunk)
    ref, _ = vo.attention(q, k, v, r, s, kcount, T, H, W, w.scale)
    assert_close(f64_of(out["o"]), ref, f"O D=64 kv_chunk={kv_chunk}")


def _random_csr(rng, rows, nT):
    """Any CSR the call accepts: empty rows, single columns, complete rows
    (which run as G units) and random ascending column subsets."""
    lens = []
    cols = []
    for _ in range(rows):
        u = rng.random()
        n = 0 if u < 0.1 else 1 if u < 0.2 else nT if u < 0.35 else int(rng.integers(2, nT))
        lens.append(n)
        cols.append(np.sort(rng.choice(nT, n, replace=False)))
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return rp, np.concatenate(cols).astype(np.int32)


def _check_csr_attention(w, q, k, v, rp, ci, o, lse, skim=None):
    """O / LSE of an arbitrary CSR against the oracle; rows without keys must
    give zeros and LSE = -inf."""
    nT = w.n_cells
    tt = vo.token_tile(w.T, w.H, w.W)
    got = f64_of(o)[0]
    lse_t = lse.cpu().numpy().astype(np.float64)[0]
    g_all, r_all = [], []
    for h in range(w.heads):
        keep = np.zeros((nT, nT), bool)
        for a in range(nT):
            row = h * nT + a
            keep[a, ci[rp[row]:rp[row + 1]]] = True
        nonempty = keep.any(axis=1)
        rows = np.flatnonzero(nonempty[tt])
        empty = np.flatnonzero(~nonempty[tt])
        qf, kf, vf = (vo.bf16_to_f64(x[0, :, h]) for x in (q, k, v))
        if skim is None:
            ref, lref = vo.attention_head_rows(qf, kf, vf, keep, tt, rows, w.scale)
        else:
            ref, lref = vo.tiered_attention_head(qf, kf, vf, keep, skim[h], tt, rows, w.scale)
        g_all.append(got[rows, h])
        r_all.append(ref)
        assert np.all(got[empty, h] == 0.0), "rows without keys must be zero"
        # LSE in token-major order: token n of tile tau sits at slot tau*64 + local index
        slot = vo.permute(np.arange(w.tokens, dtype=np.float64)[None, :, None, None], w.T, w.H, w.W)[0, 0, :, 0]
        valid = vo.permute(np.ones((1, w.tokens, 1, 1)), w.T, w.H, w.W)[0, 0, :, 0] > 0
        tok_of_slot = np.full(slot.shape, -1, np.int64)
        tok_of_slot[valid] = slot[valid].astype(np.int64)
        pos = np.full(w.tokens, -1, np.int64)
        pos[tok_of_slot[valid]] = np.flatnonzero(valid)
        assert np.abs(lse_t[h, pos[rows]] - lref).max() <= LSE_ABS
        if len(empty):
            assert np.all(np.isneginf(lse_t[h, pos[empty]]))
    assert_close(np.concatenate(g_all), np.concatenate(r_all), "O arbitrary CSR")


@pytest.mark.parametrize("D,kv_chunk", [(64, 0), (128, 0), (128, 3)])
def test_attention_arbitrary_csr(D, kv_chunk):
    """Any CSR, not only the mask builder's: empty rows, one-column rows,
    complete rows (G units) and random column subsets."""
    T, H, W, heads = 9, 10, 11, 2
    w = wl.custom(T, H, W, heads, D, radius_set=(1,), cid=413)
    q, k, v = wl.qkv(w)
    nT = w.n_cells
    rp, ci = _random_csr(np.random.default_rng(D + kv_chunk), heads * nT, nT)
    say(f"attention arbitrary CSR D={D} kv_chunk={kv_chunk} nnz={rp[-1]}")
    sh = _shape(w)
    q_t = vsa.tile_permute(bf16_to_dev(q), sh, vsa.LAYOUT_TOKEN_MAJOR)
    k_t = vsa.tile_permute(bf16_to_dev(k), sh, vsa.LAYOUT_TOKEN_MAJOR)
    v_t = vsa.tile_permute(bf16_to_dev(v), sh, vsa.LAYOUT_FEATURE_MAJOR)
    o_t, lse = vsa.attn_fwd(q_t, k_t, v_t, torch.from_numpy(rp).to(dev()),
                            torch.from_numpy(ci).to(dev()), sh, w.scale, kv_chunk)
    o = vsa.tile_unpermute(o_t, sh)
    torch.cuda.synchronize()
    _check_csr_attention(w, q, k, v, rp, ci, o, lse)


def test_attention_composed_fused_and_unfused():
    """vsa.attention (permutes, mask, forward) with the raster forward call and
    with the tile-major one: the same bits, within tolerance of the oracle."""
    w = wl.custom(9, 10, 14, 2, 64, radius_set=(1, 2), cid=416)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    kcount = 2
    say(f"attention composed T={w.T} H={w.H} W={w.W} k={kcount}")
    args = (bf16_to_dev(q), bf16_to_dev(k), bf16_to_dev(v), (w.T, w.H, w.W),
            torch.from_numpy(r).to(dev()), torch.from_numpy(s).to(dev()), kcount)
    a = vsa.attention(*args, scale=w.scale, r_max=2)
    b = vsa.attention(*args, scale=w.scale, r_max=2, fused=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b))
    ref, _ = vo.attention(q, k, v, r, s, kcount, w.T, w.H, w.W, w.scale)
    assert_close(f64_of(a), ref, "O composed")


@pytest.mark.parametrize("D,kv_chunk", [(128, 0), (64, 0), (128, 3)])
def test_attention_running_max_moves_every_tile(D, kv_chunk):
    """Scores that grow with the key tile's index: a shared direction u is added
    to every query and c(tau) * u to every key of key tile tau, with c rising by
    10 log2 units of score per tile, so each later tile of a row lifts the
    running maximum past the lazy-rescale slack (2^8) and the rescale branch
    runs on almost every tile, for routed and local rows; tile-major and raster
    calls, O and LSE against the oracle."""
    T, H, W, heads = 9, 10, 11, 2        # 27 key tiles, ragged on every axis
    w = wl.custom(T, H, W, heads, D, radius_set=(1, 2, 3), cid=430)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    kcount = 5
    q2, k2 = rising_scores(w, q, k)
    say(f"attention running max moves D={D} kv_chunk={kv_chunk}")
    out = _run_all(w, q2, k2, v, r, s, kcount, kv_chunk=kv_chunk)
    ref, lse_ref = vo.attention(q2, k2, v, r, s, kcount, T, H, W, w.scale)
    assert_close(f64_of(out["o"]), ref, "O tile-major")
    lse_t = out["lse"].cpu().numpy().astype(np.float64)
    lse_ref_t = vo.permute(lse_ref.transpose(0, 2, 1)[..., None], T, H, W)[..., 0]
    valid = vo.permute(np.ones((1, T * H * W, heads, 1)), T, H, W)[..., 0] > 0
    d = np.abs(lse_t - lse_ref_t)[valid]
    say(f"  LSE max_abs={d.max():.3e} (LSE up to {np.abs(lse_ref).max():.0f})")
    assert d.max() <= LSE_ABS
    sh = _shape(w)
    o_r, lse_r = vsa.attn_fwd_raster(bf16_to_dev(q2), out["k_t"], out["v_t"], out["rp"], out["ci"],
                                     sh, w.scale, kv_chunk)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(o_r), bits_of(out["o"]))
