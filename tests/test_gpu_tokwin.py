"""GPU parity (through the C ABI) of attention with exact per-token windows
against the CPU oracle: small and ragged grids in full (O and LSE), key
splits, grids where tile windows cover every key tile (complete rows run as
shared-key units yet windowed per token), token radii uniform per tile
(bit-identical to the block-mask call), and the Wan2.1-1.3B call with radii
from the token-budget chain on sampled query tiles."""
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


def _run(w, q, k, v, tok_r, scores, kcount, r_max, kv_chunk=0):
    sh = vsa.shape(q.shape[0], w.heads, w.D, w.T, w.H, w.W)
    q_t = vsa.tile_permute(bf16_to_dev(q), sh, vsa.LAYOUT_TOKEN_MAJOR)
    k_t = vsa.tile_permute(bf16_to_dev(k), sh, vsa.LAYOUT_TOKEN_MAJOR)
    v_t = vsa.tile_permute(bf16_to_dev(v), sh, vsa.LAYOUT_FEATURE_MAJOR)
    tr = torch.from_numpy(np.ascontiguousarray(tok_r)).to(dev())
    tile_r = vsa.tile_radius_from_tokens(tr, sh)
    rp, ci, routed = vsa.build_mask(tile_r, torch.from_numpy(scores).to(dev()), sh, kcount, r_max)
    o_t, lse = vsa.attn_fwd_token_window(q_t, k_t, v_t, rp, ci, routed, tr, sh, r_max, w.scale,
                                         kv_chunk)
    o = vsa.tile_unpermute(o_t, sh)
    torch.cuda.synchronize()
    return dict(q_t=q_t, k_t=k_t, v_t=v_t, rp=rp, ci=ci, routed=routed, tile_r=tile_r, o_t=o_t,
                lse=lse, o=o, sh=sh)


def _check_lse(out, lse_ref, T, H, W, heads):
    lse_t = out["lse"].cpu().numpy().astype(np.float64)
    lse_ref_t = vo.permute(lse_ref.transpose(0, 2, 1)[..., None], T, H, W)[..., 0]
    valid = vo.permute(np.ones((1, T * H * W, heads, 1)), T, H, W)[..., 0] > 0
    d = np.abs(lse_t - lse_ref_t)[valid]
    say(f"  LSE max_abs={d.max():.3e}")
    assert d.max() <= LSE_ABS


SMALL = [  # T, H, W, heads, D, token radius range, r_max, routed counts, kv_chunk
    (8, 16, 16, 2, 64, 4, 3, (0, 6), 0),
    (5, 6, 7, 2, 128, 3, 2, (0, 1), 0),
    (13, 9, 17, 2, 128, 5, 4, (0, 5), 0),
    (9, 10, 11, 2, 64, 4, 3, (2,), 3),
    (12, 12, 12, 2, 128, 4, 3, (0, 2), 1),
    (8, 8, 8, 3, 128, 4, 3, (0, 1), 0),        # 2x2x2 tiles: radius-2 windows cover the grid
]


@pytest.mark.parametrize("T,H,W,heads,D,rhi,r_max,kset,kv_chunk", SMALL)
def test_token_window_full_small(T, H, W, heads, D, rhi, r_max, kset, kv_chunk):
    w = wl.custom(T, H, W, heads, D, cid=420)
    q, k, v = wl.qkv(w)
    _, s = wl.radii_scores(w)
    rng = np.random.default_rng(T * H * W + D)
    tok_r = rng.integers(0, rhi + 1, size=(1, heads, T * H * W)).astype(np.uint8)
    for kcount in kset:
        say(f"token windows T={T} H={H} W={W} heads={heads} D={D} r<={rhi} r_max={r_max} "
            f"k={kcount} kv_chunk={kv_chunk}")
        out = _run(w, q, k, v, tok_r, s, kcount, r_max, kv_chunk)
        ref, lse = vo.token_window_attention(q, k, v, tok_r, s, kcount, r_max, T, H, W, w.scale)
        assert_close(f64_of(out["o"]), ref, "O")
        _check_lse(out, lse, T, H, W, heads)


def test_token_window_batch2():
    """Two batch entries with different inputs, token radii and scores."""
    T, H, W, heads, D = 9, 10, 11, 2, 128
    ws = [wl.custom(T, H, W, heads, D, cid=c) for c in (422, 423)]
    draws = [wl.qkv(w) + wl.radii_scores(w) for w in ws]
    q, k, v, _, s = (np.concatenate([d[i] for d in draws], axis=0) for i in range(5))
    rng = np.random.default_rng(424)
    tok_r = rng.integers(0, 4, size=(2, heads, T * H * W)).astype(np.uint8)
    for kcount in (0, 3):
        say(f"token windows batch=2 T={T} H={H} W={W} heads={heads} D={D} k={kcount}")
        out = _run(ws[0], q, k, v, tok_r, s, kcount, 3)
        ref, lse = vo.token_window_attention(q, k, v, tok_r, s, kcount, 3, T, H, W, ws[0].scale)
        assert_close(f64_of(out["o"]), ref, f"O batch=2 k={kcount}")


@pytest.mark.parametrize("D", [64, 128])
def test_uniform_token_radii_equal_block_mask_call(D):
    """Every token carrying its tile's radius: no key tile is windowed out, and
    the call must return the bits of the block-mask call."""
    T, H, W, heads = 11, 13, 9, 2
    w = wl.custom(T, H, W, heads, D, radius_set=(0, 1, 2, 3), cid=421)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    tok_r = np.ascontiguousarray(r[:, :, vo.token_tile(T, H, W)])
    say(f"token windows uniform D={D}")
    out = _run(w, q, k, v, tok_r, s, 3, 3)
    o_ref, lse_ref = vsa.attn_fwd(out["q_t"], out["k_t"], out["v_t"], out["rp"], out["ci"],
                                  out["sh"], w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(out["o_t"]), bits_of(o_ref))
    assert torch.equal(out["lse"], lse_ref)


def test_token_window_wan13b_sampled():
    w = wl.WORKLOADS[1]
    kcount, r_max = w.dense_counts[0], max(w.radius_set)
    say(f"token windows {w.name} k={kcount} (generating inputs)")
    q, k, v = wl.qkv(w)
    budget, tscore = wl.token_inputs(w)
    sh = vsa.shape(1, w.heads, w.D, w.T, w.H, w.W)
    tok_r = vsa.budget_to_radius(torch.from_numpy(budget).to(dev()), sh, r_max).cpu().numpy()
    scores = vsa.tile_score_from_tokens(torch.from_numpy(tscore).to(dev()), sh).cpu().numpy()
    out = _run(w, q, k, v, tok_r, scores, kcount, r_max)
    o = f64_of(out["o"])
    tt = vo.token_tile(w.T, w.H, w.W)
    rng = np.random.default_rng(5)
    tile_r = out["tile_r"].cpu().numpy()
    got_all, ref_all = [], []
    windowed_out = 0
    for h in (0, 6, 11):
        routed = vo.routed_tiles(scores[0, h], kcount)
        keep_tok = vo.token_window_keep(tok_r[0, h], routed, r_max, w.T, w.H, w.W)
        keep_tile = vo.tile_keep(np.minimum(tile_r[0, h], r_max), routed, w.T, w.H, w.W)
        windowed_out += int((keep_tile[tt] & ~keep_tok).sum())
        tiles = np.concatenate([rng.choice(np.flatnonzero(routed), 3, replace=False),
                                rng.choice(np.flatnonzero(~routed), 9, replace=False)])
        rows = np.flatnonzero(np.isin(tt, tiles))
        qf, kf, vf = (vo.bf16_to_f64(x[0, :, h]) for x in (q, k, v))
        ref, _ = vo.token_window_attention_rows(qf, kf, vf, keep_tok, tt, rows, w.scale)
        got_all.append(o[0, rows, h])
        ref_all.append(ref)
    assert_close(np.concatenate(got_all), np.concatenate(ref_all), f"{w.name} token windows")
    # the windows bite: kept tiles outside some tokens' own windows
    say(f"  (token, kept tile) pairs outside the token's window: {windowed_out}")
    assert windowed_out > 0


@pytest.mark.parametrize("D", [64, 128])
def test_token_window_running_max_moves_every_tile(D):
    """Exact per-token windows on scores that rise with the key tile's index
    (the running maximum moves on most tiles a token attends): O and LSE."""
    T, H, W, heads = 9, 10, 11, 2
    w = wl.custom(T, H, W, heads, D, cid=431)
    q, k, v = wl.qkv(w)
    _, s = wl.radii_scores(w)
    q, k = rising_scores(w, q, k)
    rng = np.random.default_rng(D + 7)
    tok_r = rng.integers(0, 4, size=(1, heads, T * H * W)).astype(np.uint8)
    for kcount in (0, 3):
        say(f"token windows running max moves D={D} k={kcount}")
        out = _run(w, q, k, v, tok_r, s, kcount, 3)
        ref, lse = vo.token_window_attention(q, k, v, tok_r, s, kcount, 3, T, H, W, w.scale)
        assert_close(f64_of(out["o"]), ref, "O")
        _check_lse(out, lse, T, H, W, heads)
