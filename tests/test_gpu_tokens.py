"""GPU parity (through the C ABI) of the token-level calls against the CPU
oracle, bit-exact: budget -> radius per query token, token radii -> tile
radius, token scores -> tile score, and the mask built from them."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import dev, say
from oracle import vsa_oracle as vo

pytestmark = pytest.mark.gpu

vsa = pytest.importorskip("block_sparse_attention_19_amd")

if not torch.cuda.is_available():  # collected on CPU hosts only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)

GRIDS = [(8, 16, 16, 2), (5, 6, 7, 3), (9, 5, 3, 2), (1, 1, 1, 1), (5, 4, 6, 1), (13, 6, 10, 2)]


def _shape(T, H, W, heads):
    return vsa.shape(1, heads, 64, T, H, W)


def _oracle_radius(budget, r_max, T, H, W):
    return np.stack([vo.budget_to_radius(budget[0, h], r_max, T, H, W)
                     for h in range(budget.shape[1])])[None]


@pytest.mark.parametrize("T,H,W,heads", GRIDS)
@pytest.mark.parametrize("r_max", [0, 3, 9])
def test_budget_to_radius_bitexact(T, H, W, heads, r_max):
    say(f"budget->radius T={T} H={H} W={W} heads={heads} r_max={r_max}")
    rng = np.random.default_rng(T * 100 + r_max)
    N = T * H * W
    budget = rng.integers(-3, N + 70, size=(1, heads, N)).astype(np.int32)
    budget[0, 0, :4] = [0, 1, N, 2 ** 31 - 1][:min(4, N)]  # edge budgets
    got = vsa.budget_to_radius(torch.from_numpy(budget).to(dev()), _shape(T, H, W, heads), r_max)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _oracle_radius(budget, r_max, T, H, W))


def test_budget_to_radius_r_max_255():
    T, H, W, heads = 9, 5, 3, 1
    N = T * H * W
    budget = np.arange(-5, N + 5, dtype=np.int32)[:N][None, None]
    budget = np.ascontiguousarray(budget)
    got = vsa.budget_to_radius(torch.from_numpy(budget).to(dev()), _shape(T, H, W, heads), 255)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _oracle_radius(budget, 255, T, H, W))


@pytest.mark.parametrize("T,H,W,heads", GRIDS + [(21, 30, 52, 12)])
def test_tile_radius_and_score_bitexact(T, H, W, heads):
    say(f"tile radius/score T={T} H={H} W={W} heads={heads}")
    rng = np.random.default_rng(T + 7 * H + 31 * W)
    N = T * H * W
    rad = rng.integers(0, 256, size=(1, heads, N)).astype(np.uint8)
    sc = rng.standard_normal((1, heads, N)).astype(np.float32)
    # special values in the IEEE total order
    specials = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45], dtype=np.float32)
    sc.reshape(-1)[: min(specials.size, sc.size)] = specials[: min(specials.size, sc.size)]
    sh = _shape(T, H, W, heads)
    gr = vsa.tile_radius_from_tokens(torch.from_numpy(rad).to(dev()), sh)
    gs = vsa.tile_score_from_tokens(torch.from_numpy(sc).to(dev()), sh)
    torch.cuda.synchronize()
    want_r = np.stack([vo.tile_radius_from_tokens(rad[0, h], T, H, W) for h in range(heads)])[None]
    want_s = np.stack([vo.tile_score_from_tokens(sc[0, h], T, H, W) for h in range(heads)])[None]
    assert np.array_equal(gr.cpu().numpy(), want_r)
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


@pytest.mark.parametrize("cid", [0, 1])
def test_token_pipeline_to_mask(cid):
    """Token budgets and scores -> tile radii and scores -> CSR, against the
    oracle's chain on the same per-token inputs (the workload's own draws)."""
    w = wl.WORKLOADS[cid]
    say(f"token pipeline {w.name}")
    budget, score = wl.token_inputs(w)
    r_max = 4
    sh = vsa.shape(w.batch, w.heads, w.D, w.T, w.H, w.W)
    k = w.dense_counts[0]
    rad_tok = vsa.budget_to_radius(torch.from_numpy(budget).to(dev()), sh, r_max)
    rad_tile = vsa.tile_radius_from_tokens(rad_tok, sh)
    sc_tile = vsa.tile_score_from_tokens(torch.from_numpy(score).to(dev()), sh)
    rp, ci, routed = vsa.build_mask(rad_tile, sc_tile, sh, k, r_max)
    torch.cuda.synchronize()
    want_tok = _oracle_radius(budget, r_max, w.T, w.H, w.W)
    assert np.array_equal(rad_tok.cpu().numpy(), want_tok)
    want_rt = np.stack([vo.tile_radius_from_tokens(want_tok[0, h], w.T, w.H, w.W)
                        for h in range(w.heads)])[None]
    want_st = np.stack([vo.tile_score_from_tokens(score[0, h], w.T, w.H, w.W)
                        for h in range(w.heads)])[None]
    assert np.array_equal(rad_tile.cpu().numpy(), want_rt)
    assert np.array_equal(sc_tile.cpu().numpy(), want_st)
    keep, rt = vo.block_mask(want_rt, want_st, k, w.T, w.H, w.W)
    row_ptr, col_idx = vo.csr(keep)
    assert np.array_equal(rp.cpu().numpy().astype(np.int64), row_ptr)
    nnz = int(row_ptr[-1])
    assert np.array_equal(ci[:nnz].cpu().numpy().astype(np.int64), col_idx)
    assert np.array_equal(routed.cpu().numpy().astype(bool), rt)
