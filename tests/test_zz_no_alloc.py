"""The allocation-free forward call (the library's fixed device workspace)
against the raster call with a caller workspace: the same kernels, so O and
LSE must be bitwise equal.  Several calls in a row on one GPU, each smaller
than the one before, so every call runs on a workspace the previous call
left filled; outputs start as NaN, so an element a call never writes shows."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_close, bf16_to_dev, bits_of, dev, f64_of, say
from oracle import vsa_oracle as vo

pytestmark = pytest.mark.gpu

vsa = pytest.importorskip("block_sparse_attention_19_amd")

if not torch.cuda.is_available():  # collected on CPU hosts only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)


def _inputs(w, kcount):
    sh = vsa.shape(w.batch, w.heads, w.D, w.T, w.H, w.W)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    qd = bf16_to_dev(q)
    k_t = vsa.tile_permute(bf16_to_dev(k), sh, vsa.LAYOUT_TOKEN_MAJOR)
    v_t = vsa.tile_permute(bf16_to_dev(v), sh, vsa.LAYOUT_FEATURE_MAJOR)
    rp, ci, _ = vsa.build_mask(torch.from_numpy(r).to(dev()), torch.from_numpy(s).to(dev()), sh,
                               kcount, max(w.radius_set))
    return sh, (q, k, v, r, s), qd, k_t, v_t, rp, ci


def _nan_outputs(w):
    o = torch.full((w.batch, w.tokens, w.heads, w.D), float("nan"), dtype=torch.bfloat16,
                   device=dev())
    lse = torch.full((w.batch, w.heads, w.tokens), float("nan"), dtype=torch.float32, device=dev())
    return o, lse


CASES = [  # largest first: each later call reuses a workspace a bigger call filled
    (1, None, None),
    ("custom", (13, 9, 17, 2, 128, (1, 2, 3, 4)), 5),
    ("custom", (8, 16, 16, 2, 64, (1, 2, 3)), 6),
    ("custom", (1, 1, 1, 1, 64, (0,)), 0),
]


def test_noalloc_matches_workspace_call_in_sequence():
    for cid, dims, kcount in CASES:
        if cid == "custom":
            T, H, W, heads, D, rset = dims
            w = wl.custom(T, H, W, heads, D, radius_set=rset, cid=440)
        else:
            w = wl.WORKLOADS[cid]
            kcount = w.dense_counts[0]
        say(f"no-alloc call {w.name} T={w.T} H={w.H} W={w.W} heads={w.heads} D={w.D} k={kcount}")
        sh, host, qd, k_t, v_t, rp, ci = _inputs(w, kcount)
        o_ref, lse_ref = _nan_outputs(w)
        vsa.attn_fwd_raster(qd, k_t, v_t, rp, ci, sh, w.scale, 0, out=o_ref, lse_out=lse_ref)
        o_na, lse_na = _nan_outputs(w)
        vsa.attn_fwd_raster_noalloc(qd, k_t, v_t, rp, ci, sh, w.scale, out=o_na, lse_out=lse_na)
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(o_na), bits_of(o_ref)), f"O differs ({w.name})"
        assert torch.equal(lse_na, lse_ref), f"LSE differs ({w.name})"
        assert torch.isfinite(o_na.float()).all().item()
        if w.tokens <= 4096:
            q, k, v, r, s = host
            ref, _ = vo.attention(q, k, v, r, s, kcount, w.T, w.H, w.W, w.scale)
            assert_close(f64_of(o_na), ref, f"O no-alloc {w.name}")
        del o_ref, lse_ref, o_na, lse_na
    torch.cuda.empty_cache()


def test_noalloc_repeat_same_shape():
    """The same call twice on the shared workspace gives the same bits."""
    w = wl.custom(9, 10, 11, 3, 128, radius_set=(1, 2), cid=441)
    sh, _, qd, k_t, v_t, rp, ci = _inputs(w, 4)
    a, la = vsa.attn_fwd_raster_noalloc(qd, k_t, v_t, rp, ci, sh, w.scale)
    b, lb = vsa.attn_fwd_raster_noalloc(qd, k_t, v_t, rp, ci, sh, w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(a), bits_of(b))
    assert torch.equal(la, lb)
