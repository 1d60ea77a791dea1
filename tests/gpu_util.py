"""Helpers shared by the GPU tests (device transfer, error statistics, input recipes)."""
import math
import sys

import numpy as np
import torch

from oracle import vsa_oracle as vo

MAX_ABS = 2e-2     # bf16-in / fp32-accumulate output tolerance (max |delta|)
MEAN_REL = 3e-3    # sum |delta| / sum |ref| over compared outputs
LSE_ABS = 2e-3     # fp32 log-sum-exp


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return vo.bf16_to_f64(bits_of(t))


def err_stats(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max()), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


def assert_close(got, ref, what=""):
    mx, mr = err_stats(got, ref)
    say(f"  {what}: max_abs={mx:.3e} mean_rel={mr:.3e} (n={ref.size})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= MAX_ABS, f"{what}: max_abs {mx} > {MAX_ABS}"
    assert mr <= MEAN_REL, f"{what}: mean_rel {mr} > {MEAN_REL}"


def rising_scores(w, q, k, a=0.5, per_tile=10.0):
    """Q and K (bf16 bits, [B, N, heads, D]) reshaped so that scores rise with
    the key tile's index: a shared direction (every feature a) is added to every
    query and, times c(tau), to every key of key tile tau, with c raising the
    score by about `per_tile` log2 units per tile.  A row's running maximum then
    passes the lazy-rescale slack on most of its tiles."""
    import workloads as wl
    tt = vo.token_tile(w.T, w.H, w.W)
    c2 = w.scale / math.log(2.0)
    step = per_tile / (c2 * w.D * a * a)
    qf = vo.bf16_to_f64(q) + a
    kf = vo.bf16_to_f64(k) + (step * tt.astype(np.float64) * a)[None, :, None, None]
    return (wl.f32_to_bf16_bits(qf.astype(np.float32)), wl.f32_to_bf16_bits(kf.astype(np.float32)))
