"""Host-side checks of bench.py (no GPU): the one-GPU guard, and the parity
report of the oracle leg, which compares the oracle rows it computes with a
given raster output."""
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402
from oracle import vsa_oracle as vo  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_oracle_leg_parity_report():
    """The oracle's own output rounded to bf16 (fp32 LSE) passes; one output
    element moved by 0.05 fails on max |dO|, and an LSE moved by 0.01 fails."""
    w = wl.WORKLOADS[0]
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    kc = w.dense_counts[0]
    o_ref, lse_ref = vo.attention(q, k, v, r, s, kc, w.T, w.H, w.W, w.scale)
    o = torch.from_numpy(o_ref.astype(np.float32)).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref.astype(np.float32))
    base, par = bench.cpu_baseline(w, q, k, v, r, s, kc, 0.5, o, lse)
    assert base["kind"] == "oracle" and base["cores"] >= 1
    assert par["pass"], par
    assert 0 < par["max_abs"] <= 2 ** -8            # bf16 rounding of |O| < 1
    assert par["lse_max_abs"] < 1e-5                 # fp32 rounding only
    assert par["rows"] == 64 * par["tiles"]          # the tiny grid has no padded tile

    o_bad = o.clone()
    o_bad[0, :, :, 3] += 0.05                        # feature 3 of every output row
    _, bad = bench.cpu_baseline(w, q, k, v, r, s, kc, 0.5, o_bad, lse)
    assert not bad["pass"] and bad["max_abs"] > 0.04

    lse_bad = lse.clone()
    lse_bad += 0.01                                  # every row
    _, bad = bench.cpu_baseline(w, q, k, v, r, s, kc, 0.5, o, lse_bad)
    assert not bad["pass"] and bad["lse_max_abs"] > 0.009
