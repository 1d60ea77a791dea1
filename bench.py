"""Benchmark of one block-sparse video attention call on one MI355X.

A step is the whole path over one batch of synthetic, HBM-resident input:
tile permute of K (token-major) and V (feature-major), CSR mask build from
per-tile radii and routing scores (on a second stream, beside the permutes),
and the block-sparse attention forward
(plan, flash kernel, split combine) of vsa_attn_fwd_raster, which gathers
each query tile's rows from the raster Q and writes every token's output row
to the raster O (the Q permute and the O unpermute, fused).  The same path
with the Q permute and the O unpermute as kernels of their own (vsa_attn_fwd
on tile-major Q and O) is timed beside it (``step_unfused_ms``).  Default workload: the
Wan2.1-1.3B 480p-shaped call, 21x30x52 latent grid (32760 tokens), 12 heads,
head_dim 128, radii in {1, 2, 3}, 20% of query tiles routed dense.

Prints ONE JSON line.  ``value`` is retained-tile bf16 TFLOP/s of the whole
step (kept tile pairs x 4*64*64*D flops over the step time); ``roofline``
rates the attention kernel alone against the bf16 MFMA peak; ``cpu_baseline``
times the fp64 CPU oracle on a bounded sample of the same workload, and
``parity`` compares the oracle rows of that sample with the step's output
(max |dO|, sum |dO| / sum |O|, worst row relative L2, max |dLSE|);
``token_level_calls`` times the per-token -> per-tile calls (budget -> radius,
tile radius, tile score) and ``skim_tier`` the MXFP4 encoding and the tiered
attention call (half / all kept pairs skimmed) at the workload's size, both
outside the step.

Beside the headline, ``configs`` measures every workload and routing point
(Wan2.1-1.3B, the Wan2.2-5B sweep of 20/0/10/40/100% routed, Wan2.1-14B,
HunyuanVideo at the fitted count and all routed): the attention call warm
(median, p10, p90, mean over per-launch events) and cold (1 GiB rewritten
before each launch, so neither the L2 nor the Infinity Cache holds K and V),
the K and V permutes, the mask build and the O unpermute in GB/s of
algorithmic bytes, the step, and the speedup over the dense-mask run of the
same shape.

    python bench.py [--gpus 1] [--steps 30] [--warmup 30] [--workload 1] [--no-configs]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "retained-tile bf16 TFLOP/s (% MFMA peak) + ms/attention call, 32760 tokens"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_traffic_wan2.1-1.3b-480p.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_19_amd", "csrc", "attn.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the clock settles over the first few dozen launches of the call (per-call
    # time falls by ~10% over the first ~25), so the default warm-up is long
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--dense-index", type=int, default=0,
                    help="which routed count of the workload's sweep")
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle sample budget (0 disables the cpu_baseline leg)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload leg (configs)")
    ap.add_argument("--no-side-legs", action="store_true",
                    help="skip the token-level, per-token-window and skim-tier legs")
    ap.add_argument("--cold-reps", type=int, default=8,
                    help="launches timed after a cache flush, per measurement")
    return ap.parse_args()


FLUSH_BYTES = 1 << 30   # rewritten before a cold launch: 4x the 256 MB Infinity Cache


def _pcts(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "mean": round(float(a.mean()), 4),
            "n": int(a.size)}


def time_launches(fn, stream, reps, flush=None):
    """Per-launch durations (ms) of fn() on `stream`, each bracketed by its own
    pair of HIP events; with `flush`, a buffer of FLUSH_BYTES is rewritten
    (read and written) before every launch, outside the bracket."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        if flush is not None:
            flush.add_(1)
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def attn_source_hash() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_figure(n_launch_units: float):
    """HBM bytes per attention launch from committed rocprofv3 counters, or None
    when they were taken on a different version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attn_source_sha") != attn_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# Output tolerance of the bf16-in / fp32-accumulate path against the fp64
# oracle (the same bounds the GPU parity tests assert): max |dO|, sum |dO| /
# sum |O|, and max |dLSE| (natural log).
PARITY_MAX_ABS, PARITY_MEAN_REL, PARITY_LSE_ABS = 2e-2, 3e-3, 2e-3


def cpu_baseline(w, q, k, v, r, s, kcount, budget_s, o_gpu=None, lse_gpu=None):
    """fp64 oracle on sampled query tiles of the same workload, until the time
    budget is spent; rated in retained-tile TFLOP/s like the GPU.

    With the step's GPU output (raster O [1, N, Hh, D] bf16 and LSE [1, Hh, N]
    fp32, host copies), the oracle rows computed for the timing are compared
    with it afterwards, outside the timed loop: returns (baseline, parity)."""
    import numpy as np
    from oracle import vsa_oracle as vo
    # the host cores this process may run on; numpy's BLAS (the oracle's
    # matrix products) is given exactly that many threads
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        limiter = None
    rng = np.random.default_rng(1234)
    tt = vo.token_tile(w.T, w.H, w.W)
    done_tiles, pairs, t0 = 0, 0, time.perf_counter()
    kept = []  # (head, tile, routed, rows, oracle O, oracle LSE) for the parity check
    while time.perf_counter() - t0 < budget_s:
        h = int(rng.integers(w.heads))
        routed = vo.routed_tiles(s[0, h], kcount)
        keep = vo.tile_keep(r[0, h], routed, w.T, w.H, w.W)
        qf, kf, vf = (vo.bf16_to_f64(x[0, :, h]) for x in (q, k, v))
        for a in rng.permutation(w.n_cells)[:8]:
            rows = np.flatnonzero(tt == a)
            ref_o, ref_lse = vo.attention_head_rows(qf, kf, vf, keep, tt, rows, w.scale)
            done_tiles += 1
            pairs += int(keep[a].sum())
            kept.append((h, int(a), bool(routed[a]), rows, ref_o, ref_lse))
    el = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    flops = pairs * 4.0 * 64 * 64 * w.D
    base = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done_tiles} query tiles ({pairs} retained tile pairs) of {w.name}, "
                      f"fp64 masked attention over all keys, {el:.1f} s; full-call "
                      f"extrapolation {el / max(done_tiles, 1) * w.heads * w.n_cells:.0f} s"}
    if o_gpu is None or not kept:
        return base, None
    # parity of the sampled rows: the step's bf16 O and fp32 LSE against the oracle
    got_o = o_gpu[0].float().numpy()       # [N, Hh, D], exact bf16 values
    got_lse = lse_gpu[0].numpy()           # [Hh, N]
    c = vo.tile_coords(w.T, w.H, w.W)
    edge = (4 * (c[:, 0] + 1) > w.T) | (4 * (c[:, 1] + 1) > w.H) | (4 * (c[:, 2] + 1) > w.W)
    max_abs, sum_d, sum_ref, row_l2, lse_abs, n_rows = 0.0, 0.0, 0.0, 0.0, 0.0, 0
    finite = True
    for h, a, _, rows, ref_o, ref_lse in kept:
        g = got_o[rows, h].astype(np.float64)
        d = np.abs(g - ref_o)
        finite &= bool(np.all(np.isfinite(g)))
        max_abs = max(max_abs, float(d.max()))
        sum_d += float(d.sum())
        sum_ref += float(np.abs(ref_o).sum())
        row_l2 = max(row_l2, float((np.linalg.norm(g - ref_o, axis=1) /
                                    np.linalg.norm(ref_o, axis=1)).max()))
        lse_abs = max(lse_abs, float(np.abs(got_lse[h, rows].astype(np.float64) - ref_lse).max()))
        n_rows += len(rows)
    mean_rel = sum_d / max(sum_ref, 1e-300)
    parity = {
        "against": "fp64 oracle (masked softmax over every key of the head)",
        "tiles": len(kept), "distinct_tiles": len({(x[0], x[1]) for x in kept}),
        "routed_tiles": sum(1 for x in kept if x[2]),
        "edge_tiles": sum(1 for x in kept if edge[x[1]]), "rows": n_rows,
        "heads": sorted({x[0] for x in kept}),
        "max_abs": max_abs, "mean_rel": mean_rel, "row_rel_l2_max": row_l2, "lse_max_abs": lse_abs,
        "tolerance": {"max_abs": PARITY_MAX_ABS, "mean_rel": PARITY_MEAN_REL,
                      "lse_max_abs": PARITY_LSE_ABS},
        "pass": bool(finite and max_abs <= PARITY_MAX_ABS and mean_rel <= PARITY_MEAN_REL
                     and lse_abs <= PARITY_LSE_ABS),
    }
    return base, parity


def token_level_calls(w, sh, dev, stream, reps):
    """Time the token-level calls (budget -> radius per query token, token
    radii / scores -> tile radii / scores) at the workload's size on its own
    per-token draws; they are latency-bound, so report microseconds and the
    HBM bytes they move."""
    import numpy as np
    import torch

    import block_sparse_attention_19_amd as vsa
    import workloads as wl
    budget, score = wl.token_inputs(w)
    bd = torch.from_numpy(budget).to(dev)
    sd = torch.from_numpy(score).to(dev)
    r_max = 4
    rad = torch.empty(budget.shape, dtype=torch.uint8, device=dev)
    tr = torch.empty((1, w.heads, w.n_cells), dtype=torch.uint8, device=dev)
    ts = torch.empty((1, w.heads, w.n_cells), dtype=torch.float32, device=dev)
    calls = {
        "budget_to_radius": (lambda: vsa.budget_to_radius(bd, sh, r_max, out=rad), 5),
        "tile_radius_from_tokens": (lambda: vsa.tile_radius_from_tokens(rad, sh, out=tr), 1),
        "tile_score_from_tokens": (lambda: vsa.tile_score_from_tokens(sd, sh, out=ts), 4),
    }
    out = {"r_max": r_max, "tokens_per_head": w.tokens, "heads": w.heads}
    for name, (fn, in_bytes) in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        n_tok = w.heads * w.tokens
        moved = n_tok * in_bytes + (n_tok if name == "budget_to_radius" else w.heads * w.n_cells * (1 if "radius" in name else 4))
        out[name] = {"us": round(us, 2), "hbm_bytes": int(moved), "GB/s": round(moved / (us * 1e-6) / 1e9, 1)}
    return out


def token_windows(w, sh, dev, stream, reps, q_t, k_t, v_t, ws, o_t, kv_chunk, kcount):
    """Exact per-token windows at the workload's size, outside the step: token
    radii from the token budgets (budget -> radius), the mask from their tile
    maxima and the tiles' largest token scores, then the attention call that
    windows each query token by its own radius, beside the block-mask call on
    the same CSR.  Both do the same tile-pair work; the windowed call masks
    the (query token, key tile) pairs outside the token's own window."""
    import numpy as np
    import torch

    import block_sparse_attention_19_amd as vsa
    import workloads as wl
    r_max = max(w.radius_set)
    budget, score = wl.token_inputs(w)
    rad = vsa.budget_to_radius(torch.from_numpy(budget).to(dev), sh, r_max)
    tr = vsa.tile_radius_from_tokens(rad, sh)
    ts = vsa.tile_score_from_tokens(torch.from_numpy(score).to(dev), sh)
    rp, ci, routed = vsa.build_mask(tr, ts, sh, kcount, r_max)
    torch.cuda.synchronize()
    nnz = int(rp[-1].item())

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_w = timed(lambda: vsa.attn_fwd_token_window(q_t, k_t, v_t, rp, ci, routed, rad, sh, r_max,
                                                   w.scale, kv_chunk, out=o_t, workspace=ws,
                                                   with_lse=False))
    ms_b = timed(lambda: vsa.attn_fwd(q_t, k_t, v_t, rp, ci, sh, w.scale, kv_chunk, out=o_t,
                                      workspace=ws, with_lse=False))
    # share of (query token, kept key tile) pairs outside the token's own
    # window, over every 16th local row (host count)
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:nnz].cpu().numpy().astype(np.int64)
    rad_h = rad.cpu().numpy()
    routed_h = routed.cpu().numpy().reshape(-1)
    a_, b_, c_ = w.grid_cells
    coords = np.stack(np.unravel_index(np.arange(w.n_cells), (a_, b_, c_)), axis=1)
    lt, lh, lw = np.unravel_index(np.arange(64), (4, 4, 4))
    out_pairs = all_pairs = 0
    for row in range(0, len(rp_h) - 1, 16):
        if routed_h[row]:
            continue
        h, a = divmod(row, w.n_cells)
        t0, h0, w0 = 4 * coords[a]
        tok = (t0 + lt, h0 + lh, w0 + lw)
        ok = (tok[0] < w.T) & (tok[1] < w.H) & (tok[2] < w.W)
        n = ((tok[0] * w.H + tok[1]) * w.W + tok[2])[ok]
        d = np.abs(coords[ci_h[rp_h[row]:rp_h[row + 1]]] - coords[a])
        dist = d[:, 0] + np.maximum(d[:, 1], d[:, 2])
        r = np.minimum(rad_h[0, h, n].astype(np.int64), r_max)
        all_pairs += r.size * dist.size
        out_pairs += int((dist[None, :] > r[:, None]).sum())
    flops = nnz * 4.0 * 64 * 64 * w.D
    return {"r_max": r_max, "retained_tile_pairs": nnz,
            "windowed_out_share_of_local_pairs": round(out_pairs / max(all_pairs, 1), 4),
            "attn_token_window": {"ms": round(ms_w, 4),
                                  "TFLOP/s": round(flops / (ms_w * 1e-3) / 1e12, 2)},
            "attn_block_mask_same_csr": {"ms": round(ms_b, 4),
                                         "TFLOP/s": round(flops / (ms_b * 1e-3) / 1e12, 2)}}


# (workload, routed-count index) of the per-workload leg, in the order run
CONFIG_POINTS = [(1, 0), (2, 0), (2, 1), (2, 2), (2, 3), (2, 4), (3, 0), (4, 0), (4, 1)]


def configs_leg(stream, cold_reps, flush):
    """Every workload and routing point: attention warm and cold, the K and V
    permutes, the mask build and the O unpermute (GB/s of algorithmic bytes),
    the step, and the dense-mask speedups.  Reps per point are scaled to the
    call's length so the leg stays within a few tens of seconds of GPU time."""
    import numpy as np
    import torch

    import block_sparse_attention_19_amd as vsa
    import workloads as wl
    dev = torch.device("cuda:0")
    out = {}
    by_cid = {}
    for cid, ki in CONFIG_POINTS:
        by_cid.setdefault(cid, []).append(ki)
    for cid, kis in by_cid.items():
        w = wl.WORKLOADS[cid]
        q, k, v = wl.qkv(w)
        r, s = wl.radii_scores(w)
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        del q, k, v
        rd, sd = torch.from_numpy(r).to(dev), torch.from_numpy(s).to(dev)
        sh = vsa.shape(w.batch, w.heads, w.D, w.T, w.H, w.W)
        nT = w.n_cells
        r_max = max(w.radius_set)
        k_t = torch.empty((1, w.heads, nT * 64, w.D), dtype=torch.bfloat16, device=dev)
        v_t = torch.empty((1, w.heads, nT, w.D, 64), dtype=torch.bfloat16, device=dev)
        o = torch.empty_like(qd)
        o_t = torch.empty_like(k_t)
        lse = torch.empty((1, w.heads, w.tokens), dtype=torch.float32, device=dev)
        ws = torch.empty(vsa.attn_workspace_bytes(sh, 0), dtype=torch.uint8, device=dev)
        tok_bytes = w.tokens * w.heads * w.D * 2
        pad_bytes = nT * 64 * w.heads * w.D * 2
        for ki in kis:
            kcount = w.dense_counts[ki]
            mbuf = vsa.mask_buffers(sh, kcount, r_max, dev)
            vsa.tile_permute(kd, sh, vsa.LAYOUT_TOKEN_MAJOR, out=k_t)
            vsa.tile_permute(vd, sh, vsa.LAYOUT_FEATURE_MAJOR, out=v_t)
            vsa.build_mask(rd, sd, sh, kcount, r_max, out=mbuf)
            torch.cuda.synchronize()
            rp, ci = mbuf[0], mbuf[1]
            nnz = int(rp[-1].item())
            flops = nnz * 4.0 * 64 * 64 * w.D

            def attn():
                vsa.attn_fwd_raster(qd, k_t, v_t, rp, ci, sh, w.scale, 0, out=o, workspace=ws,
                                    lse_out=lse)

            def step():
                vsa.tile_permute(kd, sh, vsa.LAYOUT_TOKEN_MAJOR, out=k_t)
                vsa.tile_permute(vd, sh, vsa.LAYOUT_FEATURE_MAJOR, out=v_t)
                vsa.build_mask(rd, sd, sh, kcount, r_max, out=mbuf)
                attn()

            est = max(flops / 1.0e15 * 1e3, 0.5)           # ms at about 1 PFLOP/s
            reps = int(min(30, max(4, 600.0 / est)))
            for _ in range(3):
                attn()
            warm = time_launches(attn, stream, reps)
            cold = time_launches(attn, stream, min(cold_reps, reps), flush=flush)
            steps = time_launches(step, stream, max(3, reps // 2))
            kperm = time_launches(lambda: vsa.tile_permute(kd, sh, vsa.LAYOUT_TOKEN_MAJOR, out=k_t),
                                  stream, 10)
            vperm = time_launches(lambda: vsa.tile_permute(vd, sh, vsa.LAYOUT_FEATURE_MAJOR, out=v_t),
                                  stream, 10)
            mask = time_launches(lambda: vsa.build_mask(rd, sd, sh, kcount, r_max, out=mbuf),
                                 stream, 10)
            unperm = time_launches(lambda: vsa.tile_unpermute(o_t, sh, out=o), stream, 10)
            rows = w.heads * nT
            mask_bytes = rows * (1 + 4) + 4 * (rows + 1) + 4 * nnz + rows   # radii, scores, row_ptr, col_idx, routed
            gbs = lambda b, ms: round(b / (float(np.median(ms)) * 1e-3) / 1e9, 1)
            wp = _pcts(warm)
            key = f"{w.name}@k={kcount}"
            out[key] = {
                "workload": w.name, "tokens": w.tokens, "heads": w.heads, "head_dim": w.D,
                "tiles": nT, "dense_count": kcount, "routed_fraction": round(kcount / nT, 4),
                "retained_tile_pairs": nnz, "tile_pair_density": round(nnz / (w.heads * nT * nT), 4),
                "attn_ms_warm": wp, "attn_ms_cold": _pcts(cold),
                "attn_TFLOP/s": round(flops / (wp["mean"] * 1e-3) / 1e12, 2),
                "attn_frac_of_bf16_peak": round(flops / (wp["mean"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "attn_frac_cold": round(flops / (_pcts(cold)["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "step_ms": _pcts(steps)["median"],
                "permute_k": {"ms": round(float(np.median(kperm)), 4), "GB/s": gbs(tok_bytes + pad_bytes, kperm)},
                "permute_v": {"ms": round(float(np.median(vperm)), 4), "GB/s": gbs(tok_bytes + pad_bytes, vperm)},
                "mask_build": {"ms": round(float(np.median(mask)), 4), "GB/s": gbs(mask_bytes, mask),
                               "bytes": int(mask_bytes)},
                "unpermute_o": {"ms": round(float(np.median(unperm)), 4), "GB/s": gbs(2 * tok_bytes, unperm)},
            }
            del mbuf
        del qd, kd, vd, k_t, v_t, o, o_t, lse, ws
        torch.cuda.empty_cache()
    # dense-mask speedup: the same shape with every query tile routed
    for name, sparse_k, dense_k in (("hunyuanvideo-720p-129f", wl.WORKLOADS[4].dense_counts[0],
                                     wl.WORKLOADS[4].dense_counts[1]),
                                    ("wan2.2-5b-720p", wl.WORKLOADS[2].dense_counts[0],
                                     wl.WORKLOADS[2].dense_counts[4])):
        a, b = out.get(f"{name}@k={sparse_k}"), out.get(f"{name}@k={dense_k}")
        if a and b:
            a["speedup_vs_dense_mask"] = round(b["attn_ms_warm"]["mean"] / a["attn_ms_warm"]["mean"], 3)
    return out


PEAK_FP4_TFLOPS = 10100.0  # MI355X dense FP4 MFMA (the skim tier's score products)


def skim_tier(w, sh, dev, stream, reps, q_t, k_t, v_t, rp, ci, nnz, ws, o_t, kv_chunk):
    """The low-precision tier at the workload's size, outside the step: the
    MXFP4 encoding of Q and K, and the tiered attention call with 0, 1/4, 1/2,
    3/4 and all of the kept pairs skimmed, tiers drawn i.i.d. per pair and
    (1/4, 1/2, 3/4) per key tile.  Each speedup is over the bf16 call on the
    same CSR, timed in this leg.  Its bound mixes two peaks: a skim pair's
    Q.K^T (2*64*64*D flops) at the FP4 rate, everything else (its P.V, both
    products of a refine pair) at the bf16 rate."""
    import numpy as np
    import torch

    import block_sparse_attention_19_amd as vsa
    import workloads as wl
    rows = q_t.shape[2] * w.heads
    q4 = (torch.empty(q_t.shape[:3] + (w.D // 2,), dtype=torch.uint8, device=dev),
          torch.empty(q_t.shape[:3] + (w.D // 32,), dtype=torch.uint8, device=dev))
    k4 = (torch.empty_like(q4[0]), torch.empty_like(q4[1]))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    q_ms = timed(lambda: (vsa.quantize_mxfp4(q_t, sh, *q4), vsa.quantize_mxfp4(k_t, sh, *k4)))
    moved = 2 * rows * (w.D * 2 + w.D // 2 + w.D // 32)
    out = {"quantize_qk": {"us": round(q_ms * 1e3, 2), "hbm_bytes": int(moved),
                           "GB/s": round(moved / (q_ms * 1e-3) / 1e9, 1)}}
    pair = 2.0 * 64 * 64 * w.D  # flops of one product of one kept pair
    bf16_ms = timed(lambda: vsa.attn_fwd(q_t, k_t, v_t, rp, ci, sh, w.scale, kv_chunk, out=o_t,
                                         workspace=ws, with_lse=False))
    out["bf16_call_ms"] = round(bf16_ms, 4)
    rp_h, ci_h = rp.cpu().numpy(), ci[:nnz].cpu().numpy()
    recipes = [("", p, lambda p: wl.tiers(w, nnz, p)) for p in (0.0, 0.25, 0.5, 0.75, 1.0)]
    recipes += [("_by_key_tile", p, lambda p: wl.tiers_by_key_tile(w, rp_h, ci_h, p))
                for p in (0.25, 0.5, 0.75)]
    for tag, p_skim, draw in recipes:
        tier = torch.from_numpy(draw(p_skim)).to(dev)
        n_skim = int(tier.sum().item())
        ms = timed(lambda: vsa.attn_fwd_tiered(q_t, k_t, v_t, q4, k4, rp, ci, tier, sh, w.scale,
                                               kv_chunk, out=o_t, workspace=ws, with_lse=False))
        bound_ms = ((2 * nnz - n_skim) * pair / (PEAK_BF16_TFLOPS * 1e12) +
                    n_skim * pair / (PEAK_FP4_TFLOPS * 1e12)) * 1e3
        out[f"attn_tiered_p{p_skim}{tag}"] = {
            "skim_pairs": n_skim, "ms": round(ms, 4),
            "TFLOP/s": round(2 * nnz * pair / (ms * 1e-3) / 1e12, 2),
            "mixed_peak_ms": round(bound_ms, 4), "frac": round(bound_ms / ms, 4),
            "speedup_vs_bf16_call": round(bf16_ms / ms, 3)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_attention_19_amd as vsa
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    kcount = w.dense_counts[args.dense_index]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = wl.qkv(w)
    r, s = wl.radii_scores(w)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    rd, sd = torch.from_numpy(r).to(dev), torch.from_numpy(s).to(dev)
    sh = vsa.shape(w.batch, w.heads, w.D, w.T, w.H, w.W)
    nT = w.n_cells
    r_max = max(w.radius_set)
    # every buffer is allocated before the timed region
    q_t = torch.empty((1, w.heads, nT * 64, w.D), dtype=torch.bfloat16, device=dev)
    k_t = torch.empty_like(q_t)
    v_t = torch.empty((1, w.heads, nT, w.D, 64), dtype=torch.bfloat16, device=dev)
    o_t = torch.empty_like(q_t)
    lse = torch.empty((1, w.heads, nT * 64), dtype=torch.float32, device=dev)
    o = torch.empty_like(qd)
    lse_r = torch.empty((1, w.heads, w.tokens), dtype=torch.float32, device=dev)
    mbuf = vsa.mask_buffers(sh, kcount, r_max, dev)
    ws = torch.empty(vsa.attn_workspace_bytes(sh, args.kv_chunk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    stages = ["permute_kv_and_mask", "attn"]
    # The mask build (a few small, latency-bound kernels) runs on a second
    # stream, default priority, beside the bandwidth-bound K and V permutes.
    side = torch.cuda.Stream(device=dev)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        side.wait_stream(stream)  # the previous step's attention has read the CSR
        with torch.cuda.stream(side):
            rp, ci, _ = vsa.build_mask(rd, sd, sh, kcount, r_max, out=mbuf)
        vsa.tile_permute(kd, sh, vsa.LAYOUT_TOKEN_MAJOR, out=k_t)
        vsa.tile_permute(vd, sh, vsa.LAYOUT_FEATURE_MAJOR, out=v_t)
        stream.wait_stream(side)
        mark(1)
        vsa.attn_fwd_raster(qd, k_t, v_t, rp, ci, sh, w.scale, args.kv_chunk, out=o,
                            workspace=ws, lse_out=lse_r)
        mark(2)

    def step_unfused():
        vsa.tile_permute(qd, sh, vsa.LAYOUT_TOKEN_MAJOR, out=q_t)
        vsa.tile_permute(kd, sh, vsa.LAYOUT_TOKEN_MAJOR, out=k_t)
        vsa.tile_permute(vd, sh, vsa.LAYOUT_FEATURE_MAJOR, out=v_t)
        rp, ci, _ = vsa.build_mask(rd, sd, sh, kcount, r_max, out=mbuf)
        vsa.attn_fwd(q_t, k_t, v_t, rp, ci, sh, w.scale, args.kv_chunk, out=o_t, workspace=ws,
                     lse_out=lse)
        vsa.tile_unpermute(o_t, sh, out=o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_all1.record(stream)
    torch.cuda.synchronize()
    ms_step = t_all0.elapsed_time(t_all1) / args.steps
    per_stage = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
                 for j, n in enumerate(stages)}
    # the unfused path (tile-major Q and O, permute and unpermute as kernels);
    # it also leaves the tile-major Q in q_t for the side measurements below
    u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    u0.record(stream)
    for _ in range(args.steps):
        step_unfused()
    u1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = u0.elapsed_time(u1) / args.steps
    # the tile-major call alone (the reference of the side measurements)
    rp_, ci_ = mbuf[0], mbuf[1]
    u0.record(stream)
    for _ in range(args.steps):
        vsa.attn_fwd(q_t, k_t, v_t, rp_, ci_, sh, w.scale, args.kv_chunk, out=o_t, workspace=ws,
                     lse_out=lse)
    u1.record(stream)
    torch.cuda.synchronize()
    ms_attn_tiled = u0.elapsed_time(u1) / args.steps
    # per-launch attention durations of the timed steps, and the same call
    # cold: 1 GiB rewritten before each launch (the step's K and V permutes
    # otherwise leave K and V in the Infinity Cache for the attention call)
    attn_launch_ms = [e[1].elapsed_time(e[2]) for e in evs]
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    rp_, ci_ = mbuf[0], mbuf[1]
    cold_attn = time_launches(lambda: vsa.attn_fwd_raster(qd, k_t, v_t, rp_, ci_, sh, w.scale,
                                                          args.kv_chunk, out=o, workspace=ws,
                                                          lse_out=lse_r),
                              stream, args.cold_reps, flush=flush)
    cold_step = time_launches(step, stream, args.cold_reps, flush=flush)
    # the step's output (raster O and LSE of the last step), for the parity
    # check of the oracle leg
    torch.cuda.synchronize()
    o_host, lse_host = (o.cpu(), lse_r.cpu()) if args.cpu_seconds > 0 else (None, None)
    nnz = int(mbuf[0][-1].item())
    flops = nnz * 4.0 * 64 * 64 * w.D
    # valid-token flops: each kept pair weighted by valid queries x valid keys
    rp_h = mbuf[0].cpu().numpy().astype(np.int64)
    ci_h = mbuf[1][:nnz].cpu().numpy().astype(np.int64)
    a, b, c = w.grid_cells
    per = [np.minimum(4, n - 4 * np.arange(m)) for n, m in ((w.T, a), (w.H, b), (w.W, c))]
    valid = (per[0][:, None, None] * per[1][None, :, None] * per[2][None, None, :]).ravel()
    row_tile = np.repeat(np.arange(len(rp_h) - 1) % nT, np.diff(rp_h))
    valid_flops = 4.0 * w.D * float(np.sum(valid[row_tile] * valid[ci_h]))
    attn_ms = per_stage["attn"]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Wan/HunyuanVideo-shaped Q/K/V, radii, routing scores)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "W": w.W, "tokens": w.tokens,
                   "heads": w.heads, "head_dim": w.D, "batch": w.batch, "tiles": nT,
                   "radius_set": list(w.radius_set), "dense_count": kcount,
                   "retained_tile_pairs": nnz, "tile_pair_density": round(nnz / (w.heads * nT * nT), 4),
                   "kv_chunk": args.kv_chunk, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_figure(1.0),
                     "traffic_basis": "bytes beyond the XCD L2s per attn_kernel launch "
                                      "(TCC FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel); "
                                      "the Infinity Cache may serve part of them, no counter "
                                      "separates its hits from HBM",
                     "kernel": "vsa_attn_fwd_raster (plan + attn_kernel + combine_kernel)"},
        "attn_ms_warm": _pcts(attn_launch_ms),
        "attn_ms_cold": _pcts(cold_attn),
        "attn_frac_cold": round(flops / (float(np.median(cold_attn)) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "step_ms_cold": _pcts(cold_step),
        "breakdown_ms": {k2: round(v2, 4) for k2, v2 in per_stage.items()},
        "step_unfused_ms": round(ms_unfused, 4),
        "attn_tile_major_ms": round(ms_attn_tiled, 4),
        "attn_valid_token_tflops": round(valid_flops / (attn_ms * 1e-3) / 1e12, 2),
    }
    if not args.no_side_legs:
        line["token_level_calls"] = token_level_calls(w, sh, dev, stream, args.steps)
        line["token_windows"] = token_windows(w, sh, dev, stream, args.steps, q_t, k_t, v_t, ws,
                                              o_t, args.kv_chunk, kcount)
        line["skim_tier"] = skim_tier(w, sh, dev, stream, args.steps, q_t, k_t, v_t, mbuf[0],
                                      mbuf[1], nnz, ws, o_t, args.kv_chunk)
    del q_t, o_t, lse
    if not args.no_configs:
        line["configs"] = configs_leg(stream, args.cold_reps, flush)
    if args.cpu_seconds > 0:
        line["cpu_baseline"], line["parity"] = cpu_baseline(w, q, k, v, r, s, kcount,
                                                            args.cpu_seconds, o_host, lse_host)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
