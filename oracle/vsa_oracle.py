"""fp64 CPU definition of block-sparse video attention (test infrastructure).

What is computed, and where it comes from:

* Token grid and tile-major order -- "Token Radius Attention for Efficient
  Video Generation" (TRA), pipeline step 3: tokens are reordered tile-major so
  that sparse supports become whole blocks.  Reading adopted here: cubic
  4x4x4 tiles; tiles in raster order (tt, th, tw) with tw fastest; inside a
  tile raster order (lt, lh, lw) with lw fastest; grid edges padded up to whole
  tiles with zeros.
* Local window with temporal decay -- TRA, pipeline step 2: a per-query base
  radius applied across frames with a temporal distance-decay rule, giving
  regular spatio-temporal supports.  Reading adopted here, at tile
  granularity: query tile a with radius r keeps key tile b iff
  |dt| <= r and max(|dh|, |dw|) <= r - |dt|, with (dt, dh, dw) = c(b) - c(a).
* Dense routing -- "Where Compute Matters: Heterogeneous Attention for
  Efficient Video Diffusion" (HetA-DiT), abstract: uncertain tokens go through
  dense global attention, the rest through local attention, about 20% dense.
  Reading adopted here: per (batch, head), the k query tiles with the highest
  routing score attend to every key tile; ties are broken by the IEEE-754 total
  order of the float32 score, then by lower tile index.
* Attention -- softmax(scale * q.k) v over the kept keys only, i.e. the
  block-sparse mask applied to ordinary scaled-dot-product attention; the
  block-sparse execution of TRA step 3 and of the other pages skips masked
  tiles and must reach this same result.

* Exact per-token windows -- TRA, pipeline steps 2 and 3: radii are
  assigned per query token and translated into block masks.  The block mask
  uses each tile's largest token radius; the exact variant lets every query
  token attend only the key tiles of its own radius's window (routed tiles
  still attend every key tile).

* Low-precision tier -- "Triage: Skip, Skim, or Refine Attention Tiles in
  Video Diffusion Transformers": each kept tile pair is either computed in a
  quick 4-bit version (skim) or fully (refine).  Reading adopted here: an
  input tier per kept pair; a skim pair's scores use the MXFP4 (OCP MX v1.0)
  round trips of q and k, the rest is unchanged.

The oracle works on the valid tokens only (it has no padding); padded slots
exist only in the tile-major layout.  All floating point is float64 on the
exact bfloat16 input values.
"""
from __future__ import annotations

import math
from typing import Iterable, Tuple

import numpy as np

TILE = 4          # tile edge in tokens, along t, h and w
TILE_TOKENS = 64  # TILE ** 3


# ---------------------------------------------------------------- data format

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ tile grid

def tile_grid(T: int, H: int, W: int) -> Tuple[int, int, int]:
    """Number of tiles along t, h, w (edges padded up to whole tiles)."""
    return (math.ceil(T / TILE), math.ceil(H / TILE), math.ceil(W / TILE))


def num_tiles(T: int, H: int, W: int) -> int:
    a, b, c = tile_grid(T, H, W)
    return a * b * c


def tile_coords(T: int, H: int, W: int) -> np.ndarray:
    """(nT, 3) int array: tile coordinates (tt, th, tw) of tile index tau."""
    a, b, c = tile_grid(T, H, W)
    tt, th, tw = np.meshgrid(np.arange(a), np.arange(b), np.arange(c), indexing="ij")
    return np.stack([tt.ravel(), th.ravel(), tw.ravel()], axis=1)


def token_tile(T: int, H: int, W: int) -> np.ndarray:
    """Tile index of every token, tokens in raster order n = (t*H + h)*W + w."""
    a, b, c = tile_grid(T, H, W)
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return (((t // TILE) * b + (h // TILE)) * c + (w // TILE)).ravel()


# ------------------------------------------------------------------- routing

def total_order_key(scores: np.ndarray) -> np.ndarray:
    """Map float32 values to uint32 keys whose unsigned order is the IEEE-754
    totalOrder of the floats (-NaN < -inf < ... < -0 < +0 < ... < +inf < +NaN)."""
    bits = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    neg = (bits >> np.uint32(31)).astype(bool)
    return np.where(neg, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)


def routing_order(scores: np.ndarray) -> np.ndarray:
    """Tile indices in routing order: score descending in IEEE total order,
    then tile index ascending."""
    n = scores.shape[0]
    key = total_order_key(scores).astype(np.int64)
    return np.lexsort((np.arange(n), -key))  # primary: -key, secondary: index


def routed_tiles(scores: np.ndarray, k: int) -> np.ndarray:
    """Bool [nT]: the first k tiles of the routing order.  HetA-DiT abstract:
    route the most uncertain part to dense attention."""
    n = scores.shape[0]
    if not 0 <= k <= n:
        raise ValueError("routed count out of range")
    out = np.zeros(n, dtype=bool)
    out[routing_order(scores)[:k]] = True
    return out


# --------------------------------------------------------------- tile window

def tile_keep(radii: np.ndarray, routed: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """Bool [nT, nT]: keep[a, b] -- does query tile a attend to key tile b.

    TRA step 2 (radius with temporal decay) for local tiles; HetA-DiT routing
    (every key) for routed tiles."""
    c = tile_coords(T, H, W)
    d = np.abs(c[None, :, :] - c[:, None, :])          # [a, b, 3]
    dt, dsp = d[..., 0], np.maximum(d[..., 1], d[..., 2])
    r = np.asarray(radii, dtype=np.int64)[:, None]
    local = (dt <= r) & (dsp <= r - dt)
    return local | np.asarray(routed, dtype=bool)[:, None]


def block_mask(radii: np.ndarray, scores: np.ndarray, k: int, T: int, H: int, W: int):
    """Per (b, h) tile masks: bool [B, Hh, nT, nT], and routed flags [B, Hh, nT]."""
    B, Hh, n = radii.shape
    keep = np.zeros((B, Hh, n, n), dtype=bool)
    routed = np.zeros((B, Hh, n), dtype=bool)
    for b in range(B):
        for h in range(Hh):
            routed[b, h] = routed_tiles(scores[b, h], k)
            keep[b, h] = tile_keep(radii[b, h], routed[b, h], T, H, W)
    return keep, routed


def csr(keep: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """CSR of a stack of tile masks [..., nT, nT], rows in C order of the leading
    dims then query tile.  Columns ascending (np.nonzero order).  Returns
    (row_ptr int64 [rows + 1], col_idx int64 [nnz])."""
    n = keep.shape[-1]
    flat = keep.reshape(-1, n)
    rows, cols = np.nonzero(flat)
    lengths = np.bincount(rows, minlength=flat.shape[0])
    row_ptr = np.zeros(flat.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=row_ptr[1:])
    return row_ptr, cols.astype(np.int64)


# ------------------------------------------------------------ tile-major layout

def permute(x: np.ndarray, T: int, H: int, W: int, transposed: bool = False) -> np.ndarray:
    """Raster [B, N, Hh, D] -> tile-major [B, Hh, nT*64, D], padded slots zero.

    TRA step 3, tile-major token layout.  With ``transposed`` the tile is stored
    feature-major instead: [B, Hh, nT, D, 64] (the 64 tokens of a tile are
    contiguous for each feature)."""
    B, N, Hh, D = x.shape
    assert N == T * H * W
    a, b, c = tile_grid(T, H, W)
    xp = np.zeros((B, a * TILE, b * TILE, c * TILE, Hh, D), dtype=x.dtype)
    xp[:, :T, :H, :W] = x.reshape(B, T, H, W, Hh, D)
    xp = xp.reshape(B, a, TILE, b, TILE, c, TILE, Hh, D)
    # axes: 0 B, 1 tt, 2 lt, 3 th, 4 lh, 5 tw, 6 lw, 7 Hh, 8 D
    if transposed:
        xp = xp.transpose(0, 7, 1, 3, 5, 8, 2, 4, 6)
        return np.ascontiguousarray(xp).reshape(B, Hh, a * b * c, D, TILE_TOKENS)
    xp = xp.transpose(0, 7, 1, 3, 5, 2, 4, 6, 8)
    return np.ascontiguousarray(xp).reshape(B, Hh, a * b * c * TILE_TOKENS, D)


def unpermute(xt: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """Tile-major [B, Hh, nT*64, D] -> raster [B, N, Hh, D]; padded rows dropped."""
    B, Hh, S, D = xt.shape
    a, b, c = tile_grid(T, H, W)
    assert S == a * b * c * TILE_TOKENS
    x = xt.reshape(B, Hh, a, b, c, TILE, TILE, TILE, D)
    # axes: 0 B, 1 Hh, 2 tt, 3 th, 4 tw, 5 lt, 6 lh, 7 lw, 8 D
    x = x.transpose(0, 2, 5, 3, 6, 4, 7, 1, 8)
    x = x.reshape(B, a * TILE, b * TILE, c * TILE, Hh, D)[:, :T, :H, :W]
    return np.ascontiguousarray(x).reshape(B, T * H * W, Hh, D)


# ------------------------------------------------------------------ attention

def masked_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          mask_rows: np.ndarray, scale: float):
    """Softmax attention of query rows q [R, D] over keys k, v [N, D] with a
    boolean mask [R, N] (False = key not attended).  float64.

    Returns (O [R, D], LSE [R]) with LSE = ln sum_j exp(scale * q.k_j) over kept
    keys.  Stable form: subtract the row max of the kept scores."""
    s = scale * (q @ k.T)
    s = np.where(mask_rows, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / l
    return o, (m + np.log(l))[:, 0]


def attention_head_rows(q, k, v, keep: np.ndarray, tok_tile: np.ndarray,
                        rows: np.ndarray, scale: float):
    """Rows ``rows`` (token indices) of one head.  q, k, v: float64 [N, D];
    keep: tile mask [nT, nT]; tok_tile: tile of each token."""
    mask = keep[tok_tile[rows]][:, tok_tile]   # token-level mask [R, N]
    return masked_attention_rows(q[rows], k, v, mask, scale)


def attention(q_bits, k_bits, v_bits, radii, scores, k: int, T: int, H: int, W: int,
              scale: float):
    """Full block-sparse attention, every valid query of every (b, h).

    q/k/v: bf16 bits [B, N, Hh, D].  Returns O float64 [B, N, Hh, D] and
    LSE float64 [B, Hh, N].  Cost 4*N*N*D per head: small grids only."""
    B, N, Hh, _ = q_bits.shape
    keep, _ = block_mask(radii, scores, k, T, H, W)
    tt = token_tile(T, H, W)
    O = np.zeros((B, N, Hh, v_bits.shape[-1]))
    L = np.zeros((B, Hh, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hh):
            q = bf16_to_f64(q_bits[b, :, h])
            kk = bf16_to_f64(k_bits[b, :, h])
            vv = bf16_to_f64(v_bits[b, :, h])
            O[b, :, h], L[b, h] = attention_head_rows(q, kk, vv, keep[b, h], tt, rows, scale)
    return O, L


# ------------------------------------------------ low-precision "skim" tiles
#
# "Triage: Skip, Skim, or Refine Attention Tiles in Video Diffusion
# Transformers", plain-words summary and "Route by estimated error": every
# tile is skipped, computed in a quick 4-bit version ("skim"), or computed
# with extra correction ("refine").  The pages fix neither the 4-bit format,
# nor which products it covers, nor the router's formulas.  Readings adopted
# here: the tier is an input (one byte per kept tile pair, 1 = skim); the
# 4-bit format is OCP Microscaling MXFP4 (E2M1 elements, one power-of-two E8M0
# scale per block of 32 consecutive elements along the head dimension); a skim
# pair takes its scores from the MXFP4-quantised q and k, everything after the
# scores (softmax, P.V) as for a refine pair, which is the bf16 computation.

MX_BLOCK = 32                      # elements sharing one scale
E2M1_EMAX = 2                      # exponent of the largest E2M1 binade (4..6)
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # by code & 7


def mxfp4_quantize(x: np.ndarray):
    """MXFP4 encoding along the last axis (its length a multiple of 32), as the
    OCP Microscaling Formats specification v1.0 defines it: the block scale is
    X = 2^(floor(log2(max |v|)) - emax) with emax = 2 for E2M1 (exponent -127,
    the smallest E8M0 value, for an all-zero block; clamped to [-127, 127]),
    and each v / X is rounded to the nearest E2M1 value, ties to the even code,
    magnitudes above 6 saturating to 6.

    Returns (codes uint8 [..., n]: bit 3 sign, bits 0-2 the magnitude index into
    E2M1_MAGNITUDES; exponents int32 [..., n/32]: X = 2^exponent)."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)                          # amax = f * 2^e, f in [0.5, 1)
    expo = np.where(amax > 0, e - 1 - E2M1_EMAX, -127)
    expo = np.clip(expo, -127, 127).astype(np.int32)
    y = blocks / np.ldexp(1.0, expo)[..., None]
    mag = np.abs(y)[..., None]
    dist = np.abs(mag - E2M1_MAGNITUDES)           # [..., 32, 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                            # one or two nearest values
    even = cand & ((np.arange(8) & 1) == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    codes = (idx | np.where(np.signbit(y), 8, 0)).astype(np.uint8)
    return codes.reshape(x.shape), expo


def mxfp4_dequantize(codes: np.ndarray, expo: np.ndarray) -> np.ndarray:
    """Values of MXFP4 codes: sign * E2M1 magnitude * 2^exponent of the block."""
    codes = np.asarray(codes)
    mag = E2M1_MAGNITUDES[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    blocks = val.reshape(codes.shape[:-1] + (codes.shape[-1] // MX_BLOCK, MX_BLOCK))
    out = blocks * np.ldexp(1.0, np.asarray(expo, dtype=np.int64))[..., None]
    return out.reshape(codes.shape)


def skim_values(x: np.ndarray) -> np.ndarray:
    """What a skim pair sees of q or k: the MXFP4 round trip of each vector."""
    return mxfp4_dequantize(*mxfp4_quantize(x))


def tiered_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask_rows: np.ndarray,
                          skim_rows: np.ndarray, scale: float):
    """masked_attention_rows with per-pair tiers: where skim_rows [R, N] is
    True the score is scale * (q^ . k^) of the MXFP4 round trips, elsewhere
    scale * (q . k).  Softmax and P.V are unchanged."""
    s = scale * np.where(skim_rows, skim_values(q) @ skim_values(k).T, q @ k.T)
    s = np.where(mask_rows, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l, (m + np.log(l))[:, 0]


def tiered_attention_head(q, k, v, keep: np.ndarray, skim: np.ndarray, tok_tile: np.ndarray,
                          rows: np.ndarray, scale: float):
    """Rows ``rows`` of one head with tile masks keep [nT, nT] and skim [nT, nT]
    (skim only matters where keep is True)."""
    tq = tok_tile[rows]
    return tiered_attention_rows(q[rows], k, v, keep[tq][:, tok_tile], skim[tq][:, tok_tile], scale)


def csr_tiers_to_tiles(row_ptr: np.ndarray, col_idx: np.ndarray, tier: np.ndarray, rows: int,
                       nT: int) -> np.ndarray:
    """Bool [rows, nT]: the skim flag of every kept (row, key tile) of a CSR
    with one tier byte per entry (non-zero = skim)."""
    out = np.zeros((rows, nT), dtype=bool)
    for r in range(rows):
        b, e = int(row_ptr[r]), int(row_ptr[r + 1])
        out[r, col_idx[b:e]] = np.asarray(tier[b:e]) != 0
    return out


# ------------------------------------------------------------ split merging

def merge_partials(parts: Iterable[Tuple[np.ndarray, np.ndarray, np.ndarray]]):
    """Exact merge of attention over disjoint key subsets.

    Each part is (o_unnormalised [R, D], m [R], l [R]) where, over the part's
    keys, m = max score, l = sum exp(s - m), o = sum exp(s - m) v.  Returns the
    normalised output and the LSE over the union: with M = max m_s,
    L = sum_s exp(m_s - M) l_s, O = sum_s exp(m_s - M) o_s / L, LSE = M + ln L."""
    parts = list(parts)
    M = np.max(np.stack([p[1] for p in parts]), axis=0)
    L = np.zeros_like(M)
    O = np.zeros_like(parts[0][0])
    for o, m, l in parts:
        w = np.where(np.isfinite(m), np.exp(m - M), 0.0)
        L += w * l
        O += w[:, None] * o
    return O / L[:, None], M + np.log(L)


def partial_attention(q, k, v, scale: float):
    """Unnormalised attention of q [R, D] over one key subset k, v [n, D]:
    (o, m, l) as merge_partials expects."""
    s = scale * (q @ k.T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return p @ v, m, p.sum(axis=1)


# ------------------------------------------------------------- derived counts

def window_count_closed_form(r: int) -> int:
    """Key tiles kept by an interior (unclipped) query tile of radius r:
    sum over dt in [-r, r] of the (2(r-|dt|)+1)^2 spatial square."""
    return sum((2 * (r - abs(dt)) + 1) ** 2 for dt in range(-r, r + 1))


# ------------------------------------------- token-level inputs -> tile inputs
#
# TRA's pipeline produces one budget and one radius per query *token* (steps 1
# and 2) and translates the token-level radii into block masks (step 3);
# HetA-DiT predicts a difficulty per token.  The block mask above takes one
# radius and one routing score per query *tile*.  These functions make the
# connection, with the readings: budgets count key tokens; a token's radius is
# the smallest r in [0, r_max] whose tile window (the rule of tile_keep) holds
# at least its budget of real key tokens, r_max if none does; a tile's radius
# is the largest radius among its real tokens (its window then contains every
# token's window); a tile's routing score is the largest score among its real
# tokens in the IEEE-754 total order (the tile is routed if any of its tokens
# is among the most uncertain).  Per-token arrays are [N] in raster order.

def tile_valid_tokens(T: int, H: int, W: int) -> np.ndarray:
    """int64 [nT]: real (non-padding) tokens of every tile, by counting."""
    return np.bincount(token_tile(T, H, W), minlength=num_tiles(T, H, W)).astype(np.int64)


def window_tokens(radius: int, T: int, H: int, W: int) -> np.ndarray:
    """int64 [nT]: real key tokens inside the local window of each query tile
    when every tile has radius `radius` and none is routed (brute force over
    the tile_keep matrix)."""
    n = num_tiles(T, H, W)
    keep = tile_keep(np.full(n, radius, dtype=np.int64), np.zeros(n, dtype=bool), T, H, W)
    return keep.astype(np.int64) @ tile_valid_tokens(T, H, W)


def budget_to_radius(budget: np.ndarray, r_max: int, T: int, H: int, W: int) -> np.ndarray:
    """TRA step 2 (budget -> base radius): uint8 [N] radius per query token for
    int [N] token budgets."""
    tt = token_tile(T, H, W)
    counts = np.stack([window_tokens(r, T, H, W) for r in range(r_max + 1)])  # [r_max+1, nT]
    enough = counts[:, tt] >= np.asarray(budget, dtype=np.int64)[None, :]
    radius = np.where(enough.any(axis=0), enough.argmax(axis=0), r_max)
    return radius.astype(np.uint8)


def tile_radius_from_tokens(token_radius: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """TRA step 3 (token-level radii -> block mask input): uint8 [nT], the
    largest radius among each tile's real tokens."""
    out = np.zeros(num_tiles(T, H, W), dtype=np.uint8)
    np.maximum.at(out, token_tile(T, H, W), np.asarray(token_radius, dtype=np.uint8))
    return out


def tile_score_from_tokens(token_score: np.ndarray, T: int, H: int, W: int) -> np.ndarray:
    """HetA-DiT routing at tile granularity: float32 [nT], the token score of
    each tile that is largest in the IEEE-754 total order."""
    s = np.asarray(token_score, dtype=np.float32)
    key = total_order_key(s).astype(np.int64)
    best = np.full(num_tiles(T, H, W), -1, dtype=np.int64)
    np.maximum.at(best, token_tile(T, H, W), key)
    # back from the key to the float's bits (total_order_key inverted)
    bits = np.where(best >= 2 ** 31, best - 2 ** 31, (~best) & 0xFFFFFFFF).astype(np.uint32)
    return bits.view(np.float32)


# ----------------------------------------------------- exact per-token windows
#
# TRA, pipeline step 3, turns the token-level radii into block masks; the
# block mask of a tile uses the largest radius among its tokens, so it holds
# every token's window.  Reading adopted for the exact variant: query token i
# attends the real key tokens of the key tiles inside the window of its own
# radius r_i (clamped to r_max like the tile radii) around its tile -- the
# tile_keep rule with r_i -- or of every key tile if its tile is routed.

def token_window_keep(token_radius: np.ndarray, routed: np.ndarray, r_max: int,
                      T: int, H: int, W: int) -> np.ndarray:
    """Bool [N, nT]: does query token i attend to key tile b."""
    tt = token_tile(T, H, W)
    n = num_tiles(T, H, W)
    r = np.minimum(np.asarray(token_radius, dtype=np.int64), r_max)
    out = np.zeros((len(tt), n), dtype=bool)
    for rv in np.unique(r):
        sel = r == rv
        out[sel] = tile_keep(np.full(n, rv), routed, T, H, W)[tt[sel]]
    return out


def token_window_attention_rows(q, k, v, keep_tok: np.ndarray, tok_tile: np.ndarray,
                                rows: np.ndarray, scale: float):
    """Rows ``rows`` of one head under per-token windows keep_tok [N, nT]."""
    return masked_attention_rows(q[rows], k, v, keep_tok[rows][:, tok_tile], scale)


def token_window_attention(q_bits, k_bits, v_bits, token_radius, scores, k: int, r_max: int,
                           T: int, H: int, W: int, scale: float):
    """Every valid query of every (b, h) under per-token windows.  token_radius:
    uint8 [B, Hh, N] (raster order); scores: float32 [B, Hh, nT] tile routing
    scores.  Returns O float64 [B, N, Hh, D] and LSE [B, Hh, N]."""
    B, N, Hh, _ = q_bits.shape
    tt = token_tile(T, H, W)
    O = np.zeros((B, N, Hh, v_bits.shape[-1]))
    L = np.zeros((B, Hh, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(Hh):
            keep_tok = token_window_keep(token_radius[b, h], routed_tiles(scores[b, h], k),
                                         r_max, T, H, W)
            q = bf16_to_f64(q_bits[b, :, h])
            kk = bf16_to_f64(k_bits[b, :, h])
            vv = bf16_to_f64(v_bits[b, :, h])
            O[b, :, h], L[b, h] = token_window_attention_rows(q, kk, vv, keep_tok, tt, rows, scale)
    return O, L
