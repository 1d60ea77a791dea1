// Internal definitions shared by the libvsa HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa.h"

namespace vsa {

constexpr int kTile = 4;          // tile edge in tokens (t, h and w)
constexpr int kTileTokens = 64;   // tokens per tile

struct Grid {
  int T, H, W;
  int nt, nh, nw;  // tiles along t, h, w
  int nT;          // nt * nh * nw
};

inline Grid make_grid(const vsa_shape& s) {
  Grid g;
  g.T = s.T; g.H = s.H; g.W = s.W;
  g.nt = (s.T + kTile - 1) / kTile;
  g.nh = (s.H + kTile - 1) / kTile;
  g.nw = (s.W + kTile - 1) / kTile;
  g.nT = g.nt * g.nh * g.nw;
  return g;
}

// Bitmask of the valid (inside the T x H x W grid) slots of tile `tau`.
// Slot = (lt*4 + lh)*4 + lw.
__device__ __forceinline__ uint64_t tile_valid_mask(int tau, int nh, int nw, int T, int H, int W) {
  const int tw = tau % nw;
  const int th = (tau / nw) % nh;
  const int tt = tau / (nw * nh);
  const int vt = min(kTile, T - tt * kTile);
  const int vh = min(kTile, H - th * kTile);
  const int vw = min(kTile, W - tw * kTile);
  const uint64_t wbits = (1ull << vw) - 1ull;                   // lw < vw, within a row of 4
  uint64_t row = 0;                                              // one (lt) plane of 16 slots
  for (int lh = 0; lh < vh; ++lh) row |= wbits << (4 * lh);
  uint64_t m = 0;
  for (int lt = 0; lt < vt; ++lt) m |= row << (16 * lt);
  return m;
}

struct AttnLayout {
  int64_t rows, bh, max_units, max_slots;
  size_t off_cbase, off_gbase, off_grows, off_units, off_comb, off_po, off_pml, off_ext,
      off_coord, off_iota, total;
};

// Launchers (one per source file); each returns the launch status.
hipError_t launch_permute(const vsa_shape& s, const void* x, void* xt, int layout,
                          hipStream_t stream);
hipError_t launch_unpermute(const vsa_shape& s, const void* xt, void* x, hipStream_t stream);
size_t mask_workspace_bytes(const vsa_shape& s);
hipError_t launch_budget_radius(const vsa_shape& s, const int* budget, int r_max, uint8_t* radius,
                                hipStream_t stream);
hipError_t launch_tile_radius(const vsa_shape& s, const uint8_t* token_radius, uint8_t* tile_radius,
                              hipStream_t stream);
hipError_t launch_tile_score(const vsa_shape& s, const float* token_score, float* tile_score,
                             hipStream_t stream);
hipError_t launch_build_mask(const vsa_shape& s, const uint8_t* radii, const float* scores,
                             int dense_count, int r_max, int* row_ptr, int* col_idx,
                             uint8_t* routed, void* ws, hipStream_t stream);
AttnLayout attn_layout(const vsa_shape& s, int kv_chunk);
// Inputs of the skim tier (MXFP4 Q and K, one tier byte per CSR entry).
struct SkimInputs {
  const void* q4;
  const void* q4_scales;
  const void* k4;
  const void* k4_scales;
  const uint8_t* tier;
};
// Inputs of exact per-token windows (token radii in raster order, the routed
// flag of every query tile, and the radius clamp).
struct TokenWindows {
  const uint8_t* token_radius;
  const uint8_t* routed;
  int r_max;
};
hipError_t launch_attn(const vsa_shape& s, const void* q, const void* k, const void* v,
                       const int* row_ptr, const int* col_idx, float scale, void* o, float* lse,
                       int kv_chunk, void* ws, int cus, hipStream_t stream,
                       const SkimInputs* skim = nullptr, const TokenWindows* tokw = nullptr,
                       bool raster = false);
hipError_t launch_quantize_mxfp4(const vsa_shape& s, const void* x_tiled, void* codes,
                                 void* scales, hipStream_t stream);
hipError_t attn_set_lds_limits();

void set_error(const char* fmt, ...);

}  // namespace vsa
