// Token-level inputs -> the tile inputs of the mask builder.
//
// "Token Radius Attention for Efficient Video Generation" (TRA): step 1 gives
// every query token a budget of keys, step 2 turns the budget into a base
// radius applied across frames with a temporal distance decay, and step 3
// translates the token-level radii into block-sparse masks.  "Where Compute
// Matters: Heterogeneous Attention for Efficient Video Diffusion" predicts a
// difficulty per token and routes the most uncertain ones to dense attention.
// The mask builder takes one radius and one routing score per query tile;
// these kernels produce them:
//   * budget_radius_kernel -- per query token, the smallest r in [0, r_max]
//     whose tile window (|dt| <= r, max(|dh|, |dw|) <= r - |dt|) holds at least
//     its budget of real key tokens, else r_max.  One workgroup per (b, h,
//     tile): threads r = 0..r_max count the window's tokens in closed form
//     (a sum over dt of clipped token extents) into LDS, then each of the
//     tile's tokens binary-searches the (non-decreasing) counts.
//   * tile_max kernels -- per tile, the largest radius / the largest score in
//     the IEEE-754 total order among its real tokens (the tile's window then
//     contains every token's window; the tile is routed if any token is among
//     the most uncertain).  One thread per (b, h, tile).
// All are tiny and latency-bound: per token 4 B read + 1 B written (budgets),
// per tile 64 token reads + 1 write.
#include "vsa_common.h"

namespace vsa {
namespace {

constexpr int kRadiusThreads = 256;  // covers r = 0..255

// Real tokens along one axis covered by tiles [lo, hi] (clipped to the grid).
__device__ __forceinline__ int axis_span(int X, int ntiles, int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, ntiles - 1);
  return (hi < lo) ? 0 : min(X, kTile * (hi + 1)) - kTile * lo;
}

__global__ __launch_bounds__(kRadiusThreads) void budget_radius_kernel(
    const int* __restrict__ budget, uint8_t* __restrict__ radius, int r_max, int T, int H, int W,
    int nt, int nh, int nw, int heads) {
  __shared__ int counts[kRadiusThreads];
  const int tau = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tw = tau % nw, th = (tau / nw) % nh, tt = tau / (nw * nh);
  const int r = threadIdx.x;
  if (r <= r_max) {
    int64_t tot = 0;
    for (int dt = -r; dt <= r; ++dt) {
      if (tt + dt < 0 || tt + dt >= nt) continue;
      const int s = r - abs(dt);
      tot += (int64_t)axis_span(T, nt, tt + dt, tt + dt) * axis_span(H, nh, th - s, th + s) *
             axis_span(W, nw, tw - s, tw + s);
    }
    counts[r] = (int)tot;  // <= T*H*W, which fits int32
  }
  __syncthreads();
  if (threadIdx.x >= kTileTokens) return;
  const int slot = threadIdx.x;
  const int t = tt * kTile + (slot >> 4), hh = th * kTile + ((slot >> 2) & 3),
            w = tw * kTile + (slot & 3);
  if (t >= T || hh >= H || w >= W) return;
  const int64_t N = (int64_t)T * H * W;
  const int64_t idx = ((int64_t)b * heads + h) * N + ((int64_t)t * H + hh) * W + w;
  const int want = budget[idx];
  // first r with counts[r] >= want, or r_max
  int lo = 0, hi = r_max;
  if (counts[r_max] < want) {
    lo = r_max;
  } else {
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (counts[mid] >= want) hi = mid; else lo = mid + 1;
    }
  }
  radius[idx] = (uint8_t)lo;
}

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <typename TV>
__device__ __forceinline__ uint32_t to_key(TV v);
template <>
__device__ __forceinline__ uint32_t to_key<uint8_t>(uint8_t v) { return v; }
template <>
__device__ __forceinline__ uint32_t to_key<float>(float v) { return order_key(v); }
template <typename TV>
__device__ __forceinline__ TV from_key(uint32_t k);
template <>
__device__ __forceinline__ uint8_t from_key<uint8_t>(uint32_t k) { return (uint8_t)k; }
template <>
__device__ __forceinline__ float from_key<float>(uint32_t k) { return from_order_key(k); }

template <typename TV>
__global__ __launch_bounds__(256) void tile_max_kernel(const TV* __restrict__ x, TV* __restrict__ y,
                                                       int T, int H, int W, int nh, int nw,
                                                       int nT, int64_t bh) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= bh * nT) return;
  const int64_t bhi = i / nT;
  const int tau = (int)(i % nT);
  const int tw = tau % nw, th = (tau / nw) % nh, tt = tau / (nw * nh);
  const int64_t N = (int64_t)T * H * W;
  const TV* xs = x + bhi * N;
  uint32_t best = 0;  // every tile holds at least one real token
  bool any = false;
  for (int lt = 0; lt < kTile; ++lt) {
    const int t = tt * kTile + lt;
    if (t >= T) break;
    for (int lh = 0; lh < kTile; ++lh) {
      const int hh = th * kTile + lh;
      if (hh >= H) break;
      for (int lw = 0; lw < kTile; ++lw) {
        const int w = tw * kTile + lw;
        if (w >= W) break;
        const uint32_t k = to_key<TV>(xs[((int64_t)t * H + hh) * W + w]);
        best = (!any || k > best) ? k : best;
        any = true;
      }
    }
  }
  y[i] = from_key<TV>(best);
}

}  // namespace

hipError_t launch_budget_radius(const vsa_shape& s, const int* budget, int r_max, uint8_t* radius,
                                hipStream_t stream) {
  const Grid g = make_grid(s);
  dim3 grid(g.nT, s.heads, s.batch);
  budget_radius_kernel<<<grid, kRadiusThreads, 0, stream>>>(budget, radius, r_max, s.T, s.H, s.W,
                                                            g.nt, g.nh, g.nw, s.heads);
  return hipGetLastError();
}

hipError_t launch_tile_radius(const vsa_shape& s, const uint8_t* token_radius, uint8_t* tile_radius,
                              hipStream_t stream) {
  const Grid g = make_grid(s);
  const int64_t bh = (int64_t)s.batch * s.heads;
  const int64_t n = bh * g.nT;
  tile_max_kernel<uint8_t><<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      token_radius, tile_radius, s.T, s.H, s.W, g.nh, g.nw, g.nT, bh);
  return hipGetLastError();
}

hipError_t launch_tile_score(const vsa_shape& s, const float* token_score, float* tile_score,
                             hipStream_t stream) {
  const Grid g = make_grid(s);
  const int64_t bh = (int64_t)s.batch * s.heads;
  const int64_t n = bh * g.nT;
  tile_max_kernel<float><<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      token_score, tile_score, s.T, s.H, s.W, g.nh, g.nw, g.nT, bh);
  return hipGetLastError();
}

}  // namespace vsa
