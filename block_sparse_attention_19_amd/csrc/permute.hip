// Tile-major permute / unpermute of bf16 activations.
//
// "Token Radius Attention for Efficient Video Generation", pipeline step 3:
// tokens are laid out tile-major so that every sparse support is a set of whole
// 64-token blocks.  One workgroup moves one (batch, head, tile): the 64 slots of
// a 4x4x4 tile, D features each.  Block x = tile * heads + head: consecutive
// workgroups cover the heads of one tile, so each token's raster record (all
// heads, contiguous) is streamed in one burst.  Index arithmetic is done once
// per tile and per slot (shifts only); the feature loop moves 16-byte chunks, so each token
// row is one contiguous 2*D-byte transfer on both sides.  Both directions are
// HBM-bound: per tile they read and write 64*D*2 bytes (the padded side) or
// valid*D*2 bytes (the raster side).
#include "vsa_common.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

struct TileCoord {
  int t0, h0, w0;  // first token coordinate of the tile
};

__device__ __forceinline__ TileCoord tile_origin(int tau, int nh, int nw) {
  TileCoord c;
  c.w0 = (tau % nw) * kTile;
  c.h0 = ((tau / nw) % nh) * kTile;
  c.t0 = (tau / (nw * nh)) * kTile;
  return c;
}

// Raster [B][N][Hh][D] -> token-major tiles [B][Hh][nT*64][D].
template <int D>
__global__ __launch_bounds__(kThreads) void permute_token_major(
    const uint4* __restrict__ x, uint4* __restrict__ xt, int Hh, int T, int H, int W, int nh,
    int nw, int nT) {
  constexpr int C = D / 8;                 // 16-byte chunks per token row
  constexpr int kIters = kTileTokens * C / kThreads;
  const int h = blockIdx.x % Hh, tau = blockIdx.x / Hh, b = blockIdx.y;
  const TileCoord o = tile_origin(tau, nh, nw);
  const int64_t N = (int64_t)T * H * W;
  uint4* dst = xt + (((int64_t)b * Hh + h) * nT + tau) * (kTileTokens * C);
#pragma unroll
  for (int j = 0; j < kIters; ++j) {
    const int i = threadIdx.x + j * kThreads;
    const int slot = i / C, c = i % C;
    const int t = o.t0 + (slot >> 4), hh = o.h0 + ((slot >> 2) & 3), w = o.w0 + (slot & 3);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t < T && hh < H && w < W) {
      const int64_t n = ((int64_t)t * H + hh) * W + w;
      v = x[(((int64_t)b * N + n) * Hh + h) * C + c];
    }
    dst[i] = v;
  }
}

// Raster [B][N][Hh][D] -> feature-major tiles [B][Hh][nT][D][64], through LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void permute_feature_major(
    const uint4* __restrict__ x, uint4* __restrict__ xt, int Hh, int T, int H, int W, int nh,
    int nw, int nT) {
  constexpr int C = D / 8;
  constexpr int kIters = kTileTokens * C / kThreads;
  constexpr int kStride = D + 2;           // bf16 per LDS row; +2 staggers banks
  __shared__ uint16_t tile[kTileTokens * kStride];
  const int h = blockIdx.x % Hh, tau = blockIdx.x / Hh, b = blockIdx.y;
  const TileCoord o = tile_origin(tau, nh, nw);
  const int64_t N = (int64_t)T * H * W;
#pragma unroll
  for (int j = 0; j < kIters; ++j) {
    const int i = threadIdx.x + j * kThreads;
    const int slot = i / C, c = i % C;
    const int t = o.t0 + (slot >> 4), hh = o.h0 + ((slot >> 2) & 3), w = o.w0 + (slot & 3);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t < T && hh < H && w < W) {
      const int64_t n = ((int64_t)t * H + hh) * W + w;
      v = x[(((int64_t)b * N + n) * Hh + h) * C + c];
    }
    uint32_t* row = reinterpret_cast<uint32_t*>(tile + slot * kStride + c * 8);  // 4-byte aligned
    row[0] = v.x; row[1] = v.y; row[2] = v.z; row[3] = v.w;
  }
  __syncthreads();
  // Output chunk q = d*8 + g holds slots 8g .. 8g+7 of feature d.
  uint4* dst = xt + (((int64_t)b * Hh + h) * nT + tau) * (kTileTokens * C);
#pragma unroll
  for (int j = 0; j < kIters; ++j) {
    const int q = threadIdx.x + j * kThreads;
    const int d = q >> 3, g = q & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[(8 * g + 2 * e) * kStride + d];
      const uint32_t hi = tile[(8 * g + 2 * e + 1) * kStride + d];
      w[e] = lo | (hi << 16);
    }
    dst[q] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Token-major tiles [B][Hh][nT*64][D] -> raster [B][N][Hh][D]; padded slots skipped.
template <int D>
__global__ __launch_bounds__(kThreads) void unpermute_token_major(
    const uint4* __restrict__ xt, uint4* __restrict__ x, int Hh, int T, int H, int W, int nh,
    int nw, int nT) {
  constexpr int C = D / 8;
  constexpr int kIters = kTileTokens * C / kThreads;
  const int h = blockIdx.x % Hh, tau = blockIdx.x / Hh, b = blockIdx.y;
  const TileCoord o = tile_origin(tau, nh, nw);
  const int64_t N = (int64_t)T * H * W;
  const uint4* src = xt + (((int64_t)b * Hh + h) * nT + tau) * (kTileTokens * C);
#pragma unroll
  for (int j = 0; j < kIters; ++j) {
    const int i = threadIdx.x + j * kThreads;
    const int slot = i / C, c = i % C;
    const int t = o.t0 + (slot >> 4), hh = o.h0 + ((slot >> 2) & 3), w = o.w0 + (slot & 3);
    if (t < T && hh < H && w < W) {
      const int64_t n = ((int64_t)t * H + hh) * W + w;
      x[(((int64_t)b * N + n) * Hh + h) * C + c] = src[i];
    }
  }
}

}  // namespace

hipError_t launch_permute(const vsa_shape& s, const void* x, void* xt, int layout,
                          hipStream_t stream) {
  const Grid g = make_grid(s);
  dim3 grid(g.nT * s.heads, s.batch);
  const uint4* in = static_cast<const uint4*>(x);
  uint4* out = static_cast<uint4*>(xt);
  if (layout == VSA_LAYOUT_TOKEN_MAJOR) {
    if (s.head_dim == 128)
      permute_token_major<128><<<grid, kThreads, 0, stream>>>(in, out, s.heads, s.T, s.H, s.W, g.nh, g.nw, g.nT);
    else
      permute_token_major<64><<<grid, kThreads, 0, stream>>>(in, out, s.heads, s.T, s.H, s.W, g.nh, g.nw, g.nT);
  } else {
    if (s.head_dim == 128)
      permute_feature_major<128><<<grid, kThreads, 0, stream>>>(in, out, s.heads, s.T, s.H, s.W, g.nh, g.nw, g.nT);
    else
      permute_feature_major<64><<<grid, kThreads, 0, stream>>>(in, out, s.heads, s.T, s.H, s.W, g.nh, g.nw, g.nT);
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(const vsa_shape& s, const void* xt, void* x, hipStream_t stream) {
  const Grid g = make_grid(s);
  dim3 grid(g.nT * s.heads, s.batch);
  const uint4* in = static_cast<const uint4*>(xt);
  uint4* out = static_cast<uint4*>(x);
  if (s.head_dim == 128)
    unpermute_token_major<128><<<grid, kThreads, 0, stream>>>(in, out, s.heads, s.T, s.H, s.W, g.nh, g.nw, g.nT);
  else
    unpermute_token_major<64><<<grid, kThreads, 0, stream>>>(in, out, s.heads, s.T, s.H, s.W, g.nh, g.nw, g.nT);
  return hipGetLastError();
}

}  // namespace vsa
