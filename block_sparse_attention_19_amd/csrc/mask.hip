// Mask builder: per-tile radii + routing scores -> CSR of kept key tiles.
//
// "Token Radius Attention for Efficient Video Generation" (TRA), step 2: a
// per-query radius applied across frames with a temporal distance decay; step
// 3: the radii are translated into a block-sparse mask over tile-major tiles.
// "Where Compute Matters: Heterogeneous Attention for Efficient Video
// Diffusion", abstract: a routed minority of queries takes dense attention.
//
// Three launches:
//   1. route   -- rank of every tile's score within its (batch, head); the
//                 first `dense_count` in (score desc by IEEE totalOrder, index
//                 asc) are routed.  Four threads per tile, the keys in LDS.
//                 The row length in closed form (nT if routed, else the
//                 clipped window count) goes to row_ptr[row + 1].
//   2. scan    -- in-place exclusive scan of the lengths -> row_ptr.  One
//                 workgroup, a shuffle block scan per chunk of rows staged
//                 through LDS (coalesced global reads and writes).
//   3. fill    -- one wave per row writes the ascending key-tile list: 0..nT-1
//                 for a routed row, else the window enumerated as runs of
//                 consecutive tw for each (dt, dh), which is ascending tile order.
#include "vsa_common.h"

namespace vsa {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteChunk = 4096;   // keys staged in LDS per pass
constexpr int kScanThreads = 1024;
constexpr int kScanRowsPerThread = 8;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int clip_count(int x, int s, int n) {
  return min(x + s, n - 1) - max(x - s, 0) + 1;
}

// Kept key tiles of a local query tile at (tt, th, tw) with radius r.
__device__ int window_count(int tt, int th, int tw, int r, int nt, int nh, int nw) {
  int total = 0;
  const int lo = max(-r, -tt), hi = min(r, nt - 1 - tt);
  for (int dt = lo; dt <= hi; ++dt) {
    const int s = r - abs(dt);
    total += clip_count(th, s, nh) * clip_count(tw, s, nw);
  }
  return total;
}

// kRouteSplit threads share one tile: each counts the keys ahead of it in one
// interleaved quarter of the staged keys (4-key vector reads), and the partial
// counts are summed across the group with lane shuffles.
constexpr int kRouteSplit = 4;

// The tile's row length (nT if routed, else the clipped window count) is
// written to row_ptr[row + 1] for the scan that follows.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ scores,
                                                              const uint8_t* __restrict__ radii,
                                                              uint8_t* __restrict__ routed,
                                                              int* __restrict__ row_ptr, int k,
                                                              int r_max, int nt, int nh, int nw) {
  const int nT = nt * nh * nw;
  __shared__ uint4 keys4[kRouteChunk / 4];
  uint32_t* keys = reinterpret_cast<uint32_t*>(keys4);
  const int bh = blockIdx.y;
  const int part = threadIdx.x % kRouteSplit;
  const int a = blockIdx.x * (kRouteThreads / kRouteSplit) + threadIdx.x / kRouteSplit;
  const float* sc = scores + (int64_t)bh * nT;
  const int64_t row = (int64_t)bh * nT + a;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  auto finish = [&](bool is_routed) {
    routed[row] = is_routed ? 1 : 0;
    const int r = min((int)radii[row], r_max);
    row_ptr[row + 1] = is_routed ? nT
                                 : window_count(a / (nh * nw), (a / nw) % nh, a % nw, r, nt, nh, nw);
  };
  if (k == 0 || k == nT) {
    if (a < nT && part == 0) finish(k == nT);
    return;
  }
  const uint32_t ka = (a < nT) ? order_key(sc[a]) : 0u;
  int ahead = 0;
  for (int base = 0; base < nT; base += kRouteChunk) {
    const int n = min(kRouteChunk, nT - base);
    const int n4 = (n + 3) / 4;
    __syncthreads();
    // up to 3 padding slots (last chunk only) hold 0: never greater than ka,
    // and a tie would need an index below a - base < n, which they are not
    for (int i = threadIdx.x; i < 4 * n4; i += kRouteThreads) keys[i] = (i < n) ? order_key(sc[base + i]) : 0u;
    __syncthreads();
    if (a < nT) {
      // keys before position a - base win ties, keys after it lose them
      const int split = a - base;
#pragma unroll 4
      for (int i4 = part; i4 < n4; i4 += kRouteSplit) {
        const uint4 kb = keys4[i4];
        const int i = 4 * i4;
        ahead += (kb.x > ka) || (kb.x == ka && i + 0 < split);
        ahead += (kb.y > ka) || (kb.y == ka && i + 1 < split);
        ahead += (kb.z > ka) || (kb.z == ka && i + 2 < split);
        ahead += (kb.w > ka) || (kb.w == ka && i + 3 < split);
      }
    }
  }
  // the kRouteSplit threads of a tile are consecutive lanes of one wave
#pragma unroll
  for (int d = 1; d < kRouteSplit; d <<= 1) ahead += __shfl_xor(ahead, d);
  if (a < nT && part == 0) finish(ahead < k);
}

// In-place scan of the row lengths in row_ptr[1..rows] (row_ptr[0] = 0), so
// that row_ptr becomes their exclusive scan.  Rows are taken in chunks of
// kScanRowsPerThread * kScanThreads: the chunk is staged in LDS by coalesced
// loads, each thread scans kScanRowsPerThread consecutive lengths in
// registers, a block scan of the per-thread sums plus the running total of
// earlier chunks gives each thread its offset, and the results leave through
// LDS by coalesced stores.
__global__ __launch_bounds__(kScanThreads) void scan_lengths_kernel(int64_t rows,
                                                                    int* __restrict__ row_ptr) {
  constexpr int kChunk = kScanRowsPerThread * kScanThreads;
  __shared__ int sums[kScanThreads / 64];
  __shared__ int stage[kChunk];
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  int* len_p = row_ptr + 1;
  int carry = 0;
  for (int64_t c0 = 0; c0 < rows; c0 += kChunk) {
    const int n = (int)min<int64_t>(kChunk, rows - c0);
#pragma unroll
    for (int j = 0; j < kScanRowsPerThread; ++j) {
      const int i = t + j * kScanThreads;
      stage[i] = (i < n) ? len_p[c0 + i] : 0;
    }
    __syncthreads();
    int len[kScanRowsPerThread];
    int local = 0;
#pragma unroll
    for (int j = 0; j < kScanRowsPerThread; ++j) {
      len[j] = stage[kScanRowsPerThread * t + j];
      local += len[j];
    }
    // lane shuffles within each wave, then a scan of the wave totals by the
    // first wave
    int x = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) sums[wv] = x;
    __syncthreads();
    if (wv == 0) {
      int w_ = (lane < kScanThreads / 64) ? sums[lane] : 0;
#pragma unroll
      for (int d = 1; d < kScanThreads / 64; d <<= 1) {
        const int y = __shfl_up(w_, d);
        if (lane >= d) w_ += y;
      }
      if (lane < kScanThreads / 64) sums[lane] = w_;
    }
    __syncthreads();
    int run = carry + ((wv > 0) ? sums[wv - 1] : 0) + x - local;
#pragma unroll
    for (int j = 0; j < kScanRowsPerThread; ++j) {
      run += len[j];
      stage[kScanRowsPerThread * t + j] = run;
    }
    carry += sums[kScanThreads / 64 - 1];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanRowsPerThread; ++j) {
      const int i = t + j * kScanThreads;
      if (i < n) len_p[c0 + i] = stage[i];
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void fill_kernel(const uint8_t* __restrict__ routed,
                                                   const uint8_t* __restrict__ radii, int r_max,
                                                   int64_t rows, int nt, int nh, int nw,
                                                   const int* __restrict__ row_ptr,
                                                   int* __restrict__ col_idx) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int nT = nt * nh * nw;
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  int* out = col_idx + beg;
  if (routed[row]) {
    for (int i = lane; i < nT && beg + i < end; i += 64) out[i] = i;
    return;
  }
  const int a = (int)(row % nT);
  const int tt = a / (nh * nw), th = (a / nw) % nh, tw = a % nw;
  const int r = min((int)radii[row], r_max);
  int pos = 0;
  const int lo = max(-r, -tt), hi = min(r, nt - 1 - tt);
  for (int dt = lo; dt <= hi; ++dt) {
    const int s = r - abs(dt);
    const int h0 = max(th - s, 0), h1 = min(th + s, nh - 1);
    const int w0 = max(tw - s, 0), w1 = min(tw + s, nw - 1);
    const int run = w1 - w0 + 1;
    for (int hh = h0; hh <= h1; ++hh) {
      const int base = ((tt + dt) * nh + hh) * nw + w0;
      for (int i = lane; i < run; i += 64)
        if (beg + pos + i < end) out[pos + i] = base + i;
      pos += run;
    }
  }
}

}  // namespace

size_t mask_workspace_bytes(const vsa_shape& s) {
  const Grid g = make_grid(s);
  const size_t rows = (size_t)s.batch * s.heads * g.nT;
  return (rows + 255) / 256 * 256;
}

hipError_t launch_build_mask(const vsa_shape& s, const uint8_t* radii, const float* scores,
                             int dense_count, int r_max, int* row_ptr, int* col_idx,
                             uint8_t* routed, void* ws, hipStream_t stream) {
  const Grid g = make_grid(s);
  const int bh = s.batch * s.heads;
  const int64_t rows = (int64_t)bh * g.nT;
  uint8_t* rt = routed ? routed : static_cast<uint8_t*>(ws);
  constexpr int kTilesPerBlock = kRouteThreads / kRouteSplit;
  dim3 rgrid((g.nT + kTilesPerBlock - 1) / kTilesPerBlock, bh);
  route_kernel<<<rgrid, kRouteThreads, 0, stream>>>(scores, radii, rt, row_ptr, dense_count,
                                                    r_max, g.nt, g.nh, g.nw);
  scan_lengths_kernel<<<1, kScanThreads, 0, stream>>>(rows, row_ptr);
  fill_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(rt, radii, r_max, rows, g.nt, g.nh,
                                                             g.nw, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace vsa
