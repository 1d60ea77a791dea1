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
//                 asc) are routed.  One thread per tile, the head's keys in LDS.
//   2. lengths -- row length in closed form (nT if routed, else the clipped
//                 window count), exclusive scan -> row_ptr.  One workgroup,
//                 rows in LDS-staged chunks, a block scan per chunk.
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

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ scores,
                                                              uint8_t* __restrict__ routed,
                                                              int nT, int k) {
  __shared__ uint4 keys4[kRouteChunk / 4];
  uint32_t* keys = reinterpret_cast<uint32_t*>(keys4);
  const int bh = blockIdx.y;
  const int a = blockIdx.x * kRouteThreads + threadIdx.x;
  const float* sc = scores + (int64_t)bh * nT;
  if (k == 0 || k == nT) {
    if (a < nT) routed[(int64_t)bh * nT + a] = (k == nT) ? 1 : 0;
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
#pragma unroll 8
      for (int i4 = 0; i4 < n4; ++i4) {
        const uint4 kb = keys4[i4];
        const int i = 4 * i4;
        ahead += (kb.x > ka) || (kb.x == ka && i + 0 < split);
        ahead += (kb.y > ka) || (kb.y == ka && i + 1 < split);
        ahead += (kb.z > ka) || (kb.z == ka && i + 2 < split);
        ahead += (kb.w > ka) || (kb.w == ka && i + 3 < split);
      }
    }
  }
  if (a < nT) routed[(int64_t)bh * nT + a] = (ahead < k) ? 1 : 0;
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

__device__ __forceinline__ int row_length(int64_t row, bool is_routed, int radius, int r_max, int nt,
                                          int nh, int nw, int nT) {
  if (is_routed) return nT;
  const int a = (int)(row % nT);
  const int r = min(radius, r_max);
  return window_count(a / (nh * nw), (a / nw) % nh, a % nw, r, nt, nh, nw);
}

// Row lengths and their exclusive scan.  Rows are taken in chunks of
// kScanRowsPerThread * kScanThreads: the chunk's routed flags and radii are
// staged in LDS with coalesced loads, each thread computes the lengths of
// kScanRowsPerThread consecutive rows, and a block scan of the per-thread sums
// (plus the running total of earlier chunks) gives row_ptr.
__global__ __launch_bounds__(kScanThreads) void lengths_scan_kernel(
    const uint8_t* __restrict__ routed, const uint8_t* __restrict__ radii, int r_max,
    int64_t rows, int nt, int nh, int nw, int* __restrict__ row_ptr) {
  constexpr int kChunk = kScanRowsPerThread * kScanThreads;
  __shared__ int sums[kScanThreads];
  __shared__ uint8_t s_rt[kChunk], s_rad[kChunk];
  const int nT = nt * nh * nw;
  const int t = threadIdx.x;
  if (t == 0) row_ptr[0] = 0;
  int carry = 0;
  for (int64_t c0 = 0; c0 < rows; c0 += kChunk) {
    const int n = (int)min<int64_t>(kChunk, rows - c0);
    for (int i = t; i < n; i += kScanThreads) {
      s_rt[i] = routed[c0 + i];
      s_rad[i] = radii[c0 + i];
    }
    __syncthreads();
    int len[kScanRowsPerThread];
    int local = 0;
#pragma unroll
    for (int j = 0; j < kScanRowsPerThread; ++j) {
      const int i = kScanRowsPerThread * t + j;
      len[j] = (i < n) ? row_length(c0 + i, s_rt[i] != 0, s_rad[i], r_max, nt, nh, nw, nT) : 0;
      local += len[j];
    }
    sums[t] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan over the per-thread sums.
    for (int off = 1; off < kScanThreads; off <<= 1) {
      const int v = (t >= off) ? sums[t - off] : 0;
      __syncthreads();
      sums[t] += v;
      __syncthreads();
    }
    int run = carry + sums[t] - local;
#pragma unroll
    for (int j = 0; j < kScanRowsPerThread; ++j) {
      const int i = kScanRowsPerThread * t + j;
      run += len[j];
      if (i < n) row_ptr[c0 + i + 1] = run;
    }
    carry += sums[kScanThreads - 1];
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
  dim3 rgrid((g.nT + kRouteThreads - 1) / kRouteThreads, bh);
  route_kernel<<<rgrid, kRouteThreads, 0, stream>>>(scores, rt, g.nT, dense_count);
  lengths_scan_kernel<<<1, kScanThreads, 0, stream>>>(rt, radii, r_max, rows, g.nt, g.nh, g.nw,
                                                       row_ptr);
  fill_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(rt, radii, r_max, rows, g.nt, g.nh,
                                                             g.nw, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace vsa
