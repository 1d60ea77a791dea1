// MXFP4 encoding of tile-major Q and K for the low-precision "skim" tier.
//
// "Triage: Skip, Skim, or Refine Attention Tiles in Video Diffusion
// Transformers", plain-words summary: a tile can be computed in a quick 4-bit
// version.  The 4-bit format used here is MXFP4 as the OCP Microscaling
// Formats specification v1.0 defines it, which gfx950's scaled MFMA consumes
// directly: blocks of 32 consecutive features of one token row share an E8M0
// scale X = 2^(floor(log2 max|v|) - 2), and every element is v / X rounded to
// the nearest E2M1 value (+-{0, .5, 1, 1.5, 2, 3, 4, 6}), ties to the even
// code, saturating at 6.  The scale exponent is clamped to [-127, 127] and an
// all-zero block takes -127.
//
// One thread encodes one block: 64 bytes of bf16 in, 16 bytes of codes (element
// 2i in the low nibble of byte i) and one scale byte (exponent + 127) out.  The
// scale comes from the exponent bits of the block maximum; the codes from exact
// comparisons of |v| against the rounding thresholds scaled by X (all of them
// are representable, so no rounding happens before the decision).  HBM-bound:
// 64 B read and 17 B written per block.
#include "vsa_common.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;

// floor(log2 |x|) of a non-zero bf16 magnitude (bits without the sign).
__device__ __forceinline__ int bf16_floor_log2(uint32_t mag) {
  const int e = (int)(mag >> 7);
  if (e > 0) return e - 127;
  // subnormal: mag * 2^-133, mag in [1, 127]
  return (31 - __clz((int)mag)) - 133;
}

// E2M1 magnitude code of |v| / 2^ex for a bf16 magnitude `a` (as float).
// Thresholds between neighbouring values, with the tie going to the even code:
// (.25] -> 0, (.75) -> 1, [1.25] -> 2, (1.75) -> 3, [2.5] -> 4, (3.5) -> 5,
// [5] -> 6, above -> 7.
__device__ __forceinline__ uint32_t e2m1_code(float a, float X) {
  uint32_t c;
  if (a <= 0.25f * X) c = 0;
  else if (a < 0.75f * X) c = 1;
  else if (a <= 1.25f * X) c = 2;
  else if (a < 1.75f * X) c = 3;
  else if (a <= 2.5f * X) c = 4;
  else if (a < 3.5f * X) c = 5;
  else if (a <= 5.0f * X) c = 6;
  else c = 7;
  return c;
}

__global__ __launch_bounds__(kThreads) void quantize_mxfp4_kernel(const uint4* __restrict__ x,
                                                                   uint4* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales,
                                                                   int64_t blocks) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= blocks) return;
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = x[4 * b + i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  // block maximum of the magnitudes: for finite bf16 values the integer order
  // of the magnitude bits is the order of the magnitudes
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  int ex = (amax == 0) ? -127 : bf16_floor_log2(amax) - 2;
  ex = min(127, max(-127, ex));
  // thresholds t * 2^ex are exact in fp32 for ex in [-127, 127] except below
  // 2^-149, where every candidate |v| (>= 2^-133 or 0) compares the same way
  const float X = __builtin_ldexpf(1.0f, ex);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
    const float a = __uint_as_float((bits & 0x7FFFu) << 16);
    const uint32_t c = e2m1_code(a, X) | ((bits >> 12) & 8u);
    out[i >> 3] |= c << (4 * (i & 7));
  }
  codes[b] = make_uint4(out[0], out[1], out[2], out[3]);
  scales[b] = (uint8_t)(ex + 127);
}

}  // namespace

hipError_t launch_quantize_mxfp4(const vsa_shape& s, const void* x_tiled, void* codes,
                                 void* scales, hipStream_t stream) {
  const Grid g = make_grid(s);
  const int64_t rows = (int64_t)s.batch * s.heads * g.nT * kTileTokens;
  const int64_t blocks = rows * (s.head_dim / 32);
  const int64_t grid = (blocks + kThreads - 1) / kThreads;
  quantize_mxfp4_kernel<<<(unsigned)grid, kThreads, 0, stream>>>(
      static_cast<const uint4*>(x_tiled), static_cast<uint4*>(codes),
      static_cast<uint8_t*>(scales), blocks);
  return hipGetLastError();
}

}  // namespace vsa
