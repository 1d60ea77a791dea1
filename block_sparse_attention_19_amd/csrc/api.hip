// C ABI of libvsa: argument validation on the host, then kernel launches.
// Every check runs before anything is enqueued, so a call that returns an
// error leaves the stream untouched.
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "vsa_common.h"

namespace vsa {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_cus[kMaxDevices] = {0};

// CU count of the current device (LDS limits raised once per device).
vsa_status device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("hipGetDevice failed: %s", hipGetErrorString(e));
    return VSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0) {
      set_error("hipDeviceGetAttribute(CU count) failed: %s", hipGetErrorString(e));
      return VSA_ERR_HIP;
    }
    e = attn_set_lds_limits();
    if (e != hipSuccess) {
      set_error("hipFuncSetAttribute(LDS) failed: %s", hipGetErrorString(e));
      return VSA_ERR_HIP;
    }
    g_cus[dev] = n;
  }
  *cus = g_cus[dev];
  return VSA_OK;
}

// Device-resident workspace of the allocation-free forward call: one copy per
// GPU (each device that loads the library holds its own until the process
// ends).  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(48) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch_dev[kMaxDevices] = {nullptr};

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with that device current).
vsa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("hipGetDevice failed: %s", hipGetErrorString(e));
    return VSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_error("hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return VSA_ERR_HIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return VSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

vsa_status check_shape(const vsa_shape* s) {
  if (!s) { set_error("shape is NULL"); return VSA_ERR_INVALID_ARG; }
  if (s->batch < 1 || s->heads < 1 || s->T < 1 || s->H < 1 || s->W < 1 || s->head_dim < 1) {
    set_error("shape fields must be >= 1 (batch=%d heads=%d D=%d T=%d H=%d W=%d)", s->batch,
              s->heads, s->head_dim, s->T, s->H, s->W);
    return VSA_ERR_INVALID_ARG;
  }
  if (s->head_dim != 64 && s->head_dim != 128) {
    set_error("head_dim %d not supported (64 or 128)", s->head_dim);
    return VSA_ERR_UNSUPPORTED;
  }
  if ((int64_t)s->batch * s->heads > 65535) {
    set_error("batch * heads must be <= 65535");
    return VSA_ERR_INVALID_ARG;
  }
  const int64_t nT = (int64_t)((s->T + 3) / 4) * ((s->H + 3) / 4) * ((s->W + 3) / 4);
  const int64_t rows = (int64_t)s->batch * s->heads * nT;
  // rows and padded token rows are int32 in the CSR and the unit list.
  if (nT * kTileTokens > INT_MAX || rows * kTileTokens > INT_MAX) {
    set_error("problem too large: %lld tile rows", (long long)rows);
    return VSA_ERR_OVERFLOW;
  }
  // the permutes launch heads * nT workgroups of 256 threads in one grid
  // dimension, whose work-item count is 32-bit
  if ((int64_t)s->heads * nT * 256 > (int64_t)UINT32_MAX) {
    set_error("problem too large: heads * tiles = %lld", (long long)(s->heads * nT));
    return VSA_ERR_OVERFLOW;
  }
  return VSA_OK;
}

vsa_status check_ptr(const void* p, size_t align, const char* name) {
  if (!p) { set_error("%s is NULL", name); return VSA_ERR_INVALID_ARG; }
  if (!aligned(p, align)) {
    set_error("%s is not %zu-byte aligned", name, align);
    return VSA_ERR_INVALID_ARG;
  }
  return VSA_OK;
}

vsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return VSA_OK;
  set_error("%s: %s", what, hipGetErrorString(e));
  return VSA_ERR_HIP;
}

int64_t window_bound(int64_t r, const Grid& g) {
  // Unclipped window size of radius r, capped by the tile count.
  int64_t total = 0;
  for (int64_t dt = -r; dt <= r; ++dt) {
    const int64_t s = r - (dt < 0 ? -dt : dt);
    const int64_t side_h = std::min<int64_t>(2 * s + 1, g.nh);
    const int64_t side_w = std::min<int64_t>(2 * s + 1, g.nw);
    if (dt >= g.nt || -dt >= g.nt) continue;
    total += side_h * side_w;
  }
  return std::min<int64_t>(total, g.nT);
}

#define VSA_TRY(x)                       \
  do {                                   \
    vsa_status _st = (x);                \
    if (_st != VSA_OK) return _st;       \
  } while (0)

}  // namespace
}  // namespace vsa

using namespace vsa;

extern "C" {

const char* vsa_status_string(vsa_status s) {
  switch (s) {
    case VSA_OK: return "ok";
    case VSA_ERR_INVALID_ARG: return "invalid argument";
    case VSA_ERR_UNSUPPORTED: return "unsupported";
    case VSA_ERR_CAPACITY: return "buffer too small";
    case VSA_ERR_OVERFLOW: return "index overflow";
    case VSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* vsa_last_error(void) { return g_err; }

int32_t vsa_num_tiles(const vsa_shape* s) {
  if (check_shape(s) != VSA_OK) return -1;
  return make_grid(*s).nT;
}

vsa_status vsa_tile_permute(const vsa_shape* s, const void* x, void* x_tiled, int32_t layout,
                            void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(x, 16, "x"));
  VSA_TRY(check_ptr(x_tiled, 16, "x_tiled"));
  if (layout != VSA_LAYOUT_TOKEN_MAJOR && layout != VSA_LAYOUT_FEATURE_MAJOR) {
    set_error("unknown layout %d", layout);
    return VSA_ERR_INVALID_ARG;
  }
  return hip_status(launch_permute(*s, x, x_tiled, layout, static_cast<hipStream_t>(stream)),
                    "tile permute launch");
}

vsa_status vsa_tile_unpermute(const vsa_shape* s, const void* o_tiled, void* o, void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(o_tiled, 16, "o_tiled"));
  VSA_TRY(check_ptr(o, 16, "o"));
  return hip_status(launch_unpermute(*s, o_tiled, o, static_cast<hipStream_t>(stream)),
                    "tile unpermute launch");
}

int64_t vsa_mask_nnz_bound(const vsa_shape* s, int32_t r_max, int32_t dense_count) {
  if (check_shape(s) != VSA_OK) return -1;
  const Grid g = make_grid(*s);
  if (r_max < 0 || r_max > 255 || dense_count < 0 || dense_count > g.nT) return -1;
  const int64_t bh = (int64_t)s->batch * s->heads;
  const int64_t local = window_bound(r_max, g);
  return bh * ((int64_t)dense_count * g.nT + (int64_t)(g.nT - dense_count) * local);
}

size_t vsa_mask_workspace_bytes(const vsa_shape* s) {
  if (check_shape(s) != VSA_OK) return 0;
  return mask_workspace_bytes(*s);
}

vsa_status vsa_build_mask(const vsa_shape* s, const uint8_t* radii, const float* scores,
                          int32_t dense_count, int32_t r_max, int32_t* row_ptr, int32_t* col_idx,
                          int64_t col_capacity, uint8_t* routed, void* ws, size_t ws_bytes,
                          void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(radii, 1, "radii"));
  VSA_TRY(check_ptr(scores, 4, "scores"));
  VSA_TRY(check_ptr(row_ptr, 4, "row_ptr"));
  VSA_TRY(check_ptr(col_idx, 4, "col_idx"));
  const Grid g = make_grid(*s);
  if (dense_count < 0 || dense_count > g.nT) {
    set_error("dense_count %d outside [0, %d]", dense_count, g.nT);
    return VSA_ERR_INVALID_ARG;
  }
  if (r_max < 0 || r_max > 255) {
    set_error("r_max %d outside [0, 255]", r_max);
    return VSA_ERR_INVALID_ARG;
  }
  const int64_t bound = vsa_mask_nnz_bound(s, r_max, dense_count);
  if (bound > INT_MAX) {
    set_error("nnz bound %lld exceeds int32", (long long)bound);
    return VSA_ERR_OVERFLOW;
  }
  if (col_capacity < bound) {
    set_error("col_capacity %lld < nnz bound %lld", (long long)col_capacity, (long long)bound);
    return VSA_ERR_CAPACITY;
  }
  if (!routed) {
    VSA_TRY(check_ptr(ws, 16, "ws"));
    if (ws_bytes < mask_workspace_bytes(*s)) {
      set_error("mask workspace %zu < %zu bytes", ws_bytes, mask_workspace_bytes(*s));
      return VSA_ERR_CAPACITY;
    }
  }
  return hip_status(launch_build_mask(*s, radii, scores, dense_count, r_max, row_ptr, col_idx,
                                      routed, ws, static_cast<hipStream_t>(stream)),
                    "mask launch");
}

vsa_status vsa_budget_to_radius(const vsa_shape* s, const int32_t* budget, int32_t r_max,
                                uint8_t* radius, void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(budget, 4, "budget"));
  VSA_TRY(check_ptr(radius, 1, "radius"));
  if (r_max < 0 || r_max > 255) {
    set_error("r_max %d outside [0, 255]", r_max);
    return VSA_ERR_INVALID_ARG;
  }
  return hip_status(launch_budget_radius(*s, budget, r_max, radius, static_cast<hipStream_t>(stream)),
                    "budget launch");
}

vsa_status vsa_tile_radius_from_tokens(const vsa_shape* s, const uint8_t* token_radius,
                                       uint8_t* tile_radius, void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(token_radius, 1, "token_radius"));
  VSA_TRY(check_ptr(tile_radius, 1, "tile_radius"));
  return hip_status(launch_tile_radius(*s, token_radius, tile_radius, static_cast<hipStream_t>(stream)),
                    "tile radius launch");
}

vsa_status vsa_tile_score_from_tokens(const vsa_shape* s, const float* token_score,
                                      float* tile_score, void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(token_score, 4, "token_score"));
  VSA_TRY(check_ptr(tile_score, 4, "tile_score"));
  return hip_status(launch_tile_score(*s, token_score, tile_score, static_cast<hipStream_t>(stream)),
                    "tile score launch");
}

size_t vsa_attn_workspace_bytes(const vsa_shape* s, int32_t kv_chunk) {
  if (check_shape(s) != VSA_OK || kv_chunk < 0) return 0;
  return attn_layout(*s, kv_chunk).total;
}

// Checks of the inputs, outputs and scale shared by every forward call.
static vsa_status check_attn_io(const vsa_shape* s, const void* q, const char* q_name,
                                const void* k_t, const void* v_t, const int32_t* row_ptr,
                                const int32_t* col_idx, float scale, const void* o,
                                const char* o_name, const float* lse, const char* lse_name) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(q, 16, q_name));
  VSA_TRY(check_ptr(k_t, 16, "k_t"));
  VSA_TRY(check_ptr(v_t, 16, "v_t"));
  VSA_TRY(check_ptr(row_ptr, 4, "row_ptr"));
  VSA_TRY(check_ptr(col_idx, 4, "col_idx"));
  VSA_TRY(check_ptr(o, 16, o_name));
  if (lse) VSA_TRY(check_ptr(lse, 4, lse_name));
  if (!(scale > 0.f) || scale > 3.0e38f) {
    set_error("scale must be finite and > 0");
    return VSA_ERR_INVALID_ARG;
  }
  return VSA_OK;
}

// Argument checks shared by the tile-major and the raster forward calls.
static vsa_status check_attn_args(const vsa_shape* s, const void* q, const char* q_name,
                                  const void* k_t, const void* v_t, const int32_t* row_ptr,
                                  const int32_t* col_idx, float scale, const void* o,
                                  const char* o_name, const float* lse, const char* lse_name,
                                  int32_t kv_chunk, const void* ws, size_t ws_bytes) {
  VSA_TRY(check_attn_io(s, q, q_name, k_t, v_t, row_ptr, col_idx, scale, o, o_name, lse,
                        lse_name));
  VSA_TRY(check_ptr(ws, 256, "ws"));
  if (kv_chunk < 0) {
    set_error("kv_chunk must be >= 0");
    return VSA_ERR_INVALID_ARG;
  }
  const size_t need = attn_layout(*s, kv_chunk).total;
  if (ws_bytes < need) {
    set_error("attention workspace %zu < %zu bytes", ws_bytes, need);
    return VSA_ERR_CAPACITY;
  }
  return VSA_OK;
}

vsa_status vsa_attn_fwd(const vsa_shape* s, const void* q_t, const void* k_t, const void* v_t,
                        const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o_t,
                        float* lse_t, int32_t kv_chunk, void* ws, size_t ws_bytes, void* stream) {
  VSA_TRY(check_attn_args(s, q_t, "q_t", k_t, v_t, row_ptr, col_idx, scale, o_t, "o_t", lse_t,
                          "lse_t", kv_chunk, ws, ws_bytes));
  int cus = 0;
  VSA_TRY(device_cus(&cus));
  return hip_status(launch_attn(*s, q_t, k_t, v_t, row_ptr, col_idx, scale, o_t, lse_t, kv_chunk,
                                ws, cus, static_cast<hipStream_t>(stream)),
                    "attention launch");
}

vsa_status vsa_attn_fwd_raster(const vsa_shape* s, const void* q, const void* k_t, const void* v_t,
                               const int32_t* row_ptr, const int32_t* col_idx, float scale,
                               void* o, float* lse, int32_t kv_chunk, void* ws, size_t ws_bytes,
                               void* stream) {
  VSA_TRY(check_attn_args(s, q, "q", k_t, v_t, row_ptr, col_idx, scale, o, "o", lse, "lse",
                          kv_chunk, ws, ws_bytes));
  int cus = 0;
  VSA_TRY(device_cus(&cus));
  return hip_status(launch_attn(*s, q, k_t, v_t, row_ptr, col_idx, scale, o, lse, kv_chunk, ws,
                                cus, static_cast<hipStream_t>(stream), nullptr, nullptr, true),
                    "attention launch");
}

size_t vsa_attn_noalloc_max_workspace(void) { return kScratchBytes; }

vsa_status vsa_attn_fwd_raster_noalloc(const vsa_shape* s, const void* q, const void* k_t,
                                       const void* v_t, const int32_t* row_ptr,
                                       const int32_t* col_idx, float scale, void* o, float* lse,
                                       void* stream) {
  VSA_TRY(check_attn_io(s, q, "q", k_t, v_t, row_ptr, col_idx, scale, o, "o", lse, "lse"));
  const size_t need = attn_layout(*s, 0).total;
  if (need > kScratchBytes) {
    set_error("shape needs %zu bytes of workspace; the allocation-free call holds %zu "
              "(use vsa_attn_fwd_raster with a caller workspace)",
              need, kScratchBytes);
    return VSA_ERR_CAPACITY;
  }
  void* ws = nullptr;
  VSA_TRY(scratch_address(&ws));
  int cus = 0;
  VSA_TRY(device_cus(&cus));
  return hip_status(launch_attn(*s, q, k_t, v_t, row_ptr, col_idx, scale, o, lse, 0, ws, cus,
                                static_cast<hipStream_t>(stream), nullptr, nullptr, true),
                    "attention launch");
}

vsa_status vsa_quantize_mxfp4(const vsa_shape* s, const void* x_tiled, void* codes, void* scales,
                              void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(x_tiled, 16, "x_tiled"));
  VSA_TRY(check_ptr(codes, 16, "codes"));
  VSA_TRY(check_ptr(scales, 16, "scales"));
  return hip_status(launch_quantize_mxfp4(*s, x_tiled, codes, scales,
                                          static_cast<hipStream_t>(stream)),
                    "quantize launch");
}

vsa_status vsa_attn_fwd_tiered(const vsa_shape* s, const void* q_t, const void* k_t,
                               const void* v_t, const void* q4, const void* q4_scales,
                               const void* k4, const void* k4_scales, const int32_t* row_ptr,
                               const int32_t* col_idx, const uint8_t* tier, float scale,
                               void* o_t, float* lse_t, int32_t kv_chunk, void* ws,
                               size_t ws_bytes, void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(q_t, 16, "q_t"));
  VSA_TRY(check_ptr(k_t, 16, "k_t"));
  VSA_TRY(check_ptr(v_t, 16, "v_t"));
  VSA_TRY(check_ptr(q4, 16, "q4"));
  VSA_TRY(check_ptr(q4_scales, 16, "q4_scales"));
  VSA_TRY(check_ptr(k4, 16, "k4"));
  VSA_TRY(check_ptr(k4_scales, 16, "k4_scales"));
  VSA_TRY(check_ptr(row_ptr, 4, "row_ptr"));
  VSA_TRY(check_ptr(col_idx, 4, "col_idx"));
  VSA_TRY(check_ptr(tier, 1, "tier"));
  VSA_TRY(check_ptr(o_t, 16, "o_t"));
  if (lse_t) VSA_TRY(check_ptr(lse_t, 4, "lse_t"));
  VSA_TRY(check_ptr(ws, 256, "ws"));
  if (!(scale > 0.f) || scale > 3.0e38f) {
    set_error("scale must be finite and > 0");
    return VSA_ERR_INVALID_ARG;
  }
  if (kv_chunk < 0) {
    set_error("kv_chunk must be >= 0");
    return VSA_ERR_INVALID_ARG;
  }
  const size_t need = attn_layout(*s, kv_chunk).total;
  if (ws_bytes < need) {
    set_error("attention workspace %zu < %zu bytes", ws_bytes, need);
    return VSA_ERR_CAPACITY;
  }
  int cus = 0;
  VSA_TRY(device_cus(&cus));
  const SkimInputs skim = {q4, q4_scales, k4, k4_scales, tier};
  return hip_status(launch_attn(*s, q_t, k_t, v_t, row_ptr, col_idx, scale, o_t, lse_t, kv_chunk,
                                ws, cus, static_cast<hipStream_t>(stream), &skim),
                    "attention launch");
}

vsa_status vsa_attn_fwd_token_window(const vsa_shape* s, const void* q_t, const void* k_t,
                                     const void* v_t, const int32_t* row_ptr,
                                     const int32_t* col_idx, const uint8_t* routed,
                                     const uint8_t* token_radius, int32_t r_max, float scale,
                                     void* o_t, float* lse_t, int32_t kv_chunk, void* ws,
                                     size_t ws_bytes, void* stream) {
  VSA_TRY(check_shape(s));
  VSA_TRY(check_ptr(q_t, 16, "q_t"));
  VSA_TRY(check_ptr(k_t, 16, "k_t"));
  VSA_TRY(check_ptr(v_t, 16, "v_t"));
  VSA_TRY(check_ptr(row_ptr, 4, "row_ptr"));
  VSA_TRY(check_ptr(col_idx, 4, "col_idx"));
  VSA_TRY(check_ptr(routed, 1, "routed"));
  VSA_TRY(check_ptr(token_radius, 1, "token_radius"));
  VSA_TRY(check_ptr(o_t, 16, "o_t"));
  if (lse_t) VSA_TRY(check_ptr(lse_t, 4, "lse_t"));
  VSA_TRY(check_ptr(ws, 256, "ws"));
  if (!(scale > 0.f) || scale > 3.0e38f) {
    set_error("scale must be finite and > 0");
    return VSA_ERR_INVALID_ARG;
  }
  if (kv_chunk < 0) {
    set_error("kv_chunk must be >= 0");
    return VSA_ERR_INVALID_ARG;
  }
  if (r_max < 0 || r_max > 255) {
    set_error("r_max %d outside [0, 255]", r_max);
    return VSA_ERR_INVALID_ARG;
  }
  const Grid g = make_grid(*s);
  if (g.nt >= 1024 || g.nh >= 1024 || g.nw >= 1024) {
    set_error("token windows take grids below 1024 tiles along each axis");
    return VSA_ERR_UNSUPPORTED;
  }
  const size_t need = attn_layout(*s, kv_chunk).total;
  if (ws_bytes < need) {
    set_error("attention workspace %zu < %zu bytes", ws_bytes, need);
    return VSA_ERR_CAPACITY;
  }
  int cus = 0;
  VSA_TRY(device_cus(&cus));
  const TokenWindows tw = {token_radius, routed, r_max};
  return hip_status(launch_attn(*s, q_t, k_t, v_t, row_ptr, col_idx, scale, o_t, lse_t, kv_chunk,
                                ws, cus, static_cast<hipStream_t>(stream), nullptr, &tw),
                    "attention launch");
}

}  // extern "C"
