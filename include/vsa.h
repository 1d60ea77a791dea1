/*
 * vsa.h -- block-sparse self-attention over a video DiT's spatio-temporal token
 * grid, for AMD Instinct MI355X (gfx950).  C ABI of libvsa.so.
 *
 * What the library computes
 * -------------------------
 * Tokens of a T x H x W latent grid are grouped into 4x4x4 tiles and stored
 * tile-major ("Token Radius Attention for Efficient Video Generation", TRA,
 * pipeline step 3: a tile-major token layout so that sparse supports become
 * whole blocks).  Query tile a keeps key tile b when b lies in a local window
 * whose radius r_a shrinks with temporal distance (TRA step 2: a per-query
 * base radius applied across frames with a temporal distance-decay rule); the
 * rule used here, in tile units, is
 *     |dt| <= r_a  and  max(|dh|, |dw|) <= r_a - |dt|,
 * with (dt, dh, dw) the tile-coordinate offset b - a.  A routed subset of the
 * query tiles -- the `dense_count` tiles with the highest routing score per
 * (batch, head) -- attends to every key tile instead ("Where Compute Matters:
 * Heterogeneous Attention for Efficient Video Diffusion", abstract: uncertain
 * tokens take dense global attention, the rest local attention, about 20%
 * dense).  Attention is softmax(scale * q.k) v over the kept keys.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tile grid: nTt = ceil(T/4), nTh = ceil(H/4), nTw = ceil(W/4),
 *   nT = nTt*nTh*nTw; tile index tau = (tt*nTh + th)*nTw + tw; slot of a token
 *   inside its tile = (lt*4 + lh)*4 + lw.  Raster token index
 *   n = (t*H + h)*W + w.  N = T*H*W, Npad = 64*nT.
 * - bf16 is bfloat16 stored as 16-bit words.  All device pointers must be
 *   16-byte aligned and point to device memory allocated by the caller; the
 *   library never allocates, frees, synchronises or keeps a pointer after the
 *   call returns.  Work is enqueued asynchronously on `stream` (a hipStream_t
 *   passed as void*, NULL = the null stream); inputs are only read.
 * - Arguments are checked on the host before anything is enqueued; a call that
 *   returns an error has enqueued nothing.  Faults inside kernels surface at
 *   the caller's next synchronisation of the stream.
 * - Results are deterministic: bitwise identical across runs for the same
 *   arguments.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = 1, /* null / misaligned pointer, bad size or count   */
  VSA_ERR_UNSUPPORTED = 2, /* valid request the library does not implement   */
  VSA_ERR_CAPACITY = 3,    /* an output or workspace buffer is too small     */
  VSA_ERR_OVERFLOW = 4,    /* an index would not fit the int32 layouts       */
  VSA_ERR_HIP = 5          /* the HIP runtime refused a launch               */
} vsa_status;

/* Problem shape.  head_dim must be 64 or 128; batch, heads, T, H, W >= 1. */
typedef struct vsa_shape {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t T, H, W;
} vsa_shape;

/* Layouts of a tile-major tensor (argument `layout` of vsa_tile_permute). */
enum {
  /* [B][heads][nT*64][D]: token rows of tile tau at rows tau*64 .. tau*64+63. */
  VSA_LAYOUT_TOKEN_MAJOR = 0,
  /* [B][heads][nT][D][64]: per tile, feature-major (the 64 slots of a tile
   * are contiguous for each feature).  This is the layout vsa_attn_fwd takes
   * for V. */
  VSA_LAYOUT_FEATURE_MAJOR = 1
};

/* Human-readable name of a status code (static string). */
const char* vsa_status_string(vsa_status s);

/* Number of tiles nT of a shape, or -1 if the shape is invalid. */
int32_t vsa_num_tiles(const vsa_shape* s);

/* Last error text of the calling thread (static storage, never NULL). */
const char* vsa_last_error(void);

/* ---------------------------------------------------------------- permute
 * vsa_tile_permute: gather raster tokens into the tile-major layout (TRA,
 * pipeline step 3).
 *   x        bf16 [B][N][heads][D]  (the layout a DiT's QKV projection gives)
 *   x_tiled  bf16, layout per `layout` (see above); every element is written;
 *            slots of padding tokens (outside the T x H x W grid) get +0.0.
 * Errors: INVALID_ARG for a bad shape / pointer / layout; OVERFLOW if an
 * element count exceeds 2^31 per (batch, head) plane.
 */
vsa_status vsa_tile_permute(const vsa_shape* s, const void* x, void* x_tiled,
                            int32_t layout, void* stream);

/* vsa_tile_unpermute: inverse of the token-major permute for the attention
 * output, returning each real token's row to raster order (TRA, pipeline
 * step 3: attention runs in the tile-major layout; the outputs of padding
 * slots, which hold no token, are dropped).  Padded rows of o_tiled are never
 * read.
 *   o_tiled  bf16 [B][heads][nT*64][D]
 *   o        bf16 [B][N][heads][D], every element written.
 * Errors: INVALID_ARG for a bad shape or a NULL / misaligned pointer;
 * OVERFLOW as vsa_tile_permute.
 */
vsa_status vsa_tile_unpermute(const vsa_shape* s, const void* o_tiled, void* o,
                              void* stream);

/* ------------------------------------------------------------------- mask
 * Upper bound of the number of kept (query tile, key tile) pairs when every
 * radius is <= r_max and `dense_count` tiles per (batch, head) are routed.
 * Returns -1 for an invalid shape or count.
 */
int64_t vsa_mask_nnz_bound(const vsa_shape* s, int32_t r_max, int32_t dense_count);

/* Device workspace (bytes) that vsa_build_mask needs. */
size_t vsa_mask_workspace_bytes(const vsa_shape* s);

/* vsa_build_mask: per-tile radii and routing scores -> CSR list of kept key
 * tiles per query tile (TRA step 3: radii translated into a block-sparse mask).
 *   radii        uint8 [B][heads][nT], tile units.  A radius above r_max is
 *                treated as r_max (so the output always fits the bound).
 *   scores       float32 [B][heads][nT].  Per (b, h) the dense_count tiles
 *                first in the order (score descending by IEEE-754 totalOrder,
 *                i.e. +NaN > +inf > ... > +0 > -0 > ... > -NaN; then lower tile
 *                index) are routed dense.
 *   dense_count  0 <= dense_count <= nT.
 *   r_max        0 <= r_max <= 255.
 *   row_ptr      int32 [B*heads*nT + 1]: row (b, h, a) at index
 *                (b*heads + h)*nT + a; row_ptr[0] = 0.
 *   col_idx      int32 [col_capacity]: each row's key tiles, strictly
 *                ascending, the query tile itself always present.
 *   col_capacity must be >= vsa_mask_nnz_bound(s, r_max, dense_count).
 *   routed       optional uint8 [B][heads][nT] (NULL to skip): 1 if routed.
 *   ws, ws_bytes device workspace of at least vsa_mask_workspace_bytes(s).
 * Errors: INVALID_ARG, CAPACITY (col_capacity or ws too small), OVERFLOW
 * (the nnz bound exceeds INT32_MAX).
 */
vsa_status vsa_build_mask(const vsa_shape* s, const uint8_t* radii, const float* scores,
                          int32_t dense_count, int32_t r_max, int32_t* row_ptr,
                          int32_t* col_idx, int64_t col_capacity, uint8_t* routed,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------ token-level inputs
 * The mask builder takes one radius and one routing score per query tile.
 * TRA produces a key budget and a radius per query *token* (steps 1-2) and
 * translates token-level radii into block masks (step 3); HetA-DiT predicts a
 * difficulty per token.  These three calls produce the tile inputs from
 * per-token values.  Per-token arrays are [B][heads][N], N = T*H*W, tokens in
 * raster order n = (t*H + h)*W + w.  The shape is validated as for the other
 * calls (head_dim 64 or 128), though head_dim does not enter.
 *
 * vsa_budget_to_radius (TRA step 2, budget -> base radius):
 *   budget   int32 [B][heads][N]: keys wanted by each query token (any int;
 *            <= 0 asks for nothing beyond the own tile).
 *   r_max    0 <= r_max <= 255.
 *   radius   uint8 [B][heads][N]: the smallest r in [0, r_max] whose tile
 *            window (|dt| <= r, max(|dh|,|dw|) <= r - |dt|, the rule of
 *            vsa_build_mask) holds at least `budget` real key tokens; r_max
 *            if none does.
 * Errors: INVALID_ARG.
 */
vsa_status vsa_budget_to_radius(const vsa_shape* s, const int32_t* budget, int32_t r_max,
                                uint8_t* radius, void* stream);

/* vsa_tile_radius_from_tokens (TRA step 3, token radii -> tile radius):
 *   token_radius uint8 [B][heads][N]
 *   tile_radius  uint8 [B][heads][nT]: the largest radius among the tile's
 *                real tokens, so the tile's window contains each token's.
 * Errors: INVALID_ARG.
 */
vsa_status vsa_tile_radius_from_tokens(const vsa_shape* s, const uint8_t* token_radius,
                                       uint8_t* tile_radius, void* stream);

/* vsa_tile_score_from_tokens (HetA-DiT token difficulty -> tile routing score):
 *   token_score float32 [B][heads][N], 4-byte aligned.
 *   tile_score  float32 [B][heads][nT]: the tile's token score that is largest
 *               in the IEEE-754 totalOrder (the order vsa_build_mask routes
 *               by), so a tile is routed if any of its tokens ranks high.
 * Errors: INVALID_ARG.
 */
vsa_status vsa_tile_score_from_tokens(const vsa_shape* s, const float* token_score,
                                      float* tile_score, void* stream);

/* -------------------------------------------------------------- attention
 * Device workspace (bytes) that vsa_attn_fwd needs for this shape and
 * kv_chunk (0 = automatic splitting).
 */
size_t vsa_attn_workspace_bytes(const vsa_shape* s, int32_t kv_chunk);

/* vsa_attn_fwd: block-sparse attention forward over the tile-major layout
 * (TRA, pipeline step 3: attention executed on the retained blocks of the
 * block-sparse mask only; Triage, "A tile-by-tile choice": skipped tiles cost
 * nothing).  The result is masked softmax attention over the listed key
 * tiles.  Walks only the key tiles listed in the CSR, with bf16 MFMA
 * products, fp32 online softmax and accumulation; long rows are split across
 * workgroups and merged exactly by log-sum-exp (the split never changes
 * which keys a query sees, only the fp32 summation order).
 *   q_t      bf16 [B][heads][nT*64][D]  (VSA_LAYOUT_TOKEN_MAJOR)
 *   k_t      bf16 [B][heads][nT*64][D]  (VSA_LAYOUT_TOKEN_MAJOR)
 *   v_t      bf16 [B][heads][nT][D][64] (VSA_LAYOUT_FEATURE_MAJOR)
 *   row_ptr, col_idx: a CSR over rows (b, h, a) (row_ptr non-decreasing,
 *            row_ptr[0] = 0).  Each row's columns must lie in [0, nT) and
 *            ascend strictly (no repeats), as vsa_build_mask writes them;
 *            columns outside [0, nT) are not checked and read outside k_t
 *            and v_t.  Any other CSR of that kind is accepted.  A row of
 *            exactly nT entries is therefore every key tile, and the call
 *            attends key tiles 0..nT-1 for it without reading its columns;
 *            a shorter row with a repeated column attends that tile once per
 *            occurrence.  A row with no column yields zeros and LSE = -inf.
 *   scale    softmax scale (1/sqrt(D) for standard attention), finite, > 0.
 *   o_t      bf16 [B][heads][nT*64][D]: outputs; rows of padding query slots
 *            hold unspecified values.
 *   lse_t    optional float32 [B][heads][nT*64] (NULL to skip): natural-log
 *            sum of exp(scale*q.k) over the kept valid keys.
 *   kv_chunk 0 = automatic; > 0 = split every row into chunks of at most
 *            kv_chunk key tiles (for testing split invariance).
 *   ws, ws_bytes device workspace of at least vsa_attn_workspace_bytes(s,
 *            kv_chunk); its contents need no initialisation.
 * Padding keys (slots outside the grid) are excluded from every softmax by
 * position: their K values never matter, and their V values are multiplied
 * by a probability of exactly 0 (or, for the 32 keys of time slices 2-3 of a
 * key tile with at most 2 valid time slices, not read at all), so they must
 * be finite (the permute writes +0.0 there); a NaN or infinity in a padded V
 * slot may make the outputs of the query tiles that list that key tile NaN.
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim not 64/128), CAPACITY (ws),
 * OVERFLOW.
 */
vsa_status vsa_attn_fwd(const vsa_shape* s, const void* q_t, const void* k_t,
                        const void* v_t, const int32_t* row_ptr, const int32_t* col_idx,
                        float scale, void* o_t, float* lse_t, int32_t kv_chunk,
                        void* ws, size_t ws_bytes, void* stream);

/* vsa_attn_fwd_raster: vsa_attn_fwd with the query read from, and the output
 * written to, the caller's raster layout, so that the Q permute and the O
 * unpermute of the pipeline (TRA, step 3: tile-major token layout; the padded
 * query slots' outputs are discarded) happen inside the call: each query tile
 * gathers its 64 token rows, and each real token's output row is written in
 * place.  The arithmetic is that of vsa_attn_fwd, so O and LSE are bitwise
 * those of vsa_attn_fwd followed by vsa_tile_unpermute (and the same permute
 * of the LSE).
 *   q        bf16 [B][N][heads][D] (raster, N = T*H*W), 16-byte aligned.
 *   k_t, v_t, row_ptr, col_idx, scale, kv_chunk, ws, ws_bytes: as
 *            vsa_attn_fwd (the same workspace size).
 *   o        bf16 [B][N][heads][D], every element written; 16-byte aligned.
 *            Must not overlap q.
 *   lse      optional fp32 [B][heads][N], natural-log LSE of every token;
 *            NULL to skip.
 * Errors: as vsa_attn_fwd.
 */
vsa_status vsa_attn_fwd_raster(const vsa_shape* s, const void* q, const void* k_t,
                               const void* v_t, const int32_t* row_ptr, const int32_t* col_idx,
                               float scale, void* o, float* lse, int32_t kv_chunk, void* ws,
                               size_t ws_bytes, void* stream);

/* ------------------------------------------------- allocation-free call
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the raster
 * forward call with its workspace taken from a fixed device array inside the
 * library instead of a caller buffer.  The library allocates nothing on this
 * path (no hipMalloc, no allocating library routine); the array is part of
 * the loaded code object, one copy per GPU, held until the process ends.
 *
 * vsa_attn_noalloc_max_workspace: the array's size in bytes (48 MiB); a
 * shape fits when vsa_attn_workspace_bytes(s, 0) is at most this.
 *
 * vsa_attn_fwd_raster_noalloc: vsa_attn_fwd_raster with kv_chunk = 0 and
 * that array as its workspace; the same kernels, so O and LSE are bitwise
 * those of vsa_attn_fwd_raster.  Every call on a GPU uses that GPU's one
 * array, and nothing in it needs to start at zero (each call's plan writes
 * what the call reads), but two calls in flight at once on the same GPU (on
 * different streams, or from different threads) race on it: serialise them.
 *   q, k_t, v_t, row_ptr, col_idx, scale, o, lse: as vsa_attn_fwd_raster.
 * Errors: as vsa_attn_fwd_raster; CAPACITY when the shape needs more than
 * vsa_attn_noalloc_max_workspace() bytes (nothing is enqueued then).
 */
size_t vsa_attn_noalloc_max_workspace(void);

vsa_status vsa_attn_fwd_raster_noalloc(const vsa_shape* s, const void* q, const void* k_t,
                                       const void* v_t, const int32_t* row_ptr,
                                       const int32_t* col_idx, float scale, void* o,
                                       float* lse, void* stream);

/* ----------------------------------------------------- low-precision tier
 * "Triage: Skip, Skim, or Refine Attention Tiles in Video Diffusion
 * Transformers" (plain-words summary; "Route by estimated error"): every
 * attention tile is skipped, computed in a quick 4-bit version ("skim") or
 * computed accurately ("refine").  The pages give neither the 4-bit format
 * nor the router's formulas, so here the tier of every kept (query tile, key
 * tile) pair is an input and the format is OCP MXFP4 (E2M1 elements, one E8M0
 * power-of-two scale per 32 consecutive features), which gfx950's scaled MFMA
 * consumes.  Skipped tiles are the ones absent from the CSR.
 *
 * vsa_quantize_mxfp4: MXFP4 encoding of a token-major tiled Q or K along D,
 * per the OCP Microscaling Formats specification v1.0: block scale
 * X = 2^(floor(log2 max|v|) - 2) (exponent clamped to [-127, 127]; -127 for an
 * all-zero block), each v / X rounded to the nearest of +-{0, .5, 1, 1.5, 2,
 * 3, 4, 6} with ties to the even code and saturation at 6; the sign of -0.0
 * is kept.
 *   x_tiled  bf16 [B][heads][nT*64][D] (VSA_LAYOUT_TOKEN_MAJOR), finite.
 *   codes    uint8 [B][heads][nT*64][D/2]: element 2i in the low nibble of
 *            byte i, element 2i+1 in the high nibble; a nibble is sign (bit 3)
 *            and the index (bits 0-2) into {0, .5, 1, 1.5, 2, 3, 4, 6}.
 *   scales   uint8 [B][heads][nT*64][D/32]: E8M0, exponent + 127.
 * All buffers are the caller's; codes/scales are fully written.
 * Errors: INVALID_ARG (shape, NULL or misaligned pointer: 16 bytes for all
 * three), UNSUPPORTED (head_dim not 64/128), OVERFLOW.
 */
vsa_status vsa_quantize_mxfp4(const vsa_shape* s, const void* x_tiled, void* codes, void* scales,
                              void* stream);

/* vsa_attn_fwd_tiered: vsa_attn_fwd with a tier per CSR entry.  Where
 * tier[e] != 0 the scores of that (query tile, key tile) pair are computed
 * from the MXFP4 Q and K (products of the dequantised values, fp32
 * accumulation); elsewhere from the bf16 Q and K.  Softmax, P.V (bf16 P and V)
 * and the output are as in vsa_attn_fwd; one softmax spans both tiers.
 *   q_t, k_t, v_t, row_ptr, col_idx, scale, o_t, lse_t, kv_chunk, ws,
 *   ws_bytes: as vsa_attn_fwd (the same workspace size).
 *   q4, q4_scales, k4, k4_scales: vsa_quantize_mxfp4 of q_t and k_t.
 *   tier     uint8 [nnz], one per CSR entry (same order as col_idx).
 * Errors: as vsa_attn_fwd, plus INVALID_ARG for NULL or misaligned MXFP4
 * buffers (16 bytes) or a NULL tier.
 */
vsa_status vsa_attn_fwd_tiered(const vsa_shape* s, const void* q_t, const void* k_t,
                               const void* v_t, const void* q4, const void* q4_scales,
                               const void* k4, const void* k4_scales, const int32_t* row_ptr,
                               const int32_t* col_idx, const uint8_t* tier, float scale,
                               void* o_t, float* lse_t, int32_t kv_chunk, void* ws,
                               size_t ws_bytes, void* stream);

/* ------------------------------------------------ exact per-token windows
 * "Token Radius Attention for Efficient Video Generation", pipeline steps 2
 * and 3: every query token has its own radius, and the radii become block
 * masks.  The block mask of a tile (vsa_build_mask on
 * vsa_tile_radius_from_tokens) uses the largest radius among its tokens, a
 * superset of each token's window.
 *
 * vsa_attn_fwd_token_window: vsa_attn_fwd on that CSR, with each query token
 * attending only the kept key tiles that lie inside the window of its own
 * radius r = min(token_radius, r_max) around its tile (|dt| <= r and
 * max(|dh|, |dw|) <= r - |dt| in tile coordinates); the query tiles that the
 * mask builder routed attend every kept key tile.  Every token's own tile
 * is in its window, so no valid query is left without keys.
 *   q_t, k_t, v_t, row_ptr, col_idx, scale, o_t, lse_t, kv_chunk, ws,
 *   ws_bytes: as vsa_attn_fwd (the same workspace size).  The CSR must be
 *            the mask builder's for tile radii >= each token's radius (e.g.
 *            vsa_tile_radius_from_tokens of token_radius) and the same r_max:
 *            keys outside the CSR are never attended.
 *   routed   uint8 [B][heads][nT]: the mask builder's routed flags.
 *   token_radius uint8 [B][heads][N], N = T*H*W, raster order.
 *   r_max    0 <= r_max <= 255, the clamp the mask builder applied.
 * Errors: as vsa_attn_fwd, plus INVALID_ARG for a NULL routed or
 * token_radius or an r_max outside [0, 255], and UNSUPPORTED for grids of
 * 1024 or more tiles along t, h or w.
 */
vsa_status vsa_attn_fwd_token_window(const vsa_shape* s, const void* q_t, const void* k_t,
                                     const void* v_t, const int32_t* row_ptr,
                                     const int32_t* col_idx, const uint8_t* routed,
                                     const uint8_t* token_radius, int32_t r_max, float scale,
                                     void* o_t, float* lse_t, int32_t kv_chunk, void* ws,
                                     size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H_ */
