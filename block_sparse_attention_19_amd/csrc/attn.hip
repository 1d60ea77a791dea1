// Block-sparse attention forward over tile-major Q/K/V, driven by a CSR of kept
// key tiles per query tile.
//
// The pages ("Token Radius Attention for Efficient Video Generation", step 3;
// "Triage: Skip, Skim, or Refine Attention Tiles in Video Diffusion
// Transformers", fused kernel) execute attention only on the retained tiles of
// a block-sparse mask.  The result is exactly masked softmax attention: every
// key tile a query tile does not list contributes nothing, so the kernel walks
// the listed tiles only.
//
// Execution model (CDNA4 / gfx950):
//   * A workgroup is 4 waves (256 threads).  Each wave owns 32 query rows and
//     keeps them in registers as the B operand of v_mfma_f32_32x32x16_bf16.
//   * Scores are computed transposed, S^T = K Q^T, so that every lane ends up
//     holding one query's scores: the row max / row sum are in-lane except for
//     one exchange between the two 32-lane halves, and the probabilities P^T
//     are already the B operand of the second product O^T = V^T P^T, whose
//     accumulator again holds one query per lane (one rescale factor per lane).
//   * K is staged in LDS as [64 keys][D], V as [D][64 keys] (the permute writes
//     V feature-major), both XOR-swizzled so the 16-byte operand reads of a
//     wave are bank-conflict free.  The 64 keys of a tile are read in an order
//     (bits 2 and 3 of the row index swapped) that makes each lane's 8 P values
//     one contiguous 16-byte V^T read.
//   * Online softmax in fp32, base 2 (scale * log2 e folded into one FMA), with
//     lazy rescaling: the running max only moves when a new score exceeds it
//     by more than 2^8, which keeps P <= 256 and skips most O rescales.
//   * Work units come from a device-side plan: "G" units pair two query tiles
//     of one (batch, head) whose key lists are both complete (every key tile;
//     routed rows) so one staged K/V tile feeds 4 waves; "S" units take one
//     query tile and split its key list over two wave pairs, merged in LDS at
//     the end.  Long G units are split into key chunks that write fp32
//     partials (O, running max, sum) merged exactly by a combine kernel.
//     A persistent grid (2 workgroups per CU) takes the units from 8 queues,
//     one per XCD, long units first and the local rows in row order.
//   * Three instances of the kernel: the bf16 forward; the skim tier (the
//     scores of chosen tile pairs from MXFP4 Q and K by scaled MFMA); and
//     exact per-token windows (each lane's query attends only the listed key
//     tiles inside the window of its own radius).
#include "vsa_common.h"

#include <limits.h>

#include <type_traits>

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte chunk (native vector)
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kPlanThreads = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: P stays <= 2^8
constexpr int kMinChunk = 32;          // smallest automatic key chunk (tiles)
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0), expcnt/lgkmcnt unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;
// Automatic splitting of G units starts when there are fewer than this many
// (half the resident workgroups of a 256-CU part at 2 per CU): then each is cut
// into key chunks so that about this many exist.  Fixed so workspace sizes do
// not depend on the device.
constexpr int kSplitTarget = 256;

struct Unit {
  int32_t row[2];  // CSR rows (global); S units use row[0] only
  int32_t kb, ke;  // key range [kb, ke): offsets into row[0]'s column list
  int32_t slot;    // first partial slot, or -1: write the final output
  int32_t mode;    // 0 = G (two query tiles share the keys), 1 = S (one tile, keys split)
  int32_t complete;  // 1: the row holds nT entries, so its keys are 0..nT-1 (G units always)
  int32_t pad;
};
static_assert(sizeof(Unit) == 32, "unit layout");

struct Comb {
  int32_t row, slot0, stride, n;
};

// Units are dealt to 8 queues, one per XCD: workgroup b serves queue b % 8
// first, the XCD that the hardware dispatches it to, and an empty queue sends
// its workgroups to the others.  Both parts of the order are cut into 8
// contiguous spans.  In the head (long units: front S and G units, all about
// one full row long, so equal spans balance) an XCD then runs the units of
// one or two heads at a time, which walk the same key tiles in the same order
// and share them through its L2 (dealing the head in chunks of 16 units made
// each XCD stream every head: 1.2-1.6x the L2 misses of the whole call, at the
// same speed).  In the rest (local rows, in the order of RowOrder) the units
// running at once on an XCD are neighbouring query tiles whose key windows
// overlap.
constexpr int kQueues = 8;

struct Header {
  int32_t n_units;
  int32_t pad1;
  int32_t n_comb;
  int32_t chunks_g;    // key chunks per G unit (for inspection; no kernel reads it)
  int32_t overflow;    // 1: the plan did not fit the workspace and no unit was written
                       // (cannot happen for a workspace of the size the entry points demand)
  int32_t n_head;      // units [0, n_head): front S and G units
  int32_t rest_span;   // units past n_head: queue x owns n_head + [x, x + 1) * rest_span
  int32_t head_span;   // units below n_head: queue x owns [x, x + 1) * head_span
  int32_t queue[kQueues];
  int32_t queue_rest[kQueues];
  int32_t pad[40];
};
static_assert(sizeof(Header) == 256, "header layout");

// Extent of a key tile inside the grid (tokens valid along t, h, w); a tile
// with any extent below 4 holds padding slots that must not be attended.
struct TileExtent {
  int vt, vh, vw;
  bool edge;
};

// Packed extent of a tile: vt | vh << 4 | vw << 8 | edge << 12 (written once per
// call by the plan kernel, read per key tile by the attention kernel).
__device__ __forceinline__ int pack_extent(int tau, int nh, int nw, int T, int H, int W) {
  const int tw = tau % nw, th = (tau / nw) % nh, tt = tau / (nw * nh);
  const int vt = min(kTile, T - tt * kTile), vh = min(kTile, H - th * kTile),
            vw = min(kTile, W - tw * kTile);
  const int edge = (vt < kTile) | (vh < kTile) | (vw < kTile);
  return vt | (vh << 4) | (vw << 8) | (edge << 12);
}

__device__ __forceinline__ TileExtent unpack_extent(int code) {
  TileExtent e;
  e.vt = code & 15;
  e.vh = (code >> 4) & 15;
  e.vw = (code >> 8) & 15;
  e.edge = (code >> 12) & 1;
  return e;
}

__device__ __forceinline__ TileExtent tile_extent(int tau, int nh, int nw, int T, int H, int W) {
  TileExtent e;
  const int tw = tau % nw, th = (tau / nw) % nh, tt = tau / (nw * nh);
  e.vt = min(kTile, T - tt * kTile);
  e.vh = min(kTile, H - th * kTile);
  e.vw = min(kTile, W - tw * kTile);
  e.edge = (e.vt < kTile) | (e.vh < kTile) | (e.vw < kTile);
  return e;
}

}  // namespace

// Packed tile coordinates tt | th << 10 | tw << 20 (each below 1024; the entry
// point taking token windows checks the grid).
__device__ __forceinline__ int pack_coord(int tau, int nh, int nw) {
  const int tw = tau % nw, th = (tau / nw) % nh, tt = tau / (nw * nh);
  return tt | (th << 10) | (tw << 20);
}

// Window distance of key tile c from query tile qc (packed coordinates): key
// tile c lies in the window of radius r around qc iff r >= this value (the
// rule |dt| <= r, max(|dh|, |dw|) <= r - |dt| rearranged).
__device__ __forceinline__ int window_dist(int c, int qc) {
  const int dt = abs((c & 1023) - (qc & 1023));
  const int dh = abs(((c >> 10) & 1023) - ((qc >> 10) & 1023));
  const int dw = abs(((c >> 20) & 1023) - ((qc >> 20) & 1023));
  return dt + max(dh, dw);
}

// ------------------------------------------------------------ workspace

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

AttnLayout attn_layout(const vsa_shape& s, int kv_chunk) {
  const Grid g = make_grid(s);
  AttnLayout L;
  L.bh = (int64_t)s.batch * s.heads;
  L.rows = L.bh * g.nT;
  const int64_t target = kSplitTarget;
  if (kv_chunk > 0) {
    const int64_t ch = (g.nT + kv_chunk - 1) / kv_chunk;
    L.max_units = (L.rows / 2 + L.rows) * ch + 1;
    L.max_slots = L.rows * ch;
  } else {
    L.max_units = L.rows / 2 + 2 * target + L.rows + 1;
    L.max_slots = 4 * target;
  }
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
  take(sizeof(Header));
  L.off_cbase = take(4 * (L.bh + 1));
  L.off_gbase = take(4 * (L.bh + 1));
  L.off_grows = take(4 * (L.rows + 2));
  L.off_units = take(sizeof(Unit) * L.max_units);
  L.off_comb = take(sizeof(Comb) * (L.rows + 1));
  L.off_po = take((size_t)L.max_slots * kTileTokens * s.head_dim * 4);
  L.off_pml = take((size_t)L.max_slots * kTileTokens * 2 * 4);
  L.off_ext = take(4 * (size_t)g.nT);
  L.off_coord = take(4 * (size_t)g.nT);
  L.off_iota = take(4 * (size_t)g.nT);
  L.total = o;
  return L;
}

namespace {

// ------------------------------------------------------------------ plan

struct PlanArgs {
  const int* row_ptr;
  int bh, nT, kv_chunk, target;
  int nh, nw, T, H, W;
  int blk_h, blk_w;  // spatial block of the row order (see RowOrder)
  int64_t max_units, max_slots;
  Header* hdr;
  int *cbase, *gbase, *grows, *ext, *coord, *iota;
  Unit* units;
  Comb* comb;
};

// Rows are taken in blocks of SEG * kPlanThreads positions of the plan's
// order (RowOrder below).  Wave w of the block holds positions
// 64 SEG w + 64j + lane (j < SEG): consecutive lanes write consecutive unit
// records, and the order is (wave, j, lane); their row_ptr reads gather
// within one (batch, head).  Row indices fit in 32 bits (rows * 64 tokens is
// checked against INT_MAX on the host), so all index arithmetic here is
// 32-bit.
// SEG rows per thread: 8 for the default plan; the plan that cuts rows into
// kv_chunk pieces places several units per row and takes 1, which keeps its
// state in registers (at 1024 threads a lane has 128 VGPRs; at 2 rows per
// thread it spilled 40 of them to scratch, at 8 rows 246).
constexpr int kPlanWaves = kPlanThreads / 64;
template <bool CHUNKED>
constexpr int plan_seg() { return CHUNKED ? 1 : 8; }

template <int SEG>
__device__ __forceinline__ int plan_row(int c0, int j) {
  return c0 + (int)(threadIdx.x >> 6) * (SEG * 64) + (j << 6) + (int)(threadIdx.x & 63);
}

// The order in which the plan takes the rows of one (batch, head), and so the
// order of the local-row units: the tile grid is cut into spatial blocks of
// blk_h x blk_w tiles (columns of blocks along w outermost, then blocks along
// h), and each block is taken whole, time slice by time slice, row-major
// inside a slice.  Units running at once on an XCD then hold query tiles of
// one narrow spatial block at a few neighbouring times, whose windows share
// more key tiles in its L2 than whole rows of the grid do (an LRU model of the
// L2 and measurement both favour blocks of at most 8 x 7 tiles).  Position
// `pos` of the order is tile tile(pos), and pos(tau) is its inverse: a
// bijection of [0, nT).  Grids of up to kOrderLds tiles keep the order as a
// table in LDS, larger ones evaluate tile(pos) per row.
constexpr int kOrderBlkH = 8, kOrderBlkW = 7;
constexpr int kOrderLds = 8192;
struct RowOrder {
  int nT, nt, nh, nw, blk_h, blk_w;
  __device__ __forceinline__ int pos(int tau) const {
    const int tt = tau / (nh * nw);
    const int rem = tau - tt * (nh * nw);
    const int th = rem / nw, tw = rem - th * nw;
    const int wb = tw / blk_w, hb = th / blk_h;
    const int wl = min(blk_w, nw - wb * blk_w), hl = min(blk_h, nh - hb * blk_h);
    return wb * (nt * nh * blk_w) + hb * (nt * blk_h * wl) + (tt * hl + (th - hb * blk_h)) * wl +
           (tw - wb * blk_w);
  }
  __device__ __forceinline__ int tile(int pos) const {
    const int col = nt * nh * blk_w;  // positions in a full column of blocks
    const int wb = pos / col;         // (only the last column can be narrower)
    int rem = pos - wb * col;
    const int wl = min(blk_w, nw - wb * blk_w);
    const int cell = nt * blk_h * wl;  // positions in a full block of the column
    const int hb = rem / cell;
    rem -= hb * cell;
    const int hl = min(blk_h, nh - hb * blk_h);
    const int tt = rem / (hl * wl);
    rem -= tt * (hl * wl);
    const int th = hb * blk_h + rem / wl, tw = wb * blk_w + rem % wl;
    return (tt * nh + th) * nw + tw;
  }
  // row index of iteration index i (same (batch, head): i / nT); `table`
  // holds tile(pos) for every pos when it is not null
  __device__ __forceinline__ int row(int i, const int* table) const {
    const int b = i / nT;
    const int p = i - b * nT;
    return b * nT + (table ? table[p] : tile(p));
  }
};

// Lengths of this thread's rows of the block at c0 (-1 past the last row).
template <int SEG>
__device__ __forceinline__ void load_lengths(const int* row_ptr, int rows, int c0,
                                             const RowOrder& ord, const int* table,
                                             int (&len)[SEG]) {
  int a[SEG], b[SEG];
#pragma unroll
  for (int j = 0; j < SEG; ++j) {
    const int i = plan_row<SEG>(c0, j);
    const int r = (i < rows) ? ord.row(i, table) : rows;
    a[j] = row_ptr[r];
    b[j] = row_ptr[min(r + 1, rows)];
  }
#pragma unroll
  for (int j = 0; j < SEG; ++j) len[j] = (plan_row<SEG>(c0, j) < rows) ? b[j] - a[j] : -1;
}

// Exclusive prefix of a 0/1 count over the lanes of the wave, and the wave
// total, by a ballot and bit counts.  Called by all 64 lanes.
__device__ __forceinline__ int wave_prefix_flags(int v, int* total) {
  const unsigned long long m = __ballot(v != 0);
  *total = __popcll(m);
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The same for any count, by a shuffle scan.
__device__ __forceinline__ int wave_prefix_scan(int v, int* total) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  *total = __shfl(x, 63);
  return x - v;
}

// Per-wave counts -> the sum over earlier waves (in place) and the block
// totals.  `ws` holds NV * kPlanWaves ints of LDS.
template <int NV>
__device__ __forceinline__ void wave_offsets(int (&wt)[NV], int* ws, int (&total)[NV]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) ws[k * kPlanWaves + w] = wt[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kPlanWaves; ++i) {
      const int x = ws[k * kPlanWaves + i];
      all += x;
      before += (i < w) ? x : 0;
    }
    wt[k] = before;
    total[k] = all;
  }
  __syncthreads();
}

// Row-order exclusive prefix of NV per-row counts over the block (in place),
// and the block totals; FLAGS: every count is 0 or 1.
template <int NV, bool FLAGS, int SEG>
__device__ void block_prefix_rows(int (&v)[NV][SEG], int* ws, int (&total)[NV]) {
  int wt[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    int run = 0;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      int t;
      const int pre = FLAGS ? wave_prefix_flags(v[k][j], &t) : wave_prefix_scan(v[k][j], &t);
      v[k][j] = run + pre;
      run += t;
    }
    wt[k] = run;
  }
  wave_offsets<NV>(wt, ws, total);
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int j = 0; j < SEG; ++j) v[k][j] += wt[k];
}

// Thread-order exclusive prefix of NV per-thread counts (in place), and totals.
template <int NV>
__device__ void block_prefix_threads(int (&v)[NV], int* ws, int (&total)[NV]) {
  int wt[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wave_prefix_scan(v[k], &wt[k]);
  wave_offsets<NV>(wt, ws, total);
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] += wt[k];
}

// Work plan of one call: G units (pairs of complete rows of one (batch, head),
// optionally cut into key chunks), S units (every other row, cut into chunks of
// kv_chunk keys when that is set), their order, partial-output slots and
// combine entries.  Pass 1 scans the complete rows (their count before each
// (batch, head)) and totals the S units of the other rows; the per-(batch,
// head) scan then fixes the pairing, the G chunking and every total; pass 2
// places each row.  CHUNKED: S rows are cut into kv_chunk keys (a row may
// then give several units); otherwise each S row is one unit.
template <bool CHUNKED>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs p) {
  __shared__ int ws[5 * kPlanWaves];
  __shared__ int s_chunk_g, s_sg, s_front;
  constexpr int SEG = plan_seg<CHUNKED>();
  constexpr int kBlock = SEG * kPlanThreads;
  const int nT = p.nT;  // >= 1
  const int t = threadIdx.x;
  const int rows = p.bh * nT;
  const RowOrder ord = {nT, nT / (p.nh * p.nw), p.nh, p.nw, p.blk_h, p.blk_w};
  constexpr bool chunked = CHUNKED;
  const int chunk_s = p.kv_chunk;
  // S chunks of a row of `len` keys, and the key count of chunk c
  auto n_chunks = [&](int len) { return (!chunked || len <= 0) ? 1 : (len + chunk_s - 1) / chunk_s; };
  auto chunk_len = [&](int len, int n, int c) {
    if (n == 1) return max(len, 0);
    return max(0, min(len, (c + 1) * chunk_s) - c * chunk_s);
  };
  // S units of at least half a full row go first (see the unit order below)
  auto is_front = [&](int lu) { return 2 * lu >= nT; };
  auto n_front_of = [&](int len, int n) {
    if (n == 1) return (int)is_front(max(len, 0));
    int f = 0;
    for (int c = 0; c < n; ++c) f += is_front(chunk_len(len, n, c));
    return f;
  };

  __shared__ int s_order[kOrderLds];
  const int* table = (nT <= kOrderLds) ? s_order : nullptr;
  for (int tau = t; tau < nT; tau += kPlanThreads) {
    p.ext[tau] = pack_extent(tau, p.nh, p.nw, p.T, p.H, p.W);
    p.coord[tau] = pack_coord(tau, p.nh, p.nw);
    p.iota[tau] = tau;
    if (table) s_order[ord.pos(tau)] = tau;
  }
  if (t == 0) s_front = 0;
  __syncthreads();

  // pass 1: cbase[b] = complete rows before (b, h) (a scan of the complete-row
  // flags in row order), and the S totals of the incomplete rows.  With a
  // single block the lengths stay in registers for pass 2.
  const bool one_block = rows <= kBlock;
  int len[SEG];
  int a_units = 0, a_front = 0, a_slots = 0, a_comb = 0;
  int carry_c = 0;
  for (int c0 = 0; c0 < rows; c0 += kBlock) {
    load_lengths(p.row_ptr, rows, c0, ord, table, len);
    int before[1][SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) before[0][j] = (len[j] == nT);
    int blk[1];
    block_prefix_rows<1, true>(before, ws, blk);
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      if (len[j] < 0) continue;
      const int i = plan_row<SEG>(c0, j);  // iteration index; its row is in (b, h) = i / nT
      const int b = i / nT;
      if (i == b * nT) p.cbase[b] = carry_c + before[0][j];
      if (len[j] != nT) {
        const int n = n_chunks(len[j]);
        a_units += n;
        a_front += n_front_of(len[j], n);
        if (n > 1) {
          a_slots += n;
          a_comb += 1;
        }
      }
    }
    carry_c += blk[0];
  }
  if (t == 0) p.cbase[p.bh] = carry_c;
  __syncthreads();

  // per (b, h): pairs of complete rows -> G groups (gbase = their exclusive
  // scan); a complete row left over from the pairing becomes an S unit
  const int segb = (p.bh + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(p.bh, segb * t), b1 = min(p.bh, b0 + segb);
  auto count_of = [&](int b) { return p.cbase[b + 1] - p.cbase[b]; };
  int g_sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int c = count_of(b);
    g_sum += c / 2;
    if (c & 1) {
      const int n = n_chunks(nT);
      a_units += n;
      a_front += n_front_of(nT, n);
      if (n > 1) {
        a_slots += n;
        a_comb += 1;
      }
    }
  }
  int tv[5] = {g_sum, a_units, a_front, a_slots, a_comb};
  int tot[5];
  block_prefix_threads<5>(tv, ws, tot);
  const int NG = tot[0], nSU = tot[1], nFront = tot[2], nSP = tot[3], nSC = tot[4];
  int gb = tv[0];
  for (int b = b0; b < b1; ++b) {
    p.gbase[b] = gb;
    gb += count_of(b) / 2;
  }
  if (t == 0) {
    int chunk;
    if (chunked) {
      chunk = p.kv_chunk;
    } else {
      int s = 1;
      if (NG > 0) s = max(1, (p.target + NG - 1) / NG);
      s = min(s, max(1, nT / kMinChunk));
      chunk = (nT + s - 1) / s;
    }
    chunk = max(1, min(chunk, nT));
    s_chunk_g = chunk;
    s_sg = (nT + chunk - 1) / chunk;
  }
  __syncthreads();
  const int chunk_g = s_chunk_g, sg = s_sg;
  const int64_t nGU = (int64_t)NG * sg;
  const int64_t gslots = (sg > 1) ? 2 * nGU : 0;
  const int64_t n_units = nGU + nSU;
  const int64_t n_comb = ((sg > 1) ? 2LL * NG : 0) + nSC;
  if (n_units > p.max_units || gslots + nSP > p.max_slots) {
    if (t == 0) {
      p.hdr->n_units = 0;
      p.hdr->n_comb = 0;
      p.hdr->overflow = 1;
      p.hdr->n_head = 0;
      p.hdr->rest_span = 0;
      p.hdr->head_span = 0;
      for (int x = 0; x < kQueues; ++x) p.hdr->queue[x] = p.hdr->queue_rest[x] = 0;
    }
    return;
  }
  // From here every count fits in 32 bits (bounded by max_units / max_slots).

  // Unit order: S units of at least half a full row first (complete rows left
  // over from the pairing), so that no unit as long as a G unit starts late;
  // then the G units; then the other S units in the plan's row order (spatial
  // blocks, RowOrder), so that neighbouring query tiles, whose key windows
  // overlap, run close in time on one XCD and share its L2.
  const int ngu = (int)nGU, gsl = (int)gslots;
  const int rest_base = nFront + ngu;
  const int comb_base = (sg > 1) ? 2 * NG : 0;

  // pass 2: place every row
  int carry_rest = 0, carry_slot = 0, carry_comb = 0;
  carry_c = 0;
  for (int c0 = 0; c0 < rows; c0 += kBlock) {
    if (!one_block) load_lengths(p.row_ptr, rows, c0, ord, table, len);
    int before[1][SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) before[0][j] = (len[j] == nT);
    int blk_c[1];
    block_prefix_rows<1, true>(before, ws, blk_c);
    // per row: rest-region units, then (CHUNKED) partial slots and combine entries
    constexpr int NC = CHUNKED ? 3 : 1;
    int nS[SEG];            // S chunks of the row, 0 for G members and padding
    int cnt[NC][SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      nS[j] = 0;
#pragma unroll
      for (int k = 0; k < NC; ++k) cnt[k][j] = 0;
      const int i = plan_row<SEG>(c0, j);
      const int b = min(i, rows - 1) / nT;
      const int cb_r = p.cbase[b], cnt_r = p.cbase[b + 1] - cb_r, gb_r = p.gbase[b];
      if (len[j] < 0) continue;
      const int r = ord.row(i, table);
      bool g_member = false;
      if (len[j] == nT) {
        const int jj = carry_c + before[0][j] - cb_r;  // index among the complete rows of (b, h)
        if ((unsigned)jj < (unsigned)((cnt_r / 2) * 2)) {
          p.grows[(gb_r + jj / 2) * 2 + (jj & 1)] = r;
          g_member = true;
        }
      }
      if (!g_member) {
        const int n = n_chunks(len[j]);
        nS[j] = n;
        cnt[0][j] = n - n_front_of(len[j], n);
        if constexpr (CHUNKED) {
          if (n > 1) {
            cnt[1][j] = n;
            cnt[2][j] = 1;
          }
        }
      }
    }
    int blk[NC];
    block_prefix_rows<NC, !CHUNKED>(cnt, ws, blk);
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
      const int n = nS[j];
      if (n == 0) continue;
      const int r = ord.row(plan_row<SEG>(c0, j), table);
      int pos_rest = carry_rest + cnt[0][j];
      int slot0 = -1;
      if constexpr (CHUNKED) slot0 = gsl + carry_slot + cnt[1][j];
      for (int c = 0; c < n; ++c) {
        Unit u;
        u.row[0] = r;
        u.row[1] = -1;
        u.kb = (n > 1) ? c * chunk_s : 0;
        u.ke = u.kb + chunk_len(len[j], n, c);
        u.slot = (n > 1) ? slot0 + c : -1;
        u.mode = 1;
        u.complete = (len[j] == nT) ? 1 : 0;
        u.pad = 0;
        const int at = is_front(u.ke - u.kb) ? atomicAdd(&s_front, 1) : rest_base + pos_rest++;
        if ((unsigned)at < (unsigned)n_units) p.units[at] = u;
      }
      if constexpr (CHUNKED) {
        if (n > 1) {
          Comb cb2;
          cb2.row = r;
          cb2.slot0 = slot0;
          cb2.stride = 1;
          cb2.n = n;
          const int ci = comb_base + carry_comb + cnt[2][j];
          if ((unsigned)ci < (unsigned)n_comb) p.comb[ci] = cb2;
        }
      }
    }
    carry_c += blk_c[0];
    carry_rest += blk[0];
    if constexpr (CHUNKED) {
      carry_slot += blk[1];
      carry_comb += blk[2];
    }
  }
  __syncthreads();

  // G units (their rows were placed in grows by pass 2) and their combine entries
  for (int i = t; i < ngu; i += kPlanThreads) {
    const int gi = i / sg, c = i - gi * sg;
    Unit u;
    u.row[0] = p.grows[2 * gi];
    u.row[1] = p.grows[2 * gi + 1];
    u.kb = c * chunk_g;
    u.ke = min(nT, u.kb + chunk_g);
    u.slot = (sg > 1) ? 2 * i : -1;
    u.mode = 0;
    u.complete = 1;
    u.pad = 0;
    p.units[nFront + i] = u;
  }
  if (sg > 1) {
    for (int i = t; i < 2 * NG; i += kPlanThreads) {
      const int gi = i >> 1, q = i & 1;
      Comb cb2;
      cb2.row = p.grows[2 * gi + q];
      cb2.slot0 = 2 * gi * sg + q;
      cb2.stride = 2;
      cb2.n = sg;
      p.comb[i] = cb2;
    }
  }
  if (t == 0) {
    p.hdr->n_units = (int)n_units;
    p.hdr->n_comb = (int)n_comb;
    p.hdr->chunks_g = sg;
    p.hdr->overflow = 0;
    p.hdr->n_head = nFront + ngu;
    p.hdr->rest_span = ((int)n_units - (nFront + ngu) + kQueues - 1) / kQueues;
    p.hdr->head_span = ((int)(nFront + ngu) + kQueues - 1) / kQueues;
    for (int x = 0; x < kQueues; ++x) p.hdr->queue[x] = p.hdr->queue_rest[x] = 0;
  }
}

// -------------------------------------------------------------- attention

// Where the query and the output of a tile slot live.  Tile-major (the
// permuted layout): row `row` of the CSR, slot s at element ((row * 64) + s) * D,
// LSE at row * 64 + s.  Raster (the caller's [B][N][Hh][D] layout, LSE
// [B][Hh][N]): the slot's token (t, h, w) of tile tau = row mod nT, at element
// ((b * N + n) * Hh + head) * D with n = (t * H + h) * W + w; a padded slot has
// no token (tok_at returns false and points at token 0; the query row of such
// a slot is loaded as +0.0 and its output is not written).
__device__ __forceinline__ bool tok_at(int raster, int heads, int nT, int nh, int nw, int T, int H,
                                       int W, int row, int s, int D, int64_t& off, int64_t& li) {
  if (!raster) {
    li = (int64_t)row * kTileTokens + s;
    off = li * D;
    return true;
  }
  const int64_t N = (int64_t)T * H * W;
  const int bh = row / nT, tau = row - bh * nT;
  const int tw = tau % nw, th = (tau / nw) % nh, tt = tau / (nw * nh);
  const int t = 4 * tt + (s >> 4), hh = 4 * th + ((s >> 2) & 3), w = 4 * tw + (s & 3);
  const bool ok = t < T && hh < H && w < W;
  const int64_t n = ok ? ((int64_t)t * H + hh) * W + w : 0;
  const int b = bh / heads, h = bh - b * heads;
  off = (((int64_t)b * N + n) * heads + h) * D;
  li = (int64_t)bh * N + n;
  return ok;
}
// The same mapping, bundled for the combine kernel.
struct TokMap {
  int raster, heads, nT, nh, nw, T, H, W;
  __device__ __forceinline__ bool at(int row, int s, int D, int64_t& off, int64_t& li) const {
    return tok_at(raster, heads, nT, nh, nw, T, H, W, row, s, D, off, li);
  }
};

struct AttnArgs {
  const uint16_t* q;   // [BH][nT*64][D], or raster [B][N][Hh][D] (raster)
  const uint16_t* k;   // [BH][nT*64][D]
  const uint16_t* v;   // [BH][nT][D][64]
  const int* row_ptr;
  const int* col_idx;
  uint16_t* o;         // [BH][nT*64][D], or raster [B][N][Hh][D] (raster)
  float* lse;          // [BH][nT*64], or raster [B][Hh][N]; or null
  int raster, heads;   // raster: q, o and lse in the caller's layout (tok_at)
  const int* ext;      // packed extent per key tile
  const int* iota;     // 0 .. nT-1: the key list of a complete row
  const Header* hdr;
  Header* hdr_mut;
  const Unit* units;
  float* part_o;       // [slots][64][D]
  float* part_ml;      // [slots][2][64]
  // skim tier (tiered instance only): MXFP4 Q and K, one tier byte per CSR entry
  const uint8_t* q4;   // codes [BH][nT*64][D/2]
  const uint8_t* q4s;  // E8M0 scales [BH][nT*64][D/32]
  const uint8_t* k4;
  const uint8_t* k4s;
  const uint8_t* tier; // [nnz], 1 = skim
  // exact per-token windows (token-window instance only)
  const int* coord;     // packed coordinates per key tile
  const uint8_t* tok_r; // token radii [BH][T*H*W], raster order
  const uint8_t* routed;// routed flag per CSR row
  int r_max;
  int nT, nh, nw, T, H, W;
  float c2;            // scale * log2(e)
};

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (a loop whose index
// must be a compile-time constant, e.g. an instruction's immediate operand).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

// Element i of an array that no kernel writes while this one runs (the CSR,
// the plan's tables), read through the constant address space: for a
// wave-uniform index the compiler then issues a scalar load (counted by
// lgkmcnt, not by the vmcnt that the tile copies use).
template <typename T>
__device__ __forceinline__ T ro(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// Broadcast a wave-uniform value to a scalar register (the compiler cannot
// prove uniformity of values derived from the thread index or read from LDS).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Row index of the K operand for A-operand row rho: bits 2 and 3 swapped.
__device__ __forceinline__ int sigma(int rho) {
  return (rho & 0x13) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

template <int D>
struct Cfg {
  static constexpr int kRowBytes = D * 2;             // K row in LDS
  static constexpr int kChunks = D / 8;               // 16-byte chunks per K row
  static constexpr int kTileBytes = kTileTokens * D * 2;
  static constexpr int kTileChunks = kTileBytes / 16;
  static constexpr int kSplitBytes = 2 * kTileBytes;  // K + V^T buffers of one key split
  static constexpr int kLdsBytes = 2 * kSplitBytes;   // two key splits
  static constexpr int kKSteps = D / 16;              // k-steps of Q.K^T
  static constexpr int kDBlocks = D / 32;             // 32-row blocks of O^T
};

// MXFP4 K tiles of the skim tier: a row of D features is D/32 blocks of 16
// code bytes (one 16-byte chunk each) plus D/32 E8M0 scale bytes.  In LDS a
// tile (or half tile) is its codes, rows of D/2 bytes with swizzled chunks,
// followed by its scales, rows of D/32 bytes.
template <int D>
struct Cfg4 {
  static constexpr int kC4 = D / 32;                    // blocks (chunks) per row
  static constexpr int kRowBytes = D / 2;
  static constexpr int kTileCodes = kTileTokens * kRowBytes;
  static constexpr int kTileAll = kTileCodes + kTileTokens * kC4;
  static constexpr int kHalfCodes = 32 * kRowBytes;
  static constexpr int kHalfAll = kHalfCodes + 32 * kC4;
  static constexpr int kM = D / 64;                     // scaled MFMAs per 32-key half
  static constexpr int kLdsBytes = 2 * kTileAll;        // beside the bf16 buffers
  static_assert(4 * kHalfAll == kLdsBytes, "skim buffers");
};

// LDS byte offset of chunk c of MXFP4 K row `row`: the chunk index is XORed
// with a row phase so that the 16 rows one read instruction touches per
// 16-lane group land in distinct bank groups.
template <int D>
__device__ __forceinline__ int k4_off(int row, int c) {
  constexpr int C4 = Cfg4<D>::kC4;
  return row * Cfg4<D>::kRowBytes + ((c ^ ((row / (16 / C4)) % C4)) << 4);
}

// LDS byte offset of 16-byte chunk c of K row `row` (swizzled).
template <int D>
__device__ __forceinline__ int k_off(int row, int c) {
  const int sw = (D == 128) ? (row & 15) : ((row >> 1) & 7);
  return row * Cfg<D>::kRowBytes + ((c ^ sw) << 4);
}
// LDS byte offset of 16-byte chunk c (8 keys) of V^T row d (swizzled).
__device__ __forceinline__ int v_off(int d, int c) { return d * 128 + ((c ^ ((d >> 1) & 7)) << 4); }

// Workgroup barrier for LDS hand-offs: completes this wave's LDS operations,
// then waits for every wave.  Unlike __syncthreads() it does not drain
// outstanding global loads, so tile prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
struct WaveState {
  bf16x8 qreg[Cfg<D>::kKSteps];
  f32x16 o[Cfg<D>::kDBlocks];
  float m;  // running max (log2 domain, scaled)
  float l;  // this lane's partial sum of P
  i32x4 q4[D / 64];  // skim tier: MXFP4 Q fragments (B operands)
  int q4s;           // their scales, shifted so that byte 2m is fragment m's
  int rl;            // token-window instance: this lane's query radius (255: no limit)
  int rl_raw;        // its token radius byte and its row's routed flag (0 or 1 in
  int rl_routed;     // the low bit), loaded with the unit, decoded by window_radius
  bool rl_inside;    // the lane's query slot holds a token of the grid
};

// This wave's Q fragments (B operands of S^T = K Q^T): row q of its 32 query
// rows, 8 features per 16-feature k-step (lane half h takes the upper 8).
template <int D>
__device__ __forceinline__ void load_q(WaveState<D>& st, const uint16_t* qp) {
  // qp is null for a padded slot of a raster query: its row is +0.0, as the
  // tile permute writes it (the wave's rescale decisions see the same scores)
  if (qp) {
#pragma unroll
    for (int t = 0; t < Cfg<D>::kKSteps; ++t) st.qreg[t] = *reinterpret_cast<const bf16x8*>(qp + 16 * t);
  } else {
#pragma unroll
    for (int t = 0; t < Cfg<D>::kKSteps; ++t) st.qreg[t] = bf16x8{};
  }
}

// Token-window instance: the lane's radius from the byte loaded with the unit.
// Called after the unit's first tile has been waited for, so the byte's load
// latency runs under that copy instead of ahead of it.
template <int D>
__device__ __forceinline__ void window_radius(WaveState<D>& st, int r_max) {
  st.rl = (st.rl_inside && st.rl_routed == 0) ? min(st.rl_raw, r_max) : 255;
}

// Skim tier.  This wave's MXFP4 Q fragments: for k-block m (64 features), the
// 32-feature block 2m + h of query row q, and the row's scale word shifted so
// that the scale of block 2m + h is its byte 2m.
template <int D>
__device__ __forceinline__ void load_q4(WaveState<D>& st, const uint8_t* q4row,
                                        const uint8_t* q4srow, int h) {
#pragma unroll
  for (int m = 0; m < Cfg4<D>::kM; ++m)
    st.q4[m] = *reinterpret_cast<const i32x4*>(q4row + (2 * m + h) * 16);
  const uint32_t w = (D == 128) ? *reinterpret_cast<const uint32_t*>(q4srow)
                                : (uint32_t)*reinterpret_cast<const uint16_t*>(q4srow);
  st.q4s = (int)(w >> (8 * h));
}

// One MXFP4 x MXFP4 product of K-block m: a 32x64 A (keys x features) and a
// 64x32 B (features x queries), each lane holding one 32-feature block of one
// row and that block's scale in byte OP of its scale word.
template <int OP>
__device__ __forceinline__ f32x16 mfma4(i32x4 a, i32x4 b, f32x16 c, int sa, int sb) {
  const i32x8 a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, OP, sa, OP, sb);
}

// S^T of 32 keys (rows r of an MXFP4 K buffer whose scales start at `sc`)
// against this wave's queries, accumulated into s.
template <int D>
__device__ __forceinline__ f32x16 qk32_skim(const char* k4buf, const char* sc, int row,
                                            const WaveState<D>& st, int h) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  const uint32_t w = (D == 128) ? *reinterpret_cast<const uint32_t*>(sc + row * 4)
                                : (uint32_t)*reinterpret_cast<const uint16_t*>(sc + row * 2);
  const int ws = (int)(w >> (8 * h));
  const i32x4 a0 = *reinterpret_cast<const i32x4*>(k4buf + k4_off<D>(row, h));
  s = mfma4<0>(a0, st.q4[0], s, ws, st.q4s);
  if constexpr (Cfg4<D>::kM > 1) {
    const i32x4 a1 = *reinterpret_cast<const i32x4*>(k4buf + k4_off<D>(row, 2 + h));
    s = mfma4<2>(a1, st.q4[1], s, ws, st.q4s);
  }
  return s;
}

// S^T (32 keys x 32 queries) = K Q^T for this wave's 32 query rows, from a
// block of 32 consecutive K rows (`k32`: row i of the block at i * 2D bytes,
// swizzled as k_off).  All the K operands are read before the first MFMA (a
// scheduling barrier keeps them there), so the chain waits on the LDS once,
// not once per k-step as when the compiler issues each read at its MFMA.
template <int D>
__device__ __forceinline__ f32x16 qk32(const char* k32, const WaveState<D>& st, int lane) {
  const int q = lane & 31, h = lane >> 5;
  const int krow = sigma(q);
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  bf16x8 a[Cfg<D>::kKSteps];
#pragma unroll
  for (int t = 0; t < Cfg<D>::kKSteps; ++t)
    a[t] = *reinterpret_cast<const bf16x8*>(k32 + k_off<D>(krow, 2 * t + h));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < Cfg<D>::kKSteps; ++t)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], st.qreg[t], s, 0, 0, 0);
  return s;
}

// LDS byte offset of 16-byte chunk c4 (8 keys) of row d of a half V^T tile
// (32 keys per row, 64 bytes; swizzled so 16 consecutive rows hit 16 distinct
// bank groups).
__device__ __forceinline__ int vh_off(int d, int c4) { return d * 64 + ((c4 ^ ((d >> 2) & 3)) << 4); }

// Values of lane l and lane l ^ 32 combined (v_permlane32_swap exchanges the
// two 32-lane halves; with the same register on both sides, the pair of
// results holds both halves' values in every lane).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online softmax of the 32 scores of half `kb` and O^T += V^T P^T over them.
// Register r of half kb in lane (q, h) holds key slot 32kb + 16(r/8) + 8h + r%8,
// i.e. lt = 2kb + r/8, lh = 2h + (r/4)%2, lw = r%4.
// HALF_V: `vbuf` holds only the 32 keys of this half ([D][32], vh_off);
// otherwise the whole tile ([D][64], v_off).
// EARLY_V: how many of the half's 2 * D/32 P.V operands are read from LDS
// before the softmax, so that the reads' latency runs under its VALU work;
// left to itself the compiler issues each read just before its MFMA and waits
// for it there.  Each one holds 4 registers through the softmax: the skim
// instance, near the register limit in its pair steps, reads three quarters
// of them early there.
template <int D, bool HALF_V, bool TOKR = false, int EARLY_V = 0>
__device__ __forceinline__ void softmax_pv_half(WaveState<D>& st, f32x16 s, const char* vbuf,
                                                int kb, int lane, const TileExtent& ext,
                                                float c2, int dist = 0) {
  const int q = lane & 31, h = lane >> 5;
  auto v_frag = [&](int s2, int db) {
    const int voff = HALF_V ? vh_off(32 * db + q, 2 * s2 + h) : v_off(32 * db + q, 4 * kb + 2 * s2 + h);
    return *reinterpret_cast<const bf16x8*>(vbuf + voff);
  };
  static_assert(EARLY_V >= 0 && EARLY_V <= 2 * Cfg<D>::kDBlocks, "early operand count");
  bf16x8 vf[2 * Cfg<D>::kDBlocks];
  if constexpr (EARLY_V > 0) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
        if (s2 * Cfg<D>::kDBlocks + db < EARLY_V) vf[s2 * Cfg<D>::kDBlocks + db] = v_frag(s2, db);
    // keeps the scheduler from sinking each read back to its MFMA
    __builtin_amdgcn_sched_barrier(0);
  }
  if (ext.edge) {
    const bool h_ok0 = 2 * h < ext.vh, h_ok1 = 2 * h + 1 < ext.vh;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool tw_ok = ((2 * kb + (r >> 3)) < ext.vt) && ((r & 3) < ext.vw);
      const bool ok = tw_ok && ((r & 4) ? h_ok1 : h_ok0);
      s[r] = ok ? s[r] : -INFINITY;
    }
  }
  // exact per-token windows: this lane's query attends the key tile only if
  // the tile lies inside the window of the query's own radius; otherwise its
  // tile maximum is -inf (no rescale) and its exp offset -inf (P = 0)
  const bool in = !TOKR || st.rl >= dist;
  // This lane's 16 scores decide whether the running max must move: the
  // query's max over both lane halves exceeds m + slack exactly when one
  // half's does, so the halves are combined (a cross-lane swap, which does
  // not overlap the other wave's MFMAs) only in the rare rescale branch, and
  // m stays the same in both halves.
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  if (TOKR && !in) mx = -INFINITY;
  if (__any(mx * c2 > st.m + kRescaleSlack)) {
    const float mc = max_halves(mx) * c2;
    const float mn = fmaxf(st.m, mc);
    const float alpha = (mn == -INFINITY) ? 1.f : exp2f(st.m - mn);
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    st.m = mn;
  }
  // every tile holds at least one valid key, so the running max is finite here;
  // with per-token windows a lane may not have met an attended tile yet (its
  // running max still -inf, its scores here -inf or outside the window): its
  // probabilities are then exp2(-inf) = 0
  float mneg = -st.m;
  if constexpr (TOKR) mneg = !in ? -INFINITY : (st.m == -INFINITY ? 0.f : -st.m);
  bf16x8 pb[2];
  float pf[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    pf[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, mneg));
    pb[r >> 3][r & 7] = (__bf16)pf[r];
  }
  // Row sum of the fp32 probabilities by a pairwise tree of plain adds (these
  // overlap the other wave's MFMAs; bf16 dot products do not).  P.V takes the
  // round-to-nearest bf16 P, whose rounding errors are unbiased, so numerator
  // and denominator agree to well within the bf16 tolerance.
  const float a0 = pf[0] + pf[1], a1 = pf[2] + pf[3], a2 = pf[4] + pf[5], a3 = pf[6] + pf[7];
  const float a4 = pf[8] + pf[9], a5 = pf[10] + pf[11], a6 = pf[12] + pf[13], a7 = pf[14] + pf[15];
  st.l += ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int db = 0; db < Cfg<D>::kDBlocks; ++db) {
      const bf16x8 a = (s2 * Cfg<D>::kDBlocks + db < EARLY_V) ? vf[s2 * Cfg<D>::kDBlocks + db]
                                                              : v_frag(s2, db);
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s2], st.o[db], 0, 0, 0);
    }
}

#define VSA_LDS __attribute__((address_space(3)))

// Asynchronous global -> LDS copy (global_load_lds_dwordx4): one wave moves a
// 1 KB block of a tile, lane L writing LDS bytes [16L, 16L + 16) of the block,
// so each lane fetches the global chunk that the swizzle places there.
// Completion is tracked by vmcnt; LDS reads of other buffers need no wait.
// This pointer form (the compiler forms 64-bit per-lane addresses) serves the
// small MXFP4 copies of the skim tier; the bf16 K/V tiles use the buffer form
// below.
__device__ __forceinline__ void dma16(const char* gbase, uint32_t lane_off, char* lds_block) {
  __builtin_amdgcn_global_load_lds(gbase + lane_off, (VSA_LDS void*)lds_block, 16, 0, 0);
}

// Per-lane byte offset, within a K block of rows [r0, r0 + rows-per-block),
// of the global chunk that lands at LDS position 16*lane; only r0 mod 16
// matters for the swizzle.
template <int D>
__device__ __forceinline__ uint32_t k_lane_off(int r0, int lane) {
  constexpr int kCpr = Cfg<D>::kChunks;
  const int row = r0 + lane / kCpr;
  const int sw = (D == 128) ? (row & 15) : ((row >> 1) & 7);
  return (uint32_t)((lane / kCpr) * Cfg<D>::kRowBytes + (((lane % kCpr) ^ sw) << 4));
}

// Same for a V^T block of 8 rows of 128 bytes starting at row d0.
__device__ __forceinline__ uint32_t v_lane_off(int d0, int lane) {
  const int d = d0 + (lane >> 3);
  return (uint32_t)((lane >> 3) * 128 + (((lane & 7) ^ ((d >> 1) & 7)) << 4));
}

// The same copy through a buffer resource over one tile: the descriptor is
// built from the tile's (uniform) base in scalar registers, the uniform part of
// the source offset is the scalar offset and the per-lane part a loop-invariant
// VGPR, so issuing a copy takes no vector arithmetic (the pointer form needs
// 64-bit vector adds per copy).  Reads past the tile's bytes would return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t soff,
                                       char* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (VSA_LDS void*)lds_block, 16, lane_off, soff, 0, 0);
}
// The same with an immediate offset IMM, which the hardware adds to both the
// source offset and the LDS address: the blocks of a run of consecutive 1 KB
// blocks then share one LDS base (M0) and one scalar offset, so the copy loop
// holds two scalar values per run instead of two per block.
template <int IMM>
__device__ __forceinline__ void dma16b_imm(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t soff,
                                           char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (VSA_LDS void*)lds_base, 16, lane_off, soff, IMM, 0);
}

// All blocks of one K tile and one V^T tile, spread over the 4 waves of the
// workgroup (this is wave `w`).
template <int D>
__device__ __forceinline__ void dma_tile(char* buf, const char* ktile, const char* vtile, int w,
                                         int nw, int lane, bool with_k = true) {
  constexpr int TB = Cfg<D>::kTileBytes;
  constexpr int kBlocks = TB / 1024;
  constexpr int kPer = kBlocks / 4;
  constexpr int kRpb = 1024 / Cfg<D>::kRowBytes;
  (void)nw;
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(ktile, TB), rv = tile_rsrc(vtile, TB);
  // this wave's blocks w*kPer .. w*kPer+kPer-1 (rows blk*kRpb.. of K, blk*8.. of
  // V^T); the swizzle phase depends on i only (w*kPer*kRpb % 16 == 0)
  static_assert(kPer <= 4, "immediate offsets reach 3 KB");
  const int b0 = w * kPer * 1024;
  // all K blocks, then all V blocks: the copy rewrites the LDS base (M0)
  // once per run instead of once per block
  if (with_k)
    static_for<kPer>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma16b_imm<i * 1024>(rk, k_lane_off<D>(i * kRpb, lane), b0, buf + b0);
    });
  static_for<kPer>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    dma16b_imm<i * 1024>(rv, v_lane_off(i * 8, lane), b0, buf + TB + b0);
  });
}

// Per-lane byte offset, within a 1 KB block of MXFP4 K codes, of the global
// chunk that lands at LDS position 16*lane (the swizzle phase of k4_off only
// depends on the row within the block).
template <int D>
__device__ __forceinline__ uint32_t k4_lane_off(int lane) {
  constexpr int C4 = Cfg4<D>::kC4;
  const int r = lane / C4;
  return (uint32_t)(r * Cfg4<D>::kRowBytes + (((lane % C4) ^ ((r / (16 / C4)) % C4)) << 4));
}

// The MXFP4 K codes and scales of `rows` consecutive rows (64: a tile, 32: a
// half), spread over `nwv` waves (this is wave `w` of them).
template <int D, int ROWS>
__device__ __forceinline__ void dma_k4(char* buf, const char* codes, const char* scales, int w,
                                       int nwv, int lane) {
  constexpr int kBlocks = ROWS * Cfg4<D>::kRowBytes / 1024;
  constexpr int kScaleDwords = ROWS * Cfg4<D>::kC4 / 4;  // scales move as dwords
  for (int blk = w; blk < kBlocks; blk += nwv)
    dma16(codes + blk * 1024, k4_lane_off<D>(lane), buf + blk * 1024);
  if (w == nwv - 1 && lane < kScaleDwords)
    __builtin_amdgcn_global_load_lds(scales + lane * 4, (VSA_LDS void*)(buf + ROWS * Cfg4<D>::kRowBytes),
                                     4, 0, 0);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); }

// Where a unit of the tiered instance finds its skim data: the MXFP4 K of its
// (batch, head) and the tier bytes of its rows from its first key on (G
// units: two rows, S units: t1 == t0).
struct SkimRef {
  const char* k4;
  const char* k4s;
  const uint8_t* t0;
  const uint8_t* t1;
};

// Tier bits of entry i of a G unit: bit 0 first row skims, bit 1 second row.
__device__ __forceinline__ int tier2(const SkimRef& sk, int i) {
  return (sk.t0[i] != 0 ? 1 : 0) | (sk.t1[i] != 0 ? 2 : 0);
}

// The tier bytes a step reads ahead are loaded at an index clamped into the
// unit's list and decoded only after the step: a load under a branch whose
// value is decoded inside it would be waited on at once, a global-memory
// latency before the step's copies are even issued.
struct TierBytes {
  int b0, b1;
};
__device__ __forceinline__ TierBytes tier_load(const SkimRef& sk, int i) {
  return {sk.t0[i], sk.t1[i]};
}
__device__ __forceinline__ int tier_bits(TierBytes t) {
  return (t.b0 != 0 ? 1 : 0) | (t.b1 != 0 ? 2 : 0);
}

// One key tile of a G unit from LDS buffer CUR; the next tile is copied into
// the other buffer by DMA while this one is computed on.  Both halves' score
// MFMAs are issued before the first softmax so they run under its VALU work.
//
// Tiered instance: `tc` / `tn` are the tier bits (tier2) of this tile and of
// the next; the bf16 K of a tile is copied only if a row refines it and its
// MXFP4 K (into the buffers past the bf16 ones) only if a row skims it.  V is
// always bf16.  Each query tile's waves take the products of their own row's
// tier.
template <int D, int CUR, bool TIER, bool TOKR>
__device__ __forceinline__ void g_step(WaveState<D>& st, char* smem, int jn, int code, int tc,
                                       int tn, const char* kbase, const char* vbase,
                                       const SkimRef& sk, const AttnArgs& a, int wave, int lane,
                                       int grp, int dist) {
  constexpr int TB = Cfg<D>::kTileBytes;
  const char* kbuf = smem + CUR * Cfg<D>::kSplitBytes;
  const char* vbuf = kbuf + TB;
  if (jn >= 0) {
    dma_tile<D>(smem + (CUR ^ 1) * Cfg<D>::kSplitBytes, kbase + (int64_t)jn * TB,
                vbase + (int64_t)jn * TB, wave, 4, lane, !TIER || tn != 3);
    if constexpr (TIER) {
      if (tn != 0)
        dma_k4<D, 64>(smem + Cfg<D>::kLdsBytes + (CUR ^ 1) * Cfg4<D>::kTileAll,
                      sk.k4 + (int64_t)jn * Cfg4<D>::kTileCodes,
                      sk.k4s + (int64_t)jn * kTileTokens * Cfg4<D>::kC4, wave, 4, lane);
    }
  }
  const TileExtent ext = unpack_extent(code);
  // Half 1 (time slices 2 and 3 of the key tile) holds only padding keys when
  // the tile has at most 2 valid time slices: all its scores would be -inf and
  // its probabilities exactly 0, so it is skipped.
  const bool half1 = ext.vt > 2;
  f32x16 s0, s1;
  if (TIER && ((tc >> grp) & 1)) {
    const char* k4buf = smem + Cfg<D>::kLdsBytes + CUR * Cfg4<D>::kTileAll;
    const int row = sigma(lane & 31), h = lane >> 5;
    s0 = qk32_skim<D>(k4buf, k4buf + Cfg4<D>::kTileCodes, row, st, h);
    if (half1) s1 = qk32_skim<D>(k4buf, k4buf + Cfg4<D>::kTileCodes, 32 + row, st, h);
  } else {
    s0 = qk32<D>(kbuf, st, lane);
    if (half1) s1 = qk32<D>(kbuf + 32 * Cfg<D>::kRowBytes, st, lane);
  }
  constexpr int kEarlyV = TIER ? 3 * Cfg<D>::kDBlocks / 2 : 2 * Cfg<D>::kDBlocks;
  softmax_pv_half<D, false, TOKR, kEarlyV>(st, s0, vbuf, 0, lane, ext, a.c2, dist);
  if (half1) softmax_pv_half<D, false, TOKR, kEarlyV>(st, s1, vbuf, 1, lane, ext, a.c2, dist);
  wait_dma();
  lds_barrier();
}

// G units: all 4 waves (two query tiles x two 32-row halves) share each key
// tile.  LDS holds two K/V buffers: while one is computed on, the next tile
// streams into the other (a whole step to arrive, one barrier per step).
// Column indices are read two tiles ahead and the next tile's extent one
// tile ahead, so neither load is waited on.
template <int D, bool TIER, bool TOKR>
__device__ __forceinline__ void run_steps_g(WaveState<D>& st, char* smem, const int* cols,
                                            int nkeys, const char* kbase, const char* vbase,
                                            const SkimRef& sk, const AttnArgs& a, int wave,
                                            int lane, const uint16_t* qp, int grp, int qc) {
  constexpr int TB = Cfg<D>::kTileBytes;
  const int j0 = uni(cols[0]);
  int jn = (1 < nkeys) ? uni(cols[1]) : -1;
  int code = uni(a.ext[j0]);
  int cc = TOKR ? uni(a.coord[j0]) : 0;  // coordinates of the current key tile
  int tc = 0, tn = 0;  // tier bits of the current and the next tile (tiered instance)
  if constexpr (TIER) {
    tc = uni(tier2(sk, 0));
    tn = (1 < nkeys) ? uni(tier2(sk, 1)) : 0;
  }
  dma_tile<D>(smem, kbase + (int64_t)j0 * TB, vbase + (int64_t)j0 * TB, wave, 4, lane,
              !TIER || tc != 3);
  if constexpr (TIER) {
    if (tc != 0)
      dma_k4<D, 64>(smem + Cfg<D>::kLdsBytes, sk.k4 + (int64_t)j0 * Cfg4<D>::kTileCodes,
                    sk.k4s + (int64_t)j0 * kTileTokens * Cfg4<D>::kC4, wave, 4, lane);
  }
  load_q<D>(st, qp);  // in flight with the first tile; one wait covers both
  wait_dma();
  lds_barrier();
  if constexpr (TOKR) window_radius<D>(st, a.r_max);
  for (int step = 0; step < nkeys; step += 2) {
    int jnn_v = (step + 2 < nkeys) ? ro(cols, step + 2) : -1;
    int cn_v = (jn >= 0) ? ro(a.ext, jn) : 0;
    int ccn_v = (TOKR && jn >= 0) ? ro(a.coord, jn) : 0;
    TierBytes tb{0, 0};
    if constexpr (TIER) tb = tier_load(sk, min(step + 2, nkeys - 1));
    g_step<D, 0, TIER, TOKR>(st, smem, jn, code, tc, tn, kbase, vbase, sk, a, wave, lane, grp,
                             TOKR ? window_dist(cc, qc) : 0);
    code = uni(cn_v);
    cc = uni(ccn_v);
    jn = uni(jnn_v);
    tc = tn;
    if constexpr (TIER) tn = (step + 2 < nkeys) ? uni(tier_bits(tb)) : 0;
    if (step + 1 >= nkeys) break;
    jnn_v = (step + 3 < nkeys) ? ro(cols, step + 3) : -1;
    cn_v = (jn >= 0) ? ro(a.ext, jn) : 0;
    ccn_v = (TOKR && jn >= 0) ? ro(a.coord, jn) : 0;
    if constexpr (TIER) tb = tier_load(sk, min(step + 3, nkeys - 1));
    g_step<D, 1, TIER, TOKR>(st, smem, jn, code, tc, tn, kbase, vbase, sk, a, wave, lane, grp,
                             TOKR ? window_dist(cc, qc) : 0);
    code = uni(cn_v);
    cc = uni(ccn_v);
    jn = uni(jnn_v);
    tc = tn;
    if constexpr (TIER) tn = (step + 3 < nkeys) ? uni(tier_bits(tb)) : 0;
  }
}

// Half-tile DMA for S units: the K rows of half kb (32 rows) and the V^T
// columns of half kb (32 keys of each of the D rows), the two waves of a key
// split sharing the blocks (this is wave `wi` of them).
template <int D>
__device__ __forceinline__ void dma_half(char* buf, const char* ktile, const char* vtile, int kb,
                                         int wi, int nwv, int lane, bool with_k = true) {
  constexpr int TB = Cfg<D>::kTileBytes;
  constexpr int kRpb = 1024 / Cfg<D>::kRowBytes;
  constexpr int KH = 32 * Cfg<D>::kRowBytes;   // bytes of a K half
  constexpr int kKBlocks = KH / 1024, kVBlocks = D * 64 / 1024;
  (void)nwv;
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(ktile, TB), rv = tile_rsrc(vtile, TB);
  // K: this wave's blocks wi*kKB .. of the half (the swizzle phase depends on
  // i only); source and LDS both advance 1 KB per block
  constexpr int kKB = kKBlocks / 2;
  static_assert(kKB <= 4, "immediate offsets reach 3 KB");
  const int kb0 = wi * kKB * 1024;
  if (with_k)
    static_for<kKB>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma16b_imm<i * 1024>(rk, k_lane_off<D>(i * kRpb, lane),
                           (32 * kb) * Cfg<D>::kRowBytes + kb0, buf + kb0);
    });
  // V blocks: consecutive 1 KB blocks of LDS from source rows 2 KB apart; one
  // LDS base for the run, the immediate offset moving both addresses by 1 KB
  // per block and the scalar offset adding the source's other 1 KB
  static_assert(kVBlocks / 2 <= 4, "immediate offsets reach 3 KB");
  {
    const int blk0 = wi * (kVBlocks / 2);
    const int d = blk0 * 16 + (lane >> 2);
    const int c4 = (lane & 3) ^ ((d >> 2) & 3);
    const uint32_t off = (uint32_t)((lane >> 2) * 128 + (c4 << 4));
    static_for<kVBlocks / 2>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      dma16b_imm<i * 1024>(rv, off, blk0 * 16 * 128 + kb * 64 + i * 1024, buf + KH + blk0 * 1024);
    });
  }
}

// S units: one query tile; waves 0-1 (rows 0-31, 32-63) take the key tiles at
// even positions of the list and waves 2-3 the odd ones.  Each key split
// double-buffers half tiles (32 keys of K and of V^T) in its own LDS region,
// so the two tiles a step needs fit beside their prefetches.  Tiered
// instance: a skim tile brings its MXFP4 K half instead of the bf16 one, into
// the split's half buffers past the bf16 region.
template <int D, bool TIER, bool TOKR>
__device__ __forceinline__ void run_steps_s(WaveState<D>& st, char* smem, const int* cols,
                                            int nkeys, const char* kbase, const char* vbase,
                                            const SkimRef& sk, const AttnArgs& a, int wave,
                                            int lane, int grp, const uint16_t* qp, int qc) {
  constexpr int TB = Cfg<D>::kTileBytes;
  constexpr int KH = 32 * Cfg<D>::kRowBytes;
  constexpr int BUF = KH + D * 64;                       // one half-tile buffer
  constexpr int H4 = Cfg4<D>::kHalfAll;                  // one MXFP4 K half buffer
  static_assert(4 * BUF <= Cfg<D>::kLdsBytes, "S unit buffers");
  char* region = smem + grp * 2 * BUF;
  char* region4 = smem + Cfg<D>::kLdsBytes + grp * 2 * H4;
  const int wi = wave & 1;
  const int nsteps = (nkeys + 1) / 2;
  const int krow = sigma(lane & 31), h = lane >> 5;
  int j = (grp < nkeys) ? uni(cols[grp]) : -1;
  int jn = (2 + grp < nkeys) ? uni(cols[2 + grp]) : -1;
  int code = (j >= 0) ? uni(a.ext[j]) : 0;
  int cc = (TOKR && j >= 0) ? uni(a.coord[j]) : 0;  // coordinates of the current key tile
  int t = 0, tn = 0;  // this split's current / next tile skims (tiered instance)
  if constexpr (TIER) {
    t = (j >= 0) ? uni(sk.t0[grp] != 0 ? 1 : 0) : 0;
    tn = (jn >= 0) ? uni(sk.t0[2 + grp] != 0 ? 1 : 0) : 0;
  }
  // half kb of tile jj (skim flag tt) into LDS half buffer `which`
  auto fetch = [&](int jj, int tt, int kb, int which) {
    dma_half<D>(region + which * BUF, kbase + (int64_t)jj * TB, vbase + (int64_t)jj * TB, kb, wi,
                2, lane, !TIER || !tt);
    if constexpr (TIER) {
      if (tt)
        dma_k4<D, 32>(region4 + which * H4,
                      sk.k4 + (int64_t)jj * Cfg4<D>::kTileCodes + kb * Cfg4<D>::kHalfCodes,
                      sk.k4s + ((int64_t)jj * kTileTokens + 32 * kb) * Cfg4<D>::kC4, wi, 2, lane);
    }
  };
  auto scores = [&](int tt, int which) -> f32x16 {
    if (TIER && tt) {
      const char* b4 = region4 + which * H4;
      return qk32_skim<D>(b4, b4 + Cfg4<D>::kHalfCodes, krow, st, h);
    }
    return qk32<D>(region + which * BUF, st, lane);
  };
  if (j >= 0) fetch(j, t, 0, 0);
  load_q<D>(st, qp);  // in flight with the first half tile; one wait covers both
  wait_dma();
  lds_barrier();
  if constexpr (TOKR) window_radius<D>(st, a.r_max);
  for (int i = 0; i < nsteps; ++i) {
    const int pnn = 2 * (i + 2) + grp;
    const int jnn_v = (pnn < nkeys) ? ro(cols, pnn) : -1;
    const int cn_v = (jn >= 0) ? ro(a.ext, jn) : 0;
    const int ccn_v = (TOKR && jn >= 0) ? ro(a.coord, jn) : 0;
    int tb = 0;  // raw tier byte two tiles ahead (clamped index, decoded after the step)
    if constexpr (TIER) tb = sk.t0[min(pnn, nkeys - 1)];
    const TileExtent ext = unpack_extent(code);
    const int dist = TOKR ? window_dist(cc, qc) : 0;
    if (j >= 0) {
      fetch(j, t, 1, 1);
      const f32x16 s0 = scores(t, 0);
      softmax_pv_half<D, true, TOKR, 2 * Cfg<D>::kDBlocks>(st, s0, region + KH, 0, lane, ext, a.c2, dist);
    }
    wait_dma();
    lds_barrier();
    if (jn >= 0) fetch(jn, tn, 0, 0);
    // half 1 of a tile with at most 2 valid time slices holds only padding
    // keys (scores -inf, probabilities exactly 0): skipped
    if (j >= 0 && ext.vt > 2) {
      const f32x16 s1 = scores(t, 1);
      softmax_pv_half<D, true, TOKR, 2 * Cfg<D>::kDBlocks>(st, s1, region + BUF + KH, 1, lane, ext,
                                                             a.c2, dist);
    }
    wait_dma();
    lds_barrier();
    j = jn;
    code = uni(cn_v);
    cc = uni(ccn_v);
    jn = uni(jnn_v);
    t = tn;
    if constexpr (TIER) tn = (pnn < nkeys && tb != 0) ? 1 : 0;
    tn = uni(tn);
  }
}

template <int D, bool TIER, bool TOKR>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int s_unit;
  __shared__ int s_head_done;  // this workgroup found the head of the order empty
  const int tid = threadIdx.x, wave = uni(tid >> 6), lane_top = tid & 63;
  const int nT = args.nT;
  const int n_units = args.hdr->n_units;
  const int n_head = args.hdr->n_head;
  const int rest_span = args.hdr->rest_span;
  const int head_span = args.hdr->head_span;
  const int half = wave & 1;
  const int grp = wave >> 1;  // G: which query tile; S: which key split
  const int home = blockIdx.x % kQueues;
  constexpr int TC = Cfg<D>::kTileChunks;

  if (tid == 0) s_head_done = 0;
  for (;;) {
    if (tid == 0) {
      int u = -1;
      for (int k = 0; k < kQueues && !s_head_done && u < 0; ++k) {
        const int x = (home + k) % kQueues;
        const int idx = atomicAdd(&args.hdr_mut->queue[x], 1);
        const int cand = x * head_span + idx;
        if (idx < head_span && cand < n_head) {
          u = cand;
          break;
        }
      }
      if (u < 0) {
        s_head_done = 1;
        for (int k = 0; k < kQueues && u < 0; ++k) {
          const int x = (home + k) % kQueues;
          const int idx = atomicAdd(&args.hdr_mut->queue_rest[x], 1);
          const int cand = n_head + x * rest_span + idx;
          if (idx < rest_span && cand < n_units) {
            u = cand;
            break;
          }
        }
      }
      s_unit = u;
    }
    lds_barrier();
    const int ui = uni(s_unit);
    lds_barrier();
    if (ui < 0) break;
    // The lane index is made opaque once per unit, so that the lane offsets
    // the unit's set-up derives from it are recomputed per unit rather than
    // hoisted out of the unit loop and held in registers across every step
    // (they spilled to scratch in the tiered instance).
    int lane = lane_top;
    asm volatile("" : "+v"(lane));
    const int q = lane & 31, h = lane >> 5;
    Unit u = args.units[ui];
    u.row[0] = uni(u.row[0]);
    u.row[1] = uni(u.row[1]);
    u.kb = uni(u.kb);
    u.ke = uni(u.ke);
    u.slot = uni(u.slot);
    u.mode = uni(u.mode);
    const bool g_mode = (u.mode == 0);
    const int row = (g_mode && grp) ? u.row[1] : u.row[0];
    const int64_t bh = row / nT;
    const int64_t qrow0 = (int64_t)row * kTileTokens + 32 * half;

    WaveState<D> st;
    int64_t q_off, q_li;
    const bool q_ok = tok_at(args.raster, args.heads, nT, args.nh, args.nw, args.T, args.H,
                             args.W, row, 32 * half + q, D, q_off, q_li);
    const uint16_t* qp = q_ok ? args.q + q_off + 8 * h : nullptr;
#pragma unroll
    for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] = 0.f;
    st.m = -INFINITY;
    st.l = 0.f;

    // A row of nT entries lists every key tile once (its columns ascend
    // strictly within [0, nT)), so its keys are read from the plan's 0..nT-1
    // table: both rows of a G unit walk the same keys whatever either list holds.
    u.complete = uni(u.complete);
    const int* cols = (g_mode || u.complete) ? args.iota + u.kb
                                             : args.col_idx + uni(args.row_ptr[u.row[0]]) + u.kb;
    const int nkeys = u.ke - u.kb;
    const char* kbase = reinterpret_cast<const char*>(args.k) + bh * (int64_t)nT * TC * 16;
    const char* vbase = reinterpret_cast<const char*>(args.v) + bh * (int64_t)nT * TC * 16;
    SkimRef sk = {nullptr, nullptr, nullptr, nullptr};
    if constexpr (TIER) {
      const int64_t tiles_before = bh * (int64_t)nT * kTileTokens;  // rows of earlier heads
      sk.k4 = reinterpret_cast<const char*>(args.k4) + tiles_before * Cfg4<D>::kRowBytes;
      sk.k4s = reinterpret_cast<const char*>(args.k4s) + tiles_before * Cfg4<D>::kC4;
      sk.t0 = args.tier + uni(args.row_ptr[u.row[0]]) + u.kb;
      sk.t1 = g_mode ? args.tier + uni(args.row_ptr[u.row[1]]) + u.kb : sk.t0;
      load_q4<D>(st, args.q4 + (qrow0 + q) * Cfg4<D>::kRowBytes,
                 args.q4s + (qrow0 + q) * Cfg4<D>::kC4, h);
    }
    int qc = 0;  // packed coordinates of this wave's query tile (token-window instance)
    bool windowed = TOKR;
    if constexpr (TOKR) {
      // this lane's query token and its own radius: 255 (no limit) for routed
      // rows and padded slots, whose outputs are not windowed or are dropped.
      // The radius byte is loaded at a valid index whatever the lane and
      // decoded after the first tile's wait (window_radius).
      qc = ro(args.coord, row - (int)bh * nT);
      const int qs = 32 * half + q;
      const int t = 4 * (qc & 1023) + (qs >> 4);
      const int hh = 4 * ((qc >> 10) & 1023) + ((qs >> 2) & 3);
      const int w = 4 * ((qc >> 20) & 1023) + (qs & 3);
      const bool inside = t < args.T && hh < args.H && w < args.W;
      const int64_t n = inside ? ((int64_t)t * args.H + hh) * args.W + w : 0;
      st.rl_raw = args.tok_r[bh * ((int64_t)args.T * args.H * args.W) + n];
      st.rl_routed = args.routed[row];
      st.rl_inside = inside;
      // a pair unit of two routed rows is not windowed: it takes the plain step
      windowed = !g_mode || !(uni(args.routed[u.row[0]]) && uni(args.routed[u.row[1]]));
    }
    if (g_mode && windowed)
      run_steps_g<D, TIER, TOKR>(st, smem, cols, nkeys, kbase, vbase, sk, args, wave, lane, qp,
                                 grp, qc);
    else if (g_mode)
      run_steps_g<D, TIER, false>(st, smem, cols, nkeys, kbase, vbase, sk, args, wave, lane, qp,
                                  grp, qc);
    else
      run_steps_s<D, TIER, TOKR>(st, smem, cols, nkeys, kbase, vbase, sk, args, wave, lane, grp,
                                 qp, qc);

    // S units: merge the two key splits (waves 2,3 -> waves 0,1) through LDS.
    if (!g_mode) {
      float* xo = reinterpret_cast<float*>(smem) + half * (64 * (Cfg<D>::kDBlocks * 16 + 2));
      if (grp == 1) {
#pragma unroll
        for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64 + lane] = st.o[db][r];
        xo[Cfg<D>::kDBlocks * 16 * 64 + lane] = st.m;
        xo[(Cfg<D>::kDBlocks * 16 + 1) * 64 + lane] = st.l;
      }
      lds_barrier();
      if (grp == 0) {
        const float m1 = xo[Cfg<D>::kDBlocks * 16 * 64 + lane];
        const float l1 = xo[(Cfg<D>::kDBlocks * 16 + 1) * 64 + lane];
        const float mm = fmaxf(st.m, m1);
        const float w0 = (mm == -INFINITY) ? 0.f : exp2f(st.m - mm);
        const float w1 = (mm == -INFINITY) ? 0.f : exp2f(m1 - mm);
#pragma unroll
        for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st.o[db][r] = w0 * st.o[db][r] + w1 * xo[(db * 16 + r) * 64 + lane];
        st.l = w0 * st.l + w1 * l1;
        st.m = mm;
      }
      lds_barrier();
    }

    const bool writer = g_mode || grp == 0;
    if (writer) {
      const float lt = sum_halves(st.l);
      const int qi = 32 * half + q;  // query row within the tile
      int64_t o_off, o_li;
      const bool o_ok = tok_at(args.raster, args.heads, nT, args.nh, args.nw, args.T, args.H,
                               args.W, row, qi, D, o_off, o_li);
      if (u.slot < 0 && o_ok) {
        const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
        uint16_t* op = args.o + o_off + 4 * h;
#pragma unroll
        for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            __bf16 b0 = (__bf16)(st.o[db][4 * g + 0] * inv);
            __bf16 b1 = (__bf16)(st.o[db][4 * g + 1] * inv);
            __bf16 b2 = (__bf16)(st.o[db][4 * g + 2] * inv);
            __bf16 b3 = (__bf16)(st.o[db][4 * g + 3] * inv);
            uint2 w;
            w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<uint2*>(op + 32 * db + 8 * g) = w;
          }
        if (args.lse && h == 0)
          args.lse[o_li] = (lt > 0.f) ? (st.m + log2f(lt)) * kLn2 : -INFINITY;
      } else if (u.slot >= 0) {
        const int64_t slot = u.slot + (g_mode ? grp : 0);
        float* po = args.part_o + slot * kTileTokens * D + (int64_t)qi * D + 4 * h;
#pragma unroll
        for (int db = 0; db < Cfg<D>::kDBlocks; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(po + 32 * db + 8 * g) =
                make_float4(st.o[db][4 * g], st.o[db][4 * g + 1], st.o[db][4 * g + 2], st.o[db][4 * g + 3]);
        if (h == 0) {
          args.part_ml[slot * 128 + qi] = st.m;
          args.part_ml[slot * 128 + 64 + qi] = lt;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- combine

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const Header* hdr, const Comb* comb,
                                                      const float* part_o, const float* part_ml,
                                                      uint16_t* o, float* lse, TokMap map) {
  const int n_comb = hdr->n_comb;
  constexpr int kVec = D / 4;                    // float4 per row
  for (int ci = blockIdx.x; ci < n_comb; ci += gridDim.x) {
    const Comb c = comb[ci];
    for (int i = threadIdx.x; i < kTileTokens * kVec; i += blockDim.x) {
      const int r = i / kVec, v4 = i % kVec;
      float M = -INFINITY;
      for (int s = 0; s < c.n; ++s) M = fmaxf(M, part_ml[(int64_t)(c.slot0 + s * c.stride) * 128 + r]);
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < c.n; ++s) {
        const int64_t slot = c.slot0 + (int64_t)s * c.stride;
        const float m = part_ml[slot * 128 + r];
        const float w = (M == -INFINITY) ? 0.f : exp2f(m - M);
        L += w * part_ml[slot * 128 + 64 + r];
        const float4 x = *reinterpret_cast<const float4*>(part_o + (slot * kTileTokens + r) * D + 4 * v4);
        acc.x += w * x.x; acc.y += w * x.y; acc.z += w * x.z; acc.w += w * x.w;
      }
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      __bf16 b0 = (__bf16)(acc.x * inv), b1 = (__bf16)(acc.y * inv);
      __bf16 b2 = (__bf16)(acc.z * inv), b3 = (__bf16)(acc.w * inv);
      uint2 w2;
      w2.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      w2.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      int64_t off, li;
      if (!map.at(c.row, r, D, off, li)) continue;  // a padded slot of a raster output
      *reinterpret_cast<uint2*>(o + off + 4 * v4) = w2;
      if (lse && v4 == 0) lse[li] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn(const vsa_shape& s, const void* q, const void* k, const void* v,
                       const int* row_ptr, const int* col_idx, float scale, void* o, float* lse,
                       int kv_chunk, void* ws, int cus, hipStream_t stream, const SkimInputs* skim,
                       const TokenWindows* tokw, bool raster) {
  const Grid g = make_grid(s);
  const AttnLayout L = attn_layout(s, kv_chunk);
  char* w = static_cast<char*>(ws);
  Header* hdr = reinterpret_cast<Header*>(w);
  PlanArgs pa;
  pa.row_ptr = row_ptr;
  pa.bh = (int)L.bh;
  pa.nT = g.nT;
  pa.kv_chunk = kv_chunk;
  pa.target = kSplitTarget;
  pa.max_units = L.max_units;
  pa.max_slots = L.max_slots;
  pa.hdr = hdr;
  pa.cbase = reinterpret_cast<int*>(w + L.off_cbase);
  pa.gbase = reinterpret_cast<int*>(w + L.off_gbase);
  pa.grows = reinterpret_cast<int*>(w + L.off_grows);
  pa.ext = reinterpret_cast<int*>(w + L.off_ext);
  pa.coord = reinterpret_cast<int*>(w + L.off_coord);
  pa.iota = reinterpret_cast<int*>(w + L.off_iota);
  pa.nh = g.nh;
  pa.nw = g.nw;
  pa.T = s.T;
  pa.H = s.H;
  pa.W = s.W;
  // the smallest even cut of the tile grid into blocks of at most
  // kOrderBlkH x kOrderBlkW tiles
  pa.blk_h = (g.nh + (g.nh + kOrderBlkH - 1) / kOrderBlkH - 1) / ((g.nh + kOrderBlkH - 1) / kOrderBlkH);
  pa.blk_w = (g.nw + (g.nw + kOrderBlkW - 1) / kOrderBlkW - 1) / ((g.nw + kOrderBlkW - 1) / kOrderBlkW);
  pa.units = reinterpret_cast<Unit*>(w + L.off_units);
  pa.comb = reinterpret_cast<Comb*>(w + L.off_comb);
  if (kv_chunk > 0)
    plan_kernel<true><<<1, kPlanThreads, 0, stream>>>(pa);
  else
    plan_kernel<false><<<1, kPlanThreads, 0, stream>>>(pa);

  AttnArgs aa;
  aa.q = static_cast<const uint16_t*>(q);
  aa.k = static_cast<const uint16_t*>(k);
  aa.v = static_cast<const uint16_t*>(v);
  aa.row_ptr = row_ptr;
  aa.col_idx = col_idx;
  aa.o = static_cast<uint16_t*>(o);
  aa.lse = lse;
  aa.ext = pa.ext;
  aa.iota = pa.iota;
  aa.coord = pa.coord;
  aa.tok_r = tokw ? tokw->token_radius : nullptr;
  aa.routed = tokw ? tokw->routed : nullptr;
  aa.r_max = tokw ? tokw->r_max : 0;
  aa.hdr = hdr;
  aa.hdr_mut = hdr;
  aa.units = pa.units;
  aa.part_o = reinterpret_cast<float*>(w + L.off_po);
  aa.part_ml = reinterpret_cast<float*>(w + L.off_pml);
  aa.nT = g.nT;
  aa.nh = g.nh;
  aa.nw = g.nw;
  aa.T = s.T;
  aa.H = s.H;
  aa.W = s.W;
  aa.c2 = scale * kLog2e;
  aa.raster = raster ? 1 : 0;
  aa.heads = s.heads;
  const TokMap map = {aa.raster, s.heads, g.nT, g.nh, g.nw, s.T, s.H, s.W};
  aa.q4 = skim ? static_cast<const uint8_t*>(skim->q4) : nullptr;
  aa.q4s = skim ? static_cast<const uint8_t*>(skim->q4_scales) : nullptr;
  aa.k4 = skim ? static_cast<const uint8_t*>(skim->k4) : nullptr;
  aa.k4s = skim ? static_cast<const uint8_t*>(skim->k4_scales) : nullptr;
  aa.tier = skim ? skim->tier : nullptr;
  const int grid = (int)std::min<int64_t>(L.max_units, 2LL * cus);
  if (s.head_dim == 128) {
    if (skim)
      attn_kernel<128, true, false><<<grid, kThreads, Cfg<128>::kLdsBytes + Cfg4<128>::kLdsBytes, stream>>>(aa);
    else if (tokw)
      attn_kernel<128, false, true><<<grid, kThreads, Cfg<128>::kLdsBytes, stream>>>(aa);
    else
      attn_kernel<128, false, false><<<grid, kThreads, Cfg<128>::kLdsBytes, stream>>>(aa);
    combine_kernel<128><<<std::max(1, 2 * cus), 256, 0, stream>>>(hdr, pa.comb, aa.part_o, aa.part_ml, aa.o, lse, map);
  } else {
    if (skim)
      attn_kernel<64, true, false><<<grid, kThreads, Cfg<64>::kLdsBytes + Cfg4<64>::kLdsBytes, stream>>>(aa);
    else if (tokw)
      attn_kernel<64, false, true><<<grid, kThreads, Cfg<64>::kLdsBytes, stream>>>(aa);
    else
      attn_kernel<64, false, false><<<grid, kThreads, Cfg<64>::kLdsBytes, stream>>>(aa);
    combine_kernel<64><<<std::max(1, 2 * cus), 256, 0, stream>>>(hdr, pa.comb, aa.part_o, aa.part_ml, aa.o, lse, map);
  }
  return hipGetLastError();
}

hipError_t attn_set_lds_limits() {
  const void* fns[6] = {reinterpret_cast<const void*>(attn_kernel<128, false, false>),
                        reinterpret_cast<const void*>(attn_kernel<128, true, false>),
                        reinterpret_cast<const void*>(attn_kernel<128, false, true>),
                        reinterpret_cast<const void*>(attn_kernel<64, false, false>),
                        reinterpret_cast<const void*>(attn_kernel<64, true, false>),
                        reinterpret_cast<const void*>(attn_kernel<64, false, true>)};
  const int lds[6] = {Cfg<128>::kLdsBytes, Cfg<128>::kLdsBytes + Cfg4<128>::kLdsBytes,
                      Cfg<128>::kLdsBytes, Cfg<64>::kLdsBytes,
                      Cfg<64>::kLdsBytes + Cfg4<64>::kLdsBytes, Cfg<64>::kLdsBytes};
  for (int i = 0; i < 6; ++i) {
    const hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, lds[i]);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace vsa
