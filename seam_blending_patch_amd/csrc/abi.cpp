// abi.cpp -- host side of the C ABI declared in include/seam_blend.h:
// argument and geometry validation, the per-axis geometry of the tile grid
// (clamped blend extents, crops, origins), the distinct-extent coefficient
// table layout, launch windows, GroupNorm patch/chunk layout and workspace.
// No device memory is allocated and the stream is never synchronised.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <numeric>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/seam_blend.h"
#include "sb_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int elem_bytes(int dtype) { return dtype == SB_F32 ? 4 : 2; }

// --------------------------------------------------------------------------
// tile-grid geometry
// --------------------------------------------------------------------------
struct Axis {
  int64_t n = 0, E = 0, R = 0, L = 0;
  std::vector<int64_t> ext, e; // e[k]: clamped blend extent between k-1 and k (e[0] = 0)
};

struct Grid {
  int ndim = 0;
  int64_t N = 0, C = 0;
  Axis ax[3]; // t, h, w
};

int build_grid(const int64_t grid[6], const int64_t *tile_extents, const int64_t blend_extent[3],
               const int64_t row_limit[3], Grid &G) {
  if (!grid || !tile_extents || !blend_extent || !row_limit)
    return fail(SB_EARG, "null geometry pointer");
  G.ndim = (int)grid[0];
  if (G.ndim != 4 && G.ndim != 5) return fail(SB_EARG, "ndim must be 4 or 5 (got %lld)", (long long)grid[0]);
  G.N = grid[1];
  G.C = grid[2];
  if (G.N < 0 || G.C < 0) return fail(SB_EARG, "N and C must be >= 0");
  if (G.N >= ((int64_t)1 << 31) || G.C >= ((int64_t)1 << 31) || G.N * G.C >= ((int64_t)1 << 31))
    return fail(SB_EGEOM, "N * C must be below 2^31");
  const char *names[3] = {"t", "h", "w"};
  int64_t off = 0;
  for (int a = 0; a < 3; ++a) {
    Axis &A = G.ax[a];
    A.n = grid[3 + a];
    if (A.n < 1) return fail(SB_EARG, "grid count along %s must be >= 1", names[a]);
    if (A.n > sb::kMaxAxisTiles)
      return fail(SB_EGEOM, "at most %d tiles per axis (got %lld along %s)", sb::kMaxAxisTiles,
                  (long long)A.n, names[a]);
    A.E = blend_extent[a];
    A.R = row_limit[a];
    if (G.ndim == 4 && a == 0) {
      A.E = 0;
      A.R = 1;
      if (A.n != 1) return fail(SB_EARG, "n_t must be 1 when ndim == 4");
    }
    if (A.E < 0) return fail(SB_EARG, "blend extent along %s must be >= 0", names[a]);
    if (A.R < 1) return fail(SB_EARG, "row limit along %s must be >= 1", names[a]);
    if (A.R > ((int64_t)1 << 30)) return fail(SB_EARG, "row limit along %s must be <= 2^30", names[a]);
    A.E = std::min<int64_t>(A.E, (int64_t)1 << 30); // extents are <= 2^30: the clamp e = min(E, ...) is unchanged
    A.ext.assign(tile_extents + off, tile_extents + off + A.n);
    off += A.n;
    for (int64_t k = 0; k < A.n; ++k) {
      if (A.ext[k] < 1) return fail(SB_EARG, "tile extent %s[%lld] must be >= 1", names[a], (long long)k);
      if (A.ext[k] > (int64_t)1 << 30) return fail(SB_EGEOM, "tile extent too large");
      if (k < A.n - 1 && A.ext[k] < A.R)
        return fail(SB_EGEOM, "non-last tile %s[%lld] = %lld is shorter than the row limit %lld",
                    names[a], (long long)k, (long long)A.ext[k], (long long)A.R);
    }
    if (G.ndim == 4 && a == 0 && A.ext[0] != 1) return fail(SB_EARG, "t_0 must be 1 when ndim == 4");
    A.e.assign(A.n, 0);
    for (int64_t k = 1; k < A.n; ++k) A.e[k] = std::min(A.E, std::min(A.ext[k - 1], A.ext[k]));
    for (int64_t k = 0; k < A.n; ++k) {
      const int64_t nxt = k + 1 < A.n ? A.e[k + 1] : 0;
      if (A.ext[k] < A.e[k] + nxt)
        return fail(SB_EGEOM,
                    "tile %s[%lld] = %lld is shorter than its two blend seams (%lld + %lld): the "
                    "data-parallel closed form needs a tile's head seam and tail to be disjoint",
                    names[a], (long long)k, (long long)A.ext[k], (long long)A.e[k], (long long)nxt);
    }
    A.L = (A.n - 1) * A.R + A.ext[A.n - 1];
    if (A.L > (int64_t)1 << 30) return fail(SB_EGEOM, "output extent too large");
  }
  return SB_OK;
}

// --------------------------------------------------------------------------
// device properties cached per device (no allocation)
// --------------------------------------------------------------------------
int cu_count() {
  // calls may come from several host threads: each entry is written once,
  // always with the same value
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

} // namespace

extern "C" const char *seamblend_last_error(void) { return g_err.c_str(); }

// error reporting and device properties for the other host files of the
// library (not exported)
extern "C" __attribute__((visibility("hidden"))) int sb_fail_message(int code, const char *msg) {
  return fail(code, "%s", msg);
}
extern "C" __attribute__((visibility("hidden"))) int sb_cu_count(void) { return cu_count(); }

extern "C" int vae_tile_blend_stitch_output_extents(const int64_t grid[6], const int64_t *tile_extents,
                                                    const int64_t blend_extent[3],
                                                    const int64_t row_limit[3],
                                                    int64_t out_extents[3]) {
  Grid G;
  int rc = build_grid(grid, tile_extents, blend_extent, row_limit, G);
  if (rc) return rc;
  if (!out_extents) return fail(SB_EARG, "null out_extents");
  for (int a = 0; a < 3; ++a) out_extents[a] = G.ax[a].L;
  return SB_OK;
}

extern "C" int vae_tile_blend_stitch(const void *const *tiles, const int64_t grid[6],
                                     const int64_t *tile_extents, const int64_t blend_extent[3],
                                     const int64_t row_limit[3], int dtype, void *out, void *stream) {
  Grid G;
  int rc = build_grid(grid, tile_extents, blend_extent, row_limit, G);
  if (rc) return rc;
  if (dtype != SB_F32 && dtype != SB_F16 && dtype != SB_BF16)
    return fail(SB_EARG, "unknown dtype %d", dtype);
  const Axis &At = G.ax[0], &Ah = G.ax[1], &Aw = G.ax[2];
  const int64_t planes = G.N * G.C;
  if (planes > 0) {
    // output and every tile below 2^50 elements: all byte offsets fit in 64 bits
    int64_t mt = 0, mh = 0, mw = 0;
    for (int64_t k = 0; k < At.n; ++k) mt = std::max(mt, At.ext[k]);
    for (int64_t k = 0; k < Ah.n; ++k) mh = std::max(mh, Ah.ext[k]);
    for (int64_t k = 0; k < Aw.n; ++k) mw = std::max(mw, Aw.ext[k]);
    const int64_t lim = ((int64_t)1 << 50) / planes;
    if (At.L * Ah.L > lim / Aw.L || mt * mh > lim / mw)
      return fail(SB_EGEOM, "output or tile too large (more than 2^50 elements)");
  }
  const int EB = elem_bytes(dtype);
  const int64_t ntiles = At.n * Ah.n * Aw.n;
  if (planes == 0) return SB_OK; // nothing to read or write (empty tensors may have null data)
  if (!tiles) return fail(SB_EARG, "null tiles");
  if (!out) return fail(SB_EARG, "null out");
  for (int64_t k = 0; k < ntiles; ++k) {
    if (!tiles[k]) return fail(SB_EARG, "null tile pointer %lld", (long long)k);
    if (!aligned(tiles[k], EB)) return fail(SB_EARG, "tile %lld is not aligned to its element size", (long long)k);
  }
  if (!aligned(out, EB)) return fail(SB_EARG, "out is not aligned to its element size");

  // output must not overlap any tile (address ranges)
  const uintptr_t o0 = (uintptr_t)out;
  const uintptr_t o1 = o0 + (uintptr_t)(planes * At.L * Ah.L * Aw.L * EB);
  for (int64_t tau = 0; tau < At.n; ++tau)
    for (int64_t i = 0; i < Ah.n; ++i)
      for (int64_t j = 0; j < Aw.n; ++j) {
        const uintptr_t t0 = (uintptr_t)tiles[(tau * Ah.n + i) * Aw.n + j];
        const uintptr_t t1 = t0 + (uintptr_t)(planes * At.ext[tau] * Ah.ext[i] * Aw.ext[j] * EB);
        if (t0 < o1 && o0 < t1)
          return fail(SB_EARG, "out overlaps tile (%lld,%lld,%lld)", (long long)tau, (long long)i,
                      (long long)j);
      }

  // vector width: 16-byte vectors when every row, row offset and seam boundary
  // along W is a whole number of vectors and every base is 16-byte aligned
  const int V16 = 16 / EB;
  bool vec16 = aligned(out, 16) && Aw.L % V16 == 0 && Aw.R % V16 == 0;
  for (int64_t k = 0; k < Aw.n && vec16; ++k) vec16 = Aw.ext[k] % V16 == 0 && Aw.e[k] % V16 == 0;
  for (int64_t k = 0; k < ntiles && vec16; ++k) vec16 = aligned(tiles[k], 16);
  const int V = vec16 ? V16 : 1;

  if (At.L * Ah.L * (Aw.L / V) >= ((int64_t)1 << 31))
    return fail(SB_EGEOM, "one (n, c) plane of the output exceeds 2^31 vectors");

  sb::BlendArgs A;
  std::memset(&A, 0, sizeof A);
  for (int a = 0; a < 3; ++a) {
    const Axis &X = G.ax[a];
    for (int64_t k = 0; k < X.n; ++k) {
      A.ext[a][k] = (int32_t)X.ext[k];
      if (X.e[k] > sb::kMaxBlend)
        return fail(SB_EGEOM, "clamped blend extent %lld exceeds %d", (long long)X.e[k], sb::kMaxBlend);
      // the seam's reciprocal, rounded once from float64 as the kernel's
      // coefficient formula requires
      A.rcp[a][k] = X.e[k] > 0 ? (float)(1.0 / (double)X.e[k]) : 0.f;
    }
  }
  A.out = out;
  A.n_t = (int32_t)At.n; A.n_h = (int32_t)Ah.n; A.n_w = (int32_t)Aw.n;
  for (int a = 0; a < 3; ++a) {
    A.E[a] = (int32_t)G.ax[a].E;
    A.R[a] = (int32_t)G.ax[a].R;
  }
  A.LT = (int32_t)At.L; A.LH = (int32_t)Ah.L; A.LW = (int32_t)Aw.L;
  A.div_Rt = sb::make_fastdiv((uint32_t)At.R);
  A.div_Rh = sb::make_fastdiv((uint32_t)Ah.R);
  {
    // 32-bit lane offsets when every (plane, frame) slice of a tile and every
    // band of output rows as tall as a tile stays below 2^31 bytes
    int64_t mh = 0, mw = 0;
    for (int64_t k = 0; k < Ah.n; ++k) mh = std::max(mh, Ah.ext[k]);
    for (int64_t k = 0; k < Aw.n; ++k) mw = std::max(mw, Aw.ext[k]);
    const int64_t cap = (((int64_t)1 << 31) - 1) / EB;
    A.off32 = (mh <= cap / std::max<int64_t>(mw, 1) && mh <= cap / std::max<int64_t>(Aw.L, 1)) ? 1 : 0;
  }
  {
    // nontemporal output stores when the call's traffic (every tile read,
    // the output written) is under half the 256 MB last-level cache
    // (in double: only a size class is wanted, and sums of extreme extents
    // would overflow 64-bit integers)
    double st = 0, sh = 0, sw = 0;
    for (int64_t k = 0; k < At.n; ++k) st += (double)At.ext[k];
    for (int64_t k = 0; k < Ah.n; ++k) sh += (double)Ah.ext[k];
    for (int64_t k = 0; k < Aw.n; ++k) sw += (double)Aw.ext[k];
    const double traffic = (st * sh * sw + (double)At.L * Ah.L * Aw.L) * (double)planes * EB;
    A.nt_store = traffic < (double)(128 << 20) ? 1 : 0;
  }
  // Rows per block.  Each block pays a fixed start-up (argument loads; in the
  // span layout also its column records and a barrier), so blocks are made
  // as large as the problem allows while still giving every CU several blocks: about
  // total / (cus * SB_BLEND_BLOCKS_PER_CU) vectors in the widest W segment,
  // clamped to [1024, 8192]; the band height is then aligned to the row seams
  // or balanced over the rows (below).  18 per CU, measured against 8, 12
  // and 24: the 4096x4096 workload 85.4 -> 82.4 us against 12 (bands of 32
  // rows instead of 64), the others within noise.
#ifndef SB_BLEND_BLOCKS_PER_CU
#define SB_BLEND_BLOCKS_PER_CU 18
#endif
  int64_t seg_max = 1;
  for (int64_t k = 0; k < Aw.n; ++k) {
    const int64_t crop = k < Aw.n - 1 ? Aw.R : Aw.ext[k];
    const int64_t es = std::min(Aw.e[k], crop);
    seg_max = std::max(seg_max, std::max(es, crop - es) / V);
  }
  const int cus = cu_count();
  const int64_t total_vec = planes * At.L * Ah.L * (Aw.L / V);
#ifndef SB_BLEND_PER_BLOCK_MIN
#define SB_BLEND_PER_BLOCK_MIN 1024
#endif
#ifndef SB_BLEND_PER_BLOCK_MAX
#define SB_BLEND_PER_BLOCK_MAX 8192
#endif
  const int64_t per_block = std::min<int64_t>(
      SB_BLEND_PER_BLOCK_MAX,
      std::max<int64_t>(SB_BLEND_PER_BLOCK_MIN, total_vec / ((int64_t)cus * SB_BLEND_BLOCKS_PER_CU)));
  // Span layout when every W segment is narrow (fewer than SB_BLEND_SPAN_BELOW
  // vectors): a block then owns whole tile columns, about 128 vectors of a row.
#ifndef SB_BLEND_SPAN_BELOW
#define SB_BLEND_SPAN_BELOW 16
#endif
  const bool span = Aw.n >= 2 && seg_max < SB_BLEND_SPAN_BELOW;
  int64_t span_k = 0, n_spans = 0, span_w = 0;
  if (span) {
    const int64_t col_vec = std::max<int64_t>(1, Aw.R / V);
#ifndef SB_BLEND_SPAN_VECS
#define SB_BLEND_SPAN_VECS 128
#endif
    span_k = std::min<int64_t>({(int64_t)sb::kMaxSpanCols, Aw.n,
                                std::max<int64_t>(1, (SB_BLEND_SPAN_VECS + col_vec - 1) / col_vec)});
    n_spans = (Aw.n + span_k - 1) / span_k;
    for (int64_t s = 0; s < n_spans; ++s) {
      const int64_t ja = s * span_k, jb = std::min(ja + span_k, Aw.n);
      span_w = std::max(span_w, (jb == Aw.n ? Aw.L : jb * Aw.R) - ja * Aw.R);
    }
  }
  // The span layout's launches are small (the tiled-encode latents, a few MB):
  // its blocks are sized so that the grid is about one round of resident
  // blocks (SB_BLEND_SPAN_BLOCKS_PER_CU per CU at the kernel's occupancy),
  // with at least SB_BLEND_SPAN_PER_BLOCK_MIN vectors each.  Measured against
  // the segment layout's 18 per CU and a 512-vector minimum: SD encode 2048
  // 4.95 -> 4.62 us, 64/32 encode 5.37 -> 4.59 us, the batch-4 4096 encode and
  // the 112x112 fp32 blend unchanged.
#ifndef SB_BLEND_SPAN_BLOCKS_PER_CU
#define SB_BLEND_SPAN_BLOCKS_PER_CU 4
#endif
#ifndef SB_BLEND_SPAN_PER_BLOCK_MIN
#define SB_BLEND_SPAN_PER_BLOCK_MIN 128
#endif
  const int64_t block_cols = span ? span_w / V : seg_max;
  const int64_t per_block_l = span ? std::min<int64_t>(
                                         SB_BLEND_PER_BLOCK_MAX,
                                         std::max<int64_t>(SB_BLEND_SPAN_PER_BLOCK_MIN,
                                                           total_vec / ((int64_t)cus * SB_BLEND_SPAN_BLOCKS_PER_CU)))
                                   : per_block;
  int64_t rows_pb = std::max<int64_t>(1, std::min<int64_t>(1024, per_block_l / block_cols));
  rows_pb = std::min<int64_t>(rows_pb, Ah.L);
  // Bands that start on every tile-row and row-seam boundary hold one run
  // each (one row class, whole batches): every such boundary is a multiple of
  // g = gcd(R_h, e_h(1), ..., e_h(n-1)) rows from a tile row's origin, so a
  // band height dividing g keeps them all on band edges.  Taken when a divisor
  // of g comes within a factor of 3 of the size-based height (measured on the
  // video workload: 64-row bands 68.6 us against 69.7 us for 60-row ones; in
  // the span layout a band that crosses a tile row also rebuilds its column
  // records); otherwise the bands are balanced over the rows.
  int64_t g = Ah.R;
  for (int64_t k = 1; k < Ah.n; ++k)
    if (Ah.e[k] > 0) g = std::gcd(g, Ah.e[k]);
  int64_t aligned_rows = 1;
  for (int64_t d = 1; d * d <= g; ++d)
    if (g % d == 0) {
      if (d <= rows_pb) aligned_rows = std::max(aligned_rows, d);
      if (g / d <= rows_pb) aligned_rows = std::max(aligned_rows, g / d);
    }
  if (Ah.n > 1 && aligned_rows * 3 >= rows_pb) {
    rows_pb = aligned_rows;
  } else {
    const int64_t nrb = (Ah.L + rows_pb - 1) / rows_pb;
    rows_pb = (Ah.L + nrb - 1) / nrb;
  }
  // row bands go on a grid axis of at most kMaxBlocksYZ blocks
  rows_pb = std::max<int64_t>(rows_pb, (Ah.L + sb::kMaxBlocksYZ - 1) / sb::kMaxBlocksYZ);
  A.rows_per_block = (int32_t)rows_pb;
  A.span_k = (int32_t)span_k;
  A.div_Rw = sb::make_fastdiv((uint32_t)Aw.R);
  // dynamic LDS: the span layout's column records (both layouts form their
  // seam coefficients in registers)
  const size_t lds = span ? (size_t)span_k * sizeof(sb::SpanCol) : 0;
  hipStream_t st = (hipStream_t)stream;
  const int64_t n_wseg = span ? n_spans : 2 * Aw.n - 1;

  // Launch windows.  A window covers output frames of temporal tiles
  // [t0, t1) and rows of tile rows [i0, i1); it needs the tile pointers of
  // temporal tiles [max(t0-1,0), t1) and tile rows [max(i0-1,0), i1).
  // Windows are grown greedily within the kernel-argument pointer budget.
  // Every window is planned and checked before the first launch, so a
  // geometry error leaves the output untouched.
  auto tiles_needed = [&](int64_t t0, int64_t t1, int64_t i0, int64_t i1) {
    return (t1 - std::max<int64_t>(t0 - 1, 0)) * (i1 - std::max<int64_t>(i0 - 1, 0)) * Aw.n;
  };
  struct Window {
    int64_t t0, t1, i0, i1;
  };
  std::vector<Window> wins;
  for (int64_t t0 = 0; t0 < At.n;) {
    int64_t t1 = t0 + 1;
    while (t1 < At.n && tiles_needed(t0, t1 + 1, 0, Ah.n) <= sb::kMaxWindowTiles) ++t1;
    for (int64_t i0 = 0; i0 < Ah.n;) {
      int64_t i1 = i0 + 1;
      if (tiles_needed(t0, t1, i0, i1) > sb::kMaxWindowTiles)
        return fail(SB_EGEOM, "tile grid too wide: %lld tiles per row exceed one launch window",
                    (long long)Aw.n);
      while (i1 < Ah.n && tiles_needed(t0, t1, i0, i1 + 1) <= sb::kMaxWindowTiles) ++i1;
      if (span) {
        // the span kernel's grid x takes the window's (plane, frame) pairs:
        // at least its frames, within 2^32 work-items (kMaxBlocksX blocks)
        const int64_t nF = ((t1 == At.n) ? At.L : t1 * At.R) - t0 * At.R;
        if (nF > sb::kMaxBlocksX)
          return fail(SB_EGEOM, "a launch window of %lld frames exceeds %lld blocks", (long long)nF,
                      (long long)sb::kMaxBlocksX);
      }
      wins.push_back(Window{t0, t1, i0, i1});
      i0 = i1;
    }
    t0 = t1;
  }

  for (const Window &w : wins) {
    const int64_t t0 = w.t0, t1 = w.t1, i0 = w.i0, i1 = w.i1;
    const int64_t tb = std::max<int64_t>(t0 - 1, 0), ib = std::max<int64_t>(i0 - 1, 0);
    A.taub = (int32_t)tb;
    A.ib = (int32_t)ib;
    A.ptr_nh = (int32_t)(i1 - ib);
    for (int k = 0; k < sb::kMaxWindowTiles; ++k) A.ptr[k] = nullptr;
    for (int64_t tq = tb; tq < t1; ++tq)
      for (int64_t iq = ib; iq < i1; ++iq)
        for (int64_t jq = 0; jq < Aw.n; ++jq)
          A.ptr[((tq - tb) * A.ptr_nh + (iq - ib)) * Aw.n + jq] = tiles[(tq * Ah.n + iq) * Aw.n + jq];
    const int64_t F0 = t0 * At.R, F1 = (t1 == At.n) ? At.L : t1 * At.R;
    const int64_t Y0 = i0 * Ah.R, Y1 = (i1 == Ah.n) ? Ah.L : i1 * Ah.R;
    A.F0 = (int32_t)F0; A.nF = (int32_t)(F1 - F0);
    A.Y0 = (int32_t)Y0; A.nY = (int32_t)(Y1 - Y0);
    const int64_t row_blocks = (A.nY + rows_pb - 1) / rows_pb;
    if (span) {
      // span kernel: grid x = (plane, frame) pairs of this window, y = spans,
      // z = row bands
      A.div_nF = sb::make_fastdiv((uint32_t)A.nF);
      const int64_t max_planes = std::max<int64_t>(1, sb::kMaxBlocksX / A.nF);
      for (int64_t p0 = 0; p0 < planes; p0 += max_planes) {
        const int64_t np = std::min(max_planes, planes - p0);
        A.plane0 = (int32_t)p0;
        const dim3 grid((unsigned)(np * A.nF), (unsigned)n_wseg, (unsigned)row_blocks);
        hipError_t e = sb_launch_blend_span(A, dtype, vec16 ? 1 : 0, grid, lds, st);
        if (e != hipSuccess) return fail(SB_ELAUNCH, "blend launch failed: %s", hipGetErrorString(e));
      }
    } else {
      // segment kernel: grid (W segments, row bands, (plane, frame) pairs),
      // at most kMaxBlocksYZ pairs per launch: the window's frames go in
      // ranges of at most that many, and planes as many as fit beside them
      for (int64_t fa = F0; fa < F1; fa += sb::kMaxBlocksYZ) {
        const int64_t nf = std::min<int64_t>(sb::kMaxBlocksYZ, F1 - fa);
        A.F0 = (int32_t)fa;
        A.nF = (int32_t)nf;
        A.div_nF = sb::make_fastdiv((uint32_t)nf);
        const int64_t max_planes = std::max<int64_t>(1, sb::kMaxBlocksYZ / nf);
        for (int64_t p0 = 0; p0 < planes; p0 += max_planes) {
          const int64_t np = std::min(max_planes, planes - p0);
          A.plane0 = (int32_t)p0;
          A.g_seg = (int32_t)n_wseg;
          A.g_band = (int32_t)row_blocks;
          A.g_pf = (int32_t)(np * nf);
          const dim3 grid((unsigned)n_wseg, (unsigned)row_blocks, (unsigned)(np * nf));
          hipError_t e = sb_launch_blend(A, dtype, vec16 ? 1 : 0, grid, lds, st);
          if (e != hipSuccess) return fail(SB_ELAUNCH, "blend launch failed: %s", hipGetErrorString(e));
        }
      }
    }
  }
  return SB_OK;
}

// --------------------------------------------------------------------------
// GroupNorm
// --------------------------------------------------------------------------
namespace {

// largest pass-1 grid: blocks of 512 threads (1024 for the whole-row
// layout) within 2^32 work-items in x
constexpr int64_t kMaxStatsBlocks = ((int64_t)1 << 32) / 1024 - 1;

struct GNPlan {
  sb::GNArgs a;
  bool vec16 = false;
  size_t ws_bytes = 0;
  bool empty = false;
};

int plan_groupnorm(int ndim, const int64_t *shape, int64_t groups, int split_axis, int64_t n_patches,
                   int dtype_bytes, bool allow_vec, GNPlan &P) {
  if (!shape) return fail(SB_EARG, "null shape");
  if (ndim < 3 || ndim > 5) return fail(SB_EARG, "ndim must be 3, 4 or 5 (got %d)", ndim);
  for (int k = 0; k < ndim; ++k)
    if (shape[k] < 0) return fail(SB_EARG, "negative extent");
  if (groups < 1) return fail(SB_EARG, "groups must be >= 1");
  if (shape[1] % groups != 0) return fail(SB_EARG, "C = %lld is not divisible by groups = %lld",
                                          (long long)shape[1], (long long)groups);
  if (split_axis < 2 || split_axis >= ndim)
    return fail(SB_EARG, "split_axis must be a spatial axis (2..%d), got %d", ndim - 1, split_axis);
  if (n_patches < 1 || n_patches > sb::kMaxPatches)
    return fail(SB_EARG, "n_patches must be in 1..%d", sb::kMaxPatches);
  if (shape[0] > ((int64_t)1 << 20) || shape[1] > ((int64_t)1 << 24))
    return fail(SB_EGEOM, "N or C too large");
  sb::GNArgs &a = P.a;
  std::memset(&a, 0, sizeof a);
  int64_t S = 1;
  for (int k = 2; k < ndim; ++k) {
    if (shape[k] > ((int64_t)1 << 30) || (shape[k] > 0 && S > ((int64_t)1 << 40) / shape[k]))
      return fail(SB_EGEOM, "spatial extents too large (each <= 2^30, product <= 2^40)");
    S *= shape[k];
  }
  a.N = (int32_t)shape[0];
  a.C = (int32_t)shape[1];
  a.G = (int32_t)groups;
  a.Cg = (int32_t)(shape[1] / groups);
  a.S = S;
  a.P = (int32_t)n_patches;
  a.L = (int32_t)shape[split_axis];
  int64_t inner = 1, mid = 1;
  for (int k = split_axis + 1; k < ndim; ++k) inner *= shape[k];
  for (int k = 2; k < split_axis; ++k) mid *= shape[k];
  a.inner = inner;
  a.mid = mid;
  a.len_small = (int32_t)(a.L / n_patches);
  a.n_big = (int32_t)(a.L % n_patches);
  a.len_big = a.len_small + 1;
  P.empty = shape[0] == 0 || shape[1] == 0 || S == 0;
  // vector width: every run of a patch and every plane a whole number of
  // 16-byte vectors (base alignment is checked per call)
  const int V16 = 16 / dtype_bytes;
  P.vec16 = allow_vec && S % V16 == 0 && (a.L * inner) % V16 == 0 &&
            ((int64_t)a.len_small * inner) % V16 == 0 &&
            (a.n_big == 0 || ((int64_t)a.len_big * inner) % V16 == 0);
  const int V = P.vec16 ? V16 : 1;
  // patches across the innermost axis: pass 1 reads whole rows of at most
  // 1024 vectors, one lane per column (see gn_stats_rows_kernel)
  a.rows_layout = (inner == 1 && a.L / V >= 1 && a.L / V <= 1024) ? 1 : 0;
  // a group's element and vector indices and its statistics counts are 32-bit
  if ((int64_t)a.Cg * S >= ((int64_t)1 << 31)) return fail(SB_EGEOM, "a group exceeds 2^31 elements");
  // (n, c) planes are 32-bit indices
  if ((int64_t)a.N * a.C >= ((int64_t)1 << 31)) return fail(SB_EGEOM, "N*C must be below 2^31");
  if (S / V >= ((int64_t)1 << 40)) return fail(SB_EGEOM, "plane too large");
  // chunks per patch: a power of two, P_pow2 * CPP <= 64 (one wavefront merges
  // the partials of a group), at least 8192 elements per chunk (measured best
  // for the video activation, 3-4% over 16384 and 10% over 4096, with x
  // resident in the last-level cache or not; the large activations are
  // insensitive); independent of dtype and vector width so the workspace size
  // is too
  int64_t ppow = 1;
  while (ppow < n_patches) ppow <<= 1;
  const int64_t patch_el = (int64_t)std::max(a.len_big, 1) * inner * a.Cg * mid;
  int64_t cpp = 1;
#ifndef SB_GN_CHUNK_MIN
#define SB_GN_CHUNK_MIN 8192
#endif
  // pass 1 launches at most kMaxStatsBlocks blocks (2^32 work-items of 1024
  // threads in x): more chunks only while the grid stays within that
  // (counted for the per-patch layout, which has the most blocks, so that the
  // chunk count and the workspace do not depend on the vector width)
  const int64_t units = (int64_t)a.N * a.G * n_patches; // blocks at one chunk per patch
  if (units > kMaxStatsBlocks)
    return fail(SB_EGEOM, "N*groups*patches = %lld exceeds %lld statistics blocks", (long long)units,
                (long long)kMaxStatsBlocks);
  while (cpp * 2 * ppow <= 64 && patch_el / (cpp * 2) >= SB_GN_CHUNK_MIN && units * cpp * 2 <= kMaxStatsBlocks)
    cpp *= 2;
  a.CPP = (int32_t)cpp;
  a.log2CPP = 0;
  while ((1 << a.log2CPP) < cpp) a.log2CPP++;
  a.per2 = sb::kNormThreads * sb::kNormUnroll; // vectors per pass-2 block
  a.chunks2 = (int32_t)std::max<int64_t>(1, (S / V + a.per2 - 1) / a.per2);
  // pass 2 runs on a (chunks of a plane, planes) grid: 2^32 work-items in x;
  // planes beyond the grid's y extent take further launches
  if ((int64_t)a.chunks2 * sb::kNormThreads >= ((int64_t)1 << 32)) return fail(SB_EGEOM, "plane too large");
  a.div_C = sb::make_fastdiv((uint32_t)std::max(a.C, 1));
  a.div_Cg = sb::make_fastdiv((uint32_t)std::max(a.Cg, 1));
  a.div_P = sb::make_fastdiv((uint32_t)a.P);
  a.div_G = sb::make_fastdiv((uint32_t)a.G);
  P.ws_bytes = (size_t)shape[0] * groups * n_patches * cpp * 4 * sizeof(float); // (count, m, M2, K_g)
  if (P.ws_bytes == 0) P.ws_bytes = 16;
  return SB_OK;
}

} // namespace

extern "C" size_t patch_groupnorm_workspace_bytes(int ndim, const int64_t *shape, int64_t groups,
                                                  int split_axis, int64_t n_patches) {
  GNPlan P;
  if (plan_groupnorm(ndim, shape, groups, split_axis, n_patches, 2, false, P)) return 0;
  return P.ws_bytes;
}

namespace {

// patch_groupnorm with its statistics partials either in the caller's
// workspace or (workspace == nullptr and use_static) in the library's static
// device scratch, looked up only after every host check has passed.
int groupnorm_call(const void *x, int ndim, const int64_t *shape, int64_t groups, int split_axis,
                   int64_t n_patches, float eps, const void *gamma, const void *beta, int dtype, void *out,
                   void *workspace, size_t workspace_bytes, bool use_static, float *patch_stats,
                   void *stream) {
  if (dtype != SB_F32 && dtype != SB_F16 && dtype != SB_BF16)
    return fail(SB_EARG, "unknown dtype %d", dtype);
  GNPlan P;
  int rc = plan_groupnorm(ndim, shape, groups, split_axis, n_patches, elem_bytes(dtype), true, P);
  if (rc) return rc;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(SB_EARG, "eps must be finite and >= 0");
  if (!x || !out) return fail(SB_EARG, "null x or out");
  if (P.empty) return SB_OK;
  if (use_static) {
    if (P.ws_bytes > (size_t)SB_GN_STATIC_SCRATCH_BYTES)
      return fail(SB_EWORKSPACE,
                  "the statistics of this problem need %zu bytes, more than the %zu-byte static "
                  "scratch: call patch_groupnorm with a workspace",
                  P.ws_bytes, (size_t)SB_GN_STATIC_SCRATCH_BYTES);
  } else {
    if (!workspace) return fail(SB_EARG, "null workspace");
    if (workspace_bytes < P.ws_bytes)
      return fail(SB_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                  P.ws_bytes);
  }
  if ((!use_static && !aligned(workspace, 16)) || (patch_stats && !aligned(patch_stats, 4)))
    return fail(SB_EARG, "workspace must be 16-byte and patch_stats 4-byte aligned");
  const int EB = elem_bytes(dtype);
  if (!aligned(x, EB) || !aligned(out, EB) || (gamma && !aligned(gamma, EB)) || (beta && !aligned(beta, EB)))
    return fail(SB_EARG, "x, out, gamma and beta must be aligned to the element size");
  // N*C < 2^31 and a group below 2^31 elements, so a plane holds fewer than
  // 2^31 elements and the tensor fewer than 2^62
  const uint64_t nbytes = (uint64_t)(shape[0] * shape[1] * P.a.S) * (uint64_t)EB;
  if (nbytes >= ((uint64_t)1 << 56)) return fail(SB_EGEOM, "tensor too large (2^56 bytes or more)");
  if (x != out) {
    const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)nbytes;
    const uintptr_t y0 = (uintptr_t)out, y1 = y0 + (uintptr_t)nbytes;
    if (x0 < y1 && y0 < x1) return fail(SB_EARG, "out partially overlaps x (only exact aliasing is allowed)");
  }
  bool vec16 = P.vec16 && aligned(x, 16) && aligned(out, 16);
  if (P.vec16 && !vec16) {
    // misaligned bases: the same layout with single-element vectors
    rc = plan_groupnorm(ndim, shape, groups, split_axis, n_patches, EB, false, P);
    if (rc) return rc;
  }
  if (use_static) {
    hipError_t e = sb_groupnorm_static_scratch(&workspace);
    if (e != hipSuccess)
      return fail(SB_ELAUNCH, "static scratch lookup failed: %s", hipGetErrorString(e));
  }
  sb::GNArgs &a = P.a;
  a.x = x;
  a.out = out;
  a.gamma = gamma;
  a.beta = beta;
  a.part = (float *)workspace;
  a.patch_stats = patch_stats;
  a.eps = eps;
  hipError_t e = sb_launch_groupnorm(a, dtype, vec16 ? 1 : 0, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SB_ELAUNCH, "groupnorm launch failed: %s", hipGetErrorString(e));
  return SB_OK;
}

} // namespace

extern "C" int patch_groupnorm(const void *x, int ndim, const int64_t *shape, int64_t groups,
                               int split_axis, int64_t n_patches, float eps, const void *gamma,
                               const void *beta, int dtype, void *out, void *workspace,
                               size_t workspace_bytes, float *patch_stats, void *stream) {
  return groupnorm_call(x, ndim, shape, groups, split_axis, n_patches, eps, gamma, beta, dtype, out,
                        workspace, workspace_bytes, false, patch_stats, stream);
}

extern "C" int patch_groupnorm_noalloc(const void *x, int ndim, const int64_t *shape, int64_t groups,
                                       int split_axis, int64_t n_patches, float eps, const void *gamma,
                                       const void *beta, int dtype, void *out, float *patch_stats,
                                       void *stream) {
  return groupnorm_call(x, ndim, shape, groups, split_axis, n_patches, eps, gamma, beta, dtype, out,
                        nullptr, 0, true, patch_stats, stream);
}
