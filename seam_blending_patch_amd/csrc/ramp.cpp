// ramp.cpp -- host side of vae_tile_ramp_blend: validation of a wide-tile
// layout, the runs of positions along each axis where the same tiles carry
// weight, the column chunks and row segments the kernel's blocks cover, and
// the launch windows.  No device memory is allocated and the stream is never
// synchronised.
//
// Weight of a tile along one axis (unsloth Studio PR "size seam-free VAE
// tiles from measured peaks", the Qwen-Image-2.1 wide-tile commit): none
// within the margin m of an edge it shares with another tile, then a linear
// ramp to full weight over the next r positions -- at whole distance d from a
// shared edge the factor is clamp((d - m) / r, 0, 1), positive iff d > m.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/seam_blend.h"
#include "sb_internal.h"

extern "C" int sb_fail_message(int code, const char *msg); // abi.cpp
extern "C" int sb_cu_count(void);                          // abi.cpp

namespace {

int failf(int code, const char *fmt, ...) {
  char buf[400];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return sb_fail_message(code, buf);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Run {
  int64_t p0, p1; // positions [p0, p1)
  int k0, cnt;    // tiles [k0, k0 + cnt) carry weight there
};

struct AxisLayout {
  int64_t n = 0, L = 0, m = 0, r = 1;
  std::vector<int64_t> o, s;
  std::vector<int64_t> lo, hi; // tile k has weight exactly on [lo_k, hi_k)
};

int read_axis(const char *name, int64_t n, const int64_t *o, const int64_t *s, int64_t m, int64_t r,
              AxisLayout &A) {
  if (n < 1 || n > sb::kRampMaxAxisTiles)
    return failf(SB_EARG, "tiles along %s must be in 1..%d (got %lld)", name, sb::kRampMaxAxisTiles,
                 (long long)n);
  if (m < 0 || m >= ((int64_t)1 << sb::kRampPosBits))
    return failf(SB_EARG, "margin along %s must be in 0..2^20", name);
  if (r < 1 || r >= ((int64_t)1 << sb::kRampPosBits))
    return failf(SB_EARG, "ramp along %s must be in 1..2^20", name);
  A.n = n;
  A.m = m;
  A.r = r;
  A.o.assign(o, o + n);
  A.s.assign(s, s + n);
  if (A.o[0] != 0) return failf(SB_EGEOM, "the first tile along %s must start at 0", name);
  for (int64_t k = 0; k < n; ++k) {
    if (A.s[k] < 1 || A.s[k] >= ((int64_t)1 << sb::kRampPosBits))
      return failf(SB_EARG, "tile extent %s[%lld] must be in 1..2^20", name, (long long)k);
    if (A.o[k] < 0 || A.o[k] >= ((int64_t)1 << sb::kRampPosBits))
      return failf(SB_EGEOM, "tile origin %s[%lld] must be in 0..2^20", name, (long long)k);
    if (k > 0 && A.o[k] <= A.o[k - 1])
      return failf(SB_EGEOM, "tile origins along %s must increase", name);
  }
  A.L = A.o[n - 1] + A.s[n - 1];
  if (A.L >= ((int64_t)1 << sb::kRampPosBits))
    return failf(SB_EGEOM, "output extent along %s must be below 2^20", name);
  for (int64_t k = 0; k < n; ++k)
    if (A.o[k] + A.s[k] > A.L)
      return failf(SB_EGEOM, "tile %s[%lld] ends past the last tile's end", name, (long long)k);
  A.lo.resize(n);
  A.hi.resize(n);
  for (int64_t k = 0; k < n; ++k) {
    A.lo[k] = k > 0 ? A.o[k] + m + 1 : A.o[k];
    A.hi[k] = k < n - 1 ? A.o[k] + A.s[k] - 1 - m : A.o[k] + A.s[k];
    if (A.hi[k] < A.lo[k]) A.hi[k] = A.lo[k]; // no weight anywhere
  }
  return SB_OK;
}

// Runs of positions with the same set of tiles carrying weight.  Fails when a
// position has none, more than kRampMaxCover, or a set that is not a range.
int element_runs(const char *name, const AxisLayout &A, std::vector<Run> &runs) {
  std::vector<int64_t> bp = {0, A.L};
  for (int64_t k = 0; k < A.n; ++k)
    if (A.lo[k] < A.hi[k]) {
      bp.push_back(A.lo[k]);
      bp.push_back(A.hi[k]);
    }
  std::sort(bp.begin(), bp.end());
  bp.erase(std::unique(bp.begin(), bp.end()), bp.end());
  runs.clear();
  for (size_t q = 0; q + 1 < bp.size(); ++q) {
    const int64_t p = bp[q];
    int k0 = -1, cnt = 0;
    for (int64_t k = 0; k < A.n; ++k) {
      if (A.lo[k] <= p && p < A.hi[k]) {
        if (k0 < 0) k0 = (int)k;
        else if (k != k0 + cnt)
          return failf(SB_EGEOM, "the tiles with weight at %s = %lld are not consecutive", name, (long long)p);
        ++cnt;
      }
    }
    if (cnt == 0)
      return failf(SB_EGEOM, "no tile has weight at %s = %lld (overlaps must exceed twice the margin)",
                   name, (long long)p);
    if (cnt > sb::kRampMaxCover)
      return failf(SB_EGEOM, "%d tiles carry weight at %s = %lld (at most %d)", cnt, name, (long long)p,
                   sb::kRampMaxCover);
    if (!runs.empty() && runs.back().k0 == k0 && runs.back().cnt == cnt) runs.back().p1 = bp[q + 1];
    else runs.push_back(Run{p, bp[q + 1], k0, cnt});
  }
  return SB_OK;
}

// The same runs on a grid of V-position vectors: a vector that straddles a
// change takes every tile with weight anywhere in it.  Returns false when some
// such tile does not cover the whole vector (then vectors cannot be used).
bool vector_runs(const AxisLayout &A, const std::vector<Run> &el, int64_t V, std::vector<Run> &out) {
  out.clear();
  size_t r = 0;
  for (int64_t q0 = 0; q0 < A.L; q0 += V) {
    const int64_t q1 = q0 + V;
    while (r < el.size() && el[r].p1 <= q0) ++r;
    int kmin = 1 << 30, kmax = -1;
    for (size_t t = r; t < el.size() && el[t].p0 < q1; ++t) {
      kmin = std::min(kmin, el[t].k0);
      kmax = std::max(kmax, el[t].k0 + el[t].cnt);
    }
    if (kmax - kmin > sb::kRampMaxCover) return false;
    for (int k = kmin; k < kmax; ++k)
      if (A.o[k] > q0 || A.o[k] + A.s[k] < q1) return false;
    if (!out.empty() && out.back().k0 == kmin && out.back().cnt == kmax - kmin) out.back().p1 = q1;
    else out.push_back(Run{q0, q1, kmin, kmax - kmin});
  }
  return true;
}

// The same runs on 128-byte lines (G positions): a line that straddles a
// change takes every tile with weight anywhere in it.  Those tiles carry
// exactly zero weight on the line's positions outside their weighted ranges
// (the normalised weights and the sums they enter are unchanged), and no two
// column chunks then share a line of the output or of a tile row, so no line
// is fetched or written by two blocks.  Returns false when some such tile
// does not cover the whole line, or a line would take more than
// kRampMaxCover tiles.
bool line_runs(const AxisLayout &A, const std::vector<Run> &el, int64_t G, std::vector<Run> &out) {
  out.clear();
  size_t r = 0;
  for (int64_t q0 = 0; q0 < A.L; q0 += G) {
    const int64_t q1 = std::min(q0 + G, A.L);
    while (r < el.size() && el[r].p1 <= q0) ++r;
    int kmin = 1 << 30, kmax = -1;
    for (size_t t = r; t < el.size() && el[t].p0 < q1; ++t) {
      kmin = std::min(kmin, el[t].k0);
      kmax = std::max(kmax, el[t].k0 + el[t].cnt);
    }
    if (kmax - kmin > sb::kRampMaxCover) return false;
    for (int k = kmin; k < kmax; ++k)
      if (A.o[k] > q0 || A.o[k] + A.s[k] < q1) return false;
    if (!out.empty() && out.back().k0 == kmin && out.back().cnt == kmax - kmin) out.back().p1 = q1;
    else out.push_back(Run{q0, q1, kmin, kmax - kmin});
  }
  return true;
}

// split runs into pieces of at most `single` (one tile) or `multi` (several)
// positions, each a whole number of V-position vectors
void split_runs(const std::vector<Run> &runs, int64_t single, int64_t multi, int64_t V, std::vector<Run> &out) {
  out.clear();
  for (const Run &u : runs) {
    const int64_t len = u.p1 - u.p0, cap = u.cnt == 1 ? single : multi;
    const int64_t pieces = (len + cap - 1) / cap;
    int64_t step = (len + pieces - 1) / pieces;
    step = (step + V - 1) / V * V;
    for (int64_t p = u.p0; p < u.p1; p += step) out.push_back(Run{p, std::min(p + step, u.p1), u.k0, u.cnt});
  }
}

} // namespace

extern "C" int vae_tile_ramp_blend(const void *const *tiles, const int64_t grid[6],
                                   const int64_t *tile_origins, const int64_t *tile_extents,
                                   const int64_t margin[3], const int64_t ramp[3], int dtype, void *out,
                                   void *stream) {
  if (!grid || !tile_origins || !tile_extents || !margin || !ramp)
    return sb_fail_message(SB_EARG, "null layout pointer");
  const int ndim = (int)grid[0];
  if (ndim != 4 && ndim != 5) return failf(SB_EARG, "ndim must be 4 or 5 (got %lld)", (long long)grid[0]);
  const int64_t N = grid[1], C = grid[2], n_t = grid[3], n_h = grid[4], n_w = grid[5];
  if (N < 0 || C < 0) return sb_fail_message(SB_EARG, "N and C must be >= 0");
  if (n_t != 1) return sb_fail_message(SB_EARG, "frames are not tiled: n_t must be 1");
  if (dtype != SB_F32 && dtype != SB_F16 && dtype != SB_BF16) return failf(SB_EARG, "unknown dtype %d", dtype);
  const int64_t T = tile_extents[0];
  if (tile_origins[0] != 0 || T < 1 || (ndim == 4 && T != 1))
    return sb_fail_message(SB_EARG, "the frame axis needs origin 0 and extent >= 1 (1 when ndim == 4)");
  if (n_h < 1 || n_h > sb::kRampMaxAxisTiles || n_w < 1 || n_w > sb::kRampMaxAxisTiles)
    return failf(SB_EARG, "tiles per axis must be in 1..%d", sb::kRampMaxAxisTiles);
  AxisLayout H, W;
  int rc = read_axis("h", n_h, tile_origins + 1, tile_extents + 1, margin[1], ramp[1], H);
  if (rc) return rc;
  rc = read_axis("w", n_w, tile_origins + 1 + n_h, tile_extents + 1 + n_h, margin[2], ramp[2], W);
  if (rc) return rc;
  std::vector<Run> hr, wr_el;
  if ((rc = element_runs("h", H, hr))) return rc;
  if ((rc = element_runs("w", W, wr_el))) return rc;

  if (N >= ((int64_t)1 << 31) || C >= ((int64_t)1 << 31) || T >= ((int64_t)1 << 31))
    return sb_fail_message(SB_EGEOM, "N, C and frames must be below 2^31");
  const int64_t planes = N * C * T;
  if (planes >= ((int64_t)1 << 31)) return sb_fail_message(SB_EGEOM, "N * C * frames must be below 2^31");
  if (planes > 0 && H.L * W.L > ((int64_t)1 << 50) / planes)
    return sb_fail_message(SB_EGEOM, "output too large (more than 2^50 elements)");
  if (planes == 0) return SB_OK; // nothing to read or write
  const int EB = dtype == SB_F32 ? 4 : 2;
  const int64_t ntiles = n_h * n_w;
  if (!tiles) return sb_fail_message(SB_EARG, "null tiles");
  if (!out) return sb_fail_message(SB_EARG, "null out");
  for (int64_t k = 0; k < ntiles; ++k) {
    if (!tiles[k]) return failf(SB_EARG, "null tile pointer %lld", (long long)k);
    if (!aligned(tiles[k], EB)) return failf(SB_EARG, "tile %lld is not aligned to its element size", (long long)k);
  }
  if (!aligned(out, EB)) return sb_fail_message(SB_EARG, "out is not aligned to its element size");
  {
    const uintptr_t o0 = (uintptr_t)out, o1 = o0 + (uintptr_t)(planes * H.L * W.L * EB);
    for (int64_t i = 0; i < n_h; ++i)
      for (int64_t j = 0; j < n_w; ++j) {
        const uintptr_t t0 = (uintptr_t)tiles[i * n_w + j];
        const uintptr_t t1 = t0 + (uintptr_t)(planes * H.s[i] * W.s[j] * EB);
        if (t0 < o1 && o0 < t1) return failf(SB_EARG, "out overlaps tile (%lld,%lld)", (long long)i, (long long)j);
      }
  }

  // 16-byte vectors along W when every origin, extent and row is a whole
  // number of vectors, every base is 16-byte aligned and every tile a
  // straddling vector takes covers it
  const int64_t V16 = 16 / EB;
  bool vec16 = aligned(out, 16) && W.L % V16 == 0;
  for (int64_t j = 0; j < n_w && vec16; ++j) vec16 = W.o[j] % V16 == 0 && W.s[j] % V16 == 0;
  for (int64_t k = 0; k < ntiles && vec16; ++k) vec16 = aligned(tiles[k], 16);
  std::vector<Run> wr;
  if (vec16) vec16 = vector_runs(W, wr_el, V16, wr);
  const int64_t V = vec16 ? V16 : 1;
  if (!vec16) wr = wr_el;
  // Column chunks on whole 128-byte lines when every tile origin along W is
  // on a line (then a line of the output is a line of every tile too) and
  // every straddling line can take the tiles of both sides: FLUX.1 at 1600 px
  // drops from +6.6% to +2.5% HBM traffic over the algorithmic bytes.  With
  // origins off the line grid, a chunk edge on an output line still splits a
  // tile line, and the union lines add zero-weight reads (2752x1536 layout:
  // +26.8% against +9.6% on 16-byte vectors), so those keep vector chunks.
  int64_t gran = V;
  {
    const int64_t G = 128 / EB;
    bool on_lines = vec16;
    for (int64_t j = 0; j < n_w && on_lines; ++j) on_lines = W.o[j] % G == 0;
    std::vector<Run> lr;
    if (on_lines && line_runs(W, wr_el, G, lr)) {
      wr = lr;
      gran = G;
    }
  }

  std::vector<Run> chunks;
  split_runs(wr, sb::kRampSingleVecs * V, sb::kRampMultiCols, gran, chunks);

  sb::RampArgs A;
  std::memset(&A, 0, sizeof A);
  A.out = out;
  for (int64_t i = 0; i < n_h; ++i) { A.t.oh[i] = (int32_t)H.o[i]; A.t.sh[i] = (int32_t)H.s[i]; }
  for (int64_t j = 0; j < n_w; ++j) { A.t.ow[j] = (int32_t)W.o[j]; A.t.sw[j] = (int32_t)W.s[j]; }
  A.t.n_h = (int32_t)n_h;
  A.t.n_w = (int32_t)n_w;
  A.t.LH = (int32_t)H.L;
  A.t.LW = (int32_t)W.L;
  A.t.mh = (int32_t)H.m;
  A.t.mw = (int32_t)W.m;
  A.t.inv_rh = 1.0f / (float)H.r;
  A.t.inv_rw = 1.0f / (float)W.r;

  // Rows per block: about total / (cus * SB_RAMP_BLOCKS_PER_CU) vectors per
  // block, clamped to [SB_RAMP_PER_BLOCK_MIN, SB_RAMP_PER_BLOCK_MAX], over the
  // average chunk width.
#ifndef SB_RAMP_BLOCKS_PER_CU
#define SB_RAMP_BLOCKS_PER_CU 8
#endif
  // The minimum of 640 vectors, measured against 512 (each launch timed on
  // its own): FLUX.1 1600 px 11.1-11.5 -> 9.8 us (bands of 9 rows instead of
  // 7), the other layouts unchanged (they take the per-CU size, 768 vectors).
#ifndef SB_RAMP_PER_BLOCK_MIN
#define SB_RAMP_PER_BLOCK_MIN 640
#endif
#ifndef SB_RAMP_PER_BLOCK_MAX
#define SB_RAMP_PER_BLOCK_MAX 8192
#endif
  const int64_t total_vec = planes * H.L * (W.L / V);
  const int64_t per_block = std::min<int64_t>(
      SB_RAMP_PER_BLOCK_MAX,
      std::max<int64_t>(SB_RAMP_PER_BLOCK_MIN, total_vec / ((int64_t)sb_cu_count() * SB_RAMP_BLOCKS_PER_CU)));
  const int64_t avg_chunk = std::max<int64_t>(1, (W.L / V) / (int64_t)chunks.size());
  int64_t rows_pb = std::max<int64_t>(1, std::min<int64_t>(1024, per_block / avg_chunk));
  rows_pb = std::max(std::min(rows_pb, H.L), (H.L + 59999) / 60000); // row bands fit grid.z
  A.t.rows_pb = (int32_t)rows_pb;

  bool multi_w = false, multi_h = false;
  int64_t multi_cols = 0;
  for (const Run &u : chunks)
    if (u.cnt > 1) { multi_w = true; multi_cols = std::max(multi_cols, u.p1 - u.p0); }
  for (const Run &u : hr) multi_h = multi_h || u.cnt > 1;
  const size_t lds = (size_t)sb::kRampMaxCover * ((multi_w ? multi_cols : 0) + (multi_h ? rows_pb : 0)) * sizeof(float);
  hipStream_t st = (hipStream_t)stream;

  // Launch windows: consecutive row segments whose tile rows fit the pointer
  // table; column chunks in slices of at most kRampMaxChunks.
  size_t s0 = 0;
  while (s0 < hr.size()) {
    size_t s1 = s0;
    int imin = hr[s0].k0, imax = hr[s0].k0 + hr[s0].cnt;
    int64_t bands = 0;
    while (s1 < hr.size() && (int64_t)(s1 - s0) < sb::kRampMaxSegs) {
      const int a = std::min(imin, hr[s1].k0), b = std::max(imax, hr[s1].k0 + hr[s1].cnt);
      const int64_t nb = (hr[s1].p1 - hr[s1].p0 + rows_pb - 1) / rows_pb;
      if ((int64_t)(b - a) * n_w > sb::kMaxWindowTiles || bands + nb > 65535) break;
      imin = a;
      imax = b;
      bands += nb;
      ++s1;
    }
    if (s1 == s0)
      return failf(SB_EGEOM, "%lld tiles per row: a row segment exceeds one launch window", (long long)n_w);
    A.t.ib = imin;
    for (int k = 0; k < sb::kMaxWindowTiles; ++k) A.ptr[k] = nullptr;
    for (int i = imin; i < imax; ++i)
      for (int64_t j = 0; j < n_w; ++j) A.ptr[(i - imin) * n_w + j] = tiles[i * n_w + j];
    A.t.nseg = (int32_t)(s1 - s0);
    int32_t b0 = 0;
    for (size_t s = s0; s < s1; ++s) {
      A.t.seg[s - s0] = sb::ramp_pack((uint32_t)hr[s].p0, (uint32_t)hr[s].k0, (uint32_t)hr[s].cnt);
      A.t.band0[s - s0] = b0;
      b0 += (int32_t)((hr[s].p1 - hr[s].p0 + rows_pb - 1) / rows_pb);
    }
    A.t.seg[s1 - s0] = sb::ramp_pack((uint32_t)hr[s1 - 1].p1, 0, 1);
    A.t.band0[s1 - s0] = b0;
    for (size_t c0 = 0; c0 < chunks.size(); c0 += sb::kRampMaxChunks) {
      const size_t c1 = std::min(chunks.size(), c0 + (size_t)sb::kRampMaxChunks);
      for (size_t c = c0; c < c1; ++c)
        A.t.chunk[c - c0] = sb::ramp_pack((uint32_t)chunks[c].p0, (uint32_t)chunks[c].k0, (uint32_t)chunks[c].cnt);
      A.t.chunk[c1 - c0] = sb::ramp_pack((uint32_t)chunks[c1 - 1].p1, 0, 1);
      // grid x = planes, in launches of at most kMaxBlocksX (2^32 work-items)
      for (int64_t p0 = 0; p0 < planes; p0 += sb::kMaxBlocksX) {
        A.plane0 = p0;
        const dim3 g((unsigned)std::min<int64_t>(sb::kMaxBlocksX, planes - p0), (unsigned)(c1 - c0),
                     (unsigned)b0);
        hipError_t e = sb_launch_ramp(A, dtype, vec16 ? 1 : 0, g, lds, st);
        if (e != hipSuccess) return failf(SB_ELAUNCH, "ramp blend launch failed: %s", hipGetErrorString(e));
      }
    }
    s0 = s1;
  }
  return SB_OK;
}
