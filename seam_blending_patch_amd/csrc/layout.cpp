// layout.cpp -- tile layouts along one axis (host only): where the tiles of a
// tiled decode start and how long each is, in latents.
//
// Rules (unsloth Studio PR "size seam-free VAE tiles from measured peaks",
// sections "Problem" and "Change" and its commit log):
//  * stock: a tile of T at every multiple of the stride S below the canvas,
//    the last one cut short by the edge (the "edge sliver");
//  * edge-aligned wide tiles: tiles of side t, neighbours overlapping by at
//    least ov, spread evenly so the last tile ends at the canvas edge at full
//    size; a canvas within one tile is one tile;
//  * fewest calls: the fewest tiles, then the widest side (capped at M), among
//    layouts that decode no more latents along the axis than the stock loop;
//  * smallest side: the fewest tiles of side at most M, then the smallest side
//    that still covers with the overlap (the earlier sliver rule);
//  * auto: keep the stock tiles when every tile is at least the floor tile and
//    every overlap at least the floor overlap, otherwise edge-aligned tiles of
//    max(floor, T) with overlap max(floor overlap, T - S).
// "Spread evenly" is read as origin_k = floor(k (L - t) / (n - 1)).

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "../../include/seam_blend.h"

extern "C" int sb_fail_message(int code, const char *msg); // abi.cpp

namespace {

// lengths, tiles, strides and overlaps are at most 2^30 positions: every sum
// and product below stays far inside 64 bits, and a stride of 1 over the
// longest canvas is 2^30 tiles, which max_tiles bounds before any loop runs
constexpr int64_t kMaxLength = (int64_t)1 << 30;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// evenly spread n tiles of side t over [0, L); requires n >= 1, t <= L
int spread(int64_t L, int64_t t, int64_t n, int64_t max_tiles, int64_t *o, int64_t *e) {
  if (n > max_tiles) return sb_fail_message(SB_EARG, "layout needs more tiles than max_tiles");
  for (int64_t k = 0; k < n; ++k) {
    o[k] = n == 1 ? 0 : (k * (L - t)) / (n - 1);
    e[k] = t;
  }
  return (int)n;
}

// fewest tiles of side t covering L with every overlap >= ov
int64_t tiles_needed(int64_t L, int64_t t, int64_t ov) {
  if (L <= t) return 1;
  return ceil_div(L - t, t - ov) + 1;
}

int stock(int64_t L, int64_t T, int64_t S, int64_t max_tiles, int64_t *o, int64_t *e) {
  const int64_t n = ceil_div(L, S);
  if (n > max_tiles) return sb_fail_message(SB_EARG, "layout needs more tiles than max_tiles");
  for (int64_t k = 0; k < n; ++k) {
    o[k] = k * S;
    e[k] = (T < L - k * S) ? T : L - k * S;
  }
  return (int)n;
}

} // namespace

extern "C" int vae_tile_layout(int64_t L, int rule, const int64_t params[4], int64_t max_tiles,
                               int64_t *origins, int64_t *extents, int64_t *n_tiles) {
  if (!params || !origins || !extents || !n_tiles) return sb_fail_message(SB_EARG, "null pointer");
  if (L < 1 || L > kMaxLength) return sb_fail_message(SB_EARG, "canvas length must be in 1..2^30");
  if (max_tiles < 1) return sb_fail_message(SB_EARG, "max_tiles must be >= 1");
  for (int k = 0; k < 4; ++k)
    if (params[k] < 0 || params[k] > kMaxLength)
      return sb_fail_message(SB_EARG, "layout parameters must be in 0..2^30");
  int rc = -1;
  switch (rule) {
    case SB_LAYOUT_STOCK: {
      const int64_t T = params[0], S = params[1];
      if (T < 1 || S < 1 || S > T) return sb_fail_message(SB_EARG, "need 1 <= stride <= tile");
      rc = stock(L, T, S, max_tiles, origins, extents);
      break;
    }
    case SB_LAYOUT_EDGE_ALIGNED: {
      const int64_t t = params[0], ov = params[1];
      if (t < 1 || ov < 0) return sb_fail_message(SB_EARG, "need tile >= 1 and overlap >= 0");
      if (L <= t) {
        // one tile covers the canvas: there is no neighbour to overlap
        origins[0] = 0;
        extents[0] = L;
        rc = 1;
      } else if (ov >= t) {
        return sb_fail_message(SB_EARG, "overlap must be below the tile when several tiles are needed");
      } else {
        rc = spread(L, t, tiles_needed(L, t, ov), max_tiles, origins, extents);
      }
      break;
    }
    case SB_LAYOUT_FEWEST_CALLS: {
      const int64_t T = params[0], S = params[1], ov = params[2], M = params[3];
      if (T < 1 || S < 1 || S > T || ov < 0 || M < 1) return sb_fail_message(SB_EARG, "bad fewest-calls parameters");
      // latents the stock loop decodes along the axis: n_s tiles, the full
      // ones of T and the rest cut short by the edge
      const int64_t n_s = ceil_div(L, S);
      const int64_t n_full = std::min(n_s, L >= T ? (L - T) / S + 1 : 0);
      const int64_t m = n_s - n_full; // the cut tiles k = n_full .. n_s - 1 have extents L - kS
      const int64_t budget = n_full * T + m * L - S * ((n_full + n_s - 1) * m / 2);
      if (L <= M) { // one call over the whole canvas (the stock loop decodes >= L)
        origins[0] = 0;
        extents[0] = L;
        rc = 1;
        break;
      }
      // n tiles of side t cover L with overlaps >= ov iff n t - (n - 1) ov >= L;
      // the widest side within the budget is min(M, budget / n); when even the
      // smallest covering side exceeds it, that side is still taken if the
      // exact fractional covering (L + (n - 1) ov latents) fits the budget
      // The fewest tiles of side <= M that cover: t_cov <= M iff n >= (L - ov) / (M - ov).
      // From there, n tiles decode at least L + (n - 1) ov latents, which only
      // grows with n: once that exceeds the budget, no larger n fits either.
      if (M > ov && L > ov) {
        for (int64_t n = std::max<int64_t>(2, ceil_div(L - ov, M - ov)); n <= L; ++n) {
          if (L + (n - 1) * ov > budget) break;
          const int64_t t_cov = ceil_div(L + (n - 1) * ov, n);
          if (t_cov > M || t_cov <= ov) continue;
          int64_t t = budget / n;
          if (t > M) t = M;
          if (t > L) t = L;
          if (t < t_cov) t = t_cov; // up to rounding: the exact covering fits the budget
          rc = spread(L, t, n, max_tiles, origins, extents);
          if (rc < 0) return rc; // more tiles than max_tiles
          break;
        }
      }
      if (rc < 0) return sb_fail_message(SB_EGEOM, "no layout decodes within the stock budget");
      break;
    }
    case SB_LAYOUT_SMALLEST_SIDE: {
      const int64_t ov = params[0], M = params[1];
      if (ov < 0 || M < 1 || (M <= ov && M < L)) return sb_fail_message(SB_EARG, "bad smallest-side parameters");
      if (L <= M) {
        origins[0] = 0;
        extents[0] = L;
        rc = 1;
        break;
      }
      const int64_t n = tiles_needed(L, M, ov);
      const int64_t t = ceil_div(L + (n - 1) * ov, n); // smallest side covering with n tiles
      rc = spread(L, t, n, max_tiles, origins, extents);
      break;
    }
    case SB_LAYOUT_AUTO: {
      const int64_t T = params[0], S = params[1], ft = params[2], fov = params[3];
      if (T < 1 || S < 1 || S > T || ft < 1 || fov < 0) return sb_fail_message(SB_EARG, "bad auto parameters");
      // Stock tile k has extent min(T, L - kS) and overlaps the next by
      // min(T, L - kS) - S: both shrink with k, so the last tile and the last
      // overlap are the smallest.  A single stock tile covers the canvas.
      const int64_t n = ceil_div(L, S);
      const bool keep = n == 1 || (L - (n - 1) * S >= ft && std::min(T, L - (n - 2) * S) - S >= fov);
      if (keep) {
        rc = stock(L, T, S, max_tiles, origins, extents);
      } else {
        const int64_t t = T > ft ? T : ft;
        const int64_t ov = (T - S) > fov ? (T - S) : fov;
        if (L <= t) {
          origins[0] = 0;
          extents[0] = L;
          rc = 1;
        } else if (ov >= t) {
          return sb_fail_message(SB_EARG, "floor overlap must be below the tile when several tiles are needed");
        } else {
          rc = spread(L, t, tiles_needed(L, t, ov), max_tiles, origins, extents);
        }
      }
      break;
    }
    default:
      return sb_fail_message(SB_EARG, "unknown layout rule");
  }
  if (rc < 0) return rc;
  *n_tiles = rc;
  return SB_OK;
}
