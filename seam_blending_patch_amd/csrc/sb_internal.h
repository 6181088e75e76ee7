// sb_internal.h -- shared between the host entry points and the gfx950 kernels.
// Not part of the public ABI (that is include/seam_blend.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sb {

// ---------------------------------------------------------------------------
// Division by a run-time invariant divisor with one high multiply and a shift
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, round-up variant).  For 1 <= d < 2^31 pick
// s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1; then for every
// 0 <= n < 2^31:  n / d == (umulhi(n, m) + n) >> s   (the sum fits 32 bits).
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// ---------------------------------------------------------------------------
// blend + crop + stitch launch arguments (passed by value as kernel arguments)
// ---------------------------------------------------------------------------
constexpr int kMaxAxisTiles = 64;    // tiles per axis
constexpr int kMaxWindowTiles = 192; // tile pointers per launch window
constexpr int kMaxBlend = 4096;      // largest clamped blend extent (the coefficient formula is checked up to it)
// largest grid x of the blend and ramp launches: 2^32 work-items in x at up to
// 256 threads per block
constexpr int64_t kMaxBlocksX = ((int64_t)1 << 24) - 1;
constexpr int64_t kMaxBlocksYZ = 65535; // largest grid extent in y and z

struct BlendArgs {
  void *out;
  const void *ptr[kMaxWindowTiles]; // window tiles [(tau - taub)][(i - ib)][j]
  int32_t ext[3][kMaxAxisTiles];    // extents per axis (t, h, w), global tile index
  float rcp[3][kMaxAxisTiles];      // fp32(1/e) of the seam between tiles k-1 and k per axis (0: no seam)
  int32_t n_t, n_h, n_w;
  int32_t E[3], R[3];
  int32_t LT, LH, LW;               // full output extents
  int32_t taub, ib, ptr_nh;         // pointer-table origin and tile rows in it
  int32_t F0, nF, Y0, nY;           // output frame / row range of this window
  int32_t plane0;                   // first (n, c) plane of this launch
  int32_t rows_per_block;           // output rows per block
  int32_t span_k;                   // span layout: tile columns per span (0: segment layout)
  int32_t off32;                    // every tile and output offset a block forms is below 2^31 bytes
  int32_t nt_store;                 // output stores with nontemporal hints (calls moving < 128 MB)
  int32_t g_seg, g_band, g_pf;      // segment kernel grid: W segments, row bands, (plane, frame) pairs
  FastDiv div_nF, div_Rt, div_Rh, div_Rw;
};

constexpr int kMaxSpanCols = 32; // tile columns per span (span layout)

// A pointer into global memory, typed so: loads through it are global loads,
// also when the pointer itself was read from LDS or came out of an asm
// statement (a generic pointer there would make them flat loads).
typedef const __attribute__((address_space(1))) char *GPtr;

// One tile column of a span (span layout), for one run of rows: the tiles the
// closed form reads, each offset so that operand (y, x) of the column is at
// base + y * pitch + x * elem_bytes, and the column seam; built per run in LDS.
struct SpanCol {
  GPtr m, u, l, c;               // tiles (i,j), (i-1,j), (i,j-1), (i-1,j-1) of chunk tau
  GPtr pm, pu, pl, pc;           // the same in chunk tau-1
  int64_t pitch_j, pitch_p;      // bytes per row of tile column j and j-1
  int32_t xbase, ews;            // first output column of the column's crop; its seam width
  int32_t ew;                    // the column seam's blend extent (0: none)
  float rw;                      // fp32(1/ew)
};

// ---------------------------------------------------------------------------
// GroupNorm launch arguments
// ---------------------------------------------------------------------------
constexpr int kMaxPatches = 64;
// Waves of a pass-1 block (per-patch layout): 8, measured against 4 in full
// steps (video activation 6.84-7.00 -> 6.64 us, 512x512 one 12.7 -> 12.4 us)
// and against 2 and 1 before the merge was a sum tree.
#ifndef SB_GN_STATS_WAVES
#define SB_GN_STATS_WAVES 8
#endif
constexpr int kStatsWaves = SB_GN_STATS_WAVES;
#ifndef SB_GN_NORM_UNROLL
#define SB_GN_NORM_UNROLL 4
#endif
constexpr int kNormUnroll = SB_GN_NORM_UNROLL; // vectors per thread in the normalise pass
constexpr int kNormThreads = 256;             // threads per normalise block

struct GNArgs {
  const void *x;
  void *out;
  const void *gamma;
  const void *beta;
  float *part;        // partials [N][G][P][CPP][4]: count (uint32 bits), mean of x - K_g, M2, K_g
  float *patch_stats; // optional [N][G][P][3]
  int32_t N, C, G, Cg;
  int64_t S;          // spatial elements per channel
  int32_t P, CPP, log2CPP;  // patches; pass-1 chunks (and partials) per patch, a power of two
  int32_t L;          // extent of the split axis
  int64_t inner;      // elements per step along the split axis
  int64_t mid;        // product of the spatial extents before the split axis
  int32_t len_big, len_small, n_big; // patch lengths along the split axis
  float eps;
  // pass 2
  int32_t chunks2;    // blocks per (n, c) plane
  int64_t per2;       // vectors per pass-2 block
  FastDiv div_C, div_Cg; // plane -> (n, c) and channel -> group
  FastDiv div_P, div_G;  // pass-1 block -> (n, group, patch)
  int32_t rows_layout; // pass 1 reads whole rows (patches cut the innermost axis)
  uint32_t plane0;    // first (n, c) plane of this pass-2 launch
};

constexpr int64_t kMaxGridY = 65535; // largest grid extent in y (pass-2 planes per launch)

// ---------------------------------------------------------------------------
// normalised-ramp blend launch arguments
// ---------------------------------------------------------------------------
constexpr int kRampMaxAxisTiles = 48; // tiles per axis
constexpr int kRampMaxCover = 4;      // tiles with weight at one position of an axis
constexpr int kRampMaxChunks = 128;   // column chunks per launch
constexpr int kRampMaxSegs = 32;      // row segments per launch
constexpr int kRampMultiCols = 512;   // widest column chunk with several tiles (LDS weights)
constexpr int kRampSingleVecs = 256;  // widest single-tile column chunk, in vectors
constexpr int kRampPosBits = 20;      // positions along an axis < 2^20

// A column chunk or row segment packs its first position (20 bits), its first
// tile (6 bits) and its tile count minus one (2 bits); every tile from the
// first to the last has weight somewhere in it and no other tile has any.
__host__ __device__ constexpr uint32_t ramp_pack(uint32_t p0, uint32_t k0, uint32_t cnt) {
  return p0 | (k0 << kRampPosBits) | ((cnt - 1) << 26);
}

// The tables a block decodes its work from; each block copies them to LDS
// with one cooperative load and does its lookups there.
struct alignas(16) RampTables {
  int32_t oh[kRampMaxAxisTiles], sh[kRampMaxAxisTiles]; // H origins and extents
  int32_t ow[kRampMaxAxisTiles], sw[kRampMaxAxisTiles]; // W origins and extents
  uint32_t chunk[kRampMaxChunks + 1];    // packed column chunks; the entry after the last holds its end
  uint32_t seg[kRampMaxSegs + 1];        // packed row segments; the entry after the last holds its end
  int32_t band0[kRampMaxSegs + 1];       // first row band of each segment (prefix sums)
  int32_t nseg, ib, n_h, n_w;
  int32_t LH, LW, rows_pb;
  int32_t mh, mw;                        // margins
  float inv_rh, inv_rw;                  // 1 / ramp
};
static_assert(sizeof(RampTables) % 16 == 0, "copied in 16-byte pieces");
static_assert(sizeof(RampTables) <= 16 * 256, "copied by one block in one pass");

struct RampArgs {
  RampTables t;
  void *out;
  int64_t plane0;                        // first (n, c, frame) plane of this launch
  const void *ptr[kMaxWindowTiles];      // tiles of rows [ib, ib + rows): ptr[(i - ib) * n_w + j]
};

} // namespace sb

// launchers (defined in the .hip files)
hipError_t sb_launch_blend(const sb::BlendArgs &a, int dtype, int vec16, dim3 grid, size_t lds,
                           hipStream_t st);
hipError_t sb_launch_blend_span(const sb::BlendArgs &a, int dtype, int vec16, dim3 grid, size_t lds,
                                hipStream_t st);
hipError_t sb_launch_groupnorm(const sb::GNArgs &a, int dtype, int vec16, hipStream_t st);
// the current device's address of the static GroupNorm statistics scratch
// (SB_GN_STATIC_SCRATCH_BYTES), looked up once per device
hipError_t sb_groupnorm_static_scratch(void **ptr);
hipError_t sb_launch_ramp(const sb::RampArgs &a, int dtype, int vec16, dim3 grid, size_t lds,
                          hipStream_t st);
