/*
 * seam_blend.h -- C ABI of the MI355X (gfx950) tiled-VAE decode-assembly library.
 *
 * Two operations, each behind one entry point:
 *
 *  vae_tile_blend_stitch  -- crossfade overlapping decoded tiles along rows
 *      (blend_v), columns (blend_h) and frames (blend_t), crop every tile to the
 *      row limit and stitch the result into one output, written once.
 *      Defined by: diffusers issue "[Proposal] Vectorize tiled VAE blending
 *      while preserving rounding and CUDA graph replay", section "Proposed
 *      scope" (blend_v / blend_h / blend_t; extent clamping from diffusers
 *      #2660; in-place output; per-product rounding; coefficients from float64
 *      division).
 *
 *  patch_groupnorm -- GroupNorm of a tensor viewed as spatial patches: per-patch
 *      (count, mean, M2) statistics merged with Chan's formula so that the
 *      result equals unsplit GroupNorm (global mean, variance divided by the
 *      count).  Defined by: DistVAE PR "Add tiled VAE parallelism & extended
 *      model support", the PatchGroupNorm commits and the Patchify commit
 *      (first patches one band longer).
 *
 * Conventions shared by every entry point
 *  - Pointers named "device" are HIP device pointers (any device memory the
 *    current device can read/write); everything else is host memory read
 *    during the call only.  The caller owns and allocates every buffer.  The
 *    library allocates no device memory, never synchronises the stream and
 *    keeps no state other than a thread-local error message.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream),
 *    on the device that is current when the call is made.  Results are ready
 *    when the stream reaches that point.
 *  - Return value: 0 on success, or a negative SB_E* code; the message is then
 *    available from seamblend_last_error().  Argument and geometry errors are
 *    detected on the host before anything is enqueued.  Faults during
 *    execution surface asynchronously on the stream, as for any HIP kernel.
 *  - Tensors are dense, contiguous, row-major (last index fastest).
 */
#ifndef SEAM_BLEND_H
#define SEAM_BLEND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage dtype of every tile / tensor in one call */
typedef enum { SB_F32 = 0, SB_F16 = 1, SB_BF16 = 2 } sb_dtype;

/* return codes */
#define SB_OK 0
#define SB_EARG (-1)       /* bad argument: null pointer, unknown dtype, bad rank ... */
#define SB_EGEOM (-2)      /* geometry outside what the data-parallel kernel supports */
#define SB_EWORKSPACE (-3) /* workspace smaller than patch_groupnorm_workspace_bytes() */
#define SB_ELAUNCH (-4)    /* the HIP runtime rejected a launch (message from hipGetErrorString) */

/*
 * Output extents of vae_tile_blend_stitch for a tile grid, after the same
 * validation the entry point performs (host only, no device work).
 *   grid[6]        {ndim (4 or 5), N, C, n_t, n_h, n_w}; n_t must be 1 when ndim == 4.
 *   tile_extents   n_t + n_h + n_w entries: t_0..t_{n_t-1}, h_0.., w_0..
 *                  (t_0 must be 1 when ndim == 4).
 *   blend_extent   {E_t, E_h, E_w} >= 0; E_t is ignored when ndim == 4.
 *   row_limit      {R_t, R_h, R_w} >= 1: stride between tile origins along
 *                  each axis, and the crop of every tile but the last.
 *   out_extents    receives {L_t, L_h, L_w}, L = (n - 1) * R + (last extent).
 * Geometry preconditions (else SB_EGEOM): every non-last tile is >= R long;
 * with e(k) = min(E, ext(k-1), ext(k)) the blend extent between tiles k-1 and
 * k (e(0) = 0), every tile satisfies ext(k) >= e(k) + e(k+1), so a tile's head
 * seam and tail never overlap; at most 64 tiles per axis; output planes and
 * tiles below 2^31 elements per (n, c) plane.
 */
int vae_tile_blend_stitch_output_extents(const int64_t grid[6], const int64_t *tile_extents,
                                         const int64_t blend_extent[3],
                                         const int64_t row_limit[3], int64_t out_extents[3]);

/*
 * Blend + crop + stitch of a tile grid into `out`.
 *   tiles        host array of n_t*n_h*n_w device pointers in raster order
 *                (tau, i, j): tile (tau, i, j) is a contiguous
 *                [N, C, t_tau, h_i, w_j] array (ndim 5) or [N, C, h_i, w_j]
 *                (ndim 4) of `dtype`.  Tiles are only read.
 *   grid, tile_extents, blend_extent, row_limit: as above.
 *   dtype        SB_F32, SB_F16 or SB_BF16 (tiles and output alike).
 *   out          device pointer to a contiguous [N, C, L_t, L_h, L_w] (ndim 5)
 *                or [N, C, L_h, L_w] (ndim 4) array of `dtype`; must not
 *                overlap any tile (checked, SB_EARG).
 *   stream       hipStream_t or NULL.
 * Result: for each temporal tile, tiles are blended in raster order, row seam
 * (with the tile above, as already blended) before column seam (with the tile
 * to the left, as already blended), each seam element
 *   RN_T( RN_T(a * w_a[k]) + RN_T(b * w_b[k]) ),  w_b[k] = fp32(k/e),
 *   w_a[k] = fp32(1 - k/e) from double, products and sum in fp32 without
 *   fusion;
 * every tile is cropped to R except the last along each axis; then each
 * stitched temporal chunk is blended with the previous stitched chunk (as
 * already blended) along frames and cropped.  Bit-exact for every dtype.
 * Each output element is written exactly once; no scratch memory.
 * N*C == 0 is a no-op that accepts null tile and output pointers.
 * Limits (SB_EGEOM beyond them, before any launch): clamped blend extents up
 * to 4096; a launch window takes at most 192 tile pointers, a window's tile
 * rows with the row above and its temporal tiles with the one before, so up
 * to 48 tile columns always fit and more may be refused when there are several
 * tile rows or temporal tiles; when every W seam and crop is narrower than 16
 * vectors (the narrow-seam layout) a launch window of more than 2^24 - 1
 * output frames is refused; otherwise any frame count is taken, in several
 * launches.
 */
int vae_tile_blend_stitch(const void *const *tiles, const int64_t grid[6],
                          const int64_t *tile_extents, const int64_t blend_extent[3],
                          const int64_t row_limit[3], int dtype, void *out, void *stream);

/*
 * Device workspace (bytes) patch_groupnorm needs for this problem; 0 with an
 * error message for invalid arguments.  shape: ndim entries {N, C, spatial..}.
 */
size_t patch_groupnorm_workspace_bytes(int ndim, const int64_t *shape, int64_t groups,
                                       int split_axis, int64_t n_patches);

/*
 * GroupNorm of x viewed as n_patches patches along split_axis.
 *   x            device pointer, contiguous [N, C, spatial...] of dtype, ndim 3..5.
 *   shape        host array of ndim extents; C % groups == 0; N*C < 2^31,
 *                each group (C/G * spatial elements) < 2^31 elements and the
 *                tensor < 2^56 bytes (else SB_EGEOM).
 *   split_axis   2 <= split_axis < ndim: the spatial axis the patches cut.
 *   n_patches    1..64.  Patch p covers [s_p, s_p + len_p) along split_axis
 *                with the first (L mod P) patches one longer (empty patches
 *                allowed when P > L).
 *   eps          added to the variance (fp32), >= 0.
 *   gamma, beta  device pointers to [C] of dtype, or NULL (1 and 0).
 *   out          device pointer like x; may be x itself (in place).
 *   workspace    device scratch of at least patch_groupnorm_workspace_bytes(),
 *                16-byte aligned; caller-owned, contents need not be initialised.
 *   patch_stats  optional device pointer to N*G*P*3 floats, or NULL: receives
 *                per-patch (count, mean, M2), M2 = sum of squared deviations
 *                about the patch mean, merged in fp32 over that patch's chunks;
 *                (0, 0, 0) for an empty patch.
 *   stream       hipStream_t or NULL.
 * Result: per (n, g), mean and M2 over the C/G channels and all spatial
 * positions, obtained by merging fp32 partial statistics in a fixed order:
 * count, mean = sum n_k mean_k / count, M2 = sum (M2_k + n_k (mean_k -
 * mean)^2) over the partials (Chan's merge taken over many sets at once);
 * var = M2 / count; rstd = 1/sqrt(var+eps);
 * y = (x - mean) * rstd * gamma_c + beta_c in fp32, rounded once to dtype.
 * Each thread folds its values into (count, mean, M2) a batch at a time: the
 * batch's mean and squared deviations by two passes, then a Chan merge
 * (Welford's update), so M2 is never a difference of power sums.  Statistics
 * are taken about a shift K_g (the median of five of the group's elements,
 * spread over it), so the mean is carried as K_g + m and x - mean is formed as
 * (x - K_g) - m: inputs whose mean is large against their spread keep full
 * fp32 accuracy, and up to two outlying samples never become the shift.
 * Deterministic: the same inputs give the same bits on every call.
 */
int patch_groupnorm(const void *x, int ndim, const int64_t *shape, int64_t groups,
                    int split_axis, int64_t n_patches, float eps, const void *gamma,
                    const void *beta, int dtype, void *out, void *workspace,
                    size_t workspace_bytes, float *patch_stats, void *stream);

/*
 * patch_groupnorm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results, with the statistics partials in
 * a static scratch array the library holds on each GPU instead of a
 * caller-given workspace.  The caller still passes x, out (and gamma, beta,
 * patch_stats).  Allocates nothing and calls no allocating routine; its first
 * call on a device looks the array's device address up once.
 *   Limit: problems whose partials exceed SB_GN_STATIC_SCRATCH_BYTES
 *   (patch_groupnorm_workspace_bytes() > 1 MiB, i.e. N*groups*patches*chunks
 *   above 65536) return SB_EWORKSPACE before anything is enqueued.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (for example on two streams) race and must be ordered by the caller.
 * Arguments, layout and errors otherwise as patch_groupnorm.
 */
#define SB_GN_STATIC_SCRATCH_BYTES (1u << 20)
int patch_groupnorm_noalloc(const void *x, int ndim, const int64_t *shape, int64_t groups,
                            int split_axis, int64_t n_patches, float eps, const void *gamma,
                            const void *beta, int dtype, void *out, float *patch_stats,
                            void *stream);

/*
 * Normalised-ramp blend of wide tiles (unsloth Studio PR "size seam-free VAE
 * tiles from measured peaks", the Qwen-Image-2.1 wide-tile commit, which
 * the later commits extend to every image VAE and to the tiled encode).
 * A tile has no weight within `margin` positions of an edge it shares with
 * another tile (an edge inside the canvas) and ramps linearly to full weight
 * over the next `ramp`: at whole distance d from such an edge the factor is
 * clamp((d - margin) / ramp, 0, 1); a tile's weight along an axis is the
 * product of its two edges' factors and its 2-D weight the product of its
 * axes'.  Weights are normalised to 1 at every position; the sum of weight
 * times value is accumulated in fp32 and rounded once to the storage type.
 *   tiles:        n_h * n_w device pointers, raster order (i, j); tile (i, j) is a
 *                 contiguous [N, C, (T,) h_i, w_j] array of dtype (frames are not tiled).
 *   grid:         {ndim (4 | 5), N, C, 1, n_h, n_w}, n_h and n_w in 1..48.
 *   tile_origins: 1 + n_h + n_w positions: 0 (frames), then the row origins, then the
 *                 column origins; each axis starts at 0 and increases.
 *   tile_extents: 1 + n_h + n_w extents: T (1 when ndim == 4), then h_i, then w_j.  The
 *                 canvas along an axis ends where its last tile ends (< 2^20).
 *   margin, ramp: per axis (t, h, w) in positions; [0] is ignored; margin >= 0, ramp >= 1.
 *   out:          contiguous [N, C, (T,) L_h, L_w] of dtype; must not overlap a tile.
 * Every position needs a tile with weight (overlaps wider than twice the margin),
 * and at most 4 tiles may carry weight at one position of an axis: else SB_EGEOM.
 * Enqueued on `stream`; allocates nothing; N * C == 0 is a no-op.
 */
int vae_tile_ramp_blend(const void *const *tiles, const int64_t grid[6], const int64_t *tile_origins,
                        const int64_t *tile_extents, const int64_t margin[3], const int64_t ramp[3],
                        int dtype, void *out, void *stream);

/*
 * Tile layout along one axis of a canvas of L latents (host only): writes the
 * origin and extent of each tile and their count.  Defined by the unsloth
 * Studio PR "size seam-free VAE tiles from measured peaks", sections "Problem"
 * and "Change" and its commit log (stock tiles with edge slivers; 32-latent
 * tiles with at least 16-latent overlaps spread evenly so the last ends at the
 * edge at full size; a canvas within one tile is one tile; at a sliver, the
 * fewest decoder calls, then the widest tile, decoding no more latents per
 * side than the stock loop; the earlier fewest tiles of the smallest side).
 *   rule / params:
 *     SB_LAYOUT_STOCK          {T, S}: a tile of T at every multiple of S below L,
 *                              the last cut short by the edge.
 *     SB_LAYOUT_EDGE_ALIGNED   {t, ov}: the fewest tiles of side t whose neighbours
 *                              overlap by >= ov, origin_k = floor(k (L - t) / (n - 1));
 *                              one tile of L when L <= t (whatever ov: a single tile
 *                              has no neighbour); otherwise ov < t (SB_EARG).
 *     SB_LAYOUT_FEWEST_CALLS   {T, S, ov, M}: the fewest tiles, then the widest side
 *                              t <= M, with n * t <= B, the latents the stock (T, S) loop
 *                              decodes along the axis, and overlaps >= ov; spread evenly.
 *                              Up to rounding: when no whole side fits B but the exact
 *                              covering does (L + (n - 1) ov <= B), the smallest covering
 *                              side is taken.
 *     SB_LAYOUT_SMALLEST_SIDE  {ov, M}: the fewest tiles of side <= M covering with
 *                              overlaps >= ov, then the smallest such side; spread evenly.
 *     SB_LAYOUT_AUTO           {T, S, floor_tile, floor_overlap}: the stock tiles when
 *                              every one is >= floor_tile and every overlap >=
 *                              floor_overlap, else EDGE_ALIGNED with
 *                              t = max(floor_tile, T), ov = max(floor_overlap, T - S).
 *   max_tiles: capacity of origins[] and extents[] (SB_EARG if exceeded).
 * Returns 0, SB_EARG for bad parameters, SB_EGEOM if no layout satisfies the rule.
 */
typedef enum {
  SB_LAYOUT_STOCK = 0,
  SB_LAYOUT_EDGE_ALIGNED = 1,
  SB_LAYOUT_FEWEST_CALLS = 2,
  SB_LAYOUT_SMALLEST_SIDE = 3,
  SB_LAYOUT_AUTO = 4
} sb_layout_rule;

int vae_tile_layout(int64_t L, int rule, const int64_t params[4], int64_t max_tiles,
                    int64_t *origins, int64_t *extents, int64_t *n_tiles);

/* Thread-local message describing the last non-zero return on this thread. */
const char *seamblend_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SEAM_BLEND_H */
