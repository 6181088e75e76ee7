/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for tiled-VAE decode
 * assembly (blend + crop + stitch) and for patch-split GroupNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or table with the HIP library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (-ffp-contract=off matters: every product and every sum below is its own
 * IEEE binary32 round-to-nearest-even operation, never a fused multiply-add).
 *
 * Sources (cited by page title and section):
 *  [P1] diffusers issue "[Proposal] Vectorize tiled VAE blending while
 *       preserving rounding and CUDA graph replay", section "Proposed scope":
 *       blend_v / blend_h / blend_t crossfade overlapping tiles in place, keep
 *       the extent clamping (diffusers #2660), keep per-product rounding, and
 *       build the coefficients with float64 division.
 *  [P3] DistVAE PR "Add tiled VAE parallelism & extended model support",
 *       the PatchGroupNorm commit: the split norm must equal nn.GroupNorm --
 *       global mean, variance divided by the count (no Bessel correction) --
 *       and the later commit that keeps the squared deviations about the
 *       global mean as their own reduction; the Patchify commit: bands are
 *       cut with the first ranks one band longer.
 *
 * Blend arithmetic (one element of one seam, storage type T):
 *   w_b = fp32( (double)k / e ),  w_a = fp32( 1.0 - (double)k / e )
 *   out = RN_T( RN_T(a * w_a) + RN_T(b * w_b) )      -- every * and + in fp32
 * where RN_T rounds fp32 to T to nearest even (identity for fp32).
 *
 * The blend+stitch oracle is the literal sequential algorithm: for each
 * temporal tile, walk the spatial tiles in raster order, blend the tile above
 * into the current one along H (as already modified), then the tile to the
 * left along W, all in place; crop every tile but the last along each axis to
 * the row limit and place it at k*R; then blend the previous stitched chunk
 * (as already modified) into the current one along T, crop, and place.
 * The blend extent along an axis is clamped to both tiles' extents.
 *
 * The normalised-ramp oracle ([P2], unsloth Studio PR "size seam-free VAE
 * tiles from measured peaks", the Qwen-Image-2.1 wide-tile commit) sums, in
 * double and one tile after another, each tile's value times its weight
 * divided by the sum of all tiles' weights at that position.
 *
 * The GroupNorm oracle is the plain definition of unsplit GroupNorm in
 * double: per (n, group) the mean over C/G channels and all spatial
 * positions, the variance as the mean squared deviation about that mean, and
 * y = (x - mean) / sqrt(var + eps) * gamma_c + beta_c.  Separately it emits
 * per-patch (count, mean, M2) and their Chan merge, both in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2

/* ------------------------------------------------------------------------ */
/* storage conversions, written from the IEEE 754 binary16 and bfloat16       */
/* definitions (round to nearest, ties to even; subnormals kept)             */
/* ------------------------------------------------------------------------ */
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t ex = (h >> 10) & 0x1Fu;
    uint32_t man = h & 0x3FFu;
    if (ex == 0x1F) /* inf / nan */
        return bits_f32(sign | 0x7F800000u | (man << 13));
    if (ex == 0) {
        /* zero or subnormal: value = man * 2^-24, exact in binary32 */
        float v = (float)man * (1.0f / 16777216.0f);
        return sign ? -v : v;
    }
    return bits_f32(sign | ((ex - 15 + 127) << 23) | (man << 13));
}

uint16_t oracle_f32_to_f16(float f)
{
    uint32_t x = f32_bits(f);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) {
        if (ax == 0x7F800000u) return sign | 0x7C00u;                     /* inf */
        return (uint16_t)(sign | 0x7E00u | ((ax >> 13) & 0x3FFu));       /* quiet nan */
    }
    if (ax < 0x00800000u) return sign; /* binary32 subnormal: below 2^-126, rounds to 0 */
    int ex = (int)(ax >> 23) - 127;            /* unbiased exponent */
    uint32_t sig = (ax & 0x7FFFFFu) | 0x800000u; /* value = sig * 2^(ex-23) */
    if (ex > 15) return sign | 0x7C00u;          /* >= 2^16: overflow */
    if (ex < -25) return sign;                   /* < 2^-25 = half the least subnormal */
    /* quantum of binary16 at this magnitude: 2^(ex-10) when normal, 2^-24 below 2^-14 */
    int drop = (ex >= -14) ? 13 : 13 + (-14 - ex);
    uint32_t q = sig >> drop;
    uint32_t rem = sig & ((1u << drop) - 1u);
    uint32_t half = 1u << (drop - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    if (ex >= -14) {
        uint32_t e16 = (uint32_t)(ex + 15);
        if (q == 0x800u) { q = 0x400u; e16++; }
        if (e16 >= 31) return sign | 0x7C00u;
        return (uint16_t)(sign | (e16 << 10) | (q & 0x3FFu));
    }
    /* subnormal: value = q * 2^-24 ; q == 0x400 is the least normal, same encoding */
    return (uint16_t)(sign | q);
}

float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t x = f32_bits(f);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u); /* quiet nan */
    uint32_t lsb = (x >> 16) & 1u;
    x += 0x7FFFu + lsb;
    return (uint16_t)(x >> 16);
}

/* RN_T: round an fp32 value to storage type T and widen it back (exact) */
static float round_T(float v, int dtype)
{
    if (dtype == OR_F16) return oracle_f16_to_f32(oracle_f32_to_f16(v));
    if (dtype == OR_BF16) return oracle_bf16_to_f32(oracle_f32_to_bf16(v));
    return v;
}

static float load_T(const void *p, int64_t idx, int dtype)
{
    if (dtype == OR_F16) return oracle_f16_to_f32(((const uint16_t *)p)[idx]);
    if (dtype == OR_BF16) return oracle_bf16_to_f32(((const uint16_t *)p)[idx]);
    return ((const float *)p)[idx];
}

static void store_T(void *p, int64_t idx, float v, int dtype)
{
    if (dtype == OR_F16) ((uint16_t *)p)[idx] = oracle_f32_to_f16(v);
    else if (dtype == OR_BF16) ((uint16_t *)p)[idx] = oracle_f32_to_bf16(v);
    else ((float *)p)[idx] = v;
}

/* Crossfade weights per the diffusers issue "[Proposal] Vectorize tiled VAE
 * blending while preserving rounding and CUDA graph replay", section "Proposed
 * scope": the ratio k/e is formed by a float64 division and each weight is
 * rounded once to fp32 (w_a from 1 - k/e in double, never 1 - w_b in fp32). */
void oracle_blend_coefficients(int64_t e, float *wa, float *wb)
{
    for (int64_t k = 0; k < e; ++k) {
        double q = (double)k / (double)e;
        wb[k] = (float)q;
        wa[k] = (float)(1.0 - q);
    }
}

/* One crossfaded element (same page and section): each weighted operand is
 * rounded to the storage type on its own before the two are added, and the
 * sum is rounded to the storage type again. */
float oracle_crossfade(float a, float b, float wa, float wb, int dtype)
{
    float pa = round_T(a * wa, dtype);
    float pb = round_T(b * wb, dtype);
    return round_T(pa + pb, dtype);
}

/* ------------------------------------------------------------------------ */
/* blend + crop + stitch                                                      */
/* ------------------------------------------------------------------------ */
/* A working tile: P planes (N*C) of F frames of H rows of W floats. */
typedef struct { int64_t P, F, H, W; float *v; } otile;

static float *at(const otile *t, int64_t p, int64_t f, int64_t y, int64_t x)
{
    return t->v + (((p * t->F + f) * t->H + y) * t->W + x);
}

static int64_t min3(int64_t a, int64_t b, int64_t c) { int64_t m = a < b ? a : b; return m < c ? m : c; }

/* blend_v: rows. b[.., k, :] = crossfade(a[.., H_a - e + k, :], b[.., k, :]) for k < e */
static void blend_rows(const otile *a, otile *b, int64_t E, int dtype)
{
    int64_t e = min3(E, a->H, b->H);
    if (e <= 0) return;
    float *wa = malloc(sizeof(float) * e), *wb = malloc(sizeof(float) * e);
    oracle_blend_coefficients(e, wa, wb);
    int64_t W = b->W;
    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t p = 0; p < b->P; ++p)
        for (int64_t f = 0; f < b->F; ++f)
            for (int64_t k = 0; k < e; ++k)
                for (int64_t x = 0; x < W; ++x) {
                    float av = *at(a, p, f, a->H - e + k, x);
                    float *bv = at(b, p, f, k, x);
                    *bv = oracle_crossfade(av, *bv, wa[k], wb[k], dtype);
                }
    free(wa); free(wb);
}

/* blend_h: columns. b[.., :, k] = crossfade(a[.., :, W_a - e + k], b[.., :, k]) for k < e */
static void blend_cols(const otile *a, otile *b, int64_t E, int dtype)
{
    int64_t e = min3(E, a->W, b->W);
    if (e <= 0) return;
    float *wa = malloc(sizeof(float) * e), *wb = malloc(sizeof(float) * e);
    oracle_blend_coefficients(e, wa, wb);
    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t p = 0; p < b->P; ++p)
        for (int64_t f = 0; f < b->F; ++f)
            for (int64_t y = 0; y < b->H; ++y)
                for (int64_t k = 0; k < e; ++k) {
                    float av = *at(a, p, f, y, a->W - e + k);
                    float *bv = at(b, p, f, y, k);
                    *bv = oracle_crossfade(av, *bv, wa[k], wb[k], dtype);
                }
    free(wa); free(wb);
}

/* blend_t: frames. b[.., k, :, :] = crossfade(a[.., F_a - e + k, :, :], b[.., k, :, :]) */
static void blend_frames(const otile *a, otile *b, int64_t E, int dtype)
{
    int64_t e = min3(E, a->F, b->F);
    if (e <= 0) return;
    float *wa = malloc(sizeof(float) * e), *wb = malloc(sizeof(float) * e);
    oracle_blend_coefficients(e, wa, wb);
    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t p = 0; p < b->P; ++p)
        for (int64_t k = 0; k < e; ++k)
            for (int64_t y = 0; y < b->H; ++y)
                for (int64_t x = 0; x < b->W; ++x) {
                    float av = *at(a, p, a->F - e + k, y, x);
                    float *bv = at(b, p, k, y, x);
                    *bv = oracle_crossfade(av, *bv, wa[k], wb[k], dtype);
                }
    free(wa); free(wb);
}

static int64_t out_len(int64_t n, const int64_t *ext, int64_t R) { return (n - 1) * R + ext[n - 1]; }
static int64_t crop_len(int64_t k, int64_t n, const int64_t *ext, int64_t R) { return k < n - 1 ? R : ext[n - 1]; }

/*
 * tiles: n_t*n_h*n_w host pointers, raster order (tau, i, j); tile (tau,i,j) is a
 *        contiguous [N, C, t_tau, h_i, w_j] array of dtype (t_tau = 1 for 4-D).
 * ext:   t_0..t_{n_t-1}, h_0..h_{n_h-1}, w_0..w_{n_w-1}
 * E, R:  blend extents and row limits (t, h, w)
 * out:   contiguous [N, C, L_t, L_h, L_w] of dtype, L = (n-1)R + ext_last.
 * Returns 0, or -1 when a non-last tile is shorter than the row limit (the crop
 * would then be undefined) or an argument is out of range.
 */
int oracle_blend_stitch(const void *const *tiles, int64_t N, int64_t C, int64_t n_t,
                        int64_t n_h, int64_t n_w, const int64_t *ext, const int64_t *E,
                        const int64_t *R, int dtype, void *out)
{
    const int64_t *et = ext, *eh = ext + n_t, *ew = ext + n_t + n_h;
    if (N < 0 || C < 0 || n_t < 1 || n_h < 1 || n_w < 1) return -1;
    for (int a = 0; a < 3; ++a) if (R[a] < 1 || E[a] < 0) return -1;
    for (int64_t k = 0; k < n_t; ++k) if (et[k] < 1 || (k < n_t - 1 && et[k] < R[0])) return -1;
    for (int64_t k = 0; k < n_h; ++k) if (eh[k] < 1 || (k < n_h - 1 && eh[k] < R[1])) return -1;
    for (int64_t k = 0; k < n_w; ++k) if (ew[k] < 1 || (k < n_w - 1 && ew[k] < R[2])) return -1;
    const int64_t P = N * C;
    const int64_t LT = out_len(n_t, et, R[0]), LH = out_len(n_h, eh, R[1]), LW = out_len(n_w, ew, R[2]);
    if (P == 0) return 0;

    otile prev = {0, 0, 0, 0, NULL};
    for (int64_t tau = 0; tau < n_t; ++tau) {
        const int64_t F = et[tau];
        /* working copies of this temporal tile's spatial tiles, as floats */
        otile *B = calloc((size_t)(n_h * n_w), sizeof(otile));
        for (int64_t i = 0; i < n_h; ++i)
            for (int64_t j = 0; j < n_w; ++j) {
                otile *t = &B[i * n_w + j];
                t->P = P; t->F = F; t->H = eh[i]; t->W = ew[j];
                int64_t n = P * F * eh[i] * ew[j];
                t->v = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
                const void *src = tiles[(tau * n_h + i) * n_w + j];
                #pragma omp parallel for schedule(static)
                for (int64_t q = 0; q < n; ++q) t->v[q] = load_T(src, q, dtype);
            }
        /* spatial blends, raster order, v before h, in place */
        for (int64_t i = 0; i < n_h; ++i)
            for (int64_t j = 0; j < n_w; ++j) {
                if (i > 0) blend_rows(&B[(i - 1) * n_w + j], &B[i * n_w + j], E[1], dtype);
                if (j > 0) blend_cols(&B[i * n_w + j - 1], &B[i * n_w + j], E[2], dtype);
            }
        /* crop + stitch into chunk S (all F frames kept: the next chunk blends
           against this chunk's tail frames) */
        otile S = {P, F, LH, LW, malloc(sizeof(float) * (size_t)(P * F * LH * LW))};
        for (int64_t i = 0; i < n_h; ++i)
            for (int64_t j = 0; j < n_w; ++j) {
                const otile *t = &B[i * n_w + j];
                int64_t ch = crop_len(i, n_h, eh, R[1]), cw = crop_len(j, n_w, ew, R[2]);
                #pragma omp parallel for collapse(3) schedule(static)
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t f = 0; f < F; ++f)
                        for (int64_t y = 0; y < ch; ++y)
                            for (int64_t x = 0; x < cw; ++x)
                                *at(&S, p, f, i * R[1] + y, j * R[2] + x) = *at(t, p, f, y, x);
            }
        for (int64_t q = 0; q < n_h * n_w; ++q) free(B[q].v);
        free(B);
        /* temporal blend against the previous chunk as modified */
        if (tau > 0) blend_frames(&prev, &S, E[0], dtype);
        /* crop along T and place at tau * R_t */
        int64_t ct = crop_len(tau, n_t, et, R[0]);
        #pragma omp parallel for collapse(3) schedule(static)
        for (int64_t p = 0; p < P; ++p)
            for (int64_t f = 0; f < ct; ++f)
                for (int64_t y = 0; y < LH; ++y)
                    for (int64_t x = 0; x < LW; ++x) {
                        int64_t o = ((p * LT + tau * R[0] + f) * LH + y) * LW + x;
                        store_T(out, o, *at(&S, p, f, y, x), dtype);
                    }
        free(prev.v);
        prev = S;
    }
    free(prev.v);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* GroupNorm                                                                  */
/* ------------------------------------------------------------------------ */
static int64_t prod(const int64_t *a, int from, int to)
{
    int64_t p = 1;
    for (int k = from; k < to; ++k) p *= a[k];
    return p;
}

/* [P3] PatchGroupNorm must equal nn.GroupNorm: plain unsplit GroupNorm, in double.
 * x: contiguous [N, C, spatial...] of dtype; gamma/beta: [C] of dtype or NULL.
 * y: N*C*S doubles; mean, var: N*G doubles each (may be NULL). */
int oracle_groupnorm(const void *x, int ndim, const int64_t *shape, int64_t G, double eps,
                     const void *gamma, const void *beta, int dtype, double *y,
                     double *mean_out, double *var_out)
{
    if (ndim < 3 || G < 1 || shape[1] % G != 0) return -1;
    const int64_t N = shape[0], C = shape[1], S = prod(shape, 2, ndim), Cg = C / G;
    const int64_t n = Cg * S;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < N; ++b)
        for (int64_t g = 0; g < G; ++g) {
            const int64_t base = (b * C + g * Cg) * S;
            double sum = 0.0;
            for (int64_t q = 0; q < n; ++q) sum += (double)load_T(x, base + q, dtype);
            double mean = n > 0 ? sum / (double)n : 0.0;
            double ss = 0.0;
            for (int64_t q = 0; q < n; ++q) {
                double d = (double)load_T(x, base + q, dtype) - mean;
                ss += d * d;
            }
            double var = n > 0 ? ss / (double)n : 0.0;  /* divide by the count */
            double inv = 1.0 / sqrt(var + eps);
            for (int64_t c = 0; c < Cg; ++c) {
                int64_t ch = g * Cg + c;
                double ga = gamma ? (double)load_T(gamma, ch, dtype) : 1.0;
                double be = beta ? (double)load_T(beta, ch, dtype) : 0.0;
                for (int64_t s = 0; s < S; ++s) {
                    int64_t o = base + c * S + s;
                    y[o] = ((double)load_T(x, o, dtype) - mean) * inv * ga + be;
                }
            }
            if (mean_out) mean_out[b * G + g] = mean;
            if (var_out) var_out[b * G + g] = var;
        }
    return 0;
}

/* [P3] Patchify: first (L mod P) patches are one longer */
static void patch_range(int64_t L, int64_t P, int64_t p, int64_t *start, int64_t *stop)
{
    int64_t base = L / P, extra = L % P;
    *start = p * base + (p < extra ? p : extra);
    *stop = *start + base + (p < extra ? 1 : 0);
}

/* Per-patch statistics, two-pass in double: stats[((n*G+g)*P+p)*3 + {0,1,2}] =
 * (count, mean, M2 = sum of squared deviations about the patch mean).
 * An empty patch gives (0, 0, 0). */
int oracle_patch_stats(const void *x, int ndim, const int64_t *shape, int64_t G, int split_axis,
                       int64_t P, int dtype, double *stats)
{
    if (ndim < 3 || G < 1 || shape[1] % G != 0 || split_axis < 2 || split_axis >= ndim || P < 1)
        return -1;
    const int64_t N = shape[0], C = shape[1], S = prod(shape, 2, ndim), Cg = C / G;
    const int64_t L = shape[split_axis];
    const int64_t inner = prod(shape, split_axis + 1, ndim);
    const int64_t mid = prod(shape, 2, split_axis); /* spatial dims before the split axis */
    #pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < N; ++b)
        for (int64_t g = 0; g < G; ++g)
            for (int64_t p = 0; p < P; ++p) {
                int64_t s0, s1;
                patch_range(L, P, p, &s0, &s1);
                double cnt = 0.0, sum = 0.0;
                for (int pass = 0; pass < 2; ++pass) {
                    double mean = cnt > 0 ? sum / cnt : 0.0, m2 = 0.0;
                    for (int64_t c = 0; c < Cg; ++c)
                        for (int64_t m = 0; m < mid; ++m)
                            for (int64_t l = s0; l < s1; ++l)
                                for (int64_t r = 0; r < inner; ++r) {
                                    int64_t o = (b * C + g * Cg + c) * S + (m * L + l) * inner + r;
                                    double v = (double)load_T(x, o, dtype);
                                    if (pass == 0) { cnt += 1.0; sum += v; }
                                    else m2 += (v - mean) * (v - mean);
                                }
                    if (pass == 1) {
                        double *st = stats + ((b * G + g) * P + p) * 3;
                        st[0] = cnt; st[1] = mean; st[2] = m2;
                    }
                }
            }
    return 0;
}

/* Chan et al. pairwise merge of (count, mean, M2) triples, applied in patch
 * order: delta = mean_B - mean_A; n = n_A + n_B; mean = mean_A + delta*n_B/n;
 * M2 = M2_A + M2_B + delta^2 * n_A * n_B / n.  Empty triples are skipped.
 * stats: rows*P triples; merged: rows triples. */
void oracle_chan_merge(const double *stats, int64_t rows, int64_t P, double *merged)
{
    for (int64_t r = 0; r < rows; ++r) {
        double n = 0.0, mean = 0.0, m2 = 0.0;
        for (int64_t p = 0; p < P; ++p) {
            const double *st = stats + (r * P + p) * 3;
            if (st[0] <= 0.0) continue;
            if (n == 0.0) { n = st[0]; mean = st[1]; m2 = st[2]; continue; }
            double nb = st[0], d = st[1] - mean, nn = n + nb;
            mean = mean + d * nb / nn;
            m2 = m2 + st[2] + d * d * n * nb / nn;
            n = nn;
        }
        merged[r * 3 + 0] = n; merged[r * 3 + 1] = mean; merged[r * 3 + 2] = m2;
    }
}

/* ------------------------------------------------------------------------ */
/* normalised-ramp blend of wide tiles                                        */
/* ------------------------------------------------------------------------ */
/*
 * [P2] the Qwen-Image-2.1 wide-tile commit: a tile has no weight within the
 * margin of an edge it shares with another tile (an edge inside the canvas),
 * ramps linearly to full weight over the next `ramp` positions, and the
 * weights are normalised to sum to 1 at every position; tiles are accumulated
 * one after another into a wide accumulator.  Weight along one axis at
 * position p of tile k (origin o, extent s, n tiles on the axis), with d the
 * distance in whole positions from the shared edge:
 *   lower edge shared (k > 0):     clamp((p - o - m) / r, 0, 1)
 *   upper edge shared (k < n - 1): clamp((o + s - 1 - p - m) / r, 0, 1)
 * the product of the two factors; the 2-D weight is the product of the axes'.
 */
static double clamp01(double v) { return v < 0.0 ? 0.0 : (v > 1.0 ? 1.0 : v); }

double oracle_ramp_weight(int64_t p, int64_t o, int64_t s, int64_t k, int64_t n, int64_t m,
                          int64_t r)
{
    if (p < o || p >= o + s) return 0.0;
    double w = 1.0;
    if (k > 0) w *= clamp01((double)(p - o - m) / (double)r);
    if (k < n - 1) w *= clamp01((double)(o + s - 1 - p - m) / (double)r);
    return w;
}

/*
 * tiles:  n_h*n_w host pointers, raster order; tile (i,j) is a contiguous
 *         [P, sh_i, sw_j] array of dtype (P = every leading dimension).
 * oh, sh, ow, sw: tile origins and extents along H and W.
 * out:    [P, LH, LW] doubles, the normalised weighted sum (not rounded).
 * mag:    optional [P, LH, LW] doubles, the same sum over |value|.
 * Returns 0, or -1 when a position has no tile with nonzero weight or an
 * argument is out of range.
 */
int oracle_ramp_blend(const void *const *tiles, int64_t P, int64_t n_h, int64_t n_w,
                      const int64_t *oh, const int64_t *sh, const int64_t *ow, const int64_t *sw,
                      int64_t LH, int64_t LW, int64_t mh, int64_t rh, int64_t mw, int64_t rw,
                      int dtype, double *out, double *mag)
{
    if (P < 0 || n_h < 1 || n_w < 1 || LH < 1 || LW < 1 || mh < 0 || mw < 0 || rh < 1 || rw < 1)
        return -1;
    for (int64_t i = 0; i < n_h; ++i) if (oh[i] < 0 || sh[i] < 1 || oh[i] + sh[i] > LH) return -1;
    for (int64_t j = 0; j < n_w; ++j) if (ow[j] < 0 || sw[j] < 1 || ow[j] + sw[j] > LW) return -1;
    /* the sum of the tiles' weights at every position */
    double *wsum = calloc((size_t)(LH * LW), sizeof(double));
    for (int64_t i = 0; i < n_h; ++i)
        for (int64_t j = 0; j < n_w; ++j)
            for (int64_t y = oh[i]; y < oh[i] + sh[i]; ++y)
                for (int64_t x = ow[j]; x < ow[j] + sw[j]; ++x)
                    wsum[y * LW + x] += oracle_ramp_weight(y, oh[i], sh[i], i, n_h, mh, rh) *
                                        oracle_ramp_weight(x, ow[j], sw[j], j, n_w, mw, rw);
    for (int64_t q = 0; q < LH * LW; ++q)
        if (!(wsum[q] > 0.0)) { free(wsum); return -1; }
    memset(out, 0, sizeof(double) * (size_t)(P * LH * LW));
    if (mag) memset(mag, 0, sizeof(double) * (size_t)(P * LH * LW));
    /* one tile after another, normalised weight times value into the accumulator */
    for (int64_t i = 0; i < n_h; ++i)
        for (int64_t j = 0; j < n_w; ++j) {
            const void *src = tiles[i * n_w + j];
            #pragma omp parallel for schedule(static)
            for (int64_t p = 0; p < P; ++p)
                for (int64_t y = 0; y < sh[i]; ++y)
                    for (int64_t x = 0; x < sw[j]; ++x) {
                        int64_t gy = oh[i] + y, gx = ow[j] + x;
                        double w = oracle_ramp_weight(gy, oh[i], sh[i], i, n_h, mh, rh) *
                                   oracle_ramp_weight(gx, ow[j], sw[j], j, n_w, mw, rw);
                        if (w == 0.0) continue;
                        double wn = w / wsum[gy * LW + gx];
                        double v = (double)load_T(src, (p * sh[i] + y) * sw[j] + x, dtype);
                        out[(p * LH + gy) * LW + gx] += wn * v;
                        if (mag) mag[(p * LH + gy) * LW + gx] += wn * fabs(v);
                    }
        }
    free(wsum);
    return 0;
}

/* Batch forms of the storage conversions (used by the tests that pin the
 * converters above against library conversions). */
void oracle_round_f32_array(const float *in, int64_t n, int dtype, uint16_t *out)
{
    for (int64_t q = 0; q < n; ++q)
        out[q] = dtype == OR_F16 ? oracle_f32_to_f16(in[q]) : oracle_f32_to_bf16(in[q]);
}

void oracle_widen_array(const uint16_t *in, int64_t n, int dtype, float *out)
{
    for (int64_t q = 0; q < n; ++q)
        out[q] = dtype == OR_F16 ? oracle_f16_to_f32(in[q]) : oracle_bf16_to_f32(in[q]);
}
