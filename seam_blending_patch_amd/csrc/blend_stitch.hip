// blend_stitch.hip -- fused blend + crop + stitch of overlapping decoded tiles, gfx950.
//
// What is computed (diffusers issue "[Proposal] Vectorize tiled VAE blending
// while preserving rounding and CUDA graph replay", section "Proposed scope"):
// blend_v / blend_h / blend_t crossfade the seam of each tile with the tail of
// its neighbour, in place, in raster order (row seam, then column seam), with
// the blend extent clamped to both tiles, coefficients from float64 division
// rounded once to fp32, and every product rounded to the storage dtype before
// the sum; every tile but the last along an axis is cropped to the row limit
// and the pieces are stitched.  Temporal tiles are stitched spatially first,
// then blended along frames against the previous stitched chunk.
//
// The in-place raster recursion has a closed form.  Given that no tile's head
// seam meets its own tail (ext(k) >= e(k) + e(k+1)), the neighbour operands a
// seam reads are untouched by their own blends except for one corner term, so
// each output element needs at most 4 tiles in 2-D:
//
//   s  = D[i][j][y, x]
//   if y < e_h(i):  U  = D[i-1][j][u+y, x]
//                   if x < e_w(j): U = b(D[i-1][j-1][u+y, l+x], U; x, e_w(j))
//                   s  = b(U, s; y, e_h(i))
//   if x < e_w(j):  Lf = D[i][j-1][y, l+x]
//                   if y < e_h(i): Lf = b(D[i-1][j-1][u+y, l+x], Lf; y, e_h(i))
//                   s  = b(Lf, s; x, e_w(j))
//
// with u = h(i-1) - e_h(i), l = w(j-1) - e_w(j); for frames f < e_t(tau) the
// same spatial value is taken in chunks tau-1 (frame t(tau-1) - e_t + f) and
// tau, and crossfaded along frames: 8 reads.
//
// Work layout.  Along W every tile j contributes a seam segment (its first
// min(e_w, crop) columns) and a body segment (the rest of its crop); along H
// likewise per tile row; along T per frame.  A block owns one output frame of
// one (n, c) plane, one W segment and a band of output rows, so the column
// tile, the column seam class, the temporal tile and the frame seam class are
// block-uniform; the band is split at tile-row seam boundaries into runs whose
// row class is block-uniform too.  Each run therefore executes one specialised
// path with scalar tile base addresses, no lane divergence, and a batch of
// output vectors per thread sized so that about eight 16-byte loads per lane
// are in flight (interior copy: 8 vectors; row or column seam: 4; corner: 2;
// with a frame seam, half of that).  Every tile element the output needs is
// read once, with a nontemporal hint (the corner operand once, used twice),
// and every output element is written once.  Each seam coefficient is formed
// where it is used, exactly equal to the float64 quotient rounded to fp32
// (coefficients_r below), so a block needs no tables and no barrier before
// its first loads.  Every product and sum is a separate fp32 operation (see
// crossfade below).

#include "sb_internal.h"
#include "sb_vec.h"

#ifndef SB_BLEND_NT
#define SB_BLEND_NT 1 // nontemporal hints on tile loads (each tile element is read once)
#endif
// Output stores carry nontemporal hints only when the whole call moves less
// than about half the 256 MB last-level cache (a host choice, the NTS
// template parameter): measured on the 64.5 MB 2048x2048 workload, 12% faster
// back to back and 7% after a cache flush; on the 375 MB and 524 MB ones plain
// stores are 9-14% faster (L2 write-combining helps there).
#ifndef SB_BLEND_THREADS
#define SB_BLEND_THREADS 256
#endif
// the host puts up to kMaxBlocksX blocks on grid x of a span launch
static_assert(sb::kMaxBlocksX * SB_BLEND_THREADS < ((int64_t)1 << 32), "grid x within 2^32 work-items");
#ifndef SB_BLEND_LOADS
#define SB_BLEND_LOADS 8 // 16-byte loads per lane in flight per batch
#endif
#ifndef SB_BLEND_WAVES_PER_EU
#define SB_BLEND_WAVES_PER_EU 0 // occupancy hint (0: none)
#endif
#if SB_BLEND_WAVES_PER_EU > 0
#define SB_BLEND_OCC __attribute__((amdgpu_waves_per_eu(SB_BLEND_WAVES_PER_EU)))
#else
#define SB_BLEND_OCC
#endif

namespace sb {

// One product, rounded to fp32 and then to the storage type.  The empty asm
// makes the fp32 product opaque so the compiler cannot fold the multiply and
// the narrowing into one mixed-precision FMA (v_fma_mix*), whose single
// rounding (and +0 addend) would differ from rounding to fp32 first.
template <int DT>
__device__ __forceinline__ float product(float a, float w) {
  float p = a * w;
  if constexpr (DT != DT_F32) asm("" : "+v"(p));
  return rn<DT>(p);
}

// Crossfade of one element.  The sum of two storage-type values is rounded to
// fp32 and then to the storage type; the compiler may do that addition in the
// storage type directly (v_add_f16): for binary16 and bfloat16 the result is
// the same, since fp32 carries at least 2p + 2 bits (no double-rounding error).
template <int DT>
__device__ __forceinline__ float crossfade(float a, float b, float2 c) {
  // c.x = w_a = fp32(1 - k/e), c.y = w_b = fp32(k/e)
  const float pa = product<DT>(a, c.x);
  const float pb = product<DT>(b, c.y);
  return rn<DT>(pa + pb);
}

// Crossfade of a packed pair of 16-bit elements: the products a*w_a and b*w_b
// of both elements are fp32 multiplies (kept opaque as above), each pair of
// products is rounded to the storage type by one packed conversion, and the
// two rounded products are summed with one rounding to the storage type.
// Same arithmetic as crossfade() element by element, fewer instructions.
template <int DT>
__device__ __forceinline__ uint32_t crossfade2(uint32_t a, uint32_t b, f32x2 wa, f32x2 wb) {
  const f32x2 fa = widen2<DT>(a), fb = widen2<DT>(b);
  f32x2 pa, pb;
  pa.x = fa.x * wa.x;
  pa.y = fa.y * wa.y;
  pb.x = fb.x * wb.x;
  pb.y = fb.y * wb.y;
  asm("" : "+v"(pa.x), "+v"(pa.y), "+v"(pb.x), "+v"(pb.y));
  return add2<DT>(narrow2<DT>(pa), narrow2<DT>(pb));
}

// The seam coefficients w_b = fp32(k/e) and w_a = fp32(1 - k/e), float64
// quotients rounded once to fp32, formed without a float64 division: with
// r = fp32(1/e) (computed on the host from float64, BlendArgs::rcp), the
// quotient n/e (n = k or e - k, whole numbers) is formed as q0 = n * r,
// corrected once by the exact fp32 remainder n - q0 * e (one fused
// multiply-add), q = q0 + rem * r (another).  For every 0 <= k < e <= 4096
// this gives exactly the float64-rounded weights (checked on all 8,390,656
// pairs on the host); kMaxBlend keeps e within that range.

__device__ __forceinline__ float quotient(float n, float e, float r) {
  const float q0 = n * r;
  const float rem = fmaf(-q0, e, n);
  return fmaf(rem, r, q0);
}

// (w_a, w_b) of position k of a seam of extent e, r = fp32(1/e)
__device__ __forceinline__ float2 coefficients_r(int k, int e, float r) {
  return make_float2(quotient((float)(e - k), (float)e, r), quotient((float)k, (float)e, r));
}

static_assert(kMaxBlend <= 4096, "the corrected-reciprocal coefficients are checked up to e = 4096");

// Block-uniform description of one run of rows (one tile row, one row class).
struct Run {
  const char *m, *u, *l, *c;     // tiles (i,j), (i-1,j), (i,j-1), (i-1,j-1) of chunk tau, each
                                 // offset so that operand (y, x) is base + y*pitch + x*EB
  const char *pm, *pu, *pl, *pc; // the same in chunk tau-1 (frame seams)
  int64_t pitch_j, pitch_p;      // bytes per row of tile column j and j-1
  char *o;                       // output at (row of local y = 0, first column of the segment)
  int64_t opitch;                // bytes per output row
  int y0, y1;                    // local rows [y0, y1) of tile row i
  int x0, wv;                    // first local column of the segment, vectors per row
  int eh, ew;                    // row and column seam extents (row / column seams)
  float rh, rw;                  // their reciprocals, fp32(1/eh) and fp32(1/ew)
  float2 ct;                     // frame coefficient (frame seams)
};

// q = n / d and n - q * d for 0 <= n < 2^24, d >= 1 uniform: the hardware
// reciprocal's quotient is within one of the exact one, and two compares fix it.
__device__ __forceinline__ int2 divmod_small(int n, int d, float rd) {
  int q = (int)((float)n * rd);
  q -= (q * d > n) ? 1 : 0;
  q += ((q + 1) * d <= n) ? 1 : 0;
  return make_int2(q, n - q * d);
}

// Walks the run's (rows x wv) vectors, nthreads apart, U per lane per batch.
// Each lane keeps its position (row r, vector x) and the byte offsets of that
// position in tile column j, tile column j-1 and the output, and advances all
// of them by nthreads vectors with adds and one carry test, so a vector costs
// a handful of integer operations.  OFF is the offset type: uint32_t when the
// host has checked that every offset stays below 2^31 bytes (the loads then
// take a block-uniform base plus a 32-bit lane offset), int64_t otherwise.
template <int DT, int VB, bool HS, bool WS, bool TS, class OFF, bool NTS>
__device__ __forceinline__ void run_rows(const Run &R, int tid, int nthreads) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int L = (1 + (HS ? 1 : 0) + (WS ? 1 : 0) + (HS && WS ? 1 : 0)) * (TS ? 2 : 1);
  constexpr int U = L >= SB_BLEND_LOADS ? 1 : SB_BLEND_LOADS / L; // output vectors per thread per batch
  const int nrows = R.y1 - R.y0;
  const int wv = R.wv;
  // first position (tid / wv, tid mod wv) and one step of nthreads vectors:
  // dr rows and dx vectors, plus a carry row when x passes wv
  const float rwv = __builtin_amdgcn_rcpf((float)wv);
  const int2 p0 = divmod_small(tid, wv, rwv);
  const int2 st = divmod_small(nthreads, wv, rwv);
  int r = p0.x, x = p0.y;
  const int dr = st.x, dx = st.y;
  const OFF pj = (OFF)R.pitch_j, pp = (OFF)R.pitch_p, po = (OFF)R.opitch;
  constexpr int VBY = V * EB; // bytes per vector
  const OFF xstep = (OFF)dx * VBY, xwrap = (OFF)wv * VBY;
  const OFF sj = (OFF)dr * pj + xstep, cj = pj - xwrap;
  const OFF sp = (OFF)dr * pp + xstep, cp = pp - xwrap;
  const OFF so = (OFF)dr * po + xstep, co = po - xwrap;
  const OFF x0b = (OFF)R.x0 * EB + (OFF)x * VBY;
  OFF oj = (OFF)(R.y0 + r) * pj + x0b;
  OFF op = (OFF)(R.y0 + r) * pp + x0b;
  OFF oo = (OFF)(R.y0 + r) * po + (OFF)x * VBY;

  // one batch: U output vectors per lane with every operand they read
  struct Batch {
    Vec<VB> m[U], up[U], lf[U], cn[U], pm[U], pu[U], pl[U], pc[U];
    int yy[U], xx[U];
    OFF od[U];
    bool ok[U];
  };
  // issue the loads of the lane's next U vectors and advance its position
  auto issue = [&](Batch &b) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      b.ok[k] = r < nrows;
      b.yy[k] = R.y0 + r;
      b.xx[k] = R.x0 + x * V;
      b.od[k] = oo;
      if (b.ok[k]) {
        b.m[k] = vload<VB, SB_BLEND_NT>(R.m + oj);
        if constexpr (HS) b.up[k] = vload<VB, SB_BLEND_NT>(R.u + oj);
        if constexpr (WS) b.lf[k] = vload<VB, SB_BLEND_NT>(R.l + op);
        if constexpr (HS && WS) b.cn[k] = vload<VB, SB_BLEND_NT>(R.c + op);
        if constexpr (TS) {
          b.pm[k] = vload<VB, SB_BLEND_NT>(R.pm + oj);
          if constexpr (HS) b.pu[k] = vload<VB, SB_BLEND_NT>(R.pu + oj);
          if constexpr (WS) b.pl[k] = vload<VB, SB_BLEND_NT>(R.pl + op);
          if constexpr (HS && WS) b.pc[k] = vload<VB, SB_BLEND_NT>(R.pc + op);
        }
      }
      r += dr;
      x += dx;
      oj += sj;
      op += sp;
      oo += so;
      if (x >= wv) {
        x -= wv;
        r += 1;
        oj += cj;
        op += cp;
        oo += co;
      }
    }
  };
  // blend the batch's vectors and store them
  auto process = [&](Batch &b) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (!b.ok[k]) continue;
      char *dst = R.o + b.od[k];
      if constexpr (!HS && !WS && !TS) {
        vstore<VB, NTS>(dst, b.m[k]);
      } else if constexpr (DT != DT_F32 && VB == 16) {
        // packed pairs of 16-bit elements
        constexpr int NW = Vec<VB>::NW;
        f32x2 ha, hb; // row coefficients (one per row, both lanes)
        if constexpr (HS) {
          const float2 c = coefficients_r(b.yy[k], R.eh, R.rh);
          ha.x = ha.y = c.x;
          hb.x = hb.y = c.y;
        }
        f32x2 wa[NW], wb[NW]; // column coefficients of elements 2w, 2w+1
        if constexpr (WS) {
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const float2 c0 = coefficients_r(b.xx[k] + 2 * w, R.ew, R.rw);
            const float2 c1 = coefficients_r(b.xx[k] + 2 * w + 1, R.ew, R.rw);
            wa[w].x = c0.x; wa[w].y = c1.x;
            wb[w].x = c0.y; wb[w].y = c1.y;
          }
        }
        auto spatial2 = [&](const Vec<VB> &vm, const Vec<VB> &vu, const Vec<VB> &vl,
                            const Vec<VB> &vc, Vec<VB> &o) {
          o = vm;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            uint32_t s = vm.w[w];
            if constexpr (HS) {
              uint32_t Uw = vu.w[w];
              if constexpr (WS) Uw = crossfade2<DT>(vc.w[w], Uw, wa[w], wb[w]);
              s = crossfade2<DT>(Uw, s, ha, hb);
            }
            if constexpr (WS) {
              uint32_t Lw = vl.w[w];
              if constexpr (HS) Lw = crossfade2<DT>(vc.w[w], Lw, ha, hb);
              s = crossfade2<DT>(Lw, s, wa[w], wb[w]);
            }
            o.w[w] = s;
          }
        };
        Vec<VB> S;
        spatial2(b.m[k], b.up[k], b.lf[k], b.cn[k], S);
        if constexpr (TS) {
          Vec<VB> Sp;
          spatial2(b.pm[k], b.pu[k], b.pl[k], b.pc[k], Sp);
          f32x2 ta, tb;
          ta.x = ta.y = R.ct.x;
          tb.x = tb.y = R.ct.y;
#pragma unroll
          for (int w = 0; w < NW; ++w) S.w[w] = crossfade2<DT>(Sp.w[w], S.w[w], ta, tb);
        }
        vstore<VB, NTS>(dst, S);
      } else {
        float2 chh = make_float2(0.f, 0.f);
        if constexpr (HS) chh = coefficients_r(b.yy[k], R.eh, R.rh);
        float2 cww[V];
        if constexpr (WS) {
#pragma unroll
          for (int e = 0; e < V; ++e) cww[e] = coefficients_r(b.xx[k] + e, R.ew, R.rw);
        }
        // closed form of the spatial blends for one chunk
        auto spatial = [&](const Vec<VB> &vm, const Vec<VB> &vu, const Vec<VB> &vl,
                           const Vec<VB> &vc, float *o) {
          unpack<DT, VB>(vm, o);
          if constexpr (HS) {
            float Uv[V];
            unpack<DT, VB>(vu, Uv);
            if constexpr (WS) {
              float Cn[V];
              unpack<DT, VB>(vc, Cn);
#pragma unroll
              for (int e = 0; e < V; ++e) Uv[e] = crossfade<DT>(Cn[e], Uv[e], cww[e]);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = crossfade<DT>(Uv[e], o[e], chh);
          }
          if constexpr (WS) {
            float Lf[V];
            unpack<DT, VB>(vl, Lf);
            if constexpr (HS) {
              float Cn[V];
              unpack<DT, VB>(vc, Cn);
#pragma unroll
              for (int e = 0; e < V; ++e) Lf[e] = crossfade<DT>(Cn[e], Lf[e], chh);
            }
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = crossfade<DT>(Lf[e], o[e], cww[e]);
          }
        };
        float S[V];
        spatial(b.m[k], b.up[k], b.lf[k], b.cn[k], S);
        if constexpr (TS) {
          float Sp[V];
          spatial(b.pm[k], b.pu[k], b.pl[k], b.pc[k], Sp);
#pragma unroll
          for (int e = 0; e < V; ++e) S[e] = crossfade<DT>(Sp[e], S[e], R.ct);
        }
        vstore<VB, NTS>(dst, pack<DT, VB>(S));
      }
    }
  };
  Batch A;
  while (r < nrows) {
    issue(A);
    process(A);
  }
}

typedef __attribute__((address_space(1))) char *GOut;

struct PtrPair {
  const char *a, *b; // pointer-table entries k-1 and k
};
// the pair of entry 0 starts at the output pointer, the argument word before
// the table: read with it, never used
static_assert(offsetof(BlendArgs, ptr) == sizeof(void *), "the table follows the output pointer");

// The tiles the closed form reads for one tile row of a segment: (i,j),
// (i-1,j), (i,j-1), (i-1,j-1) of chunk tau, then the same in chunk tau-1.
struct Tiles {
  const char *m, *u, *l, *c, *pm, *pu, *pl, *pc;
};

// The launch arguments a block reads before its first tile loads.
struct Head {
  int32_t nw, nh, nt, E0, E1, E2, R0, R1, R2, LT, LH, LW, taub, ib, ptr_nh, F0, nF, Y0, nY, plane0, rows_pb;
  int32_t g_seg, g_band, g_pf;
  uint32_t nFm, nFs, Rtm, Rts, Rhm, Rhs;
  char *out;
};

__device__ __forceinline__ uint32_t fdiv_ms(uint32_t n, uint32_t m, uint32_t s) {
  return (__umulhi(n, m) + n) >> s;
}

// One work item: (plane, frame) pf of the launch, W segment sw, row band bz.
template <int DT, int VB, class OFF, bool NTS>
__device__ __forceinline__ void blend_item(const BlendArgs &A, const Head &H, uint32_t pz, int sw, int bz) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  const int tid = threadIdx.x;
  constexpr int nthr = SB_BLEND_THREADS;
  const int nw = H.nw, nh = H.nh, nt = H.nt;

  // ---- block-uniform indices: arithmetic on the block index and the pinned
  //      argument fields only ----
  const uint32_t j = (uint32_t)(sw + 1) >> 1;
  const bool wseam = (sw & 1) != 0;
  const uint32_t pli = fdiv_ms(pz, H.nFm, H.nFs);
  const uint32_t plane = (uint32_t)H.plane0 + pli; // N * C < 2^31
  const uint32_t f_out = (uint32_t)H.F0 + (pz - pli * (uint32_t)H.nF);
  const uint32_t tau = min(fdiv_ms(f_out, H.Rtm, H.Rts), (uint32_t)nt - 1);
  const int f = (int)(f_out - tau * (uint32_t)H.R0);
  const int r0 = bz * H.rows_pb;
  const int r1 = min(r0 + H.rows_pb, H.nY);
  const int yo0 = H.Y0 + r0, yo1 = H.Y0 + r1;
  const uint32_t ia = min(fdiv_ms((uint32_t)yo0, H.Rhm, H.Rhs), (uint32_t)nh - 1); // first run's tile row

  // ---- the extents, seam reciprocals and tile pointers of the block's first
  //      run, all requested at once and pinned, so they arrive in one more
  //      round of scalar loads.  Tile (tq, ti, tj) of the window is entry
  //      ((tq - taub) * ptr_nh + (ti - ib)) * nw + tj; the neighbours are
  //      fixed steps back from (tau, ia, j), taken as zero steps where there
  //      is none (index 0 along that axis).  Tile columns j-1 and j are
  //      adjacent entries, loaded as one pair; at j = 0 the first of the pair
  //      is the entry (or, at entry 0, the argument word) before and is not
  //      used ----
  const uint32_t su = ia > 0 ? (uint32_t)nw : 0u;
  const uint32_t st = tau > 0 ? (uint32_t)(H.ptr_nh * nw) : 0u;
  const uint32_t jm = j > 0 ? j - 1 : 0u, iam = ia > 0 ? ia - 1 : 0u, taum = tau > 0 ? tau - 1 : 0u;
  int wj = A.ext[2][j], wjm = A.ext[2][jm];
  int tt = A.ext[0][tau], ttm = A.ext[0][taum];
  int hia = A.ext[1][ia], hiam = A.ext[1][iam];
  float rw = A.rcp[2][j], rt = A.rcp[0][tau], rh0 = A.rcp[1][ia];
  // byte offset of entry b's pair (entries b-1, b) from the start of the table
  const char *const tab = (const char *)A.ptr - sizeof(void *);
  auto pair = [&](uint32_t b) { return *(const PtrPair *)(tab + (size_t)(b * (uint32_t)sizeof(void *))); };
  const uint32_t b0 = ((tau - (uint32_t)H.taub) * (uint32_t)H.ptr_nh + (ia - (uint32_t)H.ib)) * (uint32_t)nw + j;
  auto tiles_of_row = [&](uint32_t b, uint32_t sui) {
    const PtrPair lm = pair(b), cu = pair(b - sui), plm = pair(b - st), pcu = pair(b - st - sui);
    return Tiles{lm.b, cu.b, lm.a, cu.a, plm.b, pcu.b, plm.a, pcu.a};
  };
  Tiles T = tiles_of_row(b0, su);
  {
    // pinned as global-address-space pointers: a generic pointer coming out
    // of the asm would turn every tile load into a flat load
    GPtr m = (GPtr)T.m, u = (GPtr)T.u, l = (GPtr)T.l, c = (GPtr)T.c;
    GPtr pm = (GPtr)T.pm, pu = (GPtr)T.pu, pl = (GPtr)T.pl, pc = (GPtr)T.pc;
    asm volatile("" : "+s"(wj), "+s"(wjm), "+s"(tt), "+s"(ttm), "+s"(hia), "+s"(hiam), "+s"(rw), "+s"(rt),
                 "+s"(rh0), "+s"(m), "+s"(u), "+s"(l), "+s"(c), "+s"(pm), "+s"(pu), "+s"(pl), "+s"(pc));
    T = Tiles{(const char *)m,  (const char *)u,  (const char *)l,  (const char *)c,
              (const char *)pm, (const char *)pu, (const char *)pl, (const char *)pc};
  }

  // ---- W segment: tile column j, seam or body ----
  const int wp = j > 0 ? wjm : 0;
  const int ew = j > 0 ? min(H.E2, min(wp, wj)) : 0;
  const int cw = j < nw - 1 ? H.R2 : wj;
  const int ews = min(ew, cw);
  const int x0 = wseam ? 0 : ews;
  const int x1 = wseam ? ews : cw;

  // ---- frame: temporal tile tau, local frame f ----
  const int tp = tau > 0 ? ttm : 0;
  const int et = tau > 0 ? min(H.E0, min(tp, tt)) : 0;
  const bool ts = f < et;
  const int fp = tp - et + f; // frame of chunk tau-1 blended into frame f

  if (x1 <= x0) return; // empty segment (no seam, or a tile that is all seam)

  // seam coefficients are formed per vector from (position, extent,
  // reciprocal); only the frame coefficient is block-uniform
  const float2 ct = ts ? coefficients_r(f, et, rt) : make_float2(0.f, 0.f);
  // (plane, frame) slices of the chunks tau and tau-1 read here, in frames
  const uint64_t sfm = (uint64_t)plane * (uint32_t)tt + (uint32_t)f;
  const uint64_t sfp = (uint64_t)plane * (uint32_t)tp + (uint32_t)fp;

  // ---- runs of rows with one tile row and one row class ----
  int cur = (int)ia;           // tile row whose extents and tiles are loaded
  int hi = hia, hp = hiam;     // its extent and the one above (clamped at row 0)
  float rh = rh0;              // fp32(1/e) of its row seam
  int yo = yo0;
  while (yo < yo1) {
    const int i = min((int)fdiv_ms((uint32_t)yo, H.Rhm, H.Rhs), nh - 1);
    if (i != cur) { // the band crosses into the next tile row (i > 0)
      hp = A.ext[1][i - 1];
      hi = A.ext[1][i];
      rh = A.rcp[1][i];
      T = tiles_of_row(b0 + (uint32_t)(i - (int)ia) * (uint32_t)nw, (uint32_t)nw);
      cur = i;
    }
    const int ybase = i * H.R1;
    const int eh = i > 0 ? min(H.E1, min(hp, hi)) : 0;
    const int chh = i < nh - 1 ? H.R1 : hi;
    const int ehs = min(eh, chh);
    const int yl = yo - ybase;
    const bool hs = yl < ehs;
    const int yl1 = min(hs ? ehs : chh, yl + (yo1 - yo));

    Run R;
    const int u = hp - eh, l = wp - ew;
    // plane, frame and neighbour-tail offsets folded into the tile bases, in
    // elements: rows of (tile row i or i-1) x (tile column j or j-1)
    const uint64_t rm = sfm * (uint32_t)hi, ru = sfm * (uint32_t)hp + (uint32_t)u;
    R.pitch_j = (int64_t)wj * EB;
    R.pitch_p = (int64_t)wp * EB;
    R.m = T.m + rm * (uint32_t)wj * EB;
    R.u = R.l = R.c = R.pm = R.pu = R.pl = R.pc = nullptr;
    if (hs) R.u = T.u + ru * (uint32_t)wj * EB;
    if (wseam) R.l = T.l + (rm * (uint32_t)wp + (uint32_t)l) * EB;
    if (hs && wseam) R.c = T.c + (ru * (uint32_t)wp + (uint32_t)l) * EB;
    if (ts) {
      const uint64_t qm = sfp * (uint32_t)hi, qu = sfp * (uint32_t)hp + (uint32_t)u;
      R.pm = T.pm + qm * (uint32_t)wj * EB;
      if (hs) R.pu = T.pu + qu * (uint32_t)wj * EB;
      if (wseam) R.pl = T.pl + (qm * (uint32_t)wp + (uint32_t)l) * EB;
      if (hs && wseam) R.pc = T.pc + (qu * (uint32_t)wp + (uint32_t)l) * EB;
    }
    R.opitch = (int64_t)H.LW * EB;
    R.o = H.out + ((((uint64_t)plane * (uint32_t)H.LT + (uint32_t)f_out) * (uint32_t)H.LH + (uint32_t)ybase) *
                       (uint32_t)H.LW + (uint32_t)(j * H.R2 + x0)) * EB;
    R.y0 = yl;
    R.y1 = yl1;
    R.x0 = x0;
    R.wv = (x1 - x0) / V;
    R.eh = eh;
    R.rh = rh;
    R.ew = ew;
    R.rw = rw;
    R.ct = ct;

    const int cls = (ts ? 4 : 0) | (hs ? 2 : 0) | (wseam ? 1 : 0);
    switch (cls) {
      case 0: run_rows<DT, VB, false, false, false, OFF, NTS>(R, tid, nthr); break;
      case 1: run_rows<DT, VB, false, true, false, OFF, NTS>(R, tid, nthr); break;
      case 2: run_rows<DT, VB, true, false, false, OFF, NTS>(R, tid, nthr); break;
      case 3: run_rows<DT, VB, true, true, false, OFF, NTS>(R, tid, nthr); break;
      case 4: run_rows<DT, VB, false, false, true, OFF, NTS>(R, tid, nthr); break;
      case 5: run_rows<DT, VB, false, true, true, OFF, NTS>(R, tid, nthr); break;
      case 6: run_rows<DT, VB, true, false, true, OFF, NTS>(R, tid, nthr); break;
      default: run_rows<DT, VB, true, true, true, OFF, NTS>(R, tid, nthr); break;
    }
    yo += yl1 - yl;
  }
}

template <int DT, int VB, class OFF, bool NTS>
__global__ __launch_bounds__(SB_BLEND_THREADS) SB_BLEND_OCC void blend_stitch_kernel(const BlendArgs A) {
  // Every launch argument the block decode and the first run read, read at
  // entry and pinned in scalar registers by empty asm statements, so that they
  // arrive in one round of scalar loads; left alone, the compiler spreads them
  // over a chain of dependent rounds between branches (about nine before the
  // first tile load), which took most of a small block's life.  The grid
  // extents come from the arguments too: gridDim and blockDim would be more
  // loads of their own.
  Head H;
  H.nw = A.n_w; H.nh = A.n_h; H.nt = A.n_t;
  H.E0 = A.E[0]; H.E1 = A.E[1]; H.E2 = A.E[2];
  H.R0 = A.R[0]; H.R1 = A.R[1]; H.R2 = A.R[2];
  H.LT = A.LT; H.LH = A.LH; H.LW = A.LW;
  H.taub = A.taub; H.ib = A.ib; H.ptr_nh = A.ptr_nh;
  H.F0 = A.F0; H.nF = A.nF; H.Y0 = A.Y0; H.nY = A.nY; H.plane0 = A.plane0; H.rows_pb = A.rows_per_block;
  H.g_seg = A.g_seg; H.g_band = A.g_band; H.g_pf = A.g_pf;
  H.nFm = A.div_nF.m; H.nFs = A.div_nF.s; H.Rtm = A.div_Rt.m; H.Rts = A.div_Rt.s;
  H.Rhm = A.div_Rh.m; H.Rhs = A.div_Rh.s;
  GOut out = (GOut)A.out; // pinned in the global address space (see blend_item)
  asm volatile("" : "+s"(H.nw), "+s"(H.nh), "+s"(H.nt), "+s"(H.E0), "+s"(H.E1), "+s"(H.E2), "+s"(H.R0),
               "+s"(H.R1), "+s"(H.R2), "+s"(H.LT), "+s"(H.LH), "+s"(H.LW), "+s"(H.taub), "+s"(H.ib),
               "+s"(H.ptr_nh), "+s"(H.F0));
  asm volatile("" : "+s"(H.nF), "+s"(H.Y0), "+s"(H.nY), "+s"(H.plane0), "+s"(H.rows_pb), "+s"(H.g_seg),
               "+s"(H.g_band), "+s"(H.g_pf), "+s"(H.nFm), "+s"(H.nFs), "+s"(H.Rtm), "+s"(H.Rts), "+s"(H.Rhm),
               "+s"(H.Rhs), "+s"(out));
  H.out = (char *)out;
  // The grid is (W segments, row bands, (plane, frame)), taken in reverse:
  // the last row band and the last frames first.  Row bands further down and
  // later frames are the ones that meet row and frame seams (up to 8 reads per
  // output vector), so the blocks left for the end of the grid are mostly
  // plain copies, which shortens the drain; and the blocks dispatched together
  // cover whole output rows of one frame, so the concurrent reads and writes
  // stay within a few frames (video workload: 66.0 -> 63.3 us back to back,
  // 68.5 -> 66.2 us after a flush, against (plane, frame) fastest).
  blend_item<DT, VB, OFF, NTS>(A, H, (uint32_t)(H.g_pf - 1) - blockIdx.z, H.g_seg - 1 - (int)blockIdx.x,
                               H.g_band - 1 - (int)blockIdx.y);
}

// ---------------------------------------------------------------------------
// Span layout, for narrow seams.  When every W segment is only a few vectors
// wide (small blend extents and row limits, as in tiled-encode latents), one
// segment per block leaves each wavefront reading short row pieces of many
// rows.  Here a block owns a span of whole tile columns instead and walks its
// rows left to right, so consecutive lanes read consecutive vectors; the
// column class (seam or body) and the tile column vary per lane, the row and
// frame classes stay block-uniform per run.  Same closed form and the same
// roundings (16-bit types in packed pairs, as in run_rows); the column records
// of a tile row (tile bases, seam extent and reciprocal) are built once per
// tile row in LDS, one lane per column, and the seam coefficients are formed
// in registers.
// ---------------------------------------------------------------------------
#ifndef SB_SPAN_U
#define SB_SPAN_U 2
#endif
struct SpanRun {
  char *o;                       // output at (local row 0, first column of the span)
  int64_t opitch;
  int y0, y1;                    // local rows of the tile row
  int xs0, wv, ja, nw;           // first output column, vectors per row, first tile column, n_w
  uint32_t Rwm, Rws;             // division by the column row limit R_w (magic multiplier, shift)
  int eh;                        // row seam extent of the run's tile row (row seams)
  float rh;                      // fp32(1/eh)
  float2 ct;                     // frame coefficient (frame seams)
};

template <int DT, int VB, bool HS, bool TS>
__device__ __forceinline__ void span_rows(const SpanRun &R, const SpanCol *cols, int tid, int nthreads) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int U = SB_SPAN_U; // output vectors per thread per batch
  const int nvec = (R.y1 - R.y0) * R.wv;
  const float rwv = __builtin_amdgcn_rcpf((float)R.wv);
  for (int q0 = tid; q0 < nvec; q0 += nthreads * U) {
    Vec<VB> m[U], up[U], lf[U], cn[U], pm[U], pu[U], pl[U], pc[U];
    int yy[U], xs[U], xl[U], ew[U];
    float rw[U];
    bool ok[U], ws[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int q = q0 + k * nthreads;
      ok[k] = q < nvec;
      const int2 rq = divmod_small(q, R.wv, rwv);
      const int y = R.y0 + rq.x;
      const int xo = rq.y * V;                       // column within the span
      const int x = R.xs0 + xo;                      // output column
      const int j = min((int)fdiv_ms((uint32_t)x, R.Rwm, R.Rws), R.nw - 1);
      yy[k] = y;
      xs[k] = xo;
      ws[k] = false;
      if (ok[k]) {
        const SpanCol &C = cols[j - R.ja];
        xl[k] = x - C.xbase;                         // column within tile j
        ws[k] = xl[k] < C.ews;
        ew[k] = C.ew;
        rw[k] = C.rw;
        const int64_t oj = (int64_t)y * C.pitch_j + (int64_t)xl[k] * EB;
        const int64_t op = (int64_t)y * C.pitch_p + (int64_t)xl[k] * EB;
        m[k] = vload<VB, SB_BLEND_NT>((const char *)(C.m + oj));
        if constexpr (HS) up[k] = vload<VB, SB_BLEND_NT>((const char *)(C.u + oj));
        if (ws[k]) {
          lf[k] = vload<VB, SB_BLEND_NT>((const char *)(C.l + op));
          if constexpr (HS) cn[k] = vload<VB, SB_BLEND_NT>((const char *)(C.c + op));
        }
        if constexpr (TS) {
          pm[k] = vload<VB, SB_BLEND_NT>((const char *)(C.pm + oj));
          if constexpr (HS) pu[k] = vload<VB, SB_BLEND_NT>((const char *)(C.pu + oj));
          if (ws[k]) {
            pl[k] = vload<VB, SB_BLEND_NT>((const char *)(C.pl + op));
            if constexpr (HS) pc[k] = vload<VB, SB_BLEND_NT>((const char *)(C.pc + op));
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if (!ok[k]) continue;
      char *dst = R.o + (int64_t)yy[k] * R.opitch + (int64_t)xs[k] * EB;
      if (!HS && !TS && !ws[k]) {
        vstore<VB, false>(dst, m[k]);
        continue;
      }
      if constexpr (DT != DT_F32 && VB == 16) {
        // packed pairs of 16-bit elements, as in run_rows
        constexpr int NW = Vec<VB>::NW;
        const bool w = ws[k];
        f32x2 ha, hb;
        if constexpr (HS) {
          const float2 c = coefficients_r(yy[k], R.eh, R.rh);
          ha.x = ha.y = c.x;
          hb.x = hb.y = c.y;
        }
        f32x2 wa[NW], wb[NW];
        if (w) {
#pragma unroll
          for (int e = 0; e < NW; ++e) {
            const float2 c0 = coefficients_r(xl[k] + 2 * e, ew[k], rw[k]);
            const float2 c1 = coefficients_r(xl[k] + 2 * e + 1, ew[k], rw[k]);
            wa[e].x = c0.x; wa[e].y = c1.x;
            wb[e].x = c0.y; wb[e].y = c1.y;
          }
        }
        auto spatial2 = [&](const Vec<VB> &vm, const Vec<VB> &vu, const Vec<VB> &vl, const Vec<VB> &vc,
                            Vec<VB> &o) {
          o = vm;
#pragma unroll
          for (int e = 0; e < NW; ++e) {
            uint32_t sv = vm.w[e];
            if constexpr (HS) {
              uint32_t Uw = vu.w[e];
              if (w) Uw = crossfade2<DT>(vc.w[e], Uw, wa[e], wb[e]);
              sv = crossfade2<DT>(Uw, sv, ha, hb);
            }
            if (w) {
              uint32_t Lw = vl.w[e];
              if constexpr (HS) Lw = crossfade2<DT>(vc.w[e], Lw, ha, hb);
              sv = crossfade2<DT>(Lw, sv, wa[e], wb[e]);
            }
            o.w[e] = sv;
          }
        };
        Vec<VB> S;
        spatial2(m[k], up[k], lf[k], cn[k], S);
        if constexpr (TS) {
          Vec<VB> Sp;
          spatial2(pm[k], pu[k], pl[k], pc[k], Sp);
          f32x2 ta, tb;
          ta.x = ta.y = R.ct.x;
          tb.x = tb.y = R.ct.y;
#pragma unroll
          for (int e = 0; e < NW; ++e) S.w[e] = crossfade2<DT>(Sp.w[e], S.w[e], ta, tb);
        }
        vstore<VB, false>(dst, S);
        continue;
      }
      // seam coefficients formed in registers, as in the segment layout
      float2 chh = make_float2(0.f, 0.f);
      if constexpr (HS) chh = coefficients_r(yy[k], R.eh, R.rh);
      float2 cww[V];
      if (ws[k]) {
#pragma unroll
        for (int e = 0; e < V; ++e) cww[e] = coefficients_r(xl[k] + e, ew[k], rw[k]);
      }
      const bool w = ws[k];
      auto spatial = [&](const Vec<VB> &vm, const Vec<VB> &vu, const Vec<VB> &vl, const Vec<VB> &vc,
                         float *o) {
        unpack<DT, VB>(vm, o);
        if constexpr (HS) {
          float Uv[V];
          unpack<DT, VB>(vu, Uv);
          if (w) {
            float Cn[V];
            unpack<DT, VB>(vc, Cn);
#pragma unroll
            for (int e = 0; e < V; ++e) Uv[e] = crossfade<DT>(Cn[e], Uv[e], cww[e]);
          }
#pragma unroll
          for (int e = 0; e < V; ++e) o[e] = crossfade<DT>(Uv[e], o[e], chh);
        }
        if (w) {
          float Lf[V];
          unpack<DT, VB>(vl, Lf);
          if constexpr (HS) {
            float Cn[V];
            unpack<DT, VB>(vc, Cn);
#pragma unroll
            for (int e = 0; e < V; ++e) Lf[e] = crossfade<DT>(Cn[e], Lf[e], chh);
          }
#pragma unroll
          for (int e = 0; e < V; ++e) o[e] = crossfade<DT>(Lf[e], o[e], cww[e]);
        }
      };
      float S[V];
      spatial(m[k], up[k], lf[k], cn[k], S);
      if constexpr (TS) {
        float Sp[V];
        spatial(pm[k], pu[k], pl[k], pc[k], Sp);
#pragma unroll
        for (int e = 0; e < V; ++e) S[e] = crossfade<DT>(Sp[e], S[e], R.ct);
      }
      vstore<VB, false>(dst, pack<DT, VB>(S));
    }
  }
}

template <int DT, int VB>
__global__ __launch_bounds__(SB_BLEND_THREADS) void blend_span_kernel(const BlendArgs A) {
  constexpr int EB = Elem<DT>::bytes;
  extern __shared__ float2 s_tab[]; // [span_k] SpanCol
  SpanCol *s_col = reinterpret_cast<SpanCol *>(s_tab);
  const int tid = threadIdx.x;
  constexpr int nthr = SB_BLEND_THREADS; // a constant: no implicit-argument load

  // Every launch argument the block decode reads, read at entry and pinned in
  // scalar registers (one round of scalar loads), as in blend_stitch_kernel.
  int32_t nw = A.n_w, nh = A.n_h, nt = A.n_t, E0 = A.E[0], E1 = A.E[1], E2 = A.E[2];
  int32_t R0 = A.R[0], R1 = A.R[1], R2 = A.R[2], LT = A.LT, LH = A.LH, LW = A.LW;
  int32_t taub = A.taub, ib = A.ib, ptr_nh = A.ptr_nh, F0 = A.F0, nF = A.nF, Y0 = A.Y0, nY = A.nY;
  int32_t plane0 = A.plane0, rows_pb = A.rows_per_block, span_k = A.span_k;
  uint32_t nFm = A.div_nF.m, nFs = A.div_nF.s, Rtm = A.div_Rt.m, Rts = A.div_Rt.s;
  uint32_t Rhm = A.div_Rh.m, Rhs = A.div_Rh.s, Rwm = A.div_Rw.m, Rws = A.div_Rw.s;
  GOut outp = (GOut)A.out;
  asm volatile("" : "+s"(nw), "+s"(nh), "+s"(nt), "+s"(E0), "+s"(E1), "+s"(E2), "+s"(R0), "+s"(R1), "+s"(R2),
               "+s"(LT), "+s"(LH), "+s"(LW), "+s"(taub), "+s"(ib), "+s"(ptr_nh), "+s"(F0));
  asm volatile("" : "+s"(nF), "+s"(Y0), "+s"(nY), "+s"(plane0), "+s"(rows_pb), "+s"(span_k), "+s"(nFm),
               "+s"(nFs), "+s"(Rtm), "+s"(Rts), "+s"(Rhm), "+s"(Rhs), "+s"(Rwm), "+s"(Rws), "+s"(outp));

  // ---- span: tile columns [ja, jb) ----
  const int ja = (int)blockIdx.y * span_k;
  const int jb = min(ja + span_k, nw);
  const int xs0 = ja * R2;
  const int xs1 = jb == nw ? LW : jb * R2;

  // ---- frame (block-uniform), as in blend_stitch_kernel ----
  const uint32_t pz = blockIdx.x;
  const uint32_t pli = fdiv_ms(pz, nFm, nFs);
  const uint32_t plane = (uint32_t)plane0 + pli; // N * C < 2^31
  const int f_out = F0 + (int)(pz - pli * (uint32_t)nF);
  const int tau = min((int)fdiv_ms((uint32_t)f_out, Rtm, Rts), nt - 1);
  const int f = f_out - tau * R0;
  const int r0 = (int)blockIdx.z * rows_pb;
  const int r1 = min(r0 + rows_pb, nY);
  const int yo0 = Y0 + r0, yo1 = Y0 + r1;
  const int ia = min((int)fdiv_ms((uint32_t)yo0, Rhm, Rhs), nh - 1); // first run's tile row

  // tile-pointer table: entry b's pair (entries b-1, b), as in blend_stitch_kernel
  const char *const tab = (const char *)A.ptr - sizeof(void *);
  auto pair = [&](uint32_t b) { return *(const PtrPair *)(tab + (size_t)(b * (uint32_t)sizeof(void *))); };

  // ---- one more round, all requested together: in lane t < jb - ja, the
  //      extents and reciprocal of tile column j = ja + t and its pointer
  //      pairs for the first run's tile row (and the previous chunk's); then
  //      the frame's and the first tile row's extents and reciprocals
  //      (scalar, pinned; the pin waits for them, so it comes last) ----
  const bool col_lane = tid < jb - ja;
  const int j = ja + min(tid, jb - ja - 1);
  const uint32_t st = tau > 0 ? (uint32_t)(ptr_nh * nw) : 0u;
  int wj = 0, wp = 0;
  float rwj = 0.f;
  // the pointer pairs of column j in tile row i: (i,j-1 | i,j), (i-1,j-1 |
  // i-1,j), then the same in chunk tau-1
  auto load_pairs = [&](int i, PtrPair (&p)[4]) {
    const uint32_t b = ((uint32_t)(tau - taub) * (uint32_t)ptr_nh + (uint32_t)(i - ib)) * (uint32_t)nw + (uint32_t)j;
    const uint32_t su = i > 0 ? (uint32_t)nw : 0u;
    p[0] = pair(b);
    p[1] = pair(b - su);
    if (tau > 0) {
      p[2] = pair(b - st);
      p[3] = pair(b - st - su);
    }
  };
  PtrPair p0[4] = {}; // the first run's tile row
  if (col_lane) {
    wj = A.ext[2][j];
    const int wq = A.ext[2][max(j - 1, 0)];
    wp = j > 0 ? wq : 0;
    rwj = A.rcp[2][j];
    load_pairs(ia, p0);
  }
  const int taum = tau > 0 ? tau - 1 : 0, iam = ia > 0 ? ia - 1 : 0;
  int tt = A.ext[0][tau], ttm = A.ext[0][taum], hia = A.ext[1][ia], hiam = A.ext[1][iam];
  float rt = A.rcp[0][tau], rh0 = A.rcp[1][ia];
  asm volatile("" : "+s"(tt), "+s"(ttm), "+s"(hia), "+s"(hiam), "+s"(rt), "+s"(rh0));

  const int tp = tau > 0 ? ttm : 0;
  const int et = tau > 0 ? min(E0, min(tp, tt)) : 0;
  const bool ts = f < et;
  const int fp = tp - et + f; // frame of chunk tau-1 blended into frame f
  const float2 ct = ts ? coefficients_r(f, et, rt) : make_float2(0.f, 0.f);
  // (plane, frame) slices of the chunks tau and tau-1 read here, in frames
  const uint64_t sfm = (uint64_t)plane * (uint32_t)tt + (uint32_t)f;
  const uint64_t sfp = (uint64_t)plane * (uint32_t)tp + (uint32_t)fp;

  // The column records of tile row i, one per lane t < jb - ja, from the
  // pairs load_pairs(i) fetched.  A record depends on the tile row, the
  // column and the frame only (the row-seam operands are set whenever there
  // is a tile row above; runs outside the row seam do not read them).
  auto build_cols = [&](int i, int hi, int hp, const PtrPair (&p)[4]) {
    const PtrPair &lm = p[0], &cu = p[1], &plm = p[2], &pcu = p[3];
    const int eh = i > 0 ? min(E1, min(hp, hi)) : 0;
    const int u = hp - eh;
    const int ew = j > 0 ? min(E2, min(wp, wj)) : 0;
    const int cw = j < nw - 1 ? R2 : wj;
    const int l = wp - ew;
    const uint64_t rm = sfm * (uint32_t)hi, ru = sfm * (uint32_t)hp + (uint32_t)u;
    SpanCol C;
    C.pitch_j = (int64_t)wj * EB;
    C.pitch_p = (int64_t)wp * EB;
    C.xbase = j * R2;
    C.ews = min(ew, cw);
    C.ew = ew;
    C.rw = rwj;
    C.m = (GPtr)lm.b + rm * (uint32_t)wj * EB;
    C.u = C.l = C.c = C.pm = C.pu = C.pl = C.pc = nullptr;
    if (i > 0) C.u = (GPtr)cu.b + ru * (uint32_t)wj * EB;
    if (ew > 0) C.l = (GPtr)lm.a + (rm * (uint32_t)wp + (uint32_t)l) * EB;
    if (i > 0 && ew > 0) C.c = (GPtr)cu.a + (ru * (uint32_t)wp + (uint32_t)l) * EB;
    if (ts) {
      const uint64_t qm = sfp * (uint32_t)hi, qu = sfp * (uint32_t)hp + (uint32_t)u;
      C.pm = (GPtr)plm.b + qm * (uint32_t)wj * EB;
      if (i > 0) C.pu = (GPtr)pcu.b + qu * (uint32_t)wj * EB;
      if (ew > 0) C.pl = (GPtr)plm.a + (qm * (uint32_t)wp + (uint32_t)l) * EB;
      if (i > 0 && ew > 0) C.pc = (GPtr)pcu.a + (qu * (uint32_t)wp + (uint32_t)l) * EB;
    }
    s_col[tid] = C;
  };
  if (col_lane) build_cols(ia, hia, hiam, p0);
  __syncthreads();

  int cur = ia, hi = hia, hp = hiam;
  float rh = rh0;
  int yo = yo0;
  while (yo < yo1) {
    const int i = min((int)fdiv_ms((uint32_t)yo, Rhm, Rhs), nh - 1);
    if (i != cur) { // the band crosses into the next tile row (i > 0)
      hp = A.ext[1][i - 1];
      hi = A.ext[1][i];
      rh = A.rcp[1][i];
      cur = i;
      PtrPair pi[4] = {};
      if (col_lane) load_pairs(i, pi);
      __syncthreads(); // the previous run is done with s_col
      if (col_lane) build_cols(i, hi, hp, pi);
      __syncthreads();
    }
    const int ybase = i * R1;
    const int eh = i > 0 ? min(E1, min(hp, hi)) : 0;
    const int chh = i < nh - 1 ? R1 : hi;
    const int ehs = min(eh, chh);
    const int yl = yo - ybase;
    const bool hs = yl < ehs;
    const int yl1 = min(hs ? ehs : chh, yl + (yo1 - yo));

    SpanRun R;
    R.o = (char *)outp + ((((uint64_t)plane * (uint32_t)LT + (uint32_t)f_out) * (uint32_t)LH + (uint32_t)ybase) *
                              (uint32_t)LW + (uint32_t)xs0) * EB;
    R.opitch = (int64_t)LW * EB;
    R.y0 = yl;
    R.y1 = yl1;
    R.xs0 = xs0;
    R.wv = (xs1 - xs0) / VecInfo<DT, VB>::V;
    R.ja = ja;
    R.nw = nw;
    R.Rwm = Rwm;
    R.Rws = Rws;
    R.eh = eh;
    R.rh = rh;
    R.ct = ct;
    const int cls = (ts ? 2 : 0) | (hs ? 1 : 0);
    switch (cls) {
      case 0: span_rows<DT, VB, false, false>(R, s_col, tid, nthr); break;
      case 1: span_rows<DT, VB, true, false>(R, s_col, tid, nthr); break;
      case 2: span_rows<DT, VB, false, true>(R, s_col, tid, nthr); break;
      default: span_rows<DT, VB, true, true>(R, s_col, tid, nthr); break;
    }
    yo += yl1 - yl;
  }
}
} // namespace sb

template <int DT, int VB>
static void launch_blend_typed(const sb::BlendArgs &a, dim3 grid, dim3 b, size_t lds, hipStream_t st) {
  if (a.nt_store) {
    if (a.off32) hipLaunchKernelGGL((sb::blend_stitch_kernel<DT, VB, uint32_t, true>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((sb::blend_stitch_kernel<DT, VB, int64_t, true>), grid, b, lds, st, a);
  } else {
    if (a.off32) hipLaunchKernelGGL((sb::blend_stitch_kernel<DT, VB, uint32_t, false>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((sb::blend_stitch_kernel<DT, VB, int64_t, false>), grid, b, lds, st, a);
  }
}

hipError_t sb_launch_blend(const sb::BlendArgs &a, int dtype, int vec16, dim3 grid, size_t lds,
                           hipStream_t st) {
  using namespace sb;
  dim3 b(SB_BLEND_THREADS);
  if (dtype == DT_F32) {
    if (vec16) launch_blend_typed<DT_F32, 16>(a, grid, b, lds, st);
    else launch_blend_typed<DT_F32, 4>(a, grid, b, lds, st);
  } else if (dtype == DT_F16) {
    if (vec16) launch_blend_typed<DT_F16, 16>(a, grid, b, lds, st);
    else launch_blend_typed<DT_F16, 2>(a, grid, b, lds, st);
  } else {
    if (vec16) launch_blend_typed<DT_BF16, 16>(a, grid, b, lds, st);
    else launch_blend_typed<DT_BF16, 2>(a, grid, b, lds, st);
  }
  return hipGetLastError();
}

hipError_t sb_launch_blend_span(const sb::BlendArgs &a, int dtype, int vec16, dim3 grid, size_t lds,
                                hipStream_t st) {
  using namespace sb;
  dim3 b(SB_BLEND_THREADS);
  if (dtype == DT_F32) {
    if (vec16) hipLaunchKernelGGL((blend_span_kernel<DT_F32, 16>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((blend_span_kernel<DT_F32, 4>), grid, b, lds, st, a);
  } else if (dtype == DT_F16) {
    if (vec16) hipLaunchKernelGGL((blend_span_kernel<DT_F16, 16>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((blend_span_kernel<DT_F16, 2>), grid, b, lds, st, a);
  } else {
    if (vec16) hipLaunchKernelGGL((blend_span_kernel<DT_BF16, 16>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((blend_span_kernel<DT_BF16, 2>), grid, b, lds, st, a);
  }
  return hipGetLastError();
}
