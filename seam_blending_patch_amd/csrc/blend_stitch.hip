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
// How: the in-place raster recursion has a closed form.  Given that no tile's
// head seam meets its own tail (ext(k) >= e(k) + e(k+1)), the neighbour
// operands read by a seam are untouched by their own blends except for one
// corner term, so each output element needs at most 4 tiles in 2-D:
//
//   s  = D[i][j][y, x]
//   if y < e_h(i):  U  = D[i-1][j][u+y, x]
//                   if x < e_w(j): U = b(D[i-1][j-1][u+y, l+x], U; x, e_w(j))
//                   s  = b(U, s; y, e_h(i))
//   if x < e_w(j):  Lf = D[i][j-1][y, l+x]
//                   if y < e_h(i): Lf = b(D[i-1][j-1][u+y, l+x], Lf; y, e_h(i))
//                   s  = b(Lf, s; x, e_w(j))
//
// with u = h(i-1) - e_h(i), l = w(j-1) - e_w(j), and for frames f < e_t(tau)
// of a temporal tile the same spatial value is taken in both chunks and
// crossfaded, b(S_{tau-1}[t(tau-1) - e_t + f], S_tau[f]; f, e_t): 8 reads.
//
// One thread owns one 16-byte output vector at a time (grid-stride loop over
// the output of one launch window), reads every tile element it needs exactly
// once (the corner operand twice from registers), and writes its output once
// with a nontemporal store.  Interior vectors are a plain bit copy.  The
// coefficient tables are built per block in LDS from float64 division.
// Every product and sum is a separate fp32 operation (the library is built
// with -ffp-contract=off), matching the per-product rounding rule exactly.

#include "sb_internal.h"
#include "sb_vec.h"

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

template <int DT, int VB>
__global__ __launch_bounds__(256) void blend_stitch_kernel(const BlendArgs A) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  extern __shared__ float2 s_pool[];
  __shared__ const char *s_ptr[kMaxWindowTiles];
  __shared__ int32_t s_ext[3][kMaxAxisTiles];
  __shared__ int32_t s_coff[3][kMaxAxisTiles];

  const int tid = threadIdx.x;
  for (int k = tid; k < kMaxWindowTiles; k += blockDim.x) s_ptr[k] = (const char *)A.ptr[k];
  for (int k = tid; k < 3 * kMaxAxisTiles; k += blockDim.x) {
    s_ext[k / kMaxAxisTiles][k % kMaxAxisTiles] = A.ext[k / kMaxAxisTiles][k % kMaxAxisTiles];
    s_coff[k / kMaxAxisTiles][k % kMaxAxisTiles] = A.coff[k / kMaxAxisTiles][k % kMaxAxisTiles];
  }
  // coefficient tables: w_b = fp32(y / e), w_a = fp32(1 - y / e), from double
  for (int a = 0; a < 3; ++a)
    for (int d = 0; d < A.n_dist[a]; ++d) {
      const int e = A.dist_e[a][d], off = A.dist_off[a][d];
      for (int y = tid; y < e; y += blockDim.x) {
        double q = (double)y / (double)e;
        s_pool[off + y] = make_float2((float)(1.0 - q), (float)q);
      }
    }
  __syncthreads();

  const int nw = A.n_w, nh = A.n_h, nt = A.n_t;
  const int Eh = A.E[1], Ew = A.E[2], Et = A.E[0];
  const int Rt = A.R[0], Rh = A.R[1], Rw = A.R[2];
  const uint32_t stride = gridDim.x * blockDim.x;
  char *const out = (char *)A.out;

  for (uint32_t g = blockIdx.x * blockDim.x + tid; g < A.total; g += stride) {
    // output coordinates of this vector
    const uint32_t line = fdiv(g, A.div_Wv);
    const int xv = (int)(g - line * (uint32_t)A.Wv);
    const uint32_t l2 = fdiv(line, A.div_nY);
    const int r = (int)(line - l2 * (uint32_t)A.nY);
    const uint32_t pl = fdiv(l2, A.div_nF);
    const int fo = (int)(l2 - pl * (uint32_t)A.nF);
    const int64_t plane = (int64_t)A.plane0 + pl;
    const int y_out = A.Y0 + r, f_out = A.F0 + fo, x_out = xv * V;
    // tile cell and local coordinates
    const int i = min((int)fdiv((uint32_t)y_out, A.div_Rh), nh - 1);
    const int y = y_out - i * Rh;
    const int tau = min((int)fdiv((uint32_t)f_out, A.div_Rt), nt - 1);
    const int f = f_out - tau * Rt;
    const int j = min((int)fdiv((uint32_t)x_out, A.div_Rw), nw - 1);
    const int x = x_out - j * Rw;

    const int hi = s_ext[1][i], wj = s_ext[2][j];
    const int hp = i > 0 ? s_ext[1][i - 1] : 0;
    const int wp = j > 0 ? s_ext[2][j - 1] : 0;
    const int eh = i > 0 ? min(Eh, min(hp, hi)) : 0;
    const int ew = j > 0 ? min(Ew, min(wp, wj)) : 0;
    const int tp = tau > 0 ? s_ext[0][tau - 1] : 0;
    const int et = tau > 0 ? min(Et, min(tp, s_ext[0][tau])) : 0;
    const bool hs = y < eh, ws = x < ew, ts = f < et;

    const int64_t o_off = (((plane * A.LT + f_out) * A.LH + y_out) * (int64_t)A.LW + x_out) * EB;

    // address of tile (tq, ti, tj) element (plane, fq, yq, xq)
    auto tile_at = [&](int tq, int ti, int tj, int tt, int th, int tw, int fq, int yq, int xq) {
      const char *base = s_ptr[((tq - A.taub) * A.ptr_nh + (ti - A.ib)) * nw + tj];
      return base + ((((plane * tt + fq) * th + yq) * (int64_t)tw + xq) * EB);
    };

    if (!(hs || ws || ts)) {
      const Vec<VB> s = vload<VB, true>(tile_at(tau, i, j, s_ext[0][tau], hi, wj, f, y, x));
      vstore<VB, true>(out + o_off, s);
      continue;
    }

    const int u = hs ? hp - eh : 0;
    const int l = ws ? wp - ew : 0;
    float2 chh = make_float2(0.f, 0.f);
    if (hs) chh = s_pool[s_coff[1][i] + y];
    float2 cww[V];
    if (ws) {
#pragma unroll
      for (int k = 0; k < V; ++k) cww[k] = s_pool[s_coff[2][j] + x + k];
    }

    // spatially stitched value of chunk tq at frame fq (closed form above)
    auto spatial = [&](int tq, int fq, float *o) {
      const int tt = s_ext[0][tq];
      Vec<VB> vs, vu, vl, vc;
      vs = vload<VB, true>(tile_at(tq, i, j, tt, hi, wj, fq, y, x));
      if (hs) vu = vload<VB, true>(tile_at(tq, i - 1, j, tt, hp, wj, fq, u + y, x));
      if (ws) vl = vload<VB, true>(tile_at(tq, i, j - 1, tt, hi, wp, fq, y, l + x));
      if (hs && ws) vc = vload<VB, true>(tile_at(tq, i - 1, j - 1, tt, hp, wp, fq, u + y, l + x));
      unpack<DT, VB>(vs, o);
      if (hs) {
        float U[V];
        unpack<DT, VB>(vu, U);
        if (ws) {
          float Cn[V];
          unpack<DT, VB>(vc, Cn);
#pragma unroll
          for (int k = 0; k < V; ++k) U[k] = crossfade<DT>(Cn[k], U[k], cww[k]);
        }
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = crossfade<DT>(U[k], o[k], chh);
      }
      if (ws) {
        float Lf[V];
        unpack<DT, VB>(vl, Lf);
        if (hs) {
          float Cn[V];
          unpack<DT, VB>(vc, Cn);
#pragma unroll
          for (int k = 0; k < V; ++k) Lf[k] = crossfade<DT>(Cn[k], Lf[k], chh);
        }
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = crossfade<DT>(Lf[k], o[k], cww[k]);
      }
    };

    float S[V];
    spatial(tau, f, S);
    if (ts) {
      float Sp[V];
      spatial(tau - 1, tp - et + f, Sp);
      const float2 ct = s_pool[s_coff[0][tau] + f];
#pragma unroll
      for (int k = 0; k < V; ++k) S[k] = crossfade<DT>(Sp[k], S[k], ct);
    }
    vstore<VB, true>(out + o_off, pack<DT, VB>(S));
  }
}

} // namespace sb

hipError_t sb_launch_blend(const sb::BlendArgs &a, int dtype, int vec16, int grid, size_t lds,
                           hipStream_t st) {
  using namespace sb;
  dim3 g(grid), b(256);
  if (dtype == DT_F32) {
    if (vec16) hipLaunchKernelGGL((blend_stitch_kernel<DT_F32, 16>), g, b, lds, st, a);
    else hipLaunchKernelGGL((blend_stitch_kernel<DT_F32, 4>), g, b, lds, st, a);
  } else if (dtype == DT_F16) {
    if (vec16) hipLaunchKernelGGL((blend_stitch_kernel<DT_F16, 16>), g, b, lds, st, a);
    else hipLaunchKernelGGL((blend_stitch_kernel<DT_F16, 2>), g, b, lds, st, a);
  } else {
    if (vec16) hipLaunchKernelGGL((blend_stitch_kernel<DT_BF16, 16>), g, b, lds, st, a);
    else hipLaunchKernelGGL((blend_stitch_kernel<DT_BF16, 2>), g, b, lds, st, a);
  }
  return hipGetLastError();
}
