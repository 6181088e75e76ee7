// ramp_blend.hip -- normalised-ramp blend of wide tiles for gfx950.
//
// unsloth Studio PR "size seam-free VAE tiles from measured peaks", the
// Qwen-Image-2.1 wide-tile commit: a tile has no weight within a margin of an
// edge it shares with another tile, ramps linearly to full weight over the
// next positions, the weights are normalised to 1 at every position, and the
// tiles are summed into an fp32 accumulator.  Here every output element is
// computed once from the tiles that carry weight at it:
//   out = RN_T( sum_j wx_j(x) * sum_i wy_i(y) * tile_ij[y - oh_i, x - ow_j] )
// with wy, wx the per-axis weights divided by their sum along that axis (the
// 2-D weight is the product of the axes' weights, so its normalisation
// factors into the two axes).
//
// One block covers one (n, c, frame) plane, one column chunk and one band of
// rows of one row segment.  Inside a chunk and a segment the same tiles carry
// weight everywhere (the host splits the axes at every change), so the tile
// set is uniform over the block and the loops take it as template counts.
// The normalised column weights of a chunk with several tiles, and the row
// weights of a segment with several, are built once per block in LDS.  Each
// tile element with weight is read once; each output element is written once.

#include <hip/hip_runtime.h>

#include "sb_internal.h"
#include "sb_vec.h"

#ifndef SB_RAMP_THREADS
#define SB_RAMP_THREADS 256
#endif
// the host puts up to kMaxBlocksX planes on grid x of a launch
static_assert(sb::kMaxBlocksX * SB_RAMP_THREADS < ((int64_t)1 << 32), "grid x within 2^32 work-items");
#ifndef SB_RAMP_BATCH
#define SB_RAMP_BATCH 1 // items whose loads are issued together (more costs occupancy; measured best)
#endif

namespace sb {
namespace {

// factor of one shared edge at whole distance d: clamp((d - m) / r, 0, 1)
__device__ __forceinline__ float edge_factor(int d, int m, float inv_r) {
  return fminf(fmaxf((float)(d - m) * inv_r, 0.0f), 1.0f);
}

// weight of tile k of n (origin o, extent s) at position p along one axis
__device__ __forceinline__ float axis_weight(int p, int o, int s, int k, int n, int m, float inv_r) {
  float w = 1.0f;
  if (k > 0) w *= edge_factor(p - o, m, inv_r);
  if (k < n - 1) w *= edge_factor(o + s - 1 - p, m, inv_r);
  return w;
}

// normalised weights of tiles [k0, k0 + cnt) at position p, into t[k * stride]
__device__ __forceinline__ void normalised_weights(int p, int k0, int cnt, int n, const int32_t *o,
                                                   const int32_t *s, int m, float inv_r, float *t,
                                                   int stride) {
  float w[kRampMaxCover];
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < kRampMaxCover; ++k) {
    w[k] = k < cnt ? axis_weight(p, o[k0 + k], s[k0 + k], k0 + k, n, m, inv_r) : 0.0f;
    sum += w[k];
  }
#pragma unroll
  for (int k = 0; k < kRampMaxCover; ++k)
    if (k < cnt) t[k * stride] = w[k] / sum;
}

// values the whole block shares, read from LDS: held in scalar registers
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const char *uniform(const char *p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const char *)(((uint64_t)hi << 32) | lo);
}

struct Block {
  const char *tile[kRampMaxCover][kRampMaxCover]; // [i][j]: element (y, x) at tile + (y * sw_j + x) * EB
  int32_t tw[kRampMaxCover];                      // row pitch of tile column j, in elements
  char *out;                                      // element (y, x) at out + (y * LW + x) * EB
  int32_t LW;
  int32_t x0, y0, cols, rows;
  const float *ww; // [j][c]: normalised column weights (several tiles)
  const float *wh; // [i][r]: normalised row weights (several tiles)
};

// The items of one block: (row r, vector v) for r < rows, v < cols / V,
// thread t takes items t, t + THREADS, ... walked without division.
template <int DT, int VB, int NH, int NW>
__device__ __forceinline__ void run_items(const Block &B, int nh, int nw) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int U = SB_RAMP_BATCH;
  constexpr bool RT = NH == 0; // tile counts known only at run time (up to 4 x 4)
  const int nvec = B.cols / V;
  const int step_r = SB_RAMP_THREADS / nvec, step_c = SB_RAMP_THREADS - step_r * nvec;
  int r = (int)threadIdx.x / nvec;
  int cv = (int)threadIdx.x - r * nvec;
  while (r < B.rows) {
    int ir[U], ic[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      live[u] = r < B.rows;
      ir[u] = r;
      ic[u] = cv;
      cv += step_c;
      r += step_r;
      if (cv >= nvec) {
        cv -= nvec;
        ++r;
      }
    }
    if constexpr (NH == 1 && NW == 1) {
      // one tile with weight 1: the value itself
      Vec<VB> v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u])
          v[u] = vload<VB, true>(B.tile[0][0] + ((int64_t)(B.y0 + ir[u]) * B.tw[0] + B.x0 + ic[u] * V) * EB);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u]) vstore<VB, false>(B.out + ((int64_t)(B.y0 + ir[u]) * B.LW + B.x0 + ic[u] * V) * EB, v[u]);
    } else if constexpr (!RT) {
      Vec<VB> v[U][NH][NW];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u]) {
#pragma unroll
          for (int i = 0; i < NH; ++i)
#pragma unroll
            for (int j = 0; j < NW; ++j)
              v[u][i][j] = vload<VB, true>(B.tile[i][j] +
                                           ((int64_t)(B.y0 + ir[u]) * B.tw[j] + B.x0 + ic[u] * V) * EB);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!live[u]) continue;
        float hw[NH];
#pragma unroll
        for (int i = 0; i < NH; ++i) hw[i] = NH == 1 ? 1.0f : B.wh[i * B.rows + ir[u]];
        float acc[V];
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
          float col[V];
#pragma unroll
          for (int e = 0; e < V; ++e) col[e] = 0.0f;
#pragma unroll
          for (int i = 0; i < NH; ++i) {
            float f[V];
            unpack<DT, VB>(v[u][i][j], f);
#pragma unroll
            for (int e = 0; e < V; ++e) col[e] = fmaf(hw[i], f[e], col[e]);
          }
          if constexpr (NW == 1) {
#pragma unroll
            for (int e = 0; e < V; ++e) acc[e] = col[e];
          } else {
            const float *cw = B.ww + j * B.cols + ic[u] * V;
#pragma unroll
            for (int e = 0; e < V; ++e) acc[e] = fmaf(cw[e], col[e], acc[e]);
          }
        }
        vstore<VB, false>(B.out + ((int64_t)(B.y0 + ir[u]) * B.LW + B.x0 + ic[u] * V) * EB,
                          pack<DT, VB>(acc));
      }
    } else {
      // general case: up to 4 x 4 tiles, one item at a time (the loops are
      // unrolled to the maximum so the tile table stays in registers)
#pragma unroll 1
      for (int u = 0; u < U; ++u) {
        if (!live[u]) continue;
        float acc[V];
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < kRampMaxCover; ++j) {
          if (j >= nw) break;
          float col[V];
#pragma unroll
          for (int e = 0; e < V; ++e) col[e] = 0.0f;
#pragma unroll
          for (int i = 0; i < kRampMaxCover; ++i) {
            if (i >= nh) break;
            const float hw = nh == 1 ? 1.0f : B.wh[i * B.rows + ir[u]];
            float f[V];
            unpack<DT, VB>(vload<VB, true>(B.tile[i][j] + ((int64_t)(B.y0 + ir[u]) * B.tw[j] + B.x0 + ic[u] * V) * EB), f);
#pragma unroll
            for (int e = 0; e < V; ++e) col[e] = fmaf(hw, f[e], col[e]);
          }
          const float *cw = B.ww + j * B.cols + ic[u] * V;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = nw == 1 ? col[e] : fmaf(cw[e], col[e], acc[e]);
        }
        vstore<VB, false>(B.out + ((int64_t)(B.y0 + ir[u]) * B.LW + B.x0 + ic[u] * V) * EB,
                          pack<DT, VB>(acc));
      }
    }
  }
}

template <int DT, int VB>
__global__ __launch_bounds__(SB_RAMP_THREADS) void ramp_blend_kernel(const RampArgs A) {
  extern __shared__ float lds[];
  __shared__ RampTables T;
  constexpr int EB = Elem<DT>::bytes;
  const int64_t plane = A.plane0 + blockIdx.x;
  const int c = blockIdx.y;
  const int band = blockIdx.z;
  constexpr uint32_t PM = (1u << kRampPosBits) - 1u;

  // the decode tables, copied to LDS in one cooperative load
  {
    constexpr int n16 = (int)(sizeof(RampTables) / 16);
    const uint4 *src = reinterpret_cast<const uint4 *>(&A.t);
    uint4 *dst = reinterpret_cast<uint4 *>(&T);
    for (int q = threadIdx.x; q < n16; q += SB_RAMP_THREADS) dst[q] = src[q];
  }
  __syncthreads();

  // column chunk
  const uint32_t cp = (uint32_t)uniform((int)T.chunk[c]);
  const int x0 = (int)(cp & PM), j0 = (int)((cp >> kRampPosBits) & 63u), nw = (int)(cp >> 26) + 1;
  const int x1 = uniform((int)(T.chunk[c + 1] & PM));
  // row segment holding this band (the last with band0 <= band)
  const int nseg = uniform(T.nseg);
  int s = 0;
  while (s + 1 < nseg && uniform(T.band0[s + 1]) <= band) ++s;
  const uint32_t sp = (uint32_t)uniform((int)T.seg[s]);
  const int sy0 = (int)(sp & PM), i0 = (int)((sp >> kRampPosBits) & 63u), nh = (int)(sp >> 26) + 1;
  const int sy1 = uniform((int)(T.seg[s + 1] & PM));
  const int rows_pb = uniform(T.rows_pb);
  const int y0 = sy0 + (band - uniform(T.band0[s])) * rows_pb;
  const int y1 = min(y0 + rows_pb, sy1);

  Block B;
  B.LW = uniform(T.LW);
  B.x0 = x0;
  B.y0 = y0;
  B.cols = x1 - x0;
  B.rows = y1 - y0;
  B.out = (char *)A.out + plane * (int64_t)uniform(T.LH) * B.LW * EB;
#pragma unroll
  for (int i = 0; i < kRampMaxCover; ++i)
#pragma unroll
    for (int j = 0; j < kRampMaxCover; ++j) {
      if (i < nh && j < nw) {
        const int ti = i0 + i, tj = j0 + j;
        // element (y, x) of the output at tile element (y - oh, x - ow)
        const int64_t base = (plane * T.sh[ti] - T.oh[ti]) * (int64_t)T.sw[tj] - T.ow[tj];
        // (the index is uniform, so the pointer is a scalar load of the
        // launch arguments and keeps its global address space)
        B.tile[i][j] = (const char *)A.ptr[uniform((ti - T.ib) * T.n_w + tj)] + base * EB;
      } else {
        B.tile[i][j] = nullptr;
      }
    }
#pragma unroll
  for (int j = 0; j < kRampMaxCover; ++j) B.tw[j] = j < nw ? uniform(T.sw[j0 + j]) : 0;

  // normalised weight tables for the axes with several tiles
  float *ww = lds;
  float *wh = lds + (nw > 1 ? nw * B.cols : 0);
  B.ww = ww;
  B.wh = wh;
  if (nw > 1)
    for (int q = threadIdx.x; q < B.cols; q += SB_RAMP_THREADS)
      normalised_weights(x0 + q, j0, nw, T.n_w, T.ow, T.sw, T.mw, T.inv_rw, ww + q, B.cols);
  if (nh > 1)
    for (int q = threadIdx.x; q < B.rows; q += SB_RAMP_THREADS)
      normalised_weights(y0 + q, i0, nh, T.n_h, T.oh, T.sh, T.mh, T.inv_rh, wh + q, B.rows);
  if (nw > 1 || nh > 1) __syncthreads();

  const int cls = (nh > 2 || nw > 2) ? 0 : (nh - 1) * 2 + (nw - 1);
  switch (cls) {
    case 0:
      if (nh == 1 && nw == 1) run_items<DT, VB, 1, 1>(B, 1, 1);
      else run_items<DT, VB, 0, 0>(B, nh, nw);
      break;
    case 1: run_items<DT, VB, 1, 2>(B, 1, 2); break;
    case 2: run_items<DT, VB, 2, 1>(B, 2, 1); break;
    default: run_items<DT, VB, 2, 2>(B, 2, 2); break;
  }
}

} // namespace
} // namespace sb

hipError_t sb_launch_ramp(const sb::RampArgs &a, int dtype, int vec16, dim3 grid, size_t lds, hipStream_t st) {
  using namespace sb;
  dim3 b(SB_RAMP_THREADS);
  if (dtype == DT_F32) {
    if (vec16) hipLaunchKernelGGL((ramp_blend_kernel<DT_F32, 16>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((ramp_blend_kernel<DT_F32, 4>), grid, b, lds, st, a);
  } else if (dtype == DT_F16) {
    if (vec16) hipLaunchKernelGGL((ramp_blend_kernel<DT_F16, 16>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((ramp_blend_kernel<DT_F16, 2>), grid, b, lds, st, a);
  } else {
    if (vec16) hipLaunchKernelGGL((ramp_blend_kernel<DT_BF16, 16>), grid, b, lds, st, a);
    else hipLaunchKernelGGL((ramp_blend_kernel<DT_BF16, 2>), grid, b, lds, st, a);
  }
  return hipGetLastError();
}
