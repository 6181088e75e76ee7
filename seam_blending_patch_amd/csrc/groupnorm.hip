// groupnorm.hip -- patch-split GroupNorm with Chan-merged statistics, gfx950.
//
// What is computed (DistVAE PR "Add tiled VAE parallelism & extended model
// support", PatchGroupNorm commits): GroupNorm over C/G channels and all
// spatial positions of each (n, group), with the statistics of every spatial
// patch computed separately and merged so that the result equals unsplit
// GroupNorm -- global mean, variance = M2 / count (no Bessel correction).
// Patches follow the Patchify split (first L mod P patches one longer).
//
// Every statistic is kept about a group shift K_g, the median of five of the
// group's elements spread over it.  Any value of the group would do as a
// shift; one near the mean keeps the fp32 deviations x - K_g, and the mean
// carried as K_g + m, accurate when the mean is large against the spread, and
// taking the median of five keeps up to two outlying samples from being the
// shift.  x - mean is then formed as (x - K_g) - m.
//
// Pass 1 (gn_stats_kernel): one block per (n, g, patch, chunk of the patch).
//   Each thread reads its vectors in batches of a few 16-byte loads.  A batch
//   gets its own count, mean and M2 by two passes over its registers (mean of
//   x - K_g, then the sum of squared deviations from that mean, so M2 never
//   comes from a difference of power sums), and is merged into the thread's
//   running (count, m, M2) with Chan's pairwise formula
//       d = mu_B - mu_A, n = n_A + n_B, mu = mu_A + d n_B / n,
//       M2 = M2_A + M2_B + d^2 n_A n_B / n
//   (Welford's update, a batch at a time).  The block merges its threads by
//   the many-set form of the same merge, n = sum n_l, mu = sum n_l mu_l / n,
//   M2 = sum (M2_l + n_l (mu_l - mu)^2), first across the wavefront (sums by
//   DPP shifts), then across its waves through LDS, and writes one partial
//   (count, m, M2, K_g) to the workspace; counts are integers.
// Pass 2 (gn_norm_kernel): one block per (n, c) plane chunk.  Every wave
//   requests the P x CPP partials of its group, gamma, beta and its vectors
//   of x, and merges the partials by the same many-set formula over fixed
//   sum trees -- the same order in every block, so results are deterministic
//   -- and streams y = ((x - K_g) - m) * (rstd * gamma_c) + beta_c back out
//   with nontemporal stores.  K_g comes from the workspace, not from x, so
//   out may alias x.  Wave 0 of the first block of each group writes the
//   optional per-patch statistics, from a tree of pairwise merges (chunks of
//   a patch first, then patches).

#include "sb_internal.h"
#include "sb_vec.h"

#include "../../include/seam_blend.h"

#include <algorithm>
#include <mutex>

#ifndef SB_GN_NT_STORE
#define SB_GN_NT_STORE 1 // nontemporal hints on y stores (measured faster here, unlike the blend)
#endif
#ifndef SB_GN_NT_LOAD2
// Pass-2 loads of x are plain: when x fits in the 256 MB last-level cache
// they hit the lines pass 1 just brought in (the video-decoder activation's
// normalise pass: 7.8 -> 6.9 us); on larger x the hint makes no difference.
#define SB_GN_NT_LOAD2 0
#endif

namespace sb {

// Statistics of a set of values: integer count, mean and sum of squared
// deviations from the mean (both about the group shift).
struct Stat {
  uint32_t n;
  float mean, m2;
};

// Chan, Golub & LeVeque's pairwise merge; an empty side is the identity.  The
// weight n_B / n is formed with the hardware reciprocal (within one ulp): it
// only scales the correction terms d * r and d^2 n_A r, so its rounding moves
// the merged mean and M2 by about 1e-7 of those terms, and it keeps a full
// division sequence off every level of the merge trees.
__device__ __forceinline__ Stat chan_merge(const Stat &a, const Stat &b) {
  if (b.n == 0) return a;
  if (a.n == 0) return b;
  const uint32_t n = a.n + b.n;
  const float d = b.mean - a.mean;
  const float r = (float)b.n * __builtin_amdgcn_rcpf((float)n);
  Stat o;
  o.n = n;
  o.mean = a.mean + d * r;
  o.m2 = a.m2 + b.m2 + d * d * (float)a.n * r;
  return o;
}

// The statistics of lane l + O (O = 1, 2, 4 or 8, inside the lane's row of
// 16), read with a DPP row shift (a VALU operand modifier, no LDS trip).
template <int O> __device__ __forceinline__ Stat dpp_down_stat(const Stat &s) {
  constexpr int ctrl = 0x100 + O; // row_shl:O -- lane i reads lane i + O of its row
  Stat t;
  t.n = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s.n, ctrl, 0xf, 0xf, false);
  t.mean = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s.mean), ctrl, 0xf, 0xf, false));
  t.m2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s.m2), ctrl, 0xf, 0xf, false));
  return t;
}

// One level of the wavefront merge tree inside rows: lane l (l a multiple of
// 2O) takes in lane l + O.
template <int O> __device__ __forceinline__ void tree_level(Stat &st, int lane) {
  const Stat t = dpp_down_stat<O>(st);
  if ((lane & (2 * O - 1)) == 0) st = chan_merge(st, t);
}

__device__ __forceinline__ Stat readlane_stat(const Stat &s, int l) {
  return Stat{(uint32_t)__builtin_amdgcn_readlane((int)s.n, l),
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.mean), l)),
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s.m2), l))};
}

// Sum over the wavefront by a fixed tree: DPP row shifts by 1, 2, 4 and 8
// (lane l adds lane l + o of its row of 16), then the four row leaders (lanes
// 0, 16, 32, 48) read as scalars and added in pairs.  Returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x101, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x102, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x108, 0xf, 0xf, false));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x101, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x102, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x108, 0xf, 0xf, false);
  return ((uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16)) +
         ((uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
}

// The whole wavefront's statistics from the merge of many sets at once:
// n = sum n_l, mean = sum n_l mean_l / n, M2 = sum (M2_l + n_l (mean_l -
// mean)^2) -- two rounds of plain sums (the second needs the merged mean)
// instead of a chain of pairwise merges, and every term of the M2 sum is
// non-negative.  Lanes without values (n_l = 0) add nothing.  Returned in
// every lane.
__device__ __forceinline__ Stat wave_merge(const Stat &st) {
  const float nl = (float)st.n;
  const uint32_t n = wave_sum(st.n);
  if (n == 0) return Stat{0u, 0.f, 0.f};
  const float mean = wave_sum(nl * st.mean) * __builtin_amdgcn_rcpf((float)n);
  const float d = st.mean - mean;
  return Stat{n, mean, wave_sum(fmaf(nl * d, d, st.m2))};
}

#ifndef SB_GN_STATS_BATCH
#define SB_GN_STATS_BATCH 4
#endif
constexpr int kStatsBatch = SB_GN_STATS_BATCH; // vectors per thread whose loads are in flight together

template <int DT> __device__ __forceinline__ uint32_t load_elem(const void *p, int64_t i) {
  return DT == DT_F32 ? ((const uint32_t *)p)[i] : (uint32_t)((const uint16_t *)p)[i];
}

// The group shift: the median of five of the group's elements, at offsets
// 0, len/4, len/2, 3len/4 and len-1 of its Cg * S contiguous elements from
// g0, so that up to two outlying samples never become the shift.  The median
// is element 2 of a 9-comparator sorting network on the five.
template <int DT>
__device__ __forceinline__ float group_shift(const void *x, int64_t g0, int64_t len) {
  float v[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) v[k] = widen<DT>(load_elem<DT>(x, g0 + (k < 4 ? k * (len / 4) : len - 1)));
  constexpr int net[9][2] = {{0, 1}, {3, 4}, {2, 4}, {2, 3}, {0, 3}, {0, 2}, {1, 4}, {1, 3}, {1, 2}};
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const float lo = fminf(v[net[k][0]], v[net[k][1]]), hi = fmaxf(v[net[k][0]], v[net[k][1]]);
    v[net[k][0]] = lo;
    v[net[k][1]] = hi;
  }
  return v[2];
}

// Merges one batch of up to kStatsBatch vectors (those with ok[u] set) into
// the running statistics st: the batch's own mean and M2 by two passes over
// the registers, then one Chan merge.
template <int DT, int VB>
__device__ __forceinline__ void accumulate_batch(Stat &st, const Vec<VB> (&v)[kStatsBatch],
                                                 const bool (&ok)[kStatsBatch], float K) {
  constexpr int V = VecInfo<DT, VB>::V;
  float d[kStatsBatch][V];
  float s = 0.f;
  uint32_t nb = 0;
#pragma unroll
  for (int u = 0; u < kStatsBatch; ++u) {
    if (ok[u]) {
      unpack<DT, VB>(v[u], d[u]);
#pragma unroll
      for (int k = 0; k < V; ++k) {
        d[u][k] -= K;
        s += d[u][k];
      }
      nb += V;
    }
  }
  if (nb == 0) return;
  const float mb = nb == (uint32_t)(kStatsBatch * V) ? s * (1.0f / (float)(kStatsBatch * V))
                                                      : s / (float)nb;
  float q = 0.f;
#pragma unroll
  for (int u = 0; u < kStatsBatch; ++u)
    if (ok[u]) {
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const float t = d[u][k] - mb;
        q = fmaf(t, t, q);
      }
    }
  st = chan_merge(st, Stat{nb, mb, q});
}

constexpr int kStatsThreads = 64 * kStatsWaves; // threads per pass-1 block (a constant: no launch-argument read)
// the host caps pass-1 grids counting blocks of up to 1024 threads
static_assert(kStatsThreads <= 1024, "pass-1 blocks of at most 1024 threads");

template <int DT, int VB>
__global__ __launch_bounds__(kStatsThreads) void gn_stats_kernel(const GNArgs A, FastDiv div_big,
                                                       FastDiv div_small) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  // Every launch argument the first loads depend on, read at entry and pinned
  // in scalar registers by an empty asm, so that they arrive in one round of
  // scalar loads (left alone, the compiler loads the patch-length divisor
  // through a block-dependent address, a second dependent round).
  uint32_t l2cpp = A.log2CPP, nP = A.P, nG = A.G, nbig = A.n_big, lbig = A.len_big, lsmall = A.len_small;
  uint32_t dPm = A.div_P.m, dPs = A.div_P.s, dGm = A.div_G.m, dGs = A.div_G.s;
  uint32_t bm = div_big.m, bs = div_big.s, sm = div_small.m, ss = div_small.s;
  uint32_t Cc = A.C, Cg = A.Cg, Lx = A.L;
  int64_t inner = A.inner, mid = A.mid, S = A.S;
  asm volatile("" : "+s"(l2cpp), "+s"(nP), "+s"(nG), "+s"(nbig), "+s"(lbig), "+s"(lsmall), "+s"(dPm),
               "+s"(dPs), "+s"(dGm), "+s"(dGs), "+s"(bm), "+s"(bs), "+s"(sm), "+s"(ss), "+s"(Cc), "+s"(Cg),
               "+s"(Lx), "+s"(inner), "+s"(mid), "+s"(S));
  const uint32_t cpp = 1u << l2cpp;
  const int c = b & (cpp - 1);
  const uint32_t rest = (uint32_t)b >> l2cpp;
  const uint32_t np_ = (__umulhi(rest, dPm) + rest) >> dPs; // rest = (n * G + g) * P + p
  const int p = (int)(rest - np_ * nP);
  const int n = (int)((__umulhi(np_, dGm) + np_) >> dGs);
  const int g = (int)(np_ - (uint32_t)n * nG);

  const bool big = (uint32_t)p < nbig;
  const int len = big ? lbig : lsmall;
  const int start = big ? p * lbig : nbig * lbig + (p - nbig) * lsmall;
  const uint32_t runv = (uint32_t)(((int64_t)len * inner) / V);
  const FastDiv dv{runv, big ? bm : sm, big ? bs : ss};
  const uint32_t totalv = (uint32_t)((int64_t)Cg * mid * runv);
  const uint32_t per = (totalv + cpp - 1) >> l2cpp; // chunks per patch are a power of two
  const uint32_t q0 = (uint32_t)c * per;
  const uint32_t q1 = min(q0 + per, totalv);
  const int64_t row = (int64_t)Lx * inner; // elements between consecutive runs
  const int64_t g0 = ((int64_t)n * Cc + (int64_t)g * Cg) * S;
  const char *gbase = (const char *)A.x + (g0 + (int64_t)start * inner) * EB;

  // Vectors q0 + tid + k * kStatsThreads, in batches of kStatsBatch whose loads
  // are issued together.
  Vec<VB> v[kStatsBatch];
  bool ok[kStatsBatch];
  auto load_batch = [&](uint32_t base) {
#pragma unroll
    for (int u = 0; u < kStatsBatch; ++u) {
      const uint32_t q = base + u * kStatsThreads;
      ok[u] = q < q1;
      if (ok[u]) {
        const uint32_t r = fdiv(q, dv);
        const uint32_t pos = q - r * runv;
        v[u] = vload<VB, false>(gbase + ((int64_t)r * row + (int64_t)pos * V) * EB);
      }
    }
  };
  // The first batch is issued before the group shift is read, so the two
  // share one memory latency; every later batch finds K_g in a register.
  Stat st{0u, 0.f, 0.f};
  const uint32_t step = kStatsThreads * kStatsBatch;
  uint32_t base = q0 + tid;
  load_batch(base);
  const float K = group_shift<DT>(A.x, g0, (int64_t)A.Cg * A.S);
  accumulate_batch<DT, VB>(st, v, ok, K);
  for (base += step; base < q1; base += step) {
    load_batch(base);
    accumulate_batch<DT, VB>(st, v, ok, K);
  }
  st = wave_merge(st);
  __shared__ Stat s_w[kStatsWaves];
  if ((tid & 63) == 0) s_w[tid >> 6] = st;
  __syncthreads();
  if (tid == 0) {
    // the waves merged the same way as the lanes
    uint32_t n = 0;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kStatsWaves; ++w) {
      n += s_w[w].n;
      s = fmaf((float)s_w[w].n, s_w[w].mean, s);
    }
    const float mean = n > 0 ? s * __builtin_amdgcn_rcpf((float)n) : 0.f;
    float m2 = 0.f;
#pragma unroll
    for (int w = 0; w < kStatsWaves; ++w) {
      const float d = s_w[w].mean - mean;
      m2 += fmaf((float)s_w[w].n * d, d, s_w[w].m2);
    }
    float4 *dst = reinterpret_cast<float4 *>(A.part) + b;
    *dst = make_float4(__uint_as_float(n), mean, m2, K);
  }
}

// Pass 1 when the patches cut the innermost axis (a W split): a patch run is
// then only a few vectors of each row, and reading it block by block touches
// every row of the group once per patch.  Here a block of kRowsThreads lanes
// covers whole rows instead: lane t keeps one column of the row (t mod the
// row's width in vectors) for the whole block, so each wave reads contiguous
// rows and each lane accumulates for one fixed patch.  The block's lanes are
// then merged by a fixed tree, first across the rows it read (same column),
// then across the columns of each patch, and the block writes one partial per
// patch: chunk c of every patch.  Same partial layout and merge order in pass 2.
constexpr int kRowsThreads = 1024;

// first element column of patch p along the split axis, and its length
__device__ __forceinline__ int patch_start(int p, const GNArgs &A) {
  return p < A.n_big ? p * A.len_big : A.n_big * A.len_big + (p - A.n_big) * A.len_small;
}
__device__ __forceinline__ int patch_len(int p, const GNArgs &A) {
  return p < A.n_big ? A.len_big : A.len_small;
}
// the patch holding element column x (x < L)
__device__ __forceinline__ int patch_of(int x, const GNArgs &A) {
  const int nb = A.n_big * A.len_big;
  return x < nb ? x / A.len_big : A.n_big + (x - nb) / max(A.len_small, 1);
}

template <int DT, int VB>
__global__ __launch_bounds__(kRowsThreads) void gn_stats_rows_kernel(const GNArgs A) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int c = b & (A.CPP - 1);
  const int ng = b >> A.log2CPP; // n * G + g
  const int Wv = A.L / V;        // vectors per row, 1..kRowsThreads (checked on the host)
  const int rpi = kRowsThreads / Wv; // rows per pass of the block
  const int lr = tid / Wv, col = tid - lr * Wv;
  const bool active = lr < rpi;
  const int64_t rows = (int64_t)A.Cg * A.mid; // the group is rows x L contiguous elements
  const int64_t per = (rows + A.CPP - 1) / A.CPP;
  const int64_t r0 = (int64_t)c * per;
  const int64_t r1 = min(r0 + per, rows);
  const int64_t g0 = (int64_t)ng * A.Cg * A.S;
  const char *gbase = (const char *)A.x + g0 * EB + (int64_t)col * V * EB;

  Vec<VB> v[kStatsBatch];
  bool ok[kStatsBatch];
  auto load_batch = [&](int64_t r) {
#pragma unroll
    for (int u = 0; u < kStatsBatch; ++u) {
      const int64_t rr = r + (int64_t)u * rpi;
      ok[u] = active && rr < r1;
      if (ok[u]) v[u] = vload<VB, false>(gbase + rr * A.L * EB);
    }
  };
  // first batch before the group shift, as in gn_stats_kernel
  Stat st{0u, 0.f, 0.f};
  const int64_t step = (int64_t)rpi * kStatsBatch;
  int64_t r = r0 + lr;
  load_batch(r);
  const float K = group_shift<DT>(A.x, g0, (int64_t)A.Cg * A.S);
  accumulate_batch<DT, VB>(st, v, ok, K);
  for (r += step; r < r1; r += step) {
    load_batch(r);
    accumulate_batch<DT, VB>(st, v, ok, K);
  }

  __shared__ Stat s_st[kRowsThreads];
  s_st[tid] = st;
  // rows: row lr takes in row lr + h (same column) while the rows left halve
  for (int n = rpi; n > 1;) {
    const int h = (n + 1) >> 1;
    __syncthreads();
    if (active && lr < n - h) s_st[tid] = chan_merge(s_st[tid], s_st[tid + h * Wv]);
    n = h;
  }
  __syncthreads();
  // columns of row 0: within each patch, column k takes in column k + s
  const int wmax = max(A.len_big, A.len_small) / V; // widest patch, in vectors
  int c0 = 0, c1 = 0;
  if (tid < Wv) {
    const int p = patch_of(tid * V, A);
    c0 = patch_start(p, A) / V;
    c1 = c0 + patch_len(p, A) / V;
  }
  for (int s = 1; s < wmax; s <<= 1) {
    if (tid < Wv && ((tid - c0) & (2 * s - 1)) == 0 && tid + s < c1)
      s_st[tid] = chan_merge(s_st[tid], s_st[tid + s]);
    __syncthreads();
  }
  if (tid < A.P) {
    const Stat m = patch_len(tid, A) > 0 ? s_st[patch_start(tid, A) / V] : Stat{0u, 0.f, 0.f};
    float4 *dst = reinterpret_cast<float4 *>(A.part) + ((int64_t)ng * A.P + tid) * A.CPP + c;
    *dst = make_float4(__uint_as_float(m.n), m.mean, m.m2, K);
  }
}


template <int DT, int VB>
__global__ __launch_bounds__(kNormThreads) void gn_norm_kernel(const GNArgs A) {
  constexpr int V = VecInfo<DT, VB>::V;
  constexpr int EB = Elem<DT>::bytes;
  const int tid = threadIdx.x;
  const uint32_t chunk = blockIdx.x;
  // Every launch argument the first loads depend on, read at entry and pinned
  // in scalar registers, so they arrive in one round of scalar loads (the
  // block size is a constant, not the implicit argument).
  uint32_t plane0 = A.plane0, dCm = A.div_C.m, dCs = A.div_C.s, dGm = A.div_Cg.m, dGs = A.div_Cg.s;
  uint32_t Cc = A.C, Gg = A.G, per = (uint32_t)A.per2, Kp = (uint32_t)(A.P * A.CPP);
  int64_t S = A.S;
  asm volatile("" : "+s"(plane0), "+s"(dCm), "+s"(dCs), "+s"(dGm), "+s"(dGs), "+s"(Cc), "+s"(Gg), "+s"(per),
               "+s"(Kp), "+s"(S));
  const uint32_t plane = plane0 + blockIdx.y; // < 2^31 (checked on the host)
  const uint32_t n = (__umulhi(plane, dCm) + plane) >> dCs;
  const uint32_t ch = plane - n * Cc;
  const uint32_t g = (__umulhi(ch, dGm) + ch) >> dGs;
  const uint32_t ng = n * Gg + g;
  // a channel plane is below 2^31 elements (its group is), so vector indices
  // within it are 32-bit
  const uint32_t Sv = (uint32_t)(S / V);
  const uint32_t q0 = chunk * per;
  const uint32_t q1 = min(q0 + per, Sv);
  const char *xb = (const char *)A.x + (uint64_t)plane * (uint64_t)S * EB;
  char *yb = (char *)A.out + (uint64_t)plane * (uint64_t)S * EB;

  // The group's partials (lane l holds patch l / CPP, chunk l % CPP), this
  // channel's gamma and beta, then the block's vectors of x.  gamma and beta
  // are read unconditionally (from x when absent) and x at a clamped index, so
  // no load sits behind a branch.  The small loads go first: loads return in
  // order, so the merge below waits for them alone while x is still in flight
  // (video activation 7.5 -> 6.9 us, 512x512 one 21.6 -> 21.0 us, against x
  // first).
  const int lane = tid & 63;
  const int K = (int)Kp; // partials of the group (lane l holds patch l / CPP, chunk l % CPP)
  float4 src = make_float4(0.f, 0.f, 0.f, 0.f);
  uint32_t graw, braw;
  Vec<VB> xs[kNormUnroll];
  auto load_small = [&]() {
    if (lane < K) src = reinterpret_cast<const float4 *>(A.part)[(uint64_t)ng * (uint32_t)K + lane];
    graw = load_elem<DT>(A.gamma ? A.gamma : A.x, A.gamma ? ch : 0);
    braw = load_elem<DT>(A.beta ? A.beta : A.x, A.beta ? ch : 0);
  };
  auto load_x = [&]() {
#pragma unroll
    for (int u = 0; u < kNormUnroll; ++u) {
      const uint32_t q = min(q0 + (uint32_t)(u * kNormThreads + tid), q1 - 1); // q1 > q0: the plane is non-empty
      xs[u] = vload<VB, SB_GN_NT_LOAD2>(xb + (size_t)q * (V * EB));
    }
  };
  load_small();
  load_x();
  const float gam = A.gamma ? widen<DT>(graw) : 1.0f;
  const float bet = A.beta ? widen<DT>(braw) : 0.0f;

  // the group's statistics from its partials (lane l holds partial l)
  Stat st{__float_as_uint(src.x), src.y, src.z};
  // the group shift K_g (the same in every partial of the group; lane 0 holds partial 0)
  const float Kg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src.w), 0));
  const bool writer = A.patch_stats != nullptr && chunk == 0 && ch == g * A.Cg && tid < 64;
  const int cppl = A.CPP; // lanes per patch
  if (writer) {
    // the writer wave also runs a tree of pairwise merges, levels o = 1, 2,
    // 4, 8 inside rows (DPP), then rows 0+1, 2+3 and the two halves, whose
    // levels hold each patch's statistics on the way: after the level at
    // which 2o == CPP, lane p * CPP holds patch p
    Stat t = st;
    auto record = [&](const Stat &v, int p) {
      float *d = A.patch_stats + ((size_t)ng * A.P + p) * 3;
      d[0] = (float)v.n; d[1] = v.n > 0 ? Kg + v.mean : 0.f; d[2] = v.m2;
    };
    auto record_rows = [&](int o) {
      if (2 * o == cppl && (lane & (cppl - 1)) == 0 && (lane >> A.log2CPP) < A.P) record(t, lane >> A.log2CPP);
    };
    if (cppl == 1 && lane < A.P) record(t, lane);
    tree_level<1>(t, lane);
    record_rows(1);
    tree_level<2>(t, lane);
    record_rows(2);
    tree_level<4>(t, lane);
    record_rows(4);
    tree_level<8>(t, lane);
    record_rows(8);
    const Stat lo = chan_merge(readlane_stat(t, 0), readlane_stat(t, 16));
    const Stat hi = chan_merge(readlane_stat(t, 32), readlane_stat(t, 48));
    if (cppl == 32 && lane == 0) {
      record(lo, 0);
      if (A.P > 1) record(hi, 1);
    }
    if (cppl == 64 && lane == 0) record(chan_merge(lo, hi), 0);
  }
  st = wave_merge(st);
  const float cnt = (float)st.n;
  const float mean = st.mean;
  const float m2 = st.m2;
  const float var = m2 / cnt;
  const float rstd = 1.0f / sqrtf(var + A.eps);
  const float a = rstd * gam;

#pragma unroll
  for (int u = 0; u < kNormUnroll; ++u) {
    const uint32_t q = q0 + (uint32_t)(u * kNormThreads + tid);
    if (q < q1) {
      float f[V];
      unpack<DT, VB>(xs[u], f);
#pragma unroll
      for (int k = 0; k < V; ++k) f[k] = fmaf((f[k] - Kg) - mean, a, bet);
      vstore<VB, SB_GN_NT_STORE>(yb + (size_t)q * (V * EB), pack<DT, VB>(f));
    }
  }
}

template <int DT, int VB>
static hipError_t launch_gn(const GNArgs &a, hipStream_t st) {
  constexpr int V = VecInfo<DT, VB>::V;
  const int64_t rb = ((int64_t)a.len_big * a.inner) / V;
  const int64_t rs = ((int64_t)a.len_small * a.inner) / V;
  const FastDiv db = make_fastdiv((uint32_t)(rb > 0 ? rb : 1));
  const FastDiv ds = make_fastdiv((uint32_t)(rs > 0 ? rs : 1));
  // pass 1: one block per (n, g, patch, chunk), or per (n, g, chunk of rows);
  // the host keeps the count below 2^24 (2^32 work-items)
  const unsigned blocks1 = (unsigned)((int64_t)a.N * a.G * a.P * a.CPP);
  if (a.rows_layout)
    hipLaunchKernelGGL((gn_stats_rows_kernel<DT, VB>), dim3((unsigned)((int64_t)a.N * a.G * a.CPP)),
                       dim3(kRowsThreads), 0, st, a);
  else
    hipLaunchKernelGGL((gn_stats_kernel<DT, VB>), dim3(blocks1), dim3(kStatsThreads), 0, st, a, db, ds);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // pass 2: (chunks of a plane, planes) with at most kMaxGridY planes per
  // launch; more planes take further launches on the same stream
  const int64_t planes = (int64_t)a.N * a.C;
  GNArgs w = a;
  for (int64_t p0 = 0; p0 < planes; p0 += kMaxGridY) {
    w.plane0 = (uint32_t)p0;
    const dim3 grid2((unsigned)a.chunks2, (unsigned)std::min<int64_t>(kMaxGridY, planes - p0));
    hipLaunchKernelGGL((gn_norm_kernel<DT, VB>), grid2, dim3(kNormThreads), 0, st, w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

} // namespace sb

hipError_t sb_launch_groupnorm(const sb::GNArgs &a, int dtype, int vec16, hipStream_t st) {
  using namespace sb;
  if (dtype == DT_F32) return vec16 ? launch_gn<DT_F32, 16>(a, st) : launch_gn<DT_F32, 4>(a, st);
  if (dtype == DT_F16) return vec16 ? launch_gn<DT_F16, 16>(a, st) : launch_gn<DT_F16, 2>(a, st);
  return vec16 ? launch_gn<DT_BF16, 16>(a, st) : launch_gn<DT_BF16, 2>(a, st);
}

// ---------------------------------------------------------------------------
// Static statistics scratch for patch_groupnorm_noalloc, for callers that
// cannot allocate device memory.  Every GPU the library runs on holds its own
// copy of the array until the process ends; its host-side name is not a
// device address, so the host uses only the address hipGetSymbolAddress
// returns for the current device, looked up once per device and kept.  The
// partials need no clearing: pass 1 writes every entry pass 2 reads.  Every
// call on one GPU shares that GPU's array, so calls that overlap on one GPU
// (on different streams) race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float4 scratch[SB_GN_STATIC_SCRATCH_BYTES / sizeof(float4)];

hipError_t sb_groupnorm_static_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}
