// probe.hip -- streaming probes that give the bench its in-run HBM ceilings.
//
// Not part of the library: a plain copy / read of a given number of bytes,
// with the read and write volumes of the kernel it is compared with, so that
// a kernel's time can be set beside the best time the same traffic takes on
// the same device in the same run.
//
// benchkit_stream reads nread 16-byte vectors of src and writes the first
// nwrite (<= nread) of them to dst at the same index; the vectors it reads but
// does not write are folded into a per-lane value that is stored to sink only
// if it equals a constant (so the loads cannot be dropped, and nothing is
// written in practice).  Each thread handles U vectors of its block's
// contiguous run of 256 * U vectors, all loads issued before any store.  Load
// and store flavours (nontemporal or not) are template choices.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NTL, bool NTS>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ src, int64_t nread,
                                                     u32x4 *__restrict__ dst, int64_t nwrite,
                                                     uint32_t *__restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * 256;
    if (i < nread) v[u] = NTL ? __builtin_nontemporal_load(src + i) : src[i];
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * 256;
    if (i < nwrite) {
      if (NTS) __builtin_nontemporal_store(v[u], dst + i);
      else dst[i] = v[u];
    } else if (i < nread) {
      acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

template <int U>
static hipError_t launch(const void *src, int64_t nread, void *dst, int64_t nwrite, uint32_t *sink, int ntl,
                         int nts, hipStream_t st) {
  const int64_t blocks = (nread + 256 * U - 1) / (256 * U);
  const dim3 g((unsigned)blocks), b(256);
  const u32x4 *s = (const u32x4 *)src;
  u32x4 *d = (u32x4 *)dst;
  if (ntl && nts) hipLaunchKernelGGL((stream_kernel<U, true, true>), g, b, 0, st, s, nread, d, nwrite, sink);
  else if (ntl) hipLaunchKernelGGL((stream_kernel<U, true, false>), g, b, 0, st, s, nread, d, nwrite, sink);
  else if (nts) hipLaunchKernelGGL((stream_kernel<U, false, true>), g, b, 0, st, s, nread, d, nwrite, sink);
  else hipLaunchKernelGGL((stream_kernel<U, false, false>), g, b, 0, st, s, nread, d, nwrite, sink);
  return hipGetLastError();
}

// src: device, at least read_bytes; dst: device, at least write_bytes (may be
// null when write_bytes is 0); sink: device, 256 uint32; read_bytes and
// write_bytes multiples of 16 with write_bytes <= read_bytes; 16-byte aligned
// pointers; u in {1, 2, 4, 8}.  Returns 0, or -1 for bad arguments, or -4 when
// the launch fails.
extern "C" int benchkit_stream(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                               uint32_t *sink, int u, int ntl, int nts, void *stream) {
  if (!src || !sink || read_bytes <= 0 || read_bytes % 16 || write_bytes < 0 || write_bytes % 16 ||
      write_bytes > read_bytes || (write_bytes > 0 && !dst) || ((uintptr_t)src | (uintptr_t)dst) % 16)
    return -1;
  const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
  if ((nr + 255) / 256 >= ((int64_t)1 << 24)) return -1; // grid x within 2^32 work-items
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (u) {
    case 1: e = launch<1>(src, nr, dst, nw, sink, ntl, nts, st); break;
    case 2: e = launch<2>(src, nr, dst, nw, sink, ntl, nts, st); break;
    case 4: e = launch<4>(src, nr, dst, nw, sink, ntl, nts, st); break;
    case 8: e = launch<8>(src, nr, dst, nw, sink, ntl, nts, st); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -4;
}
