// Measurement aid, not part of the method: a plain read of a device buffer with the
// loads a decode makes (128-bit, non-temporal, every CU busy), and no arithmetic.
// Its rate is the read bandwidth the decode figures can be set against.
#include "kvq8_internal.h"

namespace kvq8 {
namespace {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;
constexpr size_t PROBE_CHUNK = (size_t)PROBE_THREADS * PROBE_UNROLL;  // 16-byte words per workgroup

// Workgroup w reads words [w * PROBE_CHUNK, (w + 1) * PROBE_CHUNK): PROBE_UNROLL
// coalesced loads per thread, all in flight at once.  Many short workgroups keep
// every CU fed to the end (measured: faster than a resident grid striding over the
// buffer).  The XOR of what a thread read is stored only when it equals an
// arbitrary constant, which keeps the loads live without a store per thread.
__global__ __launch_bounds__(PROBE_THREADS) void k_stream_read(const u32x4* __restrict__ src,
                                                               size_t n16, uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * PROBE_CHUNK + threadIdx.x;
  uint32_t acc = 0;
  if (base + (PROBE_UNROLL - 1) * PROBE_THREADS < n16) {
    u32x4 v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = ldg128_nt(src + base + u * PROBE_THREADS);
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  } else {
    for (size_t i = base; i < n16; i += PROBE_THREADS) {
      const u32x4 v = ldg128_nt(src + i);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t blocks = (n16 + PROBE_CHUNK - 1) / PROBE_CHUNK;
  if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;  // past the grid's x extent
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(PROBE_THREADS), 0, st,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace kvq8
