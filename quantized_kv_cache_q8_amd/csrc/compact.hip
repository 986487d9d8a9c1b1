// Compaction of cache rows [0, P) into the FP16 [kvh][P][HD] copy that the prompt
// chunk's matrix products read (PR #3084 "FP16 K/V cache by default, int8 with
// --kv-q8", section Extra Notes: the prompt path stages the cache as fp16 halves
// of shape [kvh][P][HD]; with an FP16 cache this is a pure copy).
//   q8 : fp16_rne(float(code) * float(scale)); the fp32 product is exact, so the
//        result is the correctly rounded fp16 of code * scale.
//   F16: the rows are copied (the row stride changes from cap to P).
//   K8V4 (PR #711 "kv: --kv k8v4 streams with --kv-resident", section What): K as q8;
//        a V row is rotated back: u = (nibble - 8) * d (exact in fp32), the fp32
//        butterflies of the write path (H u), times 2^-7 (exact), fp16_rne.
// Mapping: 8 lanes per int8 row (16 codes = one 128-bit load each, 2 x 128-bit
// stores), 16 lanes per fp16 row (one 128-bit load and store each), 16 lanes per
// K8V4 V row (4 bytes of nibbles in, 8 dims = one 128-bit store out each).
#include "kvq8_internal.h"

namespace kvq8 {
namespace {

constexpr int CMP_THREADS = 256;

__global__ __launch_bounds__(CMP_THREADS) void k_compact_q8(
    const int8_t* __restrict__ kc, const int8_t* __restrict__ vc,
    const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs, int cap, int P,
    long long half, long long n_rows, uint16_t* __restrict__ k16, uint16_t* __restrict__ v16) {
  const long long gid = (long long)blockIdx.x * CMP_THREADS + threadIdx.x;
  const long long row = gid >> 3;  // over [K rows: half][V rows: n_rows - half]
  const int c = (int)(gid & 7);
  if (row >= n_rows) return;
  const int which = row >= half;
  const long long rr = which ? row - half : row;  // h * P + t
  const long long h = rr / P, t = rr % P;
  const long long src = h * cap + t;
  const uint4 w = *reinterpret_cast<const uint4*>((which ? vc : kc) + src * HD + c * 16);
  const float sc = h2f((which ? vs : ks)[src * NGRP + (c >> 2)]);
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t x = words[k];
    const float f0 = (float)(int8_t)(x) * sc, f1 = (float)(int8_t)(x >> 8) * sc;
    const float f2 = (float)(int8_t)(x >> 16) * sc, f3 = (float)(int8_t)(x >> 24) * sc;
    o[2 * k] = (uint32_t)f2h(f0) | ((uint32_t)f2h(f1) << 16);
    o[2 * k + 1] = (uint32_t)f2h(f2) | ((uint32_t)f2h(f3) << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>((which ? v16 : k16) + rr * HD + c * 16);
  dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
  dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

__global__ __launch_bounds__(CMP_THREADS) void k_compact_f16(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc, int cap, int P,
    long long n_rows, uint16_t* __restrict__ k16, uint16_t* __restrict__ v16) {
  const long long gid = (long long)blockIdx.x * CMP_THREADS + threadIdx.x;
  const long long row = gid >> 4;
  const int c = (int)(gid & 15);
  if (row >= n_rows) return;
  const long long half = n_rows / 2;
  const int which = row >= half;
  const long long rr = which ? row - half : row;
  const long long h = rr / P, t = rr % P;
  const uint4 v = *reinterpret_cast<const uint4*>((which ? vc : kc) + (h * cap + t) * HD + c * 8);
  *reinterpret_cast<uint4*>((which ? v16 : k16) + rr * HD + c * 8) = v;
}

// K8V4 V rows: 16 lanes per row (a row's lanes return together, so every shuffle
// partner is active); lane l holds dims 8l .. 8l + 7
__global__ __launch_bounds__(CMP_THREADS) void k_compact_v4(
    const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs, int cap, int P,
    long long n_rows, uint16_t* __restrict__ v16) {
  const long long gid = (long long)blockIdx.x * CMP_THREADS + threadIdx.x;
  const long long rr = gid >> 4;  // h * P + t
  const int l = (int)(gid & 15);
  if (rr >= n_rows) return;
  const long long h = rr / P, t = rr % P;
  const long long src = h * cap + t;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(vc + src * (HD / 2) + 4 * l);
  const float d = h2f(vs[src * NQ4 + (l >> 2)]);
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)((int)((w >> (4 * j)) & 15u) - 8) * d;  // exact
#pragma unroll
  for (int hh = 1; hh < 8; hh *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & hh) == 0) {
        const float a = x[j], c = x[j + hh];
        x[j] = a + c;
        x[j + hh] = a - c;
      }
#pragma unroll
  for (int m = 1; m < 16; m *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __shfl_xor(x[j], m, 64);
      x[j] = (l & m) ? p - x[j] : x[j] + p;
    }
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = (uint32_t)f2h(x[2 * k] * 0.0078125f) | ((uint32_t)f2h(x[2 * k + 1] * 0.0078125f) << 16);
  *reinterpret_cast<uint4*>(v16 + rr * HD + 8 * l) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_compact(int fmt, int kvh, const kv_session& s, int P, uint16_t* d_k16,
                          uint16_t* d_v16, hipStream_t st) {
  const long long n_rows = 2LL * kvh * P;
  const int lanes_per_row = fmt == KV_FMT_Q8 ? 8 : 16;
  const long long blocks = (n_rows * lanes_per_row + CMP_THREADS - 1) / CMP_THREADS;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (fmt == KV_FMT_Q8) {
    hipLaunchKernelGGL(k_compact_q8, dim3((unsigned)blocks), dim3(CMP_THREADS), 0, st,
                       static_cast<const int8_t*>(s.k), static_cast<const int8_t*>(s.v),
                       s.k_scale, s.v_scale, s.cap, P, n_rows / 2, n_rows, d_k16, d_v16);
  } else if (fmt == KV_FMT_K8V4) {
    const long long half = n_rows / 2;   // kvh * P rows of K, then as many of V
    const long long kb = (half * 8 + CMP_THREADS - 1) / CMP_THREADS;
    const long long vb = (half * 16 + CMP_THREADS - 1) / CMP_THREADS;
    if (vb > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_compact_q8, dim3((unsigned)kb), dim3(CMP_THREADS), 0, st,
                       static_cast<const int8_t*>(s.k), static_cast<const int8_t*>(s.k),
                       s.k_scale, s.k_scale, s.cap, P, half, half, d_k16, d_k16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_compact_v4, dim3((unsigned)vb), dim3(CMP_THREADS), 0, st,
                       static_cast<const uint8_t*>(s.v), s.v_scale, s.cap, P, half, d_v16);
  } else
    hipLaunchKernelGGL(k_compact_f16, dim3((unsigned)blocks), dim3(CMP_THREADS), 0, st,
                       static_cast<const uint16_t*>(s.k), static_cast<const uint16_t*>(s.v), s.cap,
                       P, n_rows, d_k16, d_v16);
  return hipGetLastError();
}

}  // namespace kvq8
