// Writing new cells into the cache: quantise-on-write (int8 + fp16 scale per 64 dims)
// or the FP16 store.
//
// Rule (PR #3084 "FP16 K/V cache by default, int8 with --kv-q8", section What
// changed): per 64-dim group of one head row, scale = fp16(max|x| / 127) and
// code = clamp(rint(x / scale), -127, 127).  Here: max|x| exact in fp32, IEEE fp32
// division (no reciprocal), round-to-nearest-even to fp16, division by the stored
// fp16 scale widened to fp32, rint = round half to even, code 0 when scale == 0.
//
// Mapping (wave64): one head row of 128 fp32 values is 32 lanes x float4; a
// 64-dim group is one 16-lane DPP row, so the group max is four DPP steps and
// needs no LDS and no workgroup barrier (the page's kernel needed a block-wide
// barrier for the same max; here every lane reaches the DPP steps and only the
// stores are guarded).  A wave covers two rows per step and keeps ROWS_PAIRS
// steps of loads in flight.
#include "kvq8_internal.h"

namespace kvq8 {
namespace {

constexpr int APPEND_THREADS = 256;
constexpr int ROW_PAIRS = 4;  // row pairs per wave

struct RowRef {
  int b, t, h, which;  // session, token, kv head, 0 = K / 1 = V
  long long src;       // element offset of the row in its input array
};

__device__ __forceinline__ RowRef decode_row(long long r, int n_sess, int n_tok, int kvh) {
  const long long per = (long long)n_sess * n_tok * kvh;
  RowRef o;
  o.which = r >= per;
  const long long rem = o.which ? r - per : r;
  o.h = (int)(rem % kvh);
  const long long bt = rem / kvh;
  o.t = (int)(bt % n_tok);
  o.b = (int)(bt / n_tok);
  o.src = rem * HD;
  return o;
}

template <int FMT>
__global__ __launch_bounds__(APPEND_THREADS) void k_append(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int n_sess, int n_tok,
    int kvh, const float* __restrict__ xk, const float* __restrict__ xv,
    int32_t* __restrict__ status) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;   // which row of the pair
  const int sub = lane & 31;    // float4 index within the row
  const long long n_rows = 2LL * n_sess * n_tok * kvh;
  const long long wave = (long long)blockIdx.x * (APPEND_THREADS / 64) + (threadIdx.x >> 6);

  float4 x[ROW_PAIRS];
  RowRef rr[ROW_PAIRS];
  bool in[ROW_PAIRS];
#pragma unroll
  for (int p = 0; p < ROW_PAIRS; ++p) {
    const long long r = (wave * ROW_PAIRS + p) * 2 + half;
    in[p] = r < n_rows;
    rr[p] = decode_row(in[p] ? r : 0, n_sess, n_tok, kvh);
    const float* src = (rr[p].which ? xv : xk) + rr[p].src + sub * 4;
    x[p] = in[p] ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

#pragma unroll
  for (int p = 0; p < ROW_PAIRS; ++p) {
    const RowRef& o = rr[p];
    const kv_session s = tab[o.b];
    const int len = lens[o.b];
    int bad = session_bad(s, FMT);
    if (!bad && (len < 0 || (long long)len + n_tok > s.cap)) bad = KV_DEV_RANGE;
    const bool store = in[p] && !bad;
    const long long row = (long long)o.h * s.cap + (long long)len + o.t;  // [kvh][cap] row

    if constexpr (FMT == KV_FMT_Q8) {
      float a = fmaxf(fmaxf(fabsf(x[p].x), fabsf(x[p].y)), fmaxf(fabsf(x[p].z), fabsf(x[p].w)));
      a = max16(a);                                  // group max: all 16 lanes of the group
      const uint16_t sbits = f2h(a / 127.0f);        // IEEE fp32 division, then RNE to fp16
      const float sc = h2f(sbits);
      int c[4];
      const float xs[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = sc == 0.0f ? 0.0f : rintf(xs[i] / sc);   // IEEE fp32 division
        c[i] = (int)fminf(fmaxf(r, -127.0f), 127.0f);
      }
      const uint32_t packed = (uint32_t)(c[0] & 0xFF) | ((uint32_t)(c[1] & 0xFF) << 8) |
                              ((uint32_t)(c[2] & 0xFF) << 16) | ((uint32_t)(c[3] & 0xFF) << 24);
      if (store) {
        stg32(static_cast<int8_t*>(o.which ? s.v : s.k) + row * HD + sub * 4, packed);
        if ((sub & 15) == 0) stg16((o.which ? s.v_scale : s.k_scale) + row * NGRP + (sub >> 4), sbits);
      }
    } else {
      const uint32_t lo = (uint32_t)f2h(x[p].x) | ((uint32_t)f2h(x[p].y) << 16);
      const uint32_t hi = (uint32_t)f2h(x[p].z) | ((uint32_t)f2h(x[p].w) << 16);
      if (store) {
        stg64(static_cast<uint16_t*>(o.which ? s.v : s.k) + row * HD + sub * 4, u32x2{lo, hi});
      }
    }
    if (in[p] && bad && sub == 0 && o.t == 0 && o.h == 0 && o.which == 0) flag(status, bad);
  }
}

}  // namespace

hipError_t launch_append(int fmt, int kvh, const kv_session* d_tab, const int32_t* d_len,
                         int n_sess, int n_tok, const float* d_k, const float* d_v,
                         int32_t* d_status, hipStream_t st) {
  const long long n_rows = 2LL * n_sess * n_tok * kvh;
  const long long rows_per_block = (APPEND_THREADS / 64) * ROW_PAIRS * 2;
  const long long blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(APPEND_THREADS);
  if (fmt == KV_FMT_Q8)
    hipLaunchKernelGGL(k_append<KV_FMT_Q8>, grid, block, 0, st, d_tab, d_len, n_sess, n_tok, kvh,
                       d_k, d_v, d_status);
  else
    hipLaunchKernelGGL(k_append<KV_FMT_F16>, grid, block, 0, st, d_tab, d_len, n_sess, n_tok, kvh,
                       d_k, d_v, d_status);
  return hipGetLastError();
}

}  // namespace kvq8
