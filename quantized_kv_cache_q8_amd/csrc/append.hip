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
// stores are guarded).  A wave covers two rows (tokens) per step and keeps
// ROW_PAIRS steps of loads in flight; a block covers 16 tokens of one head of K or
// of V of one session.  Inputs are read and cache rows written with non-temporal
// accesses (each byte is touched once).
//
// K8V4 (PR #711 "kv: --kv k8v4 streams with --kv-resident", section What: INT8 K and
// a rotated 4-bit V): K takes the int8 path above.  A V row is rotated, w = H x with
// H the Sylvester Hadamard matrix, by fp32 butterflies (stage h pairs dims i and i + h
// inside blocks of 2h, giving a + b and a - b; h = 1, 2, ..., 64), then quantised per
// 32 values: d = fp16(max|w| / 7), code = clamp(rint(w / d), -7, 7), stored as
// code + 8 in nibbles (byte j: value 2j low, 2j + 1 high).  Here 16 lanes hold a row,
// 8 dims each: stages 1, 2, 4 stay in a lane, stages 8 .. 64 pair lanes 1, 2, 4, 8
// apart; each output is one fp32 addition or subtraction of the same two operands as
// in the definition, so the result is bit-identical to it.  A 32-value block is 4
// lanes (a quad): its max is two DPP steps.
#include "kvq8_internal.h"

namespace kvq8 {
namespace {

constexpr int APPEND_THREADS = 256;
constexpr int ROW_PAIRS = 2;                                      // row pairs per wave
constexpr int TOK_PER_BLOCK = (APPEND_THREADS / 64) * ROW_PAIRS * 2;  // 16
static_assert(TOK_PER_BLOCK == (APPEND_THREADS / 64) * 4, "the K8V4 V path: 4 rows per wave");

// Destination row of cell c of session b in head h's rows of its arrays: row c of a
// contiguous session, or, for a paged session, row c % 64 of the pool slot its page
// table names for page c / 64 (-1: the entry lies outside the pool; the row is
// skipped and the session flagged).
struct RowMap {
  const int32_t* pages;   // NULL: contiguous
  int stride;
  __device__ __forceinline__ long long row(const kv_session& s, int b, int h, int c) const {
    if (pages == nullptr) return (long long)h * s.cap + c;
    const int sl = pages[(long long)b * stride + (c >> 6)];
    if (sl < 0 || sl >= s.cap / KV_PAGE_ROWS) return -1;
    return (long long)h * s.cap + (long long)sl * KV_PAGE_ROWS + (c & (KV_PAGE_ROWS - 1));
  }
};

// K8V4 V rows [len + t] of head h: 16 lanes per row, 4 rows per wave (TOK_PER_BLOCK
// rows per block, the same tokens the other paths cover)
__device__ __forceinline__ void append_v_rot4(const kv_session& s, int len, int n_tok, int kvh,
                                              int h, int b, const float* __restrict__ xv,
                                              const RowMap& rm, int32_t* status) {
  const int lane = threadIdx.x & 63;
  const int l = lane & 15;   // dims 8l .. 8l + 7 of the row
  const int t = blockIdx.x * TOK_PER_BLOCK + (threadIdx.x >> 6) * 4 + (lane >> 4);
  float x[8];
  if (t < n_tok) {
    const float* src = xv + (((size_t)b * n_tok + t) * kvh + h) * HD + 8 * l;
    const u32x4 p = ldg128_nt(src), q = ldg128_nt(src + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = as_f32(p[j]);
      x[4 + j] = as_f32(q[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.f;
  }
  // stages 1, 2, 4: pairs inside the lane's 8 dims
#pragma unroll
  for (int hh = 1; hh < 8; hh *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & hh) == 0) {
        const float a = x[j], c = x[j + hh];
        x[j] = a + c;
        x[j + hh] = a - c;
      }
  // stages 8 .. 64: the partner dim is in lane l ^ m; the lower lane keeps a + b,
  // the upper one a - b (a the lower dim's value)
#pragma unroll
  for (int m = 1; m < 16; m *= 2)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __shfl_xor(x[j], m, 64);
      x[j] = (l & m) ? p - x[j] : x[j] + p;
    }
  // 4-bit codes per 32 dims (a quad of lanes)
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[j]));
  a = fmaxf(a, dpp<DPP_QUAD_XOR1>(a));
  a = fmaxf(a, dpp<DPP_QUAD_XOR2>(a));
  const uint16_t dbits = f2h(a / 7.0f);   // IEEE fp32 division, then RNE to fp16
  const float d = h2f(dbits);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float r = d == 0.0f ? 0.0f : rintf(x[j] / d);   // IEEE fp32 division
    const uint32_t nib = (uint32_t)((int)fminf(fmaxf(r, -7.0f), 7.0f) + 8);
    word |= nib << (4 * j);   // dim 8l + j: byte j / 2, low nibble for even j
  }
  if (t < n_tok) {
    const long long r = rm.row(s, b, h, len + t);
    if (r < 0) {
      if (l == 0) flag(status, KV_DEV_BAD_PAGE);
      return;
    }
    const size_t row = (size_t)r;
    uint8_t* dst = static_cast<uint8_t*>(s.v) + row * (HD / 2) + 4 * l;
    __builtin_nontemporal_store(word, (KVQ8_GLOBAL uint32_t*)dst);
    if ((l & 3) == 0) stg16(s.v_scale + row * NQ4 + (l >> 2), dbits);
  }
}

// Grid: x = blocks of TOK_PER_BLOCK tokens, y = (K or V, kv head), z = session.  Every
// index comes from the block coordinates; a block writes the rows [len + t] of one
// head of one of the two arrays.
// A paged session (rm.pages set) holds cells [0, 64 stride): its rows lie in the
// pool slots of its page table.
template <int FMT>
__global__ __launch_bounds__(APPEND_THREADS) void k_append(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int n_tok, int kvh,
    const float* __restrict__ xk, const float* __restrict__ xv, int32_t* __restrict__ status,
    RowMap rm) {
  const int b = blockIdx.z;
  const int which = blockIdx.y >= (unsigned)kvh;   // 0 = K, 1 = V
  const int h = blockIdx.y - which * kvh;
  const kv_session s = tab[b];
  const int len = lens[b];
  int bad = session_bad(s, FMT);
  const long long room = rm.pages == nullptr ? (long long)s.cap : (long long)rm.stride * KV_PAGE_ROWS;
  if (!bad && (len < 0 || (long long)len + n_tok > room)) bad = KV_DEV_RANGE;
  if (bad) {   // the whole session is skipped; one thread of the session reports it
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) flag(status, bad);
    return;
  }
  if constexpr (FMT == KV_FMT_K8V4) {
    if (which) {
      append_v_rot4(s, len, n_tok, kvh, h, b, xv, rm, status);
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;   // which row of the pair
  const int sub = lane & 31;    // float4 index within the row
  const int t0 = blockIdx.x * TOK_PER_BLOCK + (threadIdx.x >> 6) * (ROW_PAIRS * 2);
  // source row (b, t, h) of [n_sess][n_tok][kvh][HD]
  const float* src = (which ? xv : xk) + ((size_t)b * n_tok * kvh + h) * HD + sub * 4;

  float4 x[ROW_PAIRS];
#pragma unroll
  for (int p = 0; p < ROW_PAIRS; ++p) {
    const int t = t0 + 2 * p + half;
    const float* ps = src + (size_t)t * kvh * HD;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < n_tok) {   // the new values are read once: non-temporal
      const u32x4 w = ldg128_nt(ps);
      v = make_float4(as_f32(w[0]), as_f32(w[1]), as_f32(w[2]), as_f32(w[3]));
    }
    x[p] = v;
  }

#pragma unroll
  for (int p = 0; p < ROW_PAIRS; ++p) {
    const int t = t0 + 2 * p + half;
    const long long r = t < n_tok ? rm.row(s, b, h, len + t) : -1;
    if (t < n_tok && r < 0 && sub == 0) flag(status, KV_DEV_BAD_PAGE);
    const bool store = r >= 0;
    const size_t row = store ? (size_t)r : 0;
    if constexpr (FMT != KV_FMT_F16) {   // int8: the Q8 arrays, and the K8V4 K
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
        // the cache rows are not read again by this kernel: non-temporal stores
        int8_t* dst = static_cast<int8_t*>(which ? s.v : s.k) + row * HD + sub * 4;
        __builtin_nontemporal_store(packed, (KVQ8_GLOBAL uint32_t*)dst);
        if ((sub & 15) == 0) stg16((which ? s.v_scale : s.k_scale) + row * NGRP + (sub >> 4), sbits);
      }
    } else {
      const uint32_t lo = (uint32_t)f2h(x[p].x) | ((uint32_t)f2h(x[p].y) << 16);
      const uint32_t hi = (uint32_t)f2h(x[p].z) | ((uint32_t)f2h(x[p].w) << 16);
      if (store) {
        uint16_t* dst = static_cast<uint16_t*>(which ? s.v : s.k) + row * HD + sub * 4;
        __builtin_nontemporal_store(u32x2{lo, hi}, (KVQ8_GLOBAL u32x2*)dst);
      }
    }
  }
}

}  // namespace

hipError_t launch_append(int fmt, int kvh, const kv_session* d_tab, const int32_t* d_len,
                         int n_sess, int n_tok, const float* d_k, const float* d_v,
                         int32_t* d_status, hipStream_t st, const int32_t* d_pages,
                         int page_stride) {
  const long long bx = ((long long)n_tok + TOK_PER_BLOCK - 1) / TOK_PER_BLOCK;
  if (bx > 0x7FFFFFFFLL || 2LL * kvh > 65535 || n_sess > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)bx, 2 * kvh, n_sess), block(APPEND_THREADS);
  const RowMap rm{d_pages, page_stride};
  if (fmt == KV_FMT_Q8)
    hipLaunchKernelGGL(k_append<KV_FMT_Q8>, grid, block, 0, st, d_tab, d_len, n_tok, kvh, d_k,
                       d_v, d_status, rm);
  else if (fmt == KV_FMT_K8V4)
    hipLaunchKernelGGL(k_append<KV_FMT_K8V4>, grid, block, 0, st, d_tab, d_len, n_tok, kvh, d_k,
                       d_v, d_status, rm);
  else
    hipLaunchKernelGGL(k_append<KV_FMT_F16>, grid, block, 0, st, d_tab, d_len, n_tok, kvh, d_k,
                       d_v, d_status, rm);
  return hipGetLastError();
}

}  // namespace kvq8
