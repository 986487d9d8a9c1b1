// Split-K decode attention over the cache, reading the cache format directly
// (PR #3084 "FP16 K/V cache by default, int8 with --kv-q8", sections What changed
// and Extra Notes: the next token's split-K decode reads the cache, FP16 or int8,
// with no conversion pass).
//
// k_decode_split: one workgroup = (split s, kv head h, session b), T tokens.
//   Each of its 4 waves owns T/4 consecutive tokens and works in two passes:
//   K pass   lane (r = lane/8, c = lane%8) holds dims [16c, 16c+16) of token r of
//            each 8-token step: 128-bit loads (int8: 16 codes; fp16: 2 x 8 halves),
//            dequant in registers, partial dots for the G query heads, the int8
//            group scale applied to the partial, and an 8-lane DPP sum; logits
//            (already in log2 units) go to LDS.
//   softmax  wave max and exp2 over its logits; p back to LDS.
//   V pass   same lane mapping, acc[g][16 dims] += p * scale * v.
//   The 4 wave partials are combined in LDS and written as one (o, lse) per
//   query head and split (o normalised, lse in log2 units).
// k_decode_merge: out = sum_j 2^(lse_j - L) o_j with L = log2 sum_j 2^lse_j.
//
// Dequantised values are exact in fp32 (a 7-bit code times an 11-bit fp16
// significand), so the only rounding is fp32 accumulation.
#include "kvq8_internal.h"

namespace kvq8 {
namespace {

// rows (8-token steps) per load batch; a wave alternates two batches
#ifndef KVQ8_DEC_U_Q8
#define KVQ8_DEC_U_Q8 4
#endif
#ifndef KVQ8_DEC_U_F16
#define KVQ8_DEC_U_F16 2
#endif
// K/V rows are read once per decode: non-temporal loads keep them out of the caches
#ifndef KVQ8_DEC_NT
#define KVQ8_DEC_NT 1
#endif
// minimum resident waves per SIMD the register allocation must allow
#ifndef KVQ8_DEC_WAVES_PER_EU
#define KVQ8_DEC_WAVES_PER_EU 1
#endif
// largest tokens per workgroup the split heuristic may pick
#ifndef KVQ8_DEC_T_MAX
#define KVQ8_DEC_T_MAX 1024
#endif

__device__ __forceinline__ u32x4 ldkv(const void* p) {
  if constexpr (KVQ8_DEC_NT) return ldg128_nt(p);
  return ldg128(p);
}

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16 values of one lane's row chunk, as fp32
template <int FMT>
struct Chunk;

template <>
struct Chunk<KV_FMT_Q8> {
  u32x4 w;  // 16 int8 codes
  __device__ __forceinline__ void load(const void* base, long long row, int c) {
    w = ldkv(static_cast<const int8_t*>(base) + row * HD + c * 16);
  }
  __device__ __forceinline__ float get(int i) const {
    return (float)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
};

template <>
struct Chunk<KV_FMT_F16> {
  u32x4 a, b;  // 16 fp16 values: dims [8c, 8c+8) and [64+8c, 64+8c+8)
  __device__ __forceinline__ void load(const void* base, long long row, int c) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row * HD + c * 8;
    a = ldkv(p);        // the 8 lanes of a row cover bytes [0, 128) of it
    b = ldkv(p + 64);   // ... and bytes [128, 256)
  }
  __device__ __forceinline__ float get(int i) const {
    const u32x4& v = i < 8 ? a : b;
    const int j = i & 7;
    return h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
  }
};

// Head dim of the i-th of the 16 values a lane (c = lane % 8) holds of a row.
template <int FMT>
__device__ __forceinline__ int lane_dim(int c, int i) {
  if constexpr (FMT == KV_FMT_Q8) return 16 * c + i;  // one 64-dim scale group per lane
  return i < 8 ? 8 * c + i : 64 + 8 * c + (i - 8);
}

// p of G query heads for one token from LDS (one 16/8/4-byte read)
template <int G>
__device__ __forceinline__ void load_p(const float* src, float (&p)[G]) {
  if constexpr (G % 4 == 0) {
#pragma unroll
    for (int g = 0; g < G; g += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + g);
      p[g] = v.x; p[g + 1] = v.y; p[g + 2] = v.z; p[g + 3] = v.w;
    }
  } else if constexpr (G == 2) {
    const float2 v = *reinterpret_cast<const float2*>(src);
    p[0] = v.x; p[1] = v.y;
  } else {
    p[0] = src[0];
  }
}

// G logits of one token to LDS (one lane per 8-lane row), as 16/8/4-byte stores
template <int G>
__device__ __forceinline__ void store_logits(float* dst, const float (&v)[G], bool valid) {
  float x[G];
#pragma unroll
  for (int g = 0; g < G; ++g) x[g] = valid ? v[g] : -INFINITY;
  if constexpr (G % 4 == 0) {
#pragma unroll
    for (int g = 0; g < G; g += 4)
      *reinterpret_cast<float4*>(dst + g) = make_float4(x[g], x[g + 1], x[g + 2], x[g + 3]);
  } else if constexpr (G == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(x[0], x[1]);
  } else {
    dst[0] = x[0];
  }
}

// One batch of U rows (8 tokens each per wave) of K or V for one lane: U x 16 values
// and, for int8, the U raw fp16 scales of the lane's 64-dim group.
template <int FMT, int U>
struct Batch {
  Chunk<FMT> ch[U];
  uint16_t sc[U];
  // rows past w1 re-read the last valid row (in bounds); callers mask them
  __device__ __forceinline__ void load(const void* vals, const uint16_t* scales, long long rowbase,
                                       int w0, int w1, int it0, int r, int c) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long row = rowbase + min(w0 + (it0 + u) * 8 + r, w1 - 1);
      ch[u].load(vals, row, c);
      if constexpr (FMT == KV_FMT_Q8) sc[u] = ldg16(scales + row * NGRP + (c >> 2));
    }
  }
  __device__ __forceinline__ float scale(int u) const {
    if constexpr (FMT == KV_FMT_Q8) return h2f(sc[u]);
    return 1.f;
  }
};

template <int FMT, int G, int U>
__global__ __launch_bounds__(DEC_THREADS)
__attribute__((amdgpu_waves_per_eu(KVQ8_DEC_WAVES_PER_EU))) void k_decode_split(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int max_len, int kvh,
    const float* __restrict__ q, float qscale, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int S, int T) {
  const int s_idx = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nqh = kvh * G;
  const kv_session ss = tab[b];
  const int len = lens[b];
  if (session_bad(ss, FMT) || len < 0 || len > ss.cap || len > max_len) return;  // merge flags
  const int t_begin = s_idx * T;
  if (t_begin >= len) return;
  const int t_end = min(t_begin + T, len);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane >> 3, c = lane & 7;
  const int Tw = T / DEC_WAVES;
  const int w0 = t_begin + wave * Tw;
  const int w1 = min(w0 + Tw, t_end);

  extern __shared__ float smem[];
  float* lg = smem + wave * Tw * G;                 // [Tw][G] logits, then p
  float* o_l = smem + DEC_WAVES * Tw * G;           // [waves][G][HD]
  float* m_l = o_l + DEC_WAVES * G * HD;            // [waves][G]
  float* l_l = m_l + DEC_WAVES * G;                 // [waves][G]

  const long long rowbase = (long long)h * ss.cap;
  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
  }

  if (w1 > w0) {
    const int n_it = (w1 - w0 + 7) >> 3;
    // Two load batches A and B alternate (a 2x-unrolled loop, no register copies):
    // while one is consumed the other is in flight.  Steps past n_it read clamped,
    // in-bounds rows and are masked.  The last K step prefetches V batch 0 into A,
    // so its loads overlap the softmax.
    Batch<FMT, U> A, B;
    A.load(ss.k, ss.k_scale, rowbase, w0, w1, 0, r, c);
    // ---- K pass ---------------------------------------------------------
    {
      float qv[G][16];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float* qp = q + ((long long)b * nqh + h * G + g) * HD;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4 v = ldg128(qp + lane_dim<FMT>(c, 4 * k));   // 4 consecutive dims
#pragma unroll
          for (int e = 0; e < 4; ++e) qv[g][4 * k + e] = as_f32(v[e]) * qscale;
        }
      }
      // U x G independent dot products, interleaved so that no FMA waits on the one
      // just before it; then the U x G 8-lane reductions, then the logit stores
      auto kstep = [&](const Batch<FMT, U>& cur, int it0) {
        float part[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int g = 0; g < G; ++g) part[u][g] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float kf = cur.ch[u].get(i);
#pragma unroll
            for (int g = 0; g < G; ++g) part[u][g] = fmaf(qv[g][i], kf, part[u][g]);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float sc = cur.scale(u);
#pragma unroll
          for (int g = 0; g < G; ++g)
            if constexpr (FMT == KV_FMT_Q8) part[u][g] *= sc;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int g = 0; g < G; ++g) part[u][g] = sum8(part[u][g]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int it = it0 + u;
          const int t = w0 + it * 8 + r;
          if (c == 0 && it < n_it) store_logits<G>(lg + (it * 8 + r) * G, part[u], t < w1);
        }
      };
      for (int it0 = 0; it0 < n_it; it0 += 2 * U) {
        B.load(ss.k, ss.k_scale, rowbase, w0, w1, it0 + U, r, c);
        kstep(A, it0);
        if (it0 + 2 * U < n_it)
          A.load(ss.k, ss.k_scale, rowbase, w0, w1, it0 + 2 * U, r, c);
        else
          A.load(ss.v, ss.v_scale, rowbase, w0, w1, 0, r, c);
        kstep(B, it0 + U);
      }
    }
    wave_lds_fence();
    // ---- softmax over the wave's tokens --------------------------------------
    const int n_loc = n_it * 8;
    for (int tl = lane; tl < n_loc; tl += 64) {
#pragma unroll
      for (int g = 0; g < G; ++g) m[g] = fmaxf(m[g], lg[tl * G + g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = wave_max(m[g]);
    for (int tl = lane; tl < n_loc; tl += 64) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = exp2f(lg[tl * G + g] - m[g]);
        lg[tl * G + g] = p;
        l[g] += p;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = wave_sum(l[g]);
    wave_lds_fence();
    // ---- V pass ---------------------------------------------------------------
    auto vstep = [&](const Batch<FMT, U>& cur, int it0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = it0 + u;
        const float sc = cur.scale(u);
        // p is 0 for rows past the end (their logits were stored as -inf); steps past
        // n_it read stale LDS (in bounds: Tw/8 is a multiple of 2U) and are zeroed
        float w[G];
        load_p<G>(lg + (it * 8 + r) * G, w);
#pragma unroll
        for (int g = 0; g < G; ++g) w[g] = (it < n_it) ? w[g] * sc : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float vf = cur.ch[u].get(i);
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g][i] = fmaf(w[g], vf, acc[g][i]);
        }
      }
    };
    for (int it0 = 0; it0 < n_it; it0 += 2 * U) {
      B.load(ss.v, ss.v_scale, rowbase, w0, w1, it0 + U, r, c);
      vstep(A, it0);
      if (it0 + 2 * U < n_it) A.load(ss.v, ss.v_scale, rowbase, w0, w1, it0 + 2 * U, r, c);
      vstep(B, it0 + U);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] = sum_rows8(acc[g][i]);
  }

  // ---- combine the 4 wave partials of the workgroup --------------------------
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<float4*>(o_l + (wave * G + g) * HD + lane_dim<FMT>(c, i)) =
            make_float4(acc[g][i], acc[g][i + 1], acc[g][i + 2], acc[g][i + 3]);
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_l[wave * G + g] = m[g];
      l_l[wave * G + g] = l[g];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * HD; idx += DEC_THREADS) {
    const int g = idx / HD, d = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, m_l[w * G + g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float mw = m_l[w * G + g];
      if (mw == -INFINITY) continue;
      const float f = exp2f(mw - M);
      L += l_l[w * G + g] * f;
      O += o_l[(w * G + g) * HD + d] * f;
    }
    const long long qrow = ((long long)b * nqh + h * G + g) * S + s_idx;
    ws_o[qrow * HD + d] = O / L;
    if (d == 0) ws_lse[qrow] = M + log2f(L);
  }
}

// block-wide max / sum over the 256 threads (waves combine through LDS)
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < DEC_WAVES; ++w) r = fmaxf(r, red[w]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < DEC_WAVES; ++w) r += red[w];
  return r;
}

// One workgroup per (query head, session).  The split lse values are read once,
// coalesced, for the max and the normaliser; each wave then sums every 4th split's
// o (2 dims per lane), 8 splits per loop trip so that many loads are in flight.
template <int FMT>
__global__ __launch_bounds__(DEC_THREADS) void k_decode_merge(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int max_len, int nqh,
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int S, int T,
    float* __restrict__ out, int32_t* __restrict__ status) {
  const int qh = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const kv_session ss = tab[b];
  const int len = lens[b];
  int bad = session_bad(ss, FMT);
  if (!bad && (len < 0 || len > ss.cap || len > max_len)) bad = KV_DEV_RANGE;
  float2* dst = reinterpret_cast<float2*>(out + ((long long)b * nqh + qh) * HD);
  if (bad || len == 0) {
    if (wave == 0) dst[lane] = make_float2(0.f, 0.f);
    if (bad && qh == 0 && threadIdx.x == 0) flag(status, bad);
    return;
  }
  __shared__ float red[DEC_WAVES];
  __shared__ float2 part[DEC_WAVES][64];
  const int Sb = (len + T - 1) / T;
  const float* lse = ws_lse + ((long long)b * nqh + qh) * S;
  const float* o = ws_o + ((long long)b * nqh + qh) * S * HD;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < Sb; j += DEC_THREADS) mx = fmaxf(mx, lse[j]);
  const float M = block_max(mx, red);
  float sm = 0.f;
  for (int j = threadIdx.x; j < Sb; j += DEC_THREADS) sm += exp2f(lse[j] - M);
  const float L = block_sum(sm, red);
  constexpr int UN = 8;
  float2 acc[UN];
#pragma unroll
  for (int k = 0; k < UN; ++k) acc[k] = make_float2(0.f, 0.f);
  int j = wave;
  for (; j + (UN - 1) * DEC_WAVES < Sb; j += UN * DEC_WAVES) {
    float2 v[UN];
    float f[UN];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int jj = j + k * DEC_WAVES;
      v[k] = reinterpret_cast<const float2*>(o + (long long)jj * HD)[lane];
      f[k] = lse[jj];
    }
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const float w = exp2f(f[k] - M);
      acc[k].x = fmaf(w, v[k].x, acc[k].x);
      acc[k].y = fmaf(w, v[k].y, acc[k].y);
    }
  }
  for (; j < Sb; j += DEC_WAVES) {
    const float w = exp2f(lse[j] - M);
    const float2 v = reinterpret_cast<const float2*>(o + (long long)j * HD)[lane];
    acc[0].x = fmaf(w, v.x, acc[0].x);
    acc[0].y = fmaf(w, v.y, acc[0].y);
  }
  float2 a = acc[0];
#pragma unroll
  for (int k = 1; k < UN; ++k) {
    a.x += acc[k].x;
    a.y += acc[k].y;
  }
  part[wave][lane] = a;
  __syncthreads();
  if (wave == 0) {
    float2 t = part[0][lane];
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) {
      t.x += part[w][lane].x;
      t.y += part[w][lane].y;
    }
    dst[lane] = make_float2(t.x / L, t.y / L);
  }
}

template <int FMT, int G>
hipError_t launch_g(const kv_session* tab, const int32_t* lens, int n_sess, int max_len, int kvh,
                    const float* q, float sm_scale, float* out, float* ws_o, float* ws_lse,
                    const DecodePlan& plan, int32_t* status, hipStream_t st) {
  constexpr int U = (FMT == KV_FMT_Q8) ? KVQ8_DEC_U_Q8 : KVQ8_DEC_U_F16;
  static_assert(U == 1 || U == 2 || U == 4 || U == 8, "U must divide 8");
  if ((plan.T / DEC_WAVES / 8) % (2 * U) != 0) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * ((size_t)plan.T * G + DEC_WAVES * G * HD + 2 * DEC_WAVES * G);
  dim3 grid(plan.S, kvh, n_sess), block(DEC_THREADS);
  hipLaunchKernelGGL((k_decode_split<FMT, G, U>), grid, block, lds, st, tab, lens, max_len, kvh, q,
                     sm_scale * LOG2E, ws_o, ws_lse, plan.S, plan.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid(kvh * G, n_sess);
  hipLaunchKernelGGL((k_decode_merge<FMT>), mgrid, block, 0, st, tab, lens, max_len, kvh * G, ws_o,
                     ws_lse, plan.S, plan.T, out, status);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int kvh, int nqh, int n_sess, int max_len) {
  const int G = nqh / kvh;
  // Largest T (tokens per workgroup) that still gives >= 2048 workgroups (8 per CU on
  // 256 CUs); at least 256, at most 8192 / G so the logits fit in 32 KB of LDS.
  int T = 8192 / G;
  if (T > KVQ8_DEC_T_MAX) T = KVQ8_DEC_T_MAX;
  while (T > 256 && (long long)n_sess * kvh * ((max_len + T - 1) / T) < 2048) T >>= 1;
  DecodePlan p;
  p.T = T;
  p.S = max_len > 0 ? (max_len + T - 1) / T : 1;
  const size_t rows = (size_t)n_sess * nqh * p.S;
  p.ws_o_bytes = (rows * HD * sizeof(float) + 255) & ~(size_t)255;
  p.ws_lse_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  return p;
}

hipError_t launch_decode(int fmt, int kvh, int nqh, const kv_session* d_tab,
                         const int32_t* d_len, int n_sess, int max_len, const float* d_q,
                         float sm_scale, float* d_out, void* d_ws, const DecodePlan& plan,
                         int32_t* d_status, hipStream_t st) {
  float* ws_o = static_cast<float*>(d_ws);
  float* ws_lse = reinterpret_cast<float*>(static_cast<char*>(d_ws) + plan.ws_o_bytes);
  const int G = nqh / kvh;
#define KVQ8_DEC(F, GG)                                                                          \
  if (fmt == F && G == GG)                                                                       \
    return launch_g<F, GG>(d_tab, d_len, n_sess, max_len, kvh, d_q, sm_scale, d_out, ws_o, ws_lse, \
                           plan, d_status, st);
  KVQ8_DEC(KV_FMT_Q8, 1)
  KVQ8_DEC(KV_FMT_Q8, 2)
  KVQ8_DEC(KV_FMT_Q8, 4)
  KVQ8_DEC(KV_FMT_Q8, 8)
  KVQ8_DEC(KV_FMT_F16, 1)
  KVQ8_DEC(KV_FMT_F16, 2)
  KVQ8_DEC(KV_FMT_F16, 4)
  KVQ8_DEC(KV_FMT_F16, 8)
#undef KVQ8_DEC
  return hipErrorInvalidValue;
}

}  // namespace kvq8
