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
  uint4 w;  // 16 int8 codes
  __device__ __forceinline__ void load(const void* base, long long row, int c) {
    w = *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(base) + row * HD + c * 16);
  }
  __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t word = i < 4 ? w.x : i < 8 ? w.y : i < 12 ? w.z : w.w;
    return (float)(int8_t)(word >> (8 * (i & 3)));
  }
};

template <>
struct Chunk<KV_FMT_F16> {
  uint4 a, b;  // 16 fp16 values
  __device__ __forceinline__ void load(const void* base, long long row, int c) {
    const uint4* p =
        reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * HD + c * 16);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void zero() { a = b = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ float get(int i) const {
    const uint4& v = i < 8 ? a : b;
    const int j = i & 7;
    const uint32_t word = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return h2f((uint16_t)(word >> (16 * (j & 1))));
  }
};

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

template <int FMT, int G, int U>
__global__ __launch_bounds__(DEC_THREADS) void k_decode_split(
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
    // ---- K pass ---------------------------------------------------------
    {
      float qv[G][16];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float4* qp =
            reinterpret_cast<const float4*>(q + ((long long)b * nqh + h * G + g) * HD + c * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 v = qp[k];
          qv[g][4 * k + 0] = v.x * qscale;
          qv[g][4 * k + 1] = v.y * qscale;
          qv[g][4 * k + 2] = v.z * qscale;
          qv[g][4 * k + 3] = v.w * qscale;
        }
      }
      for (int it0 = 0; it0 < n_it; it0 += U) {
        Chunk<FMT> ch[U];
        float sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int t = w0 + (it0 + u) * 8 + r;
          if (t < w1) {
            ch[u].load(ss.k, rowbase + t, c);
            if constexpr (FMT == KV_FMT_Q8) sc[u] = h2f(ss.k_scale[(rowbase + t) * NGRP + (c >> 2)]);
          } else {
            ch[u].zero();
            sc[u] = 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float part[G];
#pragma unroll
          for (int g = 0; g < G; ++g) part[g] = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float kf = ch[u].get(i);
#pragma unroll
            for (int g = 0; g < G; ++g) part[g] = fmaf(qv[g][i], kf, part[g]);
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if constexpr (FMT == KV_FMT_Q8) part[g] *= sc[u];
            part[g] = sum8(part[g]);
          }
          const int it = it0 + u;
          const int t = w0 + it * 8 + r;
          if (c == 0 && it < n_it) store_logits<G>(lg + (it * 8 + r) * G, part, t < w1);
        }
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
    for (int it0 = 0; it0 < n_it; it0 += U) {
      Chunk<FMT> ch[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = w0 + (it0 + u) * 8 + r;
        if (t < w1) {
          ch[u].load(ss.v, rowbase + t, c);
          if constexpr (FMT == KV_FMT_Q8) sc[u] = h2f(ss.v_scale[(rowbase + t) * NGRP + (c >> 2)]);
          else sc[u] = 1.f;
        } else {
          ch[u].zero();
          sc[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = it0 + u;
        float w[G];
#pragma unroll
        for (int g = 0; g < G; ++g) w[g] = (it < n_it) ? lg[(it * 8 + r) * G + g] * sc[u] : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float vf = ch[u].get(i);
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g][i] = fmaf(w[g], vf, acc[g][i]);
        }
      }
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
        *reinterpret_cast<float4*>(o_l + (wave * G + g) * HD + c * 16 + i) =
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
  const int Sb = (len + T - 1) / T;
  const float* lse = ws_lse + ((long long)b * nqh + qh) * S;
  const float* o = ws_o + ((long long)b * nqh + qh) * S * HD;
  float M = -INFINITY;
  for (int j = 0; j < Sb; ++j) M = fmaxf(M, lse[j]);
  float L = 0.f;
  for (int j = 0; j < Sb; ++j) L += exp2f(lse[j] - M);
  float2 a = make_float2(0.f, 0.f);
  for (int j = wave; j < Sb; j += DEC_WAVES) {
    const float f = exp2f(lse[j] - M);
    const float2 v = reinterpret_cast<const float2*>(o + (long long)j * HD)[lane];
    a.x = fmaf(f, v.x, a.x);
    a.y = fmaf(f, v.y, a.y);
  }
  __shared__ float2 part[DEC_WAVES][64];
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
  constexpr int U = (FMT == KV_FMT_Q8) ? 8 : 4;
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
  if (T > 1024) T = 1024;
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
