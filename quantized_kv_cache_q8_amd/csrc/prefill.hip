// Causal attention of a prompt chunk over the FP16 [kvh][P][HD] copy of the cache,
// on the matrix cores (PR #3084 "FP16 K/V cache by default, int8 with --kv-q8",
// section Extra Notes: prompt attention runs both of its matrix products, scores and
// weighted values, on an fp16 compaction of the cache).
//
// Workgroup = (kv head h, block of BQ = 256/G queries); its 256 rows are the
// (query, head) pairs of the G query heads sharing kv head h, so one K/V tile in
// LDS serves all of them.  8 waves, two per SIMD: wave w owns rows [32w, 32w + 32)
// as 2 blocks of 16, so its O accumulators (64 per lane) stay in ordinary VGPRs and
// one wave's matrix products overlap the other wave's softmax arithmetic.
//
// Per 64-key tile, with v_mfma_f32_16x16x32_f16 (fp16 in, fp32 accumulate):
//   S^T[key][row] = K Q^T    A = K rows from LDS, B = the wave's Q rows (registers)
//   online softmax per row in fp32 (each lane owns whole rows: row = lane % 16 of
//   each 16-row block; the 16 keys of a lane are reduced in registers, then across
//   the 4 lane groups)
//   O^T[dim][row] += V^T P^T  A = V^T from LDS, B = P^T straight from the S^T
//   accumulators (as hi + lo fp16 parts, two products), using one consistent
//   assignment of keys to MFMA k-slots for both operands, so no data moves
//   between lanes.
// K and V tiles go from global memory straight to LDS (global_load_lds_dwordx4: a
// wave's instruction fills 1 KB, lane L the 16-byte slot L), both row-major (a key
// per 256-byte row) with the 16-byte chunks of row r XOR-swizzled by r mod 16, so the
// K fragment reads touch every bank once (the V^T reads below meet two-way bank
// conflicts; a swizzle without them timed the same).  K fragments are 16-byte reads; V^T
// fragments come from two transposing reads (ds_read_b64_tr_b16: within 16 lanes,
// lane i receives element i mod 4 of the 8-byte pieces addressed by lanes 4e + i / 4,
// e = 0 .. 3, so 16 lanes addressing 4 keys x 16 dims each receive one dim of the 4
// keys).  Tiles alternate between two LDS buffers: the next tile's loads are in
// flight while the current tile computes, and one barrier per tile suffices.
// Workgroups are numbered so that consecutive ones take different kv heads: the
// hardware deals workgroups round-robin to the 8 XCDs, so with 8 kv heads each
// XCD's L2 serves the K/V of one head to every query block of that head.
#include "kvq8_internal.h"

namespace kvq8 {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int PF_ROWS = 256;    // (query, head) rows per workgroup
constexpr int PF_THREADS = 512; // 8 waves x 32 rows
constexpr int BK = 64;     // keys per tile
constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float PF_PRE = 15.0f;  // log2 scale of p (p <= 2^15)

__device__ __forceinline__ floatx4 mfma(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define KVQ8_LDSP(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int G>
__global__ __launch_bounds__(PF_THREADS) void k_prefill(
    const uint16_t* __restrict__ k16, const uint16_t* __restrict__ v16, long stride, int kvh,
    int pos0, int n_tok, const float* __restrict__ q, float qscale, float* __restrict__ out,
    int n_qblk) {
  constexpr int BQ = PF_ROWS / G;  // queries per workgroup
  const int h = blockIdx.x % kvh;
  const int qb = n_qblk - 1 - (int)(blockIdx.x / kvh);  // longest rows first
  const int q0 = qb * BQ;
  const int nqh = kvh * G;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int P = pos0 + n_tok;
  const int q_last = min(q0 + BQ, n_tok) - 1;
  const int n_tiles = (pos0 + q_last + 1 + BK - 1) / BK;

  __shared__ __attribute__((aligned(16))) _Float16 Ks[2][BK * HD];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[2][BK * HD];

  // ---- Q rows of this wave, fp16 (RNE), as B fragments of S^T = K Q^T ----------
  half8 qf[2][4];
  int lim[2];  // last key a row may attend
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int R = 32 * wave + 16 * rb + l16;
    const int i = q0 + R / G, g = R % G;
    lim[rb] = min(pos0 + i, P - 1);
    const float* src = q + ((long)i * nqh + h * G + g) * HD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 f;
      if (i < n_tok) {
        const float4 a = *reinterpret_cast<const float4*>(src + 32 * ks + 8 * g4);
        const float4 b = *reinterpret_cast<const float4*>(src + 32 * ks + 8 * g4 + 4);
        f[0] = (_Float16)a.x; f[1] = (_Float16)a.y; f[2] = (_Float16)a.z; f[3] = (_Float16)a.w;
        f[4] = (_Float16)b.x; f[5] = (_Float16)b.y; f[6] = (_Float16)b.z; f[7] = (_Float16)b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (_Float16)0.0f;
      }
      qf[rb][ks] = f;
    }
  }
  const int wave_lim_min = min(pos0 + q0 + (32 * wave) / G, P - 1);

  floatx4 o[2][8];  // O^T[dim = 16db + 4*g4 + j][row = 16rb + l16]
  float m[2], l[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[rb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: K or V of a tile into an LDS buffer ---------------------------
  // wave w's instruction u fills rows 8w + 4u .. + 3; slot (r, pc) holds chunk
  // pc ^ (r & 15) of row r.  Keys past P read key P - 1 (masked: past every row's last
  // key, and their weights are 0)
  auto tload = [&](const uint16_t* src, _Float16* dst, int tile) {
    const int k0 = tile * BK;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * wave + 4 * u + (lane >> 4);
      const int pc = lane & 15;
      const int key = min(k0 + r, P - 1);
      const uint16_t* gp = src + ((long)h * stride + key) * HD + 8 * (pc ^ (r & 15));
      __builtin_amdgcn_global_load_lds(gp, KVQ8_LDSP(void, &dst[(8 * wave + 4 * u) * HD]), 16, 0, 0);
    }
  };
  tload(k16, Ks[0], 0);
  tload(v16, Vs[0], 0);
  __builtin_amdgcn_s_waitcnt(0);   // the direct loads count as loads
  __syncthreads();
  for (int tile = 0; tile < n_tiles; ++tile) {
    const int cur = tile & 1;
    const bool more = tile + 1 < n_tiles;
    if (more) {   // buffers cur ^ 1 were last read in the previous tile, before its barrier
      tload(k16, Ks[cur ^ 1], tile + 1);
      tload(v16, Vs[cur ^ 1], tile + 1);
    }
    const int k0 = tile * BK;
    const _Float16* KsC = Ks[cur];
    const _Float16* VsC = Vs[cur];

    // ---- S^T = K Q^T --------------------------------------------------------
    floatx4 s[4][2];  // [kb][rb]: S^T[key = k0 + 16kb + 4*g4 + j][row = 16rb + l16]
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[kb][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // K fragments (16 = 4 k-steps x 4 key blocks) read from LDS one k-step (4 reads)
    // ahead of the products that use them; the scheduling barrier keeps the compiler
    // from moving each read back next to its use, so LDS latency hides behind MFMAs
    auto kfrag = [&](int i) __attribute__((always_inline)) {
      const int ks = i >> 2, kb = i & 3;
      return *reinterpret_cast<const half8*>(&KsC[(16 * kb + l16) * HD + 8 * ((4 * ks + g4) ^ l16)]);
    };
    half8 kf[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = kfrag(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 4 < 16) kf[(i + 4) % 5] = kfrag(i + 4);
      __builtin_amdgcn_sched_barrier(0);
      const half8 a = kf[i % 5];
      const int ks = i >> 2, kb = i & 3;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[kb][rb] = mfma(a, qf[rb][ks], s[kb][rb]);
    }

    // ---- online softmax (log2 units) -----------------------------------------
    // p is computed as 2^(s*qscale - m + PF_PRE): the fixed factor keeps the weights
    // that matter clear of the fp16 subnormals (p <= 2^PF_PRE stays finite in fp16); O
    // and l carry the same factor, which the final division removes.
    const bool need_mask = k0 + BK - 1 > wave_lim_min;
    // P^T fragments, k-slot (g4, e) -> key 4*g4 + e (e < 4), 16 + 4*g4 + e - 4.  P is
    // carried as hi + lo fp16 parts: hi = p with its low 13 fraction bits cleared (an
    // exact fp16 value), lo = p - hi (exact in fp32), so the P V product keeps ~22
    // significant bits of each weight instead of 11.
    if (need_mask) {   // only tiles that reach past some row's last key
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (k0 + 16 * kb + 4 * g4 + j > lim[rb]) s[kb][rb][j] = -INFINITY;
    }
    float alpha[2];
    bool moved = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, s[kb][rb][j]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mnew = fmaxf(m[rb], mx * qscale);   // qscale > 0 (checked by the caller)
      moved |= mnew != m[rb];
      alpha[rb] = __builtin_amdgcn_exp2f(m[rb] - mnew);
      m[rb] = mnew;
    }
    // O only needs rescaling when some row of the wave raised its maximum: after the
    // first tiles that is rare, and the branch is uniform
    if (__ballot(moved) != 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        l[rb] *= alpha[rb];
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rb][db] *= alpha[rb];
      }
    }
    half8 pf[2][2], pl[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mb = m[rb] - PF_PRE;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][rb][j], qscale, -mb));
          s[kb][rb][j] = p;
          ls += p;
        }
      l[rb] += ls;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // pairs (j, j+1) of key block 2*ks2 (e < 2) and 2*ks2 + 1 (e >= 2)
          const int kb = 2 * ks2 + (e >> 1), j = 2 * (e & 1);
          const float p0 = s[kb][rb][j], p1 = s[kb][rb][j + 1];
          const float h0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p0) & 0xFFFFE000u);
          const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p1) & 0xFFFFE000u);
          hw[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(h0, h1));
          lw[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0 - h0, p1 - h1));
        }
        pf[rb][ks2] = __builtin_bit_cast(half8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        pl[rb][ks2] = __builtin_bit_cast(half8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
    }

    // ---- O^T += V^T P^T -------------------------------------------------------
    // V^T fragments (16 = 2 key halves x 8 dim blocks) read two ahead of their products,
    // held in place by the scheduling barrier as above
    auto vfrag = [&](int i) __attribute__((always_inline)) {
      const int ks2 = i >> 3, db = i & 7;
      // k-slots (g4, 0 .. 7) of k-step ks2: keys 4 g4 .. + 3 and 16 + 4 g4 .. + 3 of the
      // half.  Lane l16 = 4 e + q addresses key 32 ks2 + 4 g4 + e (then + 16), dims
      // 16 db + 4q .. + 3, and receives dim 16 db + l16 of the four keys
      const int e = l16 >> 2, q = l16 & 3;
      const int c16 = 2 * db + (q >> 1);
      const int r1 = 32 * ks2 + 4 * g4 + e, r2 = r1 + 16;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          KVQ8_LDSP(v4i16, &VsC[r1 * HD + 8 * (c16 ^ (r1 & 15)) + 4 * (q & 1)]));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          KVQ8_LDSP(v4i16, &VsC[r2 * HD + 8 * (c16 ^ (r2 & 15)) + 4 * (q & 1)]));
      return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    half8 vf[3];
#pragma unroll
    for (int i = 0; i < 2; ++i) vf[i] = vfrag(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) vf[(i + 2) % 3] = vfrag(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const half8 a = vf[i % 3];
      const int ks2 = i >> 3, db = i & 7;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        o[rb][db] = mfma(a, pf[rb][ks2], o[rb][db]);
        o[rb][db] = mfma(a, pl[rb][ks2], o[rb][db]);
      }
    }

    // the next tile's direct loads have landed (they count as loads), then the barrier
    // publishes them and frees this tile's buffers
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- normalise and store ----------------------------------------------------
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float L = l[rb];
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
    const int R = 32 * wave + 16 * rb + l16;
    const int i = q0 + R / G, g = R % G;
    if (i >= n_tok) continue;
    float* dst = out + ((long)i * nqh + h * G + g) * HD;
    const float inv = 1.0f / L;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const floatx4 v = o[rb][db] * inv;
      *reinterpret_cast<float4*>(dst + 16 * db + 4 * g4) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

}  // namespace

hipError_t launch_prefill(int kvh, int nqh, const uint16_t* k16, const uint16_t* v16,
                          long row_stride, int pos0, int n_tok, const float* d_q,
                          float sm_scale, float* d_out, hipStream_t st) {
  const int G = nqh / kvh;
  const int BQ = PF_ROWS / G;
  const int n_qblk = (n_tok + BQ - 1) / BQ;
  const long long blocks = (long long)n_qblk * kvh;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const float qs = sm_scale * LOG2E_F;
  dim3 grid((unsigned)blocks), block(PF_THREADS);
  switch (G) {
    case 1: hipLaunchKernelGGL(k_prefill<1>, grid, block, 0, st, k16, v16, row_stride, kvh, pos0, n_tok, d_q, qs, d_out, n_qblk); break;
    case 2: hipLaunchKernelGGL(k_prefill<2>, grid, block, 0, st, k16, v16, row_stride, kvh, pos0, n_tok, d_q, qs, d_out, n_qblk); break;
    case 4: hipLaunchKernelGGL(k_prefill<4>, grid, block, 0, st, k16, v16, row_stride, kvh, pos0, n_tok, d_q, qs, d_out, n_qblk); break;
    case 8: hipLaunchKernelGGL(k_prefill<8>, grid, block, 0, st, k16, v16, row_stride, kvh, pos0, n_tok, d_q, qs, d_out, n_qblk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq8
