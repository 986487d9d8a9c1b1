// Split-K decode attention over the cache, reading the cache format directly
// (PR #3084 "FP16 K/V cache by default, int8 with --kv-q8", sections What changed
// and Extra Notes: the next token's split-K decode reads the cache, FP16 or int8,
// with no conversion pass).
//
// k_decode_split: grid (S splits, kv head h, session b), 8 waves per workgroup in
//   two groups of 4 (waves w and w + 4 share a SIMD).  Work is counted in 8-token
//   steps (one 128-bit load per lane covers a step of one head: 8 rows x 8 lanes).
//   The steps of a (session, head) are cut in two ranges, one per group, in
//   proportion to how fast each group runs (the older wave of a SIMD gets most
//   issue slots).  The W = 4S waves of a group take the steps of its range
//   round-robin -- wave gw owns steps gw, gw + W, gw + 2W, ... -- so they sweep
//   that range of K/V together, front by front, as one stream.
//   A wave works through its steps in chunks of CH steps, two passes per chunk:
//   K pass   lane (r = lane/8, c = lane%8) holds 16 dims of token r of a step:
//            in-register dequant, partial dots for the G query heads, the int8
//            group scale applied to the partial, an 8-lane DPP sum; logits (log2
//            units) go to LDS.
//   softmax  chunk max, rescale of the running (m, l, acc), exp2.
//   V pass   acc[g][16 dims] += p * scale * v.
//   Load batches alternate between two register sets so the next batch is in
//   flight while one is consumed.  The 8 wave partials are combined in LDS and
//   written as one (o, lse) per query head and split (o normalised, lse in log2).
//   Offsets are 32-bit, from per-head base pointers (a head holds at most 2^24
//   cells).
// k_decode_pair / k_decode_pair_mv (the int8-K formats): the same splits, with the
//   K logits on the matrix cores and the waves in pairs, one streaming K and one
//   streaming V per SIMD (described at the kernels).  k_decode_split serves FP16.
// k_decode_merge: out = sum_j 2^(lse_j - L) o_j with L = log2 sum_j 2^lse_j.
//
// Dequantised values are exact in fp32 (a 7-bit code times an 11-bit fp16
// significand); the int8 K logits are exact integer sums of the codes against a
// three-level int8 split of the query (residual about 2^-24 of the query); the rest
// of the rounding is fp32 accumulation.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kvq8_internal.h"

namespace kvq8 {
namespace {

// rows (8-token steps) per load batch; a wave alternates two batches
#ifndef KVQ8_DEC_U_Q8
#define KVQ8_DEC_U_Q8 4
#endif
#ifndef KVQ8_DEC_U_F16
#define KVQ8_DEC_U_F16 1
#endif
// most 8-token steps one wave handles (the per-wave LDS logits buffer)
#ifndef KVQ8_DEC_CH
#define KVQ8_DEC_CH 128
#endif
// K/V rows are read once per decode: non-temporal loads keep them out of the caches
#ifndef KVQ8_DEC_NT
#define KVQ8_DEC_NT 1
#endif
// minimum resident waves per SIMD the register allocation must allow
#ifndef KVQ8_DEC_WAVES_PER_EU
#define KVQ8_DEC_WAVES_PER_EU 1
#endif
#ifndef KVQ8_MAX_DEVICES
#define KVQ8_MAX_DEVICES 64
#endif

__device__ __forceinline__ u32x4 ldkv(const void* p) {
  if constexpr (KVQ8_DEC_NT) return ldg128_nt(p);
  return ldg128(p);
}
// base: the head's first row (the same for the whole wave); off: 32-bit byte offset
__device__ __forceinline__ u32x4 ldkv(const char* base, uint32_t off) { return ldkv(base + off); }
__device__ __forceinline__ u32x2 ldkv64(const char* base, uint32_t off) {
  if constexpr (KVQ8_DEC_NT) return __builtin_nontemporal_load((const KVQ8_GLOBAL u32x2*)(base + off));
  return *(const KVQ8_GLOBAL u32x2*)(base + off);
}

#ifndef KVQ8_DEC_WG_WAVES
#define KVQ8_DEC_WG_WAVES 8
#endif
// share (sixteenths) of a head's steps taken by the leading group of waves
#ifndef KVQ8_DEC_LEAD16_Q8
#define KVQ8_DEC_LEAD16_Q8 8
#endif
#ifndef KVQ8_DEC_LEAD16_F16
#define KVQ8_DEC_LEAD16_F16 8
#endif
constexpr int DEC_WAVES = KVQ8_DEC_WG_WAVES;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
// With 8 waves per workgroup, waves w and w + 4 share a SIMD and the instruction
// arbiter favours the older one, w: with equal work the younger wave of the int8
// kernel, starved of issue slots, finishes ~40 % later and runs alone at the end.
// The waves therefore form two groups: group 0 (waves 0-3) takes lead16 sixteenths
// of the head's steps, group 1 the rest, each group interleaving its steps over its
// own waves.
constexpr int GRP_WAVES = DEC_WAVES >= 8 ? DEC_WAVES / 2 : DEC_WAVES;
constexpr bool GROUPED = GRP_WAVES != DEC_WAVES;
template <int FMT>
__host__ __device__ constexpr int lead16() {
  return GROUPED ? (FMT != KV_FMT_F16 ? KVQ8_DEC_LEAD16_Q8 : KVQ8_DEC_LEAD16_F16) : 16;
}
template <int FMT>
__host__ __device__ constexpr int lead_steps(int J) {  // >= J - lead_steps(J) (lead16 >= 8)
  return (int)(((long long)J * lead16<FMT>() + 15) / 16);
}
constexpr float LOG2E = 1.4426950408889634f;

// fewest steps a wave of the leading group is given when a session is short for the
// grid's split count (the grid is sized by the longest session of the call)
#ifndef KVQ8_DEC_MIN_STEPS
#define KVQ8_DEC_MIN_STEPS 16
#endif
// Splits (workgroups) that work on a session of len cells, of the S in the grid: all
// of them for long sessions, fewer for short ones so that no wave gets a token or
// two; the split kernel and the merge both use it.
template <int FMT>
__host__ __device__ inline int active_splits(int len, int S) {
  const int Jf = lead_steps<FMT>((len + 7) >> 3);
  return min(S, max(1, (Jf + GRP_WAVES * KVQ8_DEC_MIN_STEPS - 1) / (GRP_WAVES * KVQ8_DEC_MIN_STEPS)));
}

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
  __device__ __forceinline__ void load(const char* base, uint32_t row, int c) {
    w = ldkv(base, row * HD + c * 16);
  }
  __device__ __forceinline__ float get(int i) const {
    return (float)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
};

// K8V4: the K chunk is the int8 one; a V chunk is 16 nibbles (8 bytes: w[0], w[1])
// of the rotated row, read as code + 8 (the 8 is taken out by the caller)
template <>
struct Chunk<KV_FMT_K8V4> {
  u32x4 w;
  __device__ __forceinline__ void load(const char* base, uint32_t row, int c) {
    w = ldkv(base, row * HD + c * 16);
  }
  __device__ __forceinline__ void load_v(const char* base, uint32_t row, int c) {
    const u32x2 t = ldkv64(base, row * (HD / 2) + c * 8);
    w[0] = t[0];
    w[1] = t[1];
  }
  __device__ __forceinline__ float get(int i) const {  // int8 K code
    return (float)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
};

template <>
struct Chunk<KV_FMT_F16> {
  u32x4 a, b;  // 16 fp16 values: dims [8c, 8c+8) and [64+8c, 64+8c+8)
  __device__ __forceinline__ void load(const char* base, uint32_t row, int c) {
    const uint32_t off = row * (HD * 2) + c * 16;
    a = ldkv(base, off);        // the 8 lanes of a row cover bytes [0, 128) of it
    b = ldkv(base, off + 128);  // ... and bytes [128, 256)
  }
  __device__ __forceinline__ float get(int i) const {
    const u32x4& v = i < 8 ? a : b;
    const int j = i & 7;
    return h2f((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
  }
};

// x & 0x0F0F0F0F: the low nibble of each byte, in its byte.  Kept opaque to the
// compiler, which would otherwise fold the mask into a 4-bit field extract per value
// instead of one byte-to-float conversion (v_cvt_f32_ubyteN) per value.
__device__ __forceinline__ uint32_t nibble_bytes(uint32_t x) {
  uint32_t r;
  asm("v_and_b32_e32 %0, 0x0f0f0f0f, %1" : "=v"(r) : "v"(x));
  return r;
}

// Signed byte k of w as fp32, in one instruction (a byte-select conversion with sign
// extension); written out because the compiler sometimes extracts the byte first.
__device__ __forceinline__ float i8_to_f32(uint32_t w, int k) {
  float r;
  switch (k) {
    case 0: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w)); break;
    case 1: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w)); break;
    case 2: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w)); break;
    default: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w)); break;
  }
  return r;
}

// Head dim of the i-th of the 16 values a lane (c = lane % 8) holds of a row.
template <int FMT>
__device__ __forceinline__ int lane_dim(int c, int i) {
  if constexpr (FMT != KV_FMT_F16) return 16 * c + i;  // one 64-dim scale group per lane
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

// Most steps per wave, on average over the two groups: the LDS holds each wave's
// logits (8 tokens x G heads per step).  With 8 query heads the full budget would
// not fit in the 160 KB of LDS beside the wave partials.
template <int G>
__host__ __device__ constexpr int ch_steps() { return G >= 8 ? 56 : KVQ8_DEC_CH; }
// logits budget of a wave of group 0 and of group 1, in proportion to their shares
// (group 0's rounded down to whole pairs of the largest load batch with 8 heads)
template <int FMT, int G>
__host__ __device__ constexpr int ch0() {
  return GROUPED ? 2 * ch_steps<G>() * lead16<FMT>() / 16 / 8 * 8 : ch_steps<G>();
}
template <int FMT, int G>
__host__ __device__ constexpr int ch1() { return GROUPED ? 2 * ch_steps<G>() - ch0<FMT, G>() : 0; }
static_assert(2 * KVQ8_DEC_CH <= 256, "a wave has at most 256 steps (the page map's registers)");
static_assert(KVQ8_DEC_CH % 8 == 0 && ch_steps<8>() % 8 == 0,
              "the group budgets are whole multiples of 8 steps");

// Paged sessions: a session's cells live in pages of KV_PAGE_ROWS (64) inside a pool
// (the session table's arrays, cap = 64 x slots); a page table maps page p (cells
// 64p .. 64p + 63) to its slot.  A wave's steps are 8W >= 64 rows apart, so each is in
// a page of its own: the wave keeps the slot of each of its steps in registers (lane
// l, register j: step l + 64 j; at most 256 steps per wave, which the plans keep) and
// a load reads it with one readlane.  A slot outside the pool reads slot 0 (the merge
// flags the table).
struct NoPages {
  static constexpr bool paged = false;
};
// The global step (8 tokens) of step k of wave gw, W waves sharing a head's steps:
// SP = 1 deals single steps round robin; SP = 2 or 4 deals units of SP adjacent steps,
// so a wave's steps SP j .. SP j + SP - 1 are 8 SP consecutive tokens (SP KB of int8
// codes per read).
template <int SP>
__device__ __forceinline__ int step_g(int gw, int k, int W) {
  static_assert(SP == 1 || SP == 2 || SP == 4 || SP == 8, "steps dealt in units of 1, 2, 4 or 8");
  if constexpr (SP == 1) return gw + k * W;
  // k >= 0: unsigned division and remainder are a shift and a mask
  else return SP * (gw + (int)((unsigned)k / SP) * W) + (int)((unsigned)k % SP);
}
#ifndef KVQ8_DEC_MV_SP
#define KVQ8_DEC_MV_SP 8
#endif
// steps per unit dealt to a wave of k_decode_pair_mv for one session: 8 steps, 64
// tokens, one page of a paged session and 8 KB of int8 codes per array (a batch of
// ragged sessions takes single steps: its short sessions split more evenly)
constexpr int MV_SP = KVQ8_DEC_MV_SP;
// Paged sessions: the rows of a step (8 consecutive tokens, 8-aligned) lie in one
// 64-row page, so a step's rows are one wave-uniform pool row plus the lane's row
// within the step.
// NR registers hold the slots of up to 64 NR steps per wave; SP as for step_g.
template <int NR, int SP = 1>
struct PageMap {
  static_assert(NR == 2 || NR == 4, "2 or 4 registers of slots");
  static constexpr bool paged = true;
  int slot[NR];   // lane l, register j: the slot of the page of step l + 64 j
  int last;      // the slot of the page holding row len - 1
  int len;
  int nst;       // the wave's steps (n_steps)
  __device__ __forceinline__ void init(const int32_t* pages, int stride, int b, int gw, int W,
                                       int n_steps, int n_slots, int len_, int lane) {
    const int32_t* row = pages + (long long)b * stride;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int k = lane + 64 * j;
      int sl = 0;
      if (k < n_steps) {
        sl = row[(step_g<SP>(gw, k, W) * 8) >> 6];
        if ((unsigned)sl >= (unsigned)n_slots) sl = 0;
      }
      slot[j] = sl;
    }
    len = len_;
    nst = n_steps;
    last = len_ > 0 ? row[(len_ - 1) >> 6] : 0;
    if ((unsigned)last >= (unsigned)n_slots) last = 0;
  }
  // slot of step k (k the same in every lane)
  __device__ __forceinline__ int slot_of(int k) const {
    const int j = k >> 6;
    const int v = j == 0 ? slot[0] : j == 1 ? slot[1] : j == 2 ? slot[2] : slot[3];
    return __builtin_amdgcn_readlane(v, k & 63);
  }
  // the slots of steps 64 (k / 64) .. 64 (k / 64) + 63, one per lane (k uniform)
  __device__ __forceinline__ int block(int k) const {
    const int j = k >> 6;
    if constexpr (NR == 2) return j == 0 ? slot[0] : slot[1];
    else return j == 0 ? slot[0] : j == 1 ? slot[1] : j == 2 ? slot[2] : slot[3];
  }
  // step k of wave gw (stride W), v = block(k): pb, the pool row of its first row,
  // and lim, its last row that holds a token (rows i > lim re-read row lim).  A step
  // past the wave's own (its tokens are masked; in a grouped kernel it may still lie
  // inside the session, on a page this wave has not mapped) or past the session's
  // end reads the session's last step, so k needs no clamp.
  __device__ __forceinline__ void step(int v, int k, int gw, int W, int& pb, int& lim) const {
    const int s = step_g<SP>(gw, k, W) * 8;
    const bool past = s >= len || k >= nst;
    const int s0 = past ? ((len - 1) & ~7) : s;
    const int rl = __builtin_amdgcn_readlane(v, k & 63);   // always: a select, not a branch
    const int sl = past ? last : rl;
    pb = sl * KV_PAGE_ROWS + (s0 & (KV_PAGE_ROWS - 1));
    lim = len - 1 - s0;
  }
  // the pool row of row i of step k, k per lane within one 64-step block (v = block of
  // that block)
  __device__ __forceinline__ uint32_t lane_row(int v, int k, int gw, int W, int i) const {
    const int s = step_g<SP>(gw, k, W) * 8;
    const bool past = s >= len || k >= nst;
    const int s0 = past ? ((len - 1) & ~7) : s;
    const int sk = __shfl(v, k & 63, 64);
    const int sl = past ? last : sk;
    return (uint32_t)(sl * KV_PAGE_ROWS + (s0 & (KV_PAGE_ROWS - 1)) + min(i, len - 1 - s0));
  }
};

// One batch of U steps for one lane: U x 16 values and, for int8, the U raw fp16
// scales of the lane's 64-dim group.
template <int FMT, int U>
struct Batch {
  Chunk<FMT> ch[U];
  uint16_t sc[U];
  // steps k .. k+U-1 of wave gw; tokens past len re-read the last cell (in bounds)
  // and are masked by the callers
  // vals, scales: the head's first row of values and of scales
  // V: the V array (only K8V4 lays it out differently from K)
  // kmax: steps past it re-read step kmax (a row of this wave's, still in cache)
  // pm: the page map of a paged session (rows then lie in step k + u's page)
  template <bool V, class PM = NoPages>
  __device__ __forceinline__ void load(const char* vals, const char* scales, int gw, int W, int k,
                                       int len, int r, int c, int kmax = 1 << 30,
                                       const PM& pm = PM()) {
    // paged: k is a multiple of U, which divides 64, so the batch's steps share one
    // register of the page map
    static_assert(64 % U == 0, "a batch lies in one 64-step block");
    int pv = 0;
    if constexpr (PM::paged) pv = pm.block(k);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ku = PM::paged ? k + u : min(k + u, kmax);
      uint32_t row;
      const char* vp = vals;
      const char* sp = scales;
      if constexpr (PM::paged) {
        // the step's rows from a wave-uniform base: the loads take a scalar address
        int pb, lim;
        pm.step(pv, ku, gw, W, pb, lim);
        constexpr size_t VROW = FMT == KV_FMT_F16 ? HD * 2 : (FMT == KV_FMT_K8V4 && V) ? HD / 2 : HD;
        constexpr size_t SROW = (FMT == KV_FMT_K8V4 && V) ? NQ4 * 2 : NGRP * 2;
        vp += (size_t)pb * VROW;
        sp += (size_t)pb * SROW;
        row = (uint32_t)min(r, lim);
      } else {
        row = (uint32_t)min((gw + ku * W) * 8 + r, len - 1);
      }
      if constexpr (FMT == KV_FMT_K8V4 && V) {
        ch[u].load_v(vp, row, c);
        sc[u] = ldg16(sp + (row * NQ4 + (c >> 1)) * 2);   // lane c: dims of block c / 2
      } else {
        ch[u].load(vp, row, c);
        if constexpr (FMT != KV_FMT_F16) sc[u] = ldg16(sp + (row * NGRP + (c >> 2)) * 2);
      }
    }
  }
  __device__ __forceinline__ float scale(int u) const {
    if constexpr (FMT != KV_FMT_F16) return h2f(sc[u]);
    return 1.f;
  }
};

// Register order of the G query heads in a lane's K-pass partials: slot j of lane
// c (c = lane % 8) holds head j ^ head_map(c).  The three reduction stages pair
// lane c with c^1, c^2 and 7-c; head_map makes the partner's slot j + n/2 (n the
// values still carried) hold the head of this lane's slot j, so a stage is one
// DPP add per value kept.  After log2(G) folding stages lane c holds head
// head_map(c) alone, and lanes 0 .. G-1 of a row hold distinct heads.
template <int G>
__device__ __forceinline__ int head_map(int c) {
  constexpr int A = G >= 8 ? 3 : G >= 4 ? 2 : G >= 2 ? 1 : 0;
  const int c2 = (c >> 2) & 1;
  const int f0 = (c & 1) ^ c2, f1 = ((c >> 1) & 1) ^ c2;
  if constexpr (A == 3) return (f0 << 2) | (f1 << 1) | c2;
  if constexpr (A == 2) return (f0 << 1) | f1;
  if constexpr (A == 1) return f0;
  return 0;
}

// One reduction stage over U rows of N live values: fold (N > 1) or plain add.
template <int CTRL, int U, int G, int N>
__device__ __forceinline__ void fold_stage(float (&x)[U][G]) {
  if constexpr (N > 1) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < N / 2; ++k) x[u][k] = __fadd_rn(x[u][k], dpp<CTRL>(x[u][k + N / 2]));
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) x[u][0] = __fadd_rn(x[u][0], dpp<CTRL>(x[u][0]));
  }
}

// The int8 K pass on the matrix cores (the pair kernels).  The logits of G query heads against 16
// tokens are a small integer product per 64-dim scale group: the query, in log2
// units, is split per (head, group) into three int8 levels,
//   q = s (a + b / 254 + c / 254^2),  s = max|q| / 127 over the group,
// so each level's dot products with the raw codes are exact integers, and the
// residual after three levels is at most s / (2 * 254^2), about 2^-24 of the group's
// largest query value (the precision of fp32).  One v_mfma_i32_16x16x64_i8 per group
// and 4 heads takes A = the query levels (row 4 * head + level, the fourth row of a
// head zero) and B = the codes of 16 tokens (column = token), so that lane l receives
// the three level sums of head l / 16 and token l % 16 and turns them into one logit.
// Any assignment of dims to k-slots is a valid contraction as long as A and B use
// the same one: lane l's byte j of both operands is dim 64 * group + 16 * (l / 16) + j.
// 8-token steps per K batch of the matrix-core pass (two batches alternate)
#ifndef KVQ8_DEC_UK_Q8
#define KVQ8_DEC_UK_Q8 8
#endif
template <int G>
__host__ __device__ constexpr int k_batch_rows() { return G >= 8 ? 4 : KVQ8_DEC_UK_Q8; }
constexpr int QLEV = 3;
constexpr float QBASE_INV = 1.f / 254.f;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// one int8 level of a value: clamp(rint(r / s)), and the residual it leaves
__device__ __forceinline__ int q_level(float& r, float s) {
  const float a = fminf(fmaxf(rintf(r / s), -127.f), 127.f);
  r = fmaf(-a, s, r);
  return (int)a;
}

// A K batch for the matrix-core pass: U 8-token steps as U/2 blocks of 16 tokens;
// per block and group, lane l holds the 16 codes of token n = l % 16 at dims
// 64 * group + 16 * (l / 16) .. + 15 and that token's group scale.  Token n of block
// j is row n % 8 of step k + 2j + n / 8, so its logit goes where the 8-lane layout
// of the other passes expects it.
// SC: also load each token's K scales (false: the caller fetches them per chunk)
template <int U, int SP = 1, bool SC = true>
struct KBatch {
  static_assert(U % 2 == 0, "blocks of 16 tokens are pairs of steps");
  u32x4 w[U / 2][2];
  uint16_t sc[SC ? U / 2 : 1][2];
  template <class PM = NoPages>
  __device__ __forceinline__ void load(const char* kb, const char* ksb, int gw, int W, int k,
                                       int len, int lane, int kmax = 1 << 30,
                                       const PM& pm = PM()) {
    const int n = lane & 15, kq = lane >> 4;
    static_assert(64 % U == 0, "a batch lies in one 64-step block");
    int pv = 0;
    if constexpr (PM::paged) pv = pm.block(k);   // k: a multiple of U
#pragma unroll
    for (int j = 0; j < U / 2; ++j) {
      const int k0 = min(k + 2 * j, kmax), k1 = min(k + 2 * j + 1, kmax);
      uint32_t row;
      if constexpr (PM::paged) {
        int pb0, lim0, pb1, lim1;
        pm.step(pv, k + 2 * j, gw, W, pb0, lim0);
        pm.step(pv, k + 2 * j + 1, gw, W, pb1, lim1);
        const bool second = (n >> 3) != 0;
        row = (uint32_t)((second ? pb1 : pb0) + min(n & 7, second ? lim1 : lim0));
      } else {
        // both steps' rows from wave-uniform values, then the lane's choice
        const int s0 = step_g<SP>(gw, k0, W), s1 = step_g<SP>(gw, k1, W);
        row = (uint32_t)min(((n >> 3) ? s1 : s0) * 8 + (n & 7), len - 1);
      }
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        w[j][grp] = ldkv(kb, row * HD + grp * 64 + kq * 16);
        if constexpr (SC) sc[j][grp] = ldg16(ksb + (row * NGRP + grp) * 2);
      }
    }
  }
};

// max(a, b) in one instruction (the median of a, b and +inf; no NaN quieting)
__device__ __forceinline__ float max2(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, INFINITY);
}
// the bits of a float as a signed int of the same order (negative values have their
// magnitude bits flipped; the map is its own inverse; -inf is the least value here)
__device__ __forceinline__ int ord_bits(int i) { return i ^ ((i >> 31) & 0x7FFFFFFF); }
// Max over the wave, returned wave-uniform, with cross-lane moves only: the four
// in-row stages, then each row's lane 15 into the next row, lane 31 into rows 2 and 3;
// lane 63 then holds the whole wave's max.  The stages compare the values' ordered
// bits as integers (a float max would first quiet each moved value).
__device__ __forceinline__ float wave_max_dpp(float v) {
  int x = ord_bits(__builtin_bit_cast(int, v));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, DPP_QUAD_XOR1, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, DPP_QUAD_XOR2, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, DPP_ROW_HALF_MIRROR, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, DPP_ROW_MIRROR, 0xF, 0xF, true));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false));
  return __builtin_bit_cast(float, ord_bits(__builtin_amdgcn_readlane(x, 63)));
}
// Sum over the wave, returned wave-uniform: the stages of wave_max_dpp with adds (a
// row left out of a broadcast stage adds 0).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp<DPP_QUAD_XOR1>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  v += __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// LDS of one split workgroup: per-wave logits (ch0 + ch1 = 2 ch_steps per pair of
// waves sharing a SIMD, whatever the format), the wave partials (o, m, l) and one
// discarded-store slot per lane
template <int G>
__host__ __device__ constexpr size_t split_lds_bytes() {
  return sizeof(float) * ((size_t)DEC_WAVES * ch_steps<G>() * 8 * G + DEC_WAVES * G * HD +
                          2 * DEC_WAVES * G + DEC_WAVES * 64);
}
static_assert(split_lds_bytes<1>() <= 160 * 1024 && split_lds_bytes<2>() <= 160 * 1024 &&
                  split_lds_bytes<4>() <= 160 * 1024 && split_lds_bytes<8>() <= 160 * 1024,
              "a split workgroup fits in one CU's LDS");

template <int FMT, int G, int U, int PG>
__global__ __launch_bounds__(DEC_THREADS)
__attribute__((amdgpu_waves_per_eu(KVQ8_DEC_WAVES_PER_EU))) void k_decode_split(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int max_len, int kvh,
    const float* __restrict__ q, float qscale, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int S, const int32_t* __restrict__ pages, int page_stride,
    const int32_t* __restrict__ sid) {
  constexpr int CH0 = ch0<FMT, G>(), CH1 = ch1<FMT, G>();
  static_assert(FMT == KV_FMT_F16, "the int8-K formats take the pair kernels");
  static_assert(CH0 % (2 * U) == 0 && CH1 % (2 * U) == 0, "a chunk holds whole pairs of load batches");
  static_assert(CH0 >= KVQ8_DEC_MIN_STEPS && (!GROUPED || CH1 >= KVQ8_DEC_MIN_STEPS),
                "a short session's waves (at most KVQ8_DEC_MIN_STEPS steps) fit the logits budget");
  const int s_idx = blockIdx.x, h = blockIdx.y, rk = blockIdx.z;
  const int nqh = kvh * G;
  // tab, lens: the call's sessions, or ranked longest first with sid the session of
  // each rank (batches)
  const kv_session ss = tab[rk];
  const int len = lens[rk];
  const int b = sid != nullptr ? sid[rk] : rk;
  if (session_bad(ss, FMT) || len < 0 || len > ss.cap || len > max_len) return;  // merge flags
  const int J = (len + 7) >> 3;                  // 8-token steps of this session
  const int Jf = lead_steps<FMT>(J);             // steps of group 0 (>= those of group 1)
  const int Sb = active_splits<FMT>(len, S);   // workgroups of this session
  if (s_idx >= Sb) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane >> 3, c = lane & 7;
  const int grp = wave / GRP_WAVES, wg = wave % GRP_WAVES;
  const int Jg = grp ? J - Jf : Jf;              // steps of this wave's group
  const int gw0 = s_idx * GRP_WAVES + wg;        // wave index within the group's waves
  const int gw = (grp ? Jf : 0) + gw0;           // first step of this wave
  const int W = Sb * GRP_WAVES;                  // waves per group of (session, head)
  const int n_steps = gw0 < Jg ? (Jg - 1 - gw0) / W + 1 : 0;
  // paged (PG: the page map's registers, 0 for a contiguous session): this wave's
  // steps -> pool slots; steps past the session's end read its last step
  std::conditional_t<PG != 0, PageMap<PG ? PG : 4>, NoPages> pm{};
  if constexpr (PG != 0) pm.init(pages, page_stride, b, gw, W, n_steps, ss.cap / KV_PAGE_ROWS, len, lane);
  const int kclamp = 1 << 30;   // rows past len re-read row len - 1

  extern __shared__ float smem[];
  float* lg = smem + (grp ? GRP_WAVES * CH0 + wg * CH1 : wg * CH0) * 8 * G;  // logits, then p
  float* o_l = smem + GRP_WAVES * (CH0 + CH1) * 8 * G;   // [waves][G][HD]
  float* m_l = o_l + DEC_WAVES * G * HD;         // [waves][G]
  float* l_l = m_l + DEC_WAVES * G;              // [waves][G]
  float* junk = l_l + DEC_WAVES * G + (threadIdx.x >> 6) * 64;  // discarded stores

  const size_t hrow = (size_t)h * (size_t)ss.cap;  // the head's first row
  const char* kb = static_cast<const char*>(ss.k) + hrow * HD * 2;
  const char* vb = static_cast<const char*>(ss.v) + hrow * HD * 2;
  const char* nsc = nullptr;   // FP16: no scale arrays
  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
  }

  if (n_steps > 0) {
    const int hsel = head_map<G>(c);
    float qv[G][16];  // slot g: head g ^ hsel
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float* qp = q + ((long long)b * nqh + h * G + (g ^ hsel)) * HD;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 v = ldg128(qp + lane_dim<FMT>(c, 4 * k));   // 4 consecutive dims
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[g][4 * k + e] = as_f32(v[e]) * qscale;
      }
    }
    // U x G independent dot products, interleaved so that no FMA waits on the one
    // just before it; then the 8-lane reductions, then the logit stores.  Slot j of
    // a lane holds head j ^ hsel (see head_map), so the reduction folds: each DPP
    // stage adds the partner's upper slots to this lane's lower ones and halves
    // the values carried (4 DPP adds per step for G = 4 instead of 12).
    auto kstep = [&](const Batch<FMT, U>& cur, int k0, int it0, int n_it) __attribute__((always_inline)) {
      float part[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float kf = cur.ch[u].get(0);
#pragma unroll
        for (int g = 0; g < G; ++g) part[u][g] = qv[g][0] * kf;
      }
#pragma unroll
      for (int i = 1; i < 16; ++i) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float kf = cur.ch[u].get(i);
#pragma unroll
          for (int g = 0; g < G; ++g) part[u][g] = fmaf(qv[g][i], kf, part[u][g]);
        }
      }
      // stage by stage over all U values, so that no DPP add waits on the one before
      constexpr int N1 = G > 1 ? G / 2 : 1, N2 = N1 > 1 ? N1 / 2 : 1, N3 = N2 > 1 ? N2 / 2 : 1;
      fold_stage<DPP_QUAD_XOR1, U, G, G>(part);
      fold_stage<DPP_QUAD_XOR2, U, G, N1>(part);
      fold_stage<DPP_ROW_HALF_MIRROR, U, G, N2>(part);
      static_assert(N3 == 1, "three stages reduce up to 8 heads");
      // lanes c < G of each row hold distinct heads and write them; the others
      // write to their own slots of a scratch area, so no lane is masked off
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float* dst = c < G ? lg + ((it0 + u) * 8 + r) * G + hsel : junk + lane;
        *dst = part[u][0];
      }
    };
    auto vstep = [&](const Batch<FMT, U>& cur, int it0, int n_it) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = it0 + u;
        // p is 0 for tokens past the end (their logits were stored as -inf); slots
        // past n_it hold stale LDS (in bounds: CH0, CH1 are multiples of 2U) and are zeroed
        float w[G];
        load_p<G>(lg + (it * 8 + r) * G, w);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float vf = cur.ch[u].get(i);
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g][i] = fmaf(w[g], vf, acc[g][i]);
        }
      }
    };

    // Two load batches A and B alternate (a 2x-unrolled loop, no register copies);
    // the last K batch of a chunk prefetches its first V batch, the last V batch the
    // next chunk's first K batch, so loads stay in flight across the softmax.
    // Two load batches A and B alternate (a 2x-unrolled loop, no register copies);
    // the last K batch prefetches the first V batch, whose loads then overlap the
    // softmax.  The plan gives every wave at most its group's budget (CH0 or CH1) of steps.
    const int n_it = n_steps;
    Batch<FMT, U> A, B;
    // Softmax of the logits of steps [s0, s1): the running max m moves to cover them,
    // l and the accumulators are rescaled to it, and p = 2^(logit - m) replaces each
    // logit; slots up to s_pad (the V pass reads whole pairs of batches) get p = 0.
    auto softmax = [&](int s0, int s1, int s_pad) __attribute__((always_inline)) {
      float mc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) mc[g] = -INFINITY;
      for (int tl = s0 * 8 + lane; tl < s1 * 8; tl += 64) {
        const int t = (gw + (tl >> 3) * W) * 8 + (tl & 7);
        if (t < len) {
#pragma unroll
          for (int g = 0; g < G; ++g) mc[g] = fmaxf(mc[g], lg[tl * G + g]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // finite: every step of the wave holds a token below len
        const float mn = fmaxf(m[g], wave_max_dpp(mc[g]));
        const float f = __builtin_amdgcn_exp2f(m[g] - mn);   // 0 on the first chunk (m = -inf)
        m[g] = mn;
        l[g] *= f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] *= f;
      }
      for (int tl = s0 * 8 + lane; tl < s_pad * 8; tl += 64) {
        const int t = (gw + (tl >> 3) * W) * 8 + (tl & 7);
        const bool ok = tl < s1 * 8 && t < len;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          // the bare exp2 (results below 2^-126 flush to 0)
          const float p = ok ? __builtin_amdgcn_exp2f(lg[tl * G + g] - m[g]) : 0.f;
          lg[tl * G + g] = p;
          l[g] += p;
        }
      }
    };
    auto vpass = [&](int s0, int s1) __attribute__((always_inline)) {
      for (int it0 = s0; it0 < s1; it0 += 2 * U) {
        B.template load<true>(vb, nsc, gw, W, it0 + U, len, r, c, kclamp, pm);
        vstep(A, it0, n_it);
        if (it0 + 2 * U < s1) A.template load<true>(vb, nsc, gw, W, it0 + 2 * U, len, r, c, kclamp, pm);
        vstep(B, it0 + U, n_it);
      }
    };
    // ---- K pass -----------------------------------------------------------------
    A.template load<false>(kb, nsc, gw, W, 0, len, r, c, kclamp, pm);
    for (int it0 = 0; it0 < n_it; it0 += 2 * U) {
      B.template load<false>(kb, nsc, gw, W, it0 + U, len, r, c, kclamp, pm);
      kstep(A, 0, it0, n_it);
      if (it0 + 2 * U < n_it)
        A.template load<false>(kb, nsc, gw, W, it0 + 2 * U, len, r, c, kclamp, pm);
      else
        A.template load<true>(vb, nsc, gw, W, 0, len, r, c, kclamp, pm);
      kstep(B, 0, it0 + U, n_it);
    }
    wave_lds_fence();
    softmax(0, n_it, (n_it + 2 * U - 1) / (2 * U) * (2 * U));
    wave_lds_fence();
    // ---- V pass -----------------------------------------------------------------
    vpass(0, n_it);
#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = wave_sum_dpp(l[g]);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] = sum_rows8(acc[g][i]);
  }

  // ---- combine the 8 wave partials of the workgroup --------------------------
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

// k_decode_pair: the int8-K formats (q8, K8V4), with the waves of a workgroup in
//   4 pairs.  A SIMD runs one pair: a V wave (waves 0-3, the older of the two, which
//   the arbiter favours) and a K wave (waves 4-7) that share the pair's steps,
//   gw, gw + W, gw + 2W, ... (W = 4 x the active splits), in chunks of PAIR_CH
//   steps.  The K wave streams the K codes, computes the chunk's logits on the
//   matrix cores and its softmax (running max m, rescale factor f, p = 2^(logit - m),
//   running sum l) into one of two LDS buffers; the V wave, one chunk behind,
//   rescales its accumulators by f and streams the V rows against p.  One workgroup
//   barrier per chunk hands a buffer from the K wave to the V wave and back.  Each
//   wave keeps one kind of load in flight all the time, and the V wave's arithmetic
//   overlaps the K wave's loads on the same SIMD.
#ifndef KVQ8_DEC_PAIR_CH
#define KVQ8_DEC_PAIR_CH 16
#endif
// waves per SIMD the pair kernel's registers must allow (4: two workgroups per CU)
#ifndef KVQ8_DEC_PAIR_WPE
#define KVQ8_DEC_PAIR_WPE 4
#endif
constexpr int PAIRS = DEC_WAVES / 2;
constexpr int PAIR_CH = KVQ8_DEC_PAIR_CH;
// fewest steps a pair of a split is planned to take (the plan's cap on splits)
constexpr int PAIR_MIN_STEPS = 32;
// steps per pair the plan aims for at most, so that long sessions spread over many
// workgroups (balance across CUs and sessions)
#ifndef KVQ8_DEC_PAIR_TARGET
#define KVQ8_DEC_PAIR_TARGET 256
#endif
constexpr int PAIR_TARGET_STEPS = KVQ8_DEC_PAIR_TARGET;
static_assert(PAIR_TARGET_STEPS <= 256, "a pair has at most 256 steps (4 registers of page map)");

template <int G>
__host__ __device__ constexpr size_t pair_lds_bytes() {
  return sizeof(float) * ((size_t)PAIRS * 2 * PAIR_CH * 8 * G + PAIRS * 2 * G + PAIRS * G * HD +
                          2 * PAIRS * G + DEC_WAVES * 64);
}
static_assert(pair_lds_bytes<8>() <= 160 * 1024, "a pair workgroup fits in one CU's LDS");

template <int FMT, int G, int U, int PG>
__global__ __launch_bounds__(DEC_THREADS) __attribute__((amdgpu_waves_per_eu(G >= 8 ? 2 : KVQ8_DEC_PAIR_WPE))) void k_decode_pair(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int max_len, int kvh,
    const float* __restrict__ q, float qscale, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int S, const int32_t* __restrict__ pages, int page_stride,
    const int32_t* __restrict__ sid) {
  static_assert(FMT != KV_FMT_F16, "the pair kernel reads int8 K codes");
  constexpr int UK = k_batch_rows<G>();
  static_assert(PAIR_CH % (2 * UK) == 0 && PAIR_CH % (2 * U) == 0,
                "a chunk holds whole pairs of K and of V batches");
  constexpr int NHB = G > 4 ? 2 : 1;
  const int s_idx = blockIdx.x, h = blockIdx.y, rk = blockIdx.z;
  const int nqh = kvh * G;
  // tab, lens: the call's sessions, or ranked longest first with sid the session of
  // each rank (batches)
  const kv_session ss = tab[rk];
  const int len = lens[rk];
  const int b = sid != nullptr ? sid[rk] : rk;
  // workgroup-uniform exits only (the loop below has barriers)
  if (session_bad(ss, FMT) || len < 0 || len > ss.cap || len > max_len) return;  // merge flags
  const int J = (len + 7) >> 3;
  const int Sb = active_splits<FMT>(len, S);
  if (s_idx >= Sb) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane >> 3, c = lane & 7;
  const bool kw = wave >= PAIRS;                 // the K wave of its pair
  const int pr = wave & (PAIRS - 1);
  const int gw = s_idx * PAIRS + pr;             // first step of the pair
  const int W = Sb * PAIRS;
  const int n_steps = gw < J ? (J - 1 - gw) / W + 1 : 0;
  const int n_first = s_idx * PAIRS < J ? (J - 1 - s_idx * PAIRS) / W + 1 : 0;  // pair 0's
  const int n_chunks = (n_first + PAIR_CH - 1) / PAIR_CH;   // the same for every wave
  // paged (PG: the page map's registers, 0 for a contiguous session): this pair's
  // steps -> pool slots
  std::conditional_t<PG != 0, PageMap<PG ? PG : 4>, NoPages> pm{};
  if constexpr (PG != 0) pm.init(pages, page_stride, b, gw, W, n_steps, ss.cap / KV_PAGE_ROWS, len, lane);

  extern __shared__ float smem[];
  float* pb = smem + (size_t)pr * 2 * PAIR_CH * 8 * G;      // this pair's two chunk buffers
  float* fb = smem + (size_t)PAIRS * 2 * PAIR_CH * 8 * G + pr * 2 * G;   // [2][G] factors
  float* o_l = smem + (size_t)PAIRS * 2 * PAIR_CH * 8 * G + PAIRS * 2 * G;   // [pairs][G][HD]
  float* m_l = o_l + PAIRS * G * HD;             // [pairs][G]
  float* l_l = m_l + PAIRS * G;                  // [pairs][G]
  float* junk = l_l + PAIRS * G + wave * 64;     // discarded stores

  constexpr int VB = FMT == KV_FMT_K8V4 ? HD / 2 : HD;   // bytes per V row
  constexpr int VSC = FMT == KV_FMT_K8V4 ? NQ4 : NGRP;    // V scales per row
  const size_t hrow = (size_t)h * (size_t)ss.cap;
  const char* kb = static_cast<const char*>(ss.k) + hrow * HD;
  const char* vb = static_cast<const char*>(ss.v) + hrow * VB;
  const char* ksb = reinterpret_cast<const char*>(ss.k_scale) + hrow * NGRP * 2;
  const char* vsb = reinterpret_cast<const char*>(ss.v_scale) + hrow * VSC * 2;

  float m[G], l[G];           // K wave: running max (wave-uniform), lane sums of p
  float acc[G][16], accw[G];  // V wave
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    accw[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
  }

  if (kw) {
    // ================= K wave ===================================================
    i32x4 aq[NHB][NGRP];
    float qs[NHB][NGRP][QLEV];
    {
      const int mrow = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int ga = hb * 4 + (mrow >> 2), lev = mrow & 3;   // this lane's A row
#pragma unroll
        for (int grp = 0; grp < NGRP; ++grp) {
          const float* qp =
              q + ((long long)b * nqh + h * G + min(ga, G - 1)) * HD + grp * 64 + kq * 16;
          float x[16];
          float mx = 0.f;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const u32x4 v = ldg128(qp + 4 * k);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[4 * k + e] = as_f32(v[e]) * qscale;
              mx = fmaxf(mx, fabsf(x[4 * k + e]));
            }
          }
          mx = fmaxf(mx, shfl_xor(mx, 16));
          mx = fmaxf(mx, shfl_xor(mx, 32));
          float sl[QLEV];
          sl[0] = mx > 0.f ? mx / 127.f : 1.f;
#pragma unroll
          for (int lv = 1; lv < QLEV; ++lv) sl[lv] = sl[lv - 1] * QBASE_INV;
          const bool live = ga < G && lev < QLEV;
          uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float rr = x[i];
            int a = 0;
#pragma unroll
            for (int lv = 0; lv < QLEV; ++lv) {
              const int al = q_level(rr, sl[lv]);
              a = lv == lev ? al : a;
            }
            wd[i >> 2] |= (uint32_t)((live ? a : 0) & 0xFF) << (8 * (i & 3));
          }
          aq[hb][grp] = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
#pragma unroll
          for (int lv = 0; lv < QLEV; ++lv) qs[hb][grp][lv] = __shfl(sl[lv], 4 * kq, 64);
        }
      }
    }
    // logits of the 16-token blocks of a batch whose first step is k (chunk-relative
    // k - c0) into the chunk buffer lc
    auto kstep = [&](const KBatch<UK>& cur, float* lc, int kr) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < UK / 2; ++j) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          float v = 0.f;
#pragma unroll
          for (int grp = 0; grp < NGRP; ++grp) {
            const u32x4& bw = cur.w[j][grp];
            const i32x4 bk = i32x4{(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
            const i32x4 d =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[hb][grp], bk, i32x4{0, 0, 0, 0}, 0, 0, 0);
            const float lv = fmaf((float)d[2], qs[hb][grp][2],
                                  fmaf((float)d[1], qs[hb][grp][1], (float)d[0] * qs[hb][grp][0]));
            v = fmaf(lv, h2f(cur.sc[j][grp]), v);
          }
          const int g = hb * 4 + (lane >> 4);
          float* dst = g < G ? lc + ((kr + 2 * j) * 8 + (lane & 15)) * G + g : junk + lane;
          *dst = v;
        }
      }
    };
    // One loop over the chunks' steps, the same count for every wave of the
    // workgroup; loads run on across chunk ends (steps past the pair's last one
    // re-read it), and each chunk ends with its softmax and a barrier.
    const int kmax = max(n_steps - 1, 0);
    const int total = n_chunks * PAIR_CH;
    KBatch<UK> KA, KB;
    // the loop body; pf: prefetch the next batch (not on the last iteration, so no
    // load past the loop is issued)
    auto kiter = [&](int k0, bool pf) __attribute__((always_inline)) {
      const int ch = k0 / PAIR_CH, kr = k0 - ch * PAIR_CH;
      float* lc = pb + (ch & 1) * PAIR_CH * 8 * G;
      KB.load(kb, ksb, gw, W, k0 + UK, len, lane, kmax, pm);
      kstep(KA, lc, kr);
      if (pf) KA.load(kb, ksb, gw, W, k0 + 2 * UK, len, lane, kmax, pm);
      kstep(KB, lc, kr + UK);
      if (kr + 2 * UK == PAIR_CH) {
        wave_lds_fence();
        // softmax of the chunk: the max moves to cover it, l is rescaled, p replaces
        // each logit (0 past the pair's last step, so the V wave may run whole chunks)
        const int c0 = ch * PAIR_CH;
        const int nl = max(0, min(n_steps, c0 + PAIR_CH) - c0) * 8;
        float mc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) mc[g] = -INFINITY;
        for (int tl = lane; tl < nl; tl += 64) {
          const int t = (gw + (c0 + (tl >> 3)) * W) * 8 + (tl & 7);
          if (t < len) {
#pragma unroll
            for (int g = 0; g < G; ++g) mc[g] = fmaxf(mc[g], lc[tl * G + g]);
          }
        }
        float* fc = fb + (ch & 1) * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float mn = fmaxf(m[g], wave_max_dpp(mc[g]));
          // 0 on the pair's first chunk (m = -inf); 1 while the pair has no token yet
          const float f = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[g] - mn);
          m[g] = mn;
          l[g] *= f;
          if (lane == g) fc[g] = f;
        }
        for (int tl = lane; tl < PAIR_CH * 8; tl += 64) {
          const int t = (gw + (c0 + (tl >> 3)) * W) * 8 + (tl & 7);
          const bool ok = tl < nl && t < len;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pv = ok ? __builtin_amdgcn_exp2f(lc[tl * G + g] - m[g]) : 0.f;
            lc[tl * G + g] = pv;
            l[g] += pv;
          }
        }
        __syncthreads();
      }
    };
    if (total > 0) {
      KA.load(kb, ksb, gw, W, 0, len, lane, kmax, pm);
      int k0 = 0;
      for (; k0 + 2 * UK < total; k0 += 2 * UK) kiter(k0, true);
      kiter(k0, false);
    }
    __syncthreads();   // the V wave's last chunk
#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = wave_sum_dpp(l[g]);
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        m_l[pr * G + g] = m[g];
        l_l[pr * G + g] = l[g];
      }
    }
  } else {
    // ================= V wave ===================================================
    auto vstep = [&](const Batch<FMT, U>& cur, const float* pc, int kr) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float sc = cur.scale(u);
        float w[G];
        load_p<G>(pc + ((kr + u) * 8 + r) * G, w);
#pragma unroll
        for (int g = 0; g < G; ++g) w[g] *= sc;
        if constexpr (FMT == KV_FMT_K8V4) {
#pragma unroll
          for (int g = 0; g < G; ++g) accw[g] += w[g];
          const u32x4& cw = cur.ch[u].w;
          const uint32_t nb[4] = {nibble_bytes(cw[0]), nibble_bytes(cw[0] >> 4),
                                  nibble_bytes(cw[1]), nibble_bytes(cw[1] >> 4)};
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t src = nb[2 * (i >> 3) + (i & 1)];
            const float vf = (float)((src >> (8 * ((i & 7) >> 1))) & 0xFFu);   // code + 8
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g][i] = fmaf(w[g], vf, acc[g][i]);
          }
        } else {
          const u32x4& cw = cur.ch[u].w;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float vf = i8_to_f32(cw[i >> 2], i & 3);
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g][i] = fmaf(w[g], vf, acc[g][i]);
          }
        }
      }
    };
    // the same single loop, one chunk behind the K wave
    const int kmax = max(n_steps - 1, 0);
    const int total = n_chunks * PAIR_CH;
    Batch<FMT, U> A, B;
    auto viter = [&](int k0, bool pf) __attribute__((always_inline)) {
      const int ch = k0 / PAIR_CH, kr = k0 - ch * PAIR_CH;
      const float* pc = pb + (ch & 1) * PAIR_CH * 8 * G;
      if (kr == 0) {
        if (ch > 0) __syncthreads();   // the K wave's chunk ch
        const float* fc = fb + (ch & 1) * G;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float f = fc[g];
          accw[g] *= f;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[g][i] *= f;
        }
      }
      B.template load<true>(vb, vsb, gw, W, k0 + U, len, r, c, kmax, pm);
      vstep(A, pc, kr);
      if (pf) A.template load<true>(vb, vsb, gw, W, k0 + 2 * U, len, r, c, kmax, pm);
      vstep(B, pc, kr + U);
    };
    if (total > 0) A.template load<true>(vb, vsb, gw, W, 0, len, r, c, kmax, pm);
    __syncthreads();   // the K wave's first chunk
    if (total > 0) {
      int k0 = 0;
      for (; k0 + 2 * U < total; k0 += 2 * U) viter(k0, true);
      viter(k0, false);
    }
    if (total > 0) __syncthreads();   // frees the K wave's last buffer
    if constexpr (FMT == KV_FMT_K8V4) {  // sum_t w_t (n - 8) = sum_t w_t n - 8 sum_t w_t
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = fmaf(-8.f, accw[g], acc[g][i]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] = sum_rows8(acc[g][i]);
    if (r == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 16; i += 4)
          *reinterpret_cast<float4*>(o_l + (pr * G + g) * HD + lane_dim<FMT>(c, i)) =
              make_float4(acc[g][i], acc[g][i + 1], acc[g][i + 2], acc[g][i + 3]);
    }
  }
  // ---- combine the pair partials of the workgroup ----------------------------
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * HD; idx += DEC_THREADS) {
    const int g = idx / HD, d = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < PAIRS; ++w) M = fmaxf(M, m_l[w * G + g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < PAIRS; ++w) {
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

// k_decode_pair_mv: the int8-K formats with 1, 2 or 4 query heads per kv head, both
//   products on the matrix cores, in the pairs of k_decode_pair.
//   K wave: the logits as in k_decode_pair; then, per 64-token block (8 steps), the
//     weights w = p * (V scale of the token's group of dims), each split into two bf16
//     values, hi = w truncated to bf16 and lo = (w - hi) rounded to bf16
//     (|w - hi - lo| <= 2^-16 |w|), written to LDS as a table of 16 rows (two groups
//     of dims, 4 heads, hi / lo) by the block's 64 tokens, token-major (a lane stores
//     its token's rows of one group with one 16-byte store); the V wave reads it back
//     as MFMA A operands with transposing 16-bit reads (ds_read_b64_tr_b16).  Q8 has
//     two 64-dim groups: one table.  K8V4 has four 32-dim groups of its rotated V: two
//     tables, groups 0-1 and 2-3.
//   V wave: stages the block's V rows in an LDS tile as bytes (Q8: the signed codes as
//     loaded; K8V4: each nibble n made the byte 0x80 | n << 3, two per input byte, in
//     dim order of the rotated row) and reads them back transposed (ds_read_b64_tr_b8:
//     16 lanes receive one dim each, 8 tokens per read); a Q8 code of at most 7 bits
//     becomes bf16 exactly (the upper half of its fp32 value), a K8V4 byte is the low
//     byte of the bf16 value 16 + n; one v_mfma_f32_16x16x32_bf16 per 16 dims and 32
//     tokens accumulates the rows' products in fp32 (K8V4 then takes out 24 times the
//     weights' sums: 16 + n = 24 + code).  The block's 64 tokens are the k-slots of both
//     operands in the same order.  Lane (q, i) of a 16-dim tile holds rows 4q .. 4q + 3
//     of its table; the tile's dims belong to one group, whose rows (0 .. 7 or 8 .. 15)
//     are kept.  K8V4 leaves its output in the rotated basis; the merge undoes the
//     rotation.
//   Against the vector V pass this moves the 64 FMAs a lane spends per step and 4
//   heads onto the matrix cores; the V wave keeps 12 conversions per 8 Q8 codes, or 6
//   bit operations and 6 byte permutes per 8 K8V4 values.
#ifndef KVQ8_DEC_MV_CH
#define KVQ8_DEC_MV_CH 16
#endif
constexpr int MV_CH = KVQ8_DEC_MV_CH;  // steps per chunk (Q8)
constexpr int MV_BLK = 8;              // steps per 64-token block
constexpr int MV_PITCH = 144;          // bytes per V tile row (16-byte aligned rows)
// a weight table: 64 tokens x 16 bf16 rows, token-major (32 bytes per token)
constexpr int MV_TBL = 64 * 32;        // bytes per table
static_assert(MV_CH % (2 * MV_BLK) == 0, "a chunk holds whole pairs of blocks");

// steps per chunk: K8V4's two weight tables per block take one-block chunks, so that
// two workgroups still share a CU's LDS
template <int FMT>
__host__ __device__ constexpr int mv_chunk() { return FMT == KV_FMT_K8V4 ? MV_BLK : MV_CH; }
template <int FMT>
__host__ __device__ constexpr int mv_tables() { return FMT == KV_FMT_K8V4 ? 2 : 1; }
template <int FMT, int G>
__host__ __device__ constexpr size_t mv_pair_bytes() {
  // logits of one chunk, the weight tables of two chunks, the rescale factors of two
  // chunks, the V tile
  return (size_t)mv_chunk<FMT>() * 8 * G * 4 +
         2 * (size_t)(mv_chunk<FMT>() / MV_BLK) * mv_tables<FMT>() * MV_TBL + 2 * 4 * 4 +
         64 * MV_PITCH;
}
template <int FMT, int G>
__host__ __device__ constexpr size_t mv_lds_bytes() {
  // the logit stores of lanes past G heads go to a per-wave discard area (none for G = 4)
  return PAIRS * mv_pair_bytes<FMT, G>() + (G < 4 ? DEC_WAVES * 64 * 4 : 0);
}
static_assert(mv_pair_bytes<KV_FMT_Q8, 4>() % 16 == 0 && mv_pair_bytes<KV_FMT_Q8, 2>() % 16 == 0 &&
                  mv_pair_bytes<KV_FMT_Q8, 1>() % 16 == 0 &&
                  mv_pair_bytes<KV_FMT_K8V4, 4>() % 16 == 0 &&
                  mv_pair_bytes<KV_FMT_K8V4, 2>() % 16 == 0 &&
                  mv_pair_bytes<KV_FMT_K8V4, 1>() % 16 == 0,
              "pair regions keep 16-byte alignment");
static_assert(PAIRS * mv_pair_bytes<KV_FMT_K8V4, 1>() >=
                  sizeof(float) * (PAIRS * 4 * HD + 2 * PAIRS * 4),
              "the final partials fit in the pair regions");
static_assert(mv_lds_bytes<KV_FMT_Q8, 4>() <= 80 * 1024 && mv_lds_bytes<KV_FMT_K8V4, 4>() <= 80 * 1024,
              "two workgroups share a CU's 160 KB of LDS");

typedef int i32x2 __attribute__((ext_vector_type(2)));
#define KVQ8_LDS __attribute__((address_space(3)))
// transposing 8-byte LDS read: within each 16 lanes, lane i receives byte i % 8 of
// the 8 bytes addressed by lanes 2 j + i / 8, j = 0 .. 7
__device__ __forceinline__ i32x2 lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((KVQ8_LDS i32x2*)(KVQ8_LDS uint8_t*)p);
}
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
// two transposing 16-bit LDS reads (ds_read_b64_tr_b16: within each 16 lanes, lane i
// receives element i % 4 of the 8 bytes addressed by lanes 4 e + i / 4, e = 0 .. 3)
// joined as one 8-element bf16 operand, p0's four elements first
__device__ __forceinline__ bf16x8 lds_tr16x2(const uint8_t* p0, const uint8_t* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((KVQ8_LDS i16x4*)(KVQ8_LDS uint8_t*)p0);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((KVQ8_LDS i16x4*)(KVQ8_LDS uint8_t*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// G consecutive floats of LDS in one read (16-byte aligned for G = 4, 8-byte for 2)
template <int G>
__device__ __forceinline__ void lds_floats(const float* p, float (&o)[G]) {
  if constexpr (G == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p);
    o[0] = t[0]; o[1] = t[1]; o[2] = t[2]; o[3] = t[3];
  } else if constexpr (G == 2) {
    const f32x2 t = *reinterpret_cast<const f32x2*>(p);
    o[0] = t[0]; o[1] = t[1];
  } else {
    o[0] = p[0];
  }
}
// 8 int8 codes (the bytes of c, in order) as 8 bf16, exactly: the upper half of each
// code's fp32 value
__device__ __forceinline__ bf16x8 codes_bf16(i32x2 c) {
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t src = (uint32_t)(d < 2 ? c.x : c.y);
    const uint32_t f0 = __builtin_bit_cast(uint32_t, i8_to_f32(src, 2 * (d & 1)));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, i8_to_f32(src, 2 * (d & 1) + 1));
    o[d] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
}
// K8V4 in the matrix-core V pass: 8 nibbles n (one 32-bit word, value j in bits
// 4j .. 4j + 3) as the bytes 0x80 | n << 3 in value order (two words), the low byte of
// the bf16 value 16 + n (0x4180 + 8 n): the bf16 operand is then one byte permute per
// two values, and the pass sums w (16 + n) = w (24 + code), from which the weights'
// own sum times 24 is taken out.
__device__ __forceinline__ void nibbles_to_biased(uint32_t x, uint32_t& o0, uint32_t& o1) {
  const uint32_t lo = ((x << 3) & 0x78787878u) | 0x80808080u;   // values 0, 2, 4, 6
  const uint32_t hi = ((x >> 1) & 0x78787878u) | 0x80808080u;   // values 1, 3, 5, 7
  o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}
// 8 biased bytes b (the bytes of c, in order) as the bf16 values 0x41 << 8 | b
__device__ __forceinline__ bf16x8 biased_bf16(i32x2 c) {
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    o[d] = __builtin_amdgcn_perm(0x41414141u, (uint32_t)(d < 2 ? c.x : c.y),
                                 (d & 1) ? 0x04030402u : 0x04010400u);
  return __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
}
template <int FMT, int G, int PG, int SP>
__global__ __launch_bounds__(DEC_THREADS) __attribute__((amdgpu_waves_per_eu(KVQ8_DEC_PAIR_WPE)))
void k_decode_pair_mv(const kv_session* __restrict__ tab, const int32_t* __restrict__ lens,
                      int max_len, int kvh, const float* __restrict__ q, float qscale,
                      float* __restrict__ ws_o, float* __restrict__ ws_lse, int S,
                      const int32_t* __restrict__ pages, int page_stride,
                      const int32_t* __restrict__ sid) {
  static_assert(FMT == KV_FMT_Q8 || FMT == KV_FMT_K8V4, "int8 K codes");
  static_assert(G <= 4, "one block of 4 heads");
  constexpr bool K4 = FMT == KV_FMT_K8V4;
  constexpr int CHK = mv_chunk<FMT>();           // steps per chunk
  constexpr int UK = CHK / 2;                    // steps per K batch: two per chunk
  constexpr int NT = mv_tables<FMT>();           // weight tables per block
  static_assert(CHK % MV_BLK == 0 && (UK == MV_BLK || 2 * UK == MV_BLK),
                "a chunk is whole blocks; a K batch is a block or half of one");
  constexpr int NCB = CHK / MV_BLK;              // blocks per chunk
  constexpr int VROW = K4 ? HD / 2 : HD;         // bytes per V row
  constexpr int VSC = K4 ? NQ4 : NGRP;           // V scales per row
  const int s_idx = blockIdx.x, h = blockIdx.y, rk = blockIdx.z;
  const int nqh = kvh * G;
  // tab, lens: the call's sessions, or ranked longest first with sid the session of
  // each rank (batches)
  const kv_session ss = tab[rk];
  const int len = lens[rk];
  const int b = sid != nullptr ? sid[rk] : rk;
  // workgroup-uniform exits only (the loops below have barriers)
  if (session_bad(ss, FMT) || len < 0 || len > ss.cap || len > max_len) return;  // merge flags
  const int J = (len + 7) >> 3;
  const int Sb = active_splits<FMT>(len, S);
  if (s_idx >= Sb) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane >> 3, c = lane & 7;
  const bool kw = wave >= PAIRS;
  const int pr = wave & (PAIRS - 1);
  const int gw = s_idx * PAIRS + pr;
  const int W = Sb * PAIRS;
  // steps dealt in units of SP (step_g<SP>): the J steps form NU units, unit u to
  // wave u mod W; the wave holding the last unit has J - SP (NU - 1) steps of it
  const int NU = (J + SP - 1) / SP;
  const int nu = gw < NU ? (NU - 1 - gw) / W + 1 : 0;
  const int n_steps = nu ? min(SP * nu, J - SP * (gw + (nu - 1) * W) + SP * (nu - 1)) : 0;
  // steps the pairs run through: pair 0 holds the most units (a bound on every pair's
  // steps), rounded to whole pairs of blocks (whole chunks; the V wave takes blocks in
  // pairs)
  const int n_first = s_idx * PAIRS < NU ? SP * ((NU - 1 - s_idx * PAIRS) / W + 1) : 0;
  const int total = (n_first + 2 * MV_BLK - 1) / (2 * MV_BLK) * (2 * MV_BLK);
  const int kmax = max(n_steps - 1, 0);
  // paged (PG: the page map's registers, 0 for a contiguous session): this pair's
  // steps -> pool slots; steps past the session's end read its last step
  std::conditional_t<PG != 0, PageMap<PG ? PG : 4, SP>, NoPages> pm{};
  if constexpr (PG != 0) pm.init(pages, page_stride, b, gw, W, n_steps, ss.cap / KV_PAGE_ROWS, len, lane);

  extern __shared__ float smem[];
  uint8_t* reg = reinterpret_cast<uint8_t*>(smem) + (size_t)pr * mv_pair_bytes<FMT, G>();
  float* lc = reinterpret_cast<float*>(reg);                            // [CHK*8][G]
  uint8_t* at = reg + (size_t)CHK * 8 * G * 4;                          // [2][NCB][NT][TBL]
  float* fb = reinterpret_cast<float*>(at + 2 * NCB * NT * MV_TBL);     // [2][4]
  uint8_t* tile = reinterpret_cast<uint8_t*>(fb + 8);                   // [64][PITCH]
  // discarded logit stores of lanes past G heads (only G < 4 has such lanes)
  float* junk = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) +
                                         PAIRS * mv_pair_bytes<FMT, G>()) + wave * 64;
  // after the loops every pair region is free: the partials reuse them
  float* o_l = smem;                         // [pairs][G][HD]
  float* m_l = o_l + PAIRS * G * HD;         // [pairs][G]
  float* l_l = m_l + PAIRS * G;              // [pairs][G]

  const size_t hrow = (size_t)h * (size_t)ss.cap;
  const char* kb = static_cast<const char*>(ss.k) + hrow * HD;
  const char* vb = static_cast<const char*>(ss.v) + hrow * VROW;
  const char* ksb = reinterpret_cast<const char*>(ss.k_scale) + hrow * NGRP * 2;
  const char* vsb = reinterpret_cast<const char*>(ss.v_scale) + hrow * VSC * 2;
  // the pool row (contiguous: the row) of token 64 bl + lane of the chunk starting at
  // step ch CHK: row lane % 8 of its step
  // Step sb + i of a wave, sb a multiple of 8 (so of SP) and i < 8, is its step sb
  // plus step_g(0, i): the lane's part of the step (step i = lane / 8 of the 8 that
  // start at sb) is one constant, the rest wave-uniform.
  // step_g grows with the step, so steps past the wave's last (masked tokens) clamp to
  // that step's rows, which the wave reads anyway.
  const int lane_step = step_g<SP>(0, lane >> 3, W);
  const int step_last = step_g<SP>(gw, kmax, W);
  auto chunk_row = [&](int ch, int bl) __attribute__((always_inline)) {
    const int st = ch * CHK + bl * 8 + (lane >> 3);
    if constexpr (PG != 0) return pm.lane_row(pm.block(ch * CHK + bl * 8), st, gw, W, lane & 7);
    else
      return (uint32_t)min(
          min(step_g<SP>(gw, ch * CHK + bl * 8, W) + lane_step, step_last) * 8 + (lane & 7), len - 1);
  };

  if (kw) {
    // ================= K wave ===================================================
    float m[G], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
    }
    i32x4 aq[NGRP];
    float qs[NGRP][QLEV];
    {
      const int mrow = lane & 15, kq = lane >> 4;
      const int ga = mrow >> 2, lev = mrow & 3;
#pragma unroll
      for (int grp = 0; grp < NGRP; ++grp) {
        const float* qp =
            q + ((long long)b * nqh + h * G + min(ga, G - 1)) * HD + grp * 64 + kq * 16;
        float x[16];
        float mx = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4 v = ldg128(qp + 4 * k);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[4 * k + e] = as_f32(v[e]) * qscale;
            mx = fmaxf(mx, fabsf(x[4 * k + e]));
          }
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        float sl[QLEV];
        sl[0] = mx > 0.f ? mx / 127.f : 1.f;
#pragma unroll
        for (int lv = 1; lv < QLEV; ++lv) sl[lv] = sl[lv - 1] * QBASE_INV;
        const bool live = ga < G && lev < QLEV;
        uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float rr = x[i];
          int a = 0;
#pragma unroll
          for (int lv = 0; lv < QLEV; ++lv) {
            const int al = q_level(rr, sl[lv]);
            a = lv == lev ? al : a;
          }
          wd[i >> 2] |= (uint32_t)((live ? a : 0) & 0xFF) << (8 * (i & 3));
        }
        aq[grp] = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
#pragma unroll
        for (int lv = 0; lv < QLEV; ++lv) qs[grp][lv] = __shfl(sl[lv], 4 * kq, 64);
      }
    }
    // the K scales of the batch's tokens come from the chunk's scale words: token
    // n = lane % 16 of 16-token piece j of the batch (first step kr of its chunk) is
    // lane 8 kr + 16 j + n (mod 64) of its 64-token block (ksw: that block's word)
    auto kstep = [&](const KBatch<UK, SP, false>& cur, int kr, uint32_t ksw)
        __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < UK / 2; ++j) {
        const uint32_t kw2 =
            (uint32_t)__shfl((int)ksw, ((8 * kr) & 63) + 16 * j + (lane & 15), 64);
        const float ks[NGRP] = {h2f((uint16_t)(kw2 & 0xFFFFu)), h2f((uint16_t)(kw2 >> 16))};
        float v = 0.f;
#pragma unroll
        for (int grp = 0; grp < NGRP; ++grp) {
          const u32x4& bw = cur.w[j][grp];
          const i32x4 bk = i32x4{(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3]};
          const i32x4 d =
              __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[grp], bk, i32x4{0, 0, 0, 0}, 0, 0, 0);
          const float lv = fmaf((float)d[2], qs[grp][2],
                                fmaf((float)d[1], qs[grp][1], (float)d[0] * qs[grp][0]));
          v = fmaf(lv, ks[grp], v);
        }
        const int g = lane >> 4;
        float* dst = g < G ? lc + ((kr + 2 * j) * 8 + (lane & 15)) * G + g : junk + lane;
        *dst = v;
      }
    };
    // the K scale words of a chunk: lane l of block bl holds both 64-dim group scales
    // (4 bytes) of token 64 bl + l of the chunk, one 32-bit load per lane and block
    uint32_t ksn[NCB], ksx[NCB] = {};   // this chunk's and the next one's
    auto k_scales = [&](int ch, uint32_t (&dst)[NCB]) __attribute__((always_inline)) {
#pragma unroll
      for (int bl = 0; bl < NCB; ++bl)
        dst[bl] = *(const KVQ8_GLOBAL uint32_t*)(ksb + chunk_row(ch, bl) * NGRP * 2);
    };
    // the V scales of a chunk, loaded as it starts: per lane and block the token's
    // VSC fp16 scales
    uint32_t svn[NCB][VSC / 2];
    auto chunk_start = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
      for (int bl = 0; bl < NCB; ++bl) {
        const uint32_t row = chunk_row(ch, bl);
        if constexpr (K4) {
          const u32x2 t = *(const KVQ8_GLOBAL u32x2*)(vsb + row * VSC * 2);
          svn[bl][0] = t[0];
          svn[bl][1] = t[1];
        } else {
          svn[bl][0] = *(const KVQ8_GLOBAL uint32_t*)(vsb + row * VSC * 2);
        }
      }
      if ((ch + 1) * CHK < total) k_scales(ch + 1, ksx);
    };
    // the chunk's softmax, then per block the weight tables; a barrier hands them over
    auto chunk_end = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
      for (int bl = 0; bl < NCB; ++bl) ksn[bl] = ksx[bl];
      wave_lds_fence();
      const int c0 = ch * CHK;
      const int nl = max(0, min(n_steps, c0 + CHK) - c0) * 8;
      // the lane's token of each block: whether it is one of the session's tokens,
      // its logits (all heads, one read)
      bool ok[NCB];
      float mc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) mc[g] = -INFINITY;
#pragma unroll
      for (int bl = 0; bl < NCB; ++bl) {
        const int tl = bl * 64 + lane;
        const int t = (step_g<SP>(gw, c0 + bl * 8, W) + lane_step) * 8 + (lane & 7);
        ok[bl] = tl < nl && t < len;
        float lg[G];
        lds_floats<G>(lc + tl * G, lg);
#pragma unroll
        for (int g = 0; g < G; ++g) mc[g] = max2(mc[g], ok[bl] ? lg[g] : -INFINITY);
      }
      float f[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = max2(m[g], wave_max_dpp(mc[g]));
        f[g] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[g] - mn);
        m[g] = mn;
        l[g] *= f[g];
      }
      if (lane == 0) {
        float* fc = fb + (ch & 1) * 4;
#pragma unroll
        for (int g = 0; g < G; ++g) fc[g] = f[g];
      }
      // Table layout (table grp / 2, row m = 8 (grp % 2) + 2 head + part): token
      // t = 8 g8 + j of the block (lane t) keeps its 16 rows in 32 bytes at
      // 256 g8 + 128 ((j / 4) ^ s) + 32 (j % 4), s = g8 % 2, rows 8 h .. 8 h + 7 in the
      // 16-byte half h ^ s: one 16-byte store per token and group, and the 16 lanes of
      // a store (or of a transposing read in the V wave) cover all 64 banks.  Rows of
      // heads past G hold 0.
      const int g8k = lane >> 3, jk = lane & 7, swk = g8k & 1;
      uint8_t* atc = at + (ch & 1) * NCB * NT * MV_TBL + g8k * 256 + ((jk >> 2) ^ swk) * 128 +
                     (jk & 3) * 32;
#pragma unroll
      for (int bl = 0; bl < NCB; ++bl) {
        float sv[VSC];
#pragma unroll
        for (int k = 0; k < VSC / 2; ++k) {
          sv[2 * k] = h2f((uint16_t)(svn[bl][k] & 0xFFFFu));
          sv[2 * k + 1] = h2f((uint16_t)(svn[bl][k] >> 16));
        }
        // p = 2^(logit - max), 0 for a token past the session's end (whose logit slot
        // may hold anything); results below 2^-126 flush to 0
        float lg[G], p[G];
        lds_floats<G>(lc + (bl * 64 + lane) * G, lg);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = __builtin_amdgcn_exp2f(lg[g] - m[g]);
          p[g] = ok[bl] ? e : 0.f;
          l[g] += p[g];
        }
        // the weights w = p * s_v and their bf16 split: hi = w truncated to bf16, lo =
        // the rest rounded to bf16 (|w - hi - lo| <= 2^-16 |w|), two heads' lo at once;
        // rows 2 g, 2 g + 1 of a group are one word: hi (w's upper half), lo
#pragma unroll
        for (int grp = 0; grp < VSC; ++grp) {
          uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int g = 0; g < G; g += 2) {
            uint32_t wb[2] = {0u, 0u};
            float lo[2] = {0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              if (g + e < G) {
                const float w = p[g + e] * sv[grp];
                wb[e] = __builtin_bit_cast(uint32_t, w);
                lo[e] = w - __builtin_bit_cast(float, wb[e] & 0xFFFF0000u);
              }
            }
            const uint32_t lob =
                __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo[0], lo[1]}, bf16x2));
            d[g] = __builtin_amdgcn_perm(lob, wb[0], 0x05040302u);
            if (g + 1 < G) d[g + 1] = __builtin_amdgcn_perm(lob, wb[1], 0x07060302u);
          }
          *reinterpret_cast<u32x4*>(atc + (bl * NT + (grp >> 1)) * MV_TBL + ((grp & 1) ^ swk) * 16) =
              u32x4{d[0], d[1], d[2], d[3]};
        }
      }
      __syncthreads();
    };
    KBatch<UK, SP, false> KA, KB;
    if (total > 0) {
      k_scales(0, ksn);
      KA.load(kb, ksb, gw, W, 0, len, lane, kmax, pm);
    }
    // one chunk per iteration, two K batches of it (the second's scale word is that of
    // its block: the chunk's second block for Q8, the same block for K8V4)
    for (int k0 = 0; k0 < total; k0 += CHK) {
      const int ch = k0 / CHK;
      chunk_start(ch);
      KB.load(kb, ksb, gw, W, k0 + UK, len, lane, kmax, pm);
      kstep(KA, 0, ksn[0]);
      KA.load(kb, ksb, gw, W, k0 + 2 * UK, len, lane, kmax, pm);
      kstep(KB, UK, ksn[(8 * UK) / 64]);
      chunk_end(ch);
    }
    __syncthreads();   // the V wave's last chunk
#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = wave_sum_dpp(l[g]);
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        m_l[pr * G + g] = m[g];
        l_l[pr * G + g] = l[g];
      }
    }
  } else {
    // ================= V wave ===================================================
    const int qv = lane >> 4, iv = lane & 15;
    // the lane's LDS bases: the 8 bytes of a weight table its two transposing 16-bit
    // reads address (lane 4 e + c of the 16: rows 4 c .. 4 c + 3 of the e-th token of
    // tokens 8 g8 .. 8 g8 + 3, then of 8 g8 + 4 .. 8 g8 + 7, g8 = 4 hh + qv); the tile
    // bytes its transposing 8-bit reads start at (token group qv, dims 8 (iv % 2) ..)
    const int swv = qv & 1;
    const uint8_t* a_lane = at + qv * 256 + (iv >> 2) * 32 + (((iv & 3) >> 1) ^ swv) * 16 + (iv & 1) * 8;
    const int a_r0 = swv * 128, a_r1 = (swv ^ 1) * 128;
    const uint8_t* t_lane = tile + (8 * qv + (iv >> 1)) * MV_PITCH + 8 * (iv & 1);
    // D tile jd (dims 16 jd ..): lane (qv, iv) holds rows 4 qv .. 4 qv + 3 of dim
    // 16 jd + iv of its table, rows m = 8 (group % 2) + 2 head + part; heads ha, ha + 1
    const int ha = 2 * (qv & 1);
    f32x4 acc[8];
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) acc[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K8V4: 24 times the sum of each table row's weights (rows as in acc)
    f32x4 wsum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // a lane's 16 dims of one row of a step: Q8 the 16 codes, K8V4 8 bytes of nibbles
    using VW = std::conditional_t<K4, u32x2, u32x4>;
    auto vload = [&](VW (&vw)[MV_BLK], int blk) __attribute__((always_inline)) {
      int pv = 0;
      if constexpr (PG != 0) pv = pm.block(blk * MV_BLK);   // the block's 8 steps share it
#pragma unroll
      for (int u = 0; u < MV_BLK; ++u) {
        const char* base = vb;
        uint32_t row;
        if constexpr (PG != 0) {
          int pb, lim;
          pm.step(pv, blk * MV_BLK + u, gw, W, pb, lim);
          base += (size_t)pb * VROW;
          row = (uint32_t)min(r, lim);
        } else {
          row = (uint32_t)min(step_g<SP>(gw, min(blk * MV_BLK + u, kmax), W) * 8 + r, len - 1);
        }
        if constexpr (K4) vw[u] = ldkv64(base, row * VROW + c * 8);
        else vw[u] = ldkv(base, row * VROW + c * 16);
      }
    };
    auto vblock = [&](const VW (&vw)[MV_BLK], int blk) __attribute__((always_inline)) {
      const int ch = blk / NCB, bl = blk - ch * NCB;
      if (bl == 0) {
        if (ch > 0) __syncthreads();   // the K wave's chunk ch
        const float fa = fb[(ch & 1) * 4 + min(ha, G - 1)];
        const float fc = fb[(ch & 1) * 4 + min(ha + 1, G - 1)];
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) {
          acc[jd][0] *= fa;
          acc[jd][1] *= fa;
          acc[jd][2] *= fc;
          acc[jd][3] *= fc;
        }
        if constexpr (K4) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            wsum[t][0] *= fa;
            wsum[t][1] *= fa;
            wsum[t][2] *= fc;
            wsum[t][3] *= fc;
          }
        }
      }
      // the block's rows, token u * 8 + r, as signed codes in dim order
#pragma unroll
      for (int u = 0; u < MV_BLK; ++u) {
        u32x4 cw;
        if constexpr (K4) {
          uint32_t o[4];
          nibbles_to_biased(vw[u][0], o[0], o[1]);
          nibbles_to_biased(vw[u][1], o[2], o[3]);
          cw = u32x4{o[0], o[1], o[2], o[3]};
        } else {
          cw = vw[u];
        }
        *reinterpret_cast<u32x4*>(tile + (u * 8 + r) * MV_PITCH + c * 16) = cw;
      }
      wave_lds_fence();
      const uint8_t* atb = a_lane + ((ch & 1) * NCB + bl) * NT * MV_TBL;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // tokens 8 g8 .. 8 g8 + 7 of the block, g8 = 4 hh + qv
        bf16x8 aw[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          aw[t] = lds_tr16x2(atb + t * MV_TBL + hh * 1024 + a_r0, atb + t * MV_TBL + hh * 1024 + a_r1);
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) {
          // B: the codes of tokens 8 g8 + 0 .. 7, dim 16 jd + iv, as bf16 (exact; K8V4:
          // 16 + n)
          const i32x2 cb = lds_tr8(t_lane + hh * 32 * MV_PITCH + 16 * jd);
          acc[jd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              aw[K4 ? jd >> 2 : 0], K4 ? biased_bf16(cb) : codes_bf16(cb), acc[jd], 0, 0, 0);
        }
        if constexpr (K4) {
          // 24 per weight: B = 24.0 in every slot
          const bf16x8 b24 = __builtin_bit_cast(bf16x8, u32x4{0x41C041C0u, 0x41C041C0u,
                                                              0x41C041C0u, 0x41C041C0u});
#pragma unroll
          for (int t = 0; t < NT; ++t)
            wsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t], b24, wsum[t], 0, 0, 0);
        }
      }
      wave_lds_fence();
    };
    const int nblk = total / MV_BLK;
    VW VA[MV_BLK], VB[MV_BLK];
    if (nblk > 0) vload(VA, 0);
    __syncthreads();   // the K wave's first chunk
    for (int blk = 0; blk < nblk; blk += 2) {
      vload(VB, blk + 1);
      vblock(VA, blk);
      vload(VA, blk + 2);
      vblock(VB, blk + 1);
    }
    if (nblk > 0) __syncthreads();   // frees the K wave's last buffers
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      // the tile's dims belong to group jd / 4 (Q8) or jd / 2 (K8V4); its rows are
      // 0 .. 7 or 8 .. 15 of the table
      const int half = K4 ? (jd >> 1) & 1 : jd >> 2;
      f32x4 a = acc[jd];
      if constexpr (K4) a -= wsum[jd >> 2];   // w (24 + code) - 24 w
      if ((qv >> 1) == half) {
        if (ha < G) o_l[(pr * G + ha) * HD + jd * 16 + iv] = a[0] + a[1];
        if (ha + 1 < G) o_l[(pr * G + ha + 1) * HD + jd * 16 + iv] = a[2] + a[3];
      }
    }
  }
  // ---- combine the pair partials of the workgroup ----------------------------
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * HD; idx += DEC_THREADS) {
    const int g = idx / HD, d = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < PAIRS; ++w) M = fmaxf(M, m_l[w * G + g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < PAIRS; ++w) {
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

// A batch's sessions ranked longest first, so that the split workgroups of the long
// sessions, which hold the most steps each, are dispatched first and the short ones
// fill in behind them (the grid's last dimension is the rank).  One workgroup: a
// counting sort on ORD_BUCKETS length classes (len * (ORD_BUCKETS - 1) / max_len,
// a length outside 0 .. max_len in the last class); within a class the order is
// whatever the atomics give, which changes no output: a session's arithmetic
// depends on its own length only.  Writes the ranked session table, lengths and
// session index of each rank.
constexpr int ORD_THREADS = 1024;
constexpr int ORD_BUCKETS = ORD_THREADS;
__global__ __launch_bounds__(ORD_THREADS) void k_session_order(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int n_sess,
    int max_len, kv_session* __restrict__ stab, int32_t* __restrict__ slen,
    int32_t* __restrict__ sid) {
  __shared__ int cnt[2][ORD_BUCKETS];
  const int t = threadIdx.x;
  const long long span = max(max_len, 1);
  auto cls = [&](int len) {   // 0: longest
    const int k = len <= 0 || len > max_len ? 0 : (int)((long long)len * (ORD_BUCKETS - 1) / span);
    return ORD_BUCKETS - 1 - k;
  };
  cnt[0][t] = 0;
  __syncthreads();
  for (int b = t; b < n_sess; b += ORD_THREADS) atomicAdd(&cnt[0][cls(lens[b])], 1);
  __syncthreads();
  // inclusive scan of the class counts (Hillis-Steele over the two buffers)
  int src = 0;
  for (int d = 1; d < ORD_BUCKETS; d *= 2) {
    const int v = cnt[src][t] + (t >= d ? cnt[src][t - d] : 0);
    cnt[src ^ 1][t] = v;
    src ^= 1;
    __syncthreads();
  }
  // the first rank of class t
  const int first = t > 0 ? cnt[src][t - 1] : 0;
  __syncthreads();
  cnt[src][t] = first;
  __syncthreads();
  for (int b = t; b < n_sess; b += ORD_THREADS) {
    const int len = lens[b];
    const int r = atomicAdd(&cnt[src][cls(len)], 1);
    stab[r] = tab[b];
    slen[r] = len;
    sid[r] = b;
  }
}

// One workgroup of 256 threads per (session, query head).  Thread t holds dims
// 4 (t % 32) .. + 3 of the splits j = t / 32 + 8 k (k = 0 .. 7) of a chunk of 64
// splits; every wave also holds the chunk's 64 lse values, one per lane, and forms
// the chunk's max and weights itself.  The first chunk's partials and lse are loaded
// at entry, before the session entry and length arrive (the workspace holds S splits
// of every row, so the loads are in bounds whatever the session), so one call costs
// about one memory round trip.  Splits past the session's count (active_splits) are
// excluded by selects, never by multiplying stale values by a zero weight.  The 8 split
// groups are summed through LDS: out = sum_j 2^(lse_j - L) o_j, L = log2 sum_j 2^lse_j.
// Paged: the workgroups of a session's query heads each check a slice of its page
// table.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_SG = MERGE_THREADS / 32;   // split groups of a chunk
constexpr int MERGE_CHUNK = 64;                // splits per chunk (one per lane)
constexpr int MERGE_PER = MERGE_CHUNK / MERGE_SG;   // splits per thread and chunk
template <int FMT>
__global__ __launch_bounds__(MERGE_THREADS) void k_decode_merge(
    const kv_session* __restrict__ tab, const int32_t* __restrict__ lens, int max_len, int nqh,
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse, int S,
    float* __restrict__ out, int32_t* __restrict__ status, const int32_t* __restrict__ pages,
    int page_stride) {
  __shared__ float4 red[MERGE_SG][32];
  const int row = blockIdx.x;
  const int b = row / nqh, qh = row - b * nqh;
  const int t = threadIdx.x, lane = t & 63;
  const int dq = t & 31, sg = t >> 5;
  const float* lse = ws_lse + (long long)row * S;
  const float4* o = reinterpret_cast<const float4*>(ws_o + (long long)row * S * HD);
  float4 v[MERGE_PER];
  float f;
  auto load_chunk = [&](int j0) __attribute__((always_inline)) {
    const int last = min(S - 1, j0 + MERGE_CHUNK - 1);
#pragma unroll
    for (int k = 0; k < MERGE_PER; ++k)
      v[k] = o[(long long)min(j0 + sg + MERGE_SG * k, last) * (HD / 4) + dq];
    f = lse[min(j0 + lane, last)];
  };
  load_chunk(0);
  const kv_session ss = tab[b];
  const int len = lens[b];
  int bad = session_bad(ss, FMT);
  if (!bad && (len < 0 || len > ss.cap || len > max_len)) bad = KV_DEV_RANGE;
  float4* dst = reinterpret_cast<float4*>(out + (long long)row * HD);
  if (bad || len == 0) {   // workgroup-uniform
    if (t < 32) dst[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (bad && qh == 0 && t == 0) flag(status, bad);
    return;
  }
  if (pages != nullptr) {
    // this head's slice of the session's page table (the split kernels read a slot
    // outside the pool as slot 0)
    const int n_slots = ss.cap / KV_PAGE_ROWS;
    const int n_pages = (len + KV_PAGE_ROWS - 1) / KV_PAGE_ROWS;
    const int per = (n_pages + nqh - 1) / nqh;
    const int p1 = min(n_pages, (qh + 1) * per);
    bool bad_page = false;
    for (int pg = qh * per + t; pg < p1; pg += MERGE_THREADS) {
      const int sl = pages[(long long)b * page_stride + pg];
      bad_page |= sl < 0 || sl >= n_slots;
    }
    if (__builtin_amdgcn_ballot_w64(bad_page) != 0 && lane == 0) flag(status, KV_DEV_BAD_PAGE);
  }
  // the splits that worked on this session (the same count the split kernel used)
  const int Sb = active_splits<FMT>(len, S);
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < Sb; j0 += MERGE_CHUNK) {
    if (j0 > 0) load_chunk(j0);
    const int n = min(MERGE_CHUNK, Sb - j0);   // workgroup-uniform
    const float fl = lane < n ? f : -INFINITY;
    const float Mn = fmaxf(M, wave_max_dpp(fl));   // finite: the chunk holds split j0
    // the bare exp2: a split more than 126 below the max adds nothing
    const float w = lane < n ? __builtin_amdgcn_exp2f(f - Mn) : 0.f;
    const float alpha = __builtin_amdgcn_exp2f(M - Mn);   // 0 on the first chunk (M = -inf)
    L = fmaf(L, alpha, wave_sum_dpp(w));
    acc.x *= alpha;
    acc.y *= alpha;
    acc.z *= alpha;
    acc.w *= alpha;
#pragma unroll
    for (int k = 0; k < MERGE_PER; ++k) {
      const int js = sg + MERGE_SG * k;
      const float wk = __shfl(w, js, 64);
      if (js < n) {
        acc.x = fmaf(wk, v[k].x, acc.x);
        acc.y = fmaf(wk, v[k].y, acc.y);
        acc.z = fmaf(wk, v[k].z, acc.z);
        acc.w = fmaf(wk, v[k].w, acc.w);
      }
    }
    M = Mn;
  }
  red[sg][dq] = acc;
  __syncthreads();
  if constexpr (FMT == KV_FMT_K8V4) {
    // the merged row is in the rotated basis: V = H (code d) / 128, so out = H res / 128.
    // Lane t of wave 0 holds dims 2t, 2t + 1: stage 1 in the lane, stages 2 .. 64 pair
    // lanes 1 .. 32 apart (the lower lane keeps a + b, the upper a - b)
    if (t < 64) {
      const float* rf = reinterpret_cast<const float*>(red);
      float r0 = 0.f, r1 = 0.f;
#pragma unroll
      for (int g = 0; g < MERGE_SG; ++g) {
        r0 += rf[g * HD + 2 * t];
        r1 += rf[g * HD + 2 * t + 1];
      }
      r0 = r0 / L;
      r1 = r1 / L;
      float u0 = r0 + r1, u1 = r0 - r1;
#pragma unroll
      for (int mk = 1; mk < 64; mk *= 2) {
        const float p0 = __shfl_xor(u0, mk, 64), p1 = __shfl_xor(u1, mk, 64);
        u0 = (t & mk) ? p0 - u0 : u0 + p0;
        u1 = (t & mk) ? p1 - u1 : u1 + p1;
      }
      reinterpret_cast<float2*>(dst)[t] = make_float2(u0 * 0.0078125f, u1 * 0.0078125f);
    }
  } else {
    if (t < 32) {
      float4 r = red[0][t];
#pragma unroll
      for (int g = 1; g < MERGE_SG; ++g) {
        const float4 e = red[g][t];
        r.x += e.x;
        r.y += e.y;
        r.z += e.z;
        r.w += e.w;
      }
      dst[t] = make_float4(r.x / L, r.y / L, r.z / L, r.w / L);
    }
  }
}

// steps per load batch: int8 takes 4 (its loads are half the size), except with 8
// query heads, where the batch registers would not fit beside the partials
template <int FMT, int G>
constexpr int batch_rows() {
  return FMT != KV_FMT_F16 ? (G >= 8 ? 2 : KVQ8_DEC_U_Q8) : KVQ8_DEC_U_F16;
}

// the int8-K formats take the pair kernels
template <int FMT>
constexpr bool use_pair() { return FMT != KV_FMT_F16; }
// the int8-K formats with 1, 2 or 4 query heads per kv head: V products on the matrix cores
template <int FMT, int G>
constexpr bool use_mv() { return FMT != KV_FMT_F16 && G <= 4; }


// Split workgroups of one kernel instance that fit on the current device at once
// (CUs x resident workgroups per CU), cached per device; 0 when unknown.
template <int FMT, int G>
int resident_splits() {
  static std::atomic<int> cache[KVQ8_MAX_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= KVQ8_MAX_DEVICES) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  hipError_t e;
  if constexpr (use_mv<FMT, G>())
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_pair_mv<FMT, G, 0, MV_SP>,
                                                     DEC_THREADS, mv_lds_bytes<FMT, G>());
  else if constexpr (use_pair<FMT>())
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, k_decode_pair<FMT, G, batch_rows<FMT, G>(), 0>, DEC_THREADS, pair_lds_bytes<G>());
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, k_decode_split<FMT, G, batch_rows<FMT, G>(), 0>, DEC_THREADS, split_lds_bytes<G>());
  if (e != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  v = per_cu * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

int resident(int fmt, int G) {
#define KVQ8_RES(F, GG) \
  if (fmt == F && G == GG) return resident_splits<F, GG>();
  KVQ8_RES(KV_FMT_K8V4, 1)
  KVQ8_RES(KV_FMT_K8V4, 2)
  KVQ8_RES(KV_FMT_K8V4, 4)
  KVQ8_RES(KV_FMT_K8V4, 8)
  KVQ8_RES(KV_FMT_Q8, 1)
  KVQ8_RES(KV_FMT_Q8, 2)
  KVQ8_RES(KV_FMT_Q8, 4)
  KVQ8_RES(KV_FMT_Q8, 8)
  KVQ8_RES(KV_FMT_F16, 1)
  KVQ8_RES(KV_FMT_F16, 2)
  KVQ8_RES(KV_FMT_F16, 4)
  KVQ8_RES(KV_FMT_F16, 8)
#undef KVQ8_RES
  return 0;
}

template <int FMT, int G, bool PG>
hipError_t launch_split(const kv_session* tab, const int32_t* lens, const int32_t* sid,
                        int n_sess, int max_len, int kvh, const float* q, float sm_scale,
                        float* ws_o, float* ws_lse, const DecodePlan& plan, const int32_t* pages,
                        int page_stride, hipStream_t st) {
  constexpr int U = batch_rows<FMT, G>();
  static_assert(U == 1 || U == 2 || U == 4 || U == 8, "U must divide the group budgets / 2");
  dim3 grid(plan.S, kvh, n_sess), block(DEC_THREADS);
  if constexpr (use_mv<FMT, G>()) {
    // the page map's registers as for k_decode_pair below
    const long long J = ((long long)max_len + 7) / 8;
    const long long per_pair = (J + (long long)PAIRS * plan.S - 1) / ((long long)PAIRS * plan.S);
    const bool one = n_sess == 1;
#define KVQ8_MV_LAUNCH(P, SPV)                                                                 \
  hipLaunchKernelGGL((k_decode_pair_mv<FMT, G, P, SPV>), grid, block, (mv_lds_bytes<FMT, G>()), st, tab, lens, \
                     max_len, kvh, q, sm_scale * LOG2E, ws_o, ws_lse, plan.S, pages, page_stride, sid)
    if constexpr (!PG) {
      if (one) KVQ8_MV_LAUNCH(0, MV_SP);
      else KVQ8_MV_LAUNCH(0, 1);
    } else if (per_pair <= 128) {
      if (one) KVQ8_MV_LAUNCH(2, MV_SP);
      else KVQ8_MV_LAUNCH(2, 1);
    } else {
      if (one) KVQ8_MV_LAUNCH(4, MV_SP);
      else KVQ8_MV_LAUNCH(4, 1);
    }
#undef KVQ8_MV_LAUNCH
  } else if constexpr (use_pair<FMT>()) {
    if constexpr (!PG) {
      hipLaunchKernelGGL((k_decode_pair<FMT, G, U, 0>), grid, block, pair_lds_bytes<G>(), st, tab,
                         lens, max_len, kvh, q, sm_scale * LOG2E, ws_o, ws_lse, plan.S, pages,
                         page_stride, sid);
    } else {
      // the page map in 2 registers when no pair has more than 128 steps, else in 4
      // with V batches of at most 2 steps, so the V wave stays within its registers.
      // A session of J_b steps runs on Sb = active_splits splits: Sb = S gives a pair
      // at most ceil(J / (PAIRS S)) steps (J: the steps of max_len); a smaller Sb is
      // at least Jf / (PAIRS MIN_STEPS), Jf >= J_b lead16 / 16, so a pair has at most
      // 16 MIN_STEPS / lead16 steps.
      static_assert(KVQ8_DEC_MIN_STEPS * 16 <= 128 * lead16<FMT>(),
                    "a session short for the grid fits the 2-register page map");
      const long long J = ((long long)max_len + 7) / 8;
      const long long per_pair = (J + (long long)PAIRS * plan.S - 1) / ((long long)PAIRS * plan.S);
      constexpr int U4 = U > 2 ? 2 : U;
      if (per_pair <= 128)
        hipLaunchKernelGGL((k_decode_pair<FMT, G, U, 2>), grid, block, pair_lds_bytes<G>(), st,
                           tab, lens, max_len, kvh, q, sm_scale * LOG2E, ws_o, ws_lse, plan.S,
                           pages, page_stride, sid);
      else
        hipLaunchKernelGGL((k_decode_pair<FMT, G, U4, 4>), grid, block, pair_lds_bytes<G>(), st,
                           tab, lens, max_len, kvh, q, sm_scale * LOG2E, ws_o, ws_lse, plan.S,
                           pages, page_stride, sid);
    }
  } else {
    hipLaunchKernelGGL((k_decode_split<FMT, G, U, PG ? 4 : 0>), grid, block, split_lds_bytes<G>(),
                       st, tab, lens, max_len, kvh, q, sm_scale * LOG2E, ws_o, ws_lse, plan.S,
                       pages, page_stride, sid);
  }
  return hipGetLastError();
}

template <int FMT, int G>
hipError_t launch_g(const kv_session* tab, const int32_t* lens, int n_sess, int max_len, int kvh,
                    const float* q, float sm_scale, float* out, float* ws_o, float* ws_lse,
                    void* ws_ord, const DecodePlan& plan, int32_t* status, const int32_t* pages,
                    int page_stride, hipStream_t st) {
  // a batch runs its sessions longest first: the split kernels read the ranked copy
  const kv_session* stab = tab;
  const int32_t* slen = lens;
  const int32_t* sid = nullptr;
  if (plan.ws_ord_bytes != 0) {
    kv_session* rt = static_cast<kv_session*>(ws_ord);
    int32_t* rl = reinterpret_cast<int32_t*>(rt + n_sess);
    int32_t* ri = rl + n_sess;
    hipLaunchKernelGGL(k_session_order, dim3(1), dim3(ORD_THREADS), 0, st, tab, lens, n_sess,
                       max_len, rt, rl, ri);
    stab = rt;
    slen = rl;
    sid = ri;
  }
  hipError_t e = pages != nullptr
                     ? launch_split<FMT, G, true>(stab, slen, sid, n_sess, max_len, kvh, q, sm_scale,
                                                  ws_o, ws_lse, plan, pages, page_stride, st)
                     : launch_split<FMT, G, false>(stab, slen, sid, n_sess, max_len, kvh, q,
                                                   sm_scale, ws_o, ws_lse, plan, nullptr, 0, st);
  if (e != hipSuccess) return e;
  const int n_rows = n_sess * kvh * G;
  hipLaunchKernelGGL((k_decode_merge<FMT>), dim3(n_rows), dim3(MERGE_THREADS), 0, st, tab, lens,
                     max_len, kvh * G, ws_o, ws_lse, plan.S, out, status, pages, page_stride);
  return hipGetLastError();
}

}  // namespace

DecodePlan decode_plan(int fmt, int kvh, int nqh, int n_sess, int max_len) {
  // Splits per (session, kv head): enough that no wave has more steps than its
  // group's logits budget (CH0 or CH1), then
  // raised so that the grid is a whole number of rounds of resident workgroups (a
  // last, partly filled round would leave CUs idle), but not past one split per 4
  // steps (so every workgroup has work).
  const long long J = ((long long)max_len + 7) / 8;
  const bool q8 = fmt != KV_FMT_F16;   // the int8 K formats share the q8 plan
  const long long Jf = q8 ? lead_steps<KV_FMT_Q8>((int)J) : lead_steps<KV_FMT_F16>((int)J);
  const long long J1 = J - Jf;
  const int G = nqh / kvh;
  long long CH0 = 0, CH1 = 0;
#define KVQ8_CHB(GG)                                                          \
  if (G == GG) {                                                              \
    CH0 = q8 ? ch0<KV_FMT_Q8, GG>() : ch0<KV_FMT_F16, GG>();                  \
    CH1 = q8 ? ch1<KV_FMT_Q8, GG>() : ch1<KV_FMT_F16, GG>();                  \
  }
  KVQ8_CHB(1) KVQ8_CHB(2) KVQ8_CHB(4) KVQ8_CHB(8)
#undef KVQ8_CHB
  if (CH0 <= 0) CH0 = 1;  // unsupported G: rejected before any launch
  const long long P = (long long)kvh * n_sess;
  long long S0, Smax;
  if (q8) {
    // pairs take any number of steps (in chunks): aim at most PAIR_TARGET_STEPS per
    // pair, and at least PAIR_MIN_STEPS
    S0 = std::max(1LL, (J + PAIRS * PAIR_TARGET_STEPS - 1) / (PAIRS * PAIR_TARGET_STEPS));
    Smax = std::max(S0, J / (PAIRS * PAIR_MIN_STEPS));
  } else {
    // every wave within its group's LDS budget of logits (CH0 or CH1 steps)
    S0 = std::max(1LL, (Jf + GRP_WAVES * CH0 - 1) / (GRP_WAVES * CH0));
    if (CH1 > 0) S0 = std::max(S0, (J1 + GRP_WAVES * CH1 - 1) / (GRP_WAVES * CH1));
    Smax = std::max(S0, (Jf + GRP_WAVES - 1) / GRP_WAVES);
  }
  long long S = S0;
  const long long C = resident(fmt, nqh / kvh);
  if (C > 0) {
    const long long rounds = (P * S0 + C - 1) / C;
    S = std::max(S0, (rounds * C + P - 1) / P);
  }
  S = std::min(S, Smax);
  DecodePlan p;
  p.S = (int)S;
  const size_t rows = (size_t)n_sess * nqh * p.S;
  p.ws_o_bytes = (rows * HD * sizeof(float) + 255) & ~(size_t)255;
  p.ws_lse_bytes = (rows * sizeof(float) + 255) & ~(size_t)255;
  p.ws_ord_bytes = n_sess > 1
                       ? ((size_t)n_sess * (sizeof(kv_session) + 2 * sizeof(int32_t)) + 255) & ~(size_t)255
                       : 0;
  return p;
}

// The fixed scratch of kv_decode_attn_static: room for the split partials of one
// call (KV_DECODE_STATIC_WS_BYTES).  Each device holds its own copy at its own
// address; host code reaches it only through the address hipGetSymbolAddress gives,
// fetched once per device with that device current.
static __device__ __align__(256) unsigned char scratch[KV_DECODE_STATIC_WS_BYTES];

void* static_workspace() {
  static std::atomic<void*> addr[KVQ8_MAX_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= KVQ8_MAX_DEVICES) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  addr[dev].store(q, std::memory_order_release);   // the same value from any racing thread
  return q;
}

hipError_t launch_decode(int fmt, int kvh, int nqh, const kv_session* d_tab,
                         const int32_t* d_len, int n_sess, int max_len, const float* d_q,
                         float sm_scale, float* d_out, void* d_ws, const DecodePlan& plan,
                         int32_t* d_status, hipStream_t st, const int32_t* d_pages,
                         int page_stride) {
  float* ws_o = static_cast<float*>(d_ws);
  float* ws_lse = reinterpret_cast<float*>(static_cast<char*>(d_ws) + plan.ws_o_bytes);
  void* ws_ord = static_cast<char*>(d_ws) + plan.ws_o_bytes + plan.ws_lse_bytes;
  const int G = nqh / kvh;
#define KVQ8_DEC(F, GG)                                                                          \
  if (fmt == F && G == GG)                                                                       \
    return launch_g<F, GG>(d_tab, d_len, n_sess, max_len, kvh, d_q, sm_scale, d_out, ws_o, ws_lse, \
                           ws_ord, plan, d_status, d_pages, page_stride, st);
  KVQ8_DEC(KV_FMT_K8V4, 1)
  KVQ8_DEC(KV_FMT_K8V4, 2)
  KVQ8_DEC(KV_FMT_K8V4, 4)
  KVQ8_DEC(KV_FMT_K8V4, 8)
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
