// Internal declarations shared by the HIP translation units of libkvq8.
// gfx950 (CDNA4) only: wave64, DPP cross-lane operations, MFMA for the prompt chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq8.h"

namespace kvq8 {

constexpr int HD = 128;        // head_dim supported by the kernels
constexpr int NGRP = HD / KV_GROUP;  // fp16 scales per head row (2)

// ---------------------------------------------------------------------------
// Cross-lane operations (DPP, within a 16-lane row; no LDS traffic)
// ---------------------------------------------------------------------------
// DPP control words
constexpr int DPP_QUAD_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;      // lane i <-> 15-i within 16 lanes
constexpr int DPP_ROW_ROR8 = 0x128;       // rotate a 16-lane row by 8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// sum over the 8 lanes {8k .. 8k+7}; every lane of the 8 gets the total
__device__ __forceinline__ float sum8(float v) {
  v += dpp<DPP_QUAD_XOR1>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_ROW_HALF_MIRROR>(v);
  return v;
}

// max over the 16 lanes {16k .. 16k+15}; every lane of the 16 gets it
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int m) {
  return __shfl_xor(v, m, 64);
}

// sum over lanes with equal (lane & 7): the 8 lanes {c, c+8, ..., c+56}
__device__ __forceinline__ float sum_rows8(float v) {
  v += dpp<DPP_ROW_ROR8>(v);  // lane i + lane (i+8) mod 16 within the row
  v += shfl_xor(v, 16);
  v += shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor(v, m);
  return v;
}

// ---------------------------------------------------------------------------
// fp16 bit helpers (IEEE binary16; conversions round to nearest even)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---------------------------------------------------------------------------
// Device-side check of a session table entry (host cannot see device tables)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int session_bad(const kv_session& s, int fmt) {
  const uintptr_t kv = reinterpret_cast<uintptr_t>(s.k) | reinterpret_cast<uintptr_t>(s.v);
  const uintptr_t sc =
      reinterpret_cast<uintptr_t>(s.k_scale) | reinterpret_cast<uintptr_t>(s.v_scale);
  if (s.k == nullptr || s.v == nullptr || (kv & 15)) return KV_DEV_BAD_SESSION;
  if (fmt == KV_FMT_Q8) {
    if (s.k_scale == nullptr || s.v_scale == nullptr || (sc & 15)) return KV_DEV_BAD_SESSION;
  } else if (sc != 0) {
    return KV_DEV_BAD_SESSION;
  }
  if (s.cap <= 0 || (s.cap & 63)) return KV_DEV_BAD_SESSION;
  return 0;
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status != nullptr && bits) atomicOr(status, bits);
}

// ---------------------------------------------------------------------------
// Launchers (validated arguments only; return hipError_t of the launch)
// ---------------------------------------------------------------------------
hipError_t launch_append(int fmt, int kvh, const kv_session* d_tab, const int32_t* d_len,
                         int n_sess, int n_tok, const float* d_k, const float* d_v,
                         int32_t* d_status, hipStream_t st);

struct DecodePlan {
  int T;      // tokens per split (per workgroup)
  int S;      // splits per session (grid x)
  size_t ws_o_bytes, ws_lse_bytes;
};
DecodePlan decode_plan(int kvh, int nqh, int n_sess, int max_len);
hipError_t launch_decode(int fmt, int kvh, int nqh, const kv_session* d_tab,
                         const int32_t* d_len, int n_sess, int max_len, const float* d_q,
                         float sm_scale, float* d_out, void* d_ws, const DecodePlan& plan,
                         int32_t* d_status, hipStream_t st);

hipError_t launch_compact(int fmt, int kvh, const kv_session& sess, int P, uint16_t* d_k16,
                          uint16_t* d_v16, hipStream_t st);

hipError_t launch_prefill(int kvh, int nqh, const uint16_t* k16, const uint16_t* v16,
                          long row_stride, int pos0, int n_tok, const float* d_q,
                          float sm_scale, float* d_out, hipStream_t st);

}  // namespace kvq8
