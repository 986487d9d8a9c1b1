// Internal declarations shared by the HIP translation units of libkvq8.
// gfx950 (CDNA4) only: wave64, DPP cross-lane operations, MFMA for the prompt chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq8.h"

namespace kvq8 {

constexpr int HD = 128;        // head_dim supported by the kernels
constexpr int NGRP = HD / KV_GROUP;  // fp16 scales per head row (2)
constexpr int NQ4 = HD / KV_Q4_BLOCK;  // fp16 scales per K8V4 V row (4)
// most cells per session: a head's rows (<= 256 B each) stay within 32-bit offsets
constexpr int KV_MAX_CAP = 1 << 24;
// Most kv heads of a shape (grids put 2 x n_kv_heads on their y extent).
constexpr int KV_MAX_KV_HEADS = 1024;
// Most sessions one decode call takes (the grid's z extent).
constexpr int KV_DEC_MAX_SESS = 65535;

// ---------------------------------------------------------------------------
// Cross-lane operations (DPP, within a 16-lane row; no LDS traffic)
// ---------------------------------------------------------------------------
// DPP control words
constexpr int DPP_QUAD_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;      // lane i <-> 15-i within 16 lanes
constexpr int DPP_ROW_ROR8 = 0x128;       // rotate a 16-lane row by 8

// every control used here reads a lane inside the same 16-lane row, so no source is
// out of range; bound_ctrl lets the compiler fold the move into the consuming add
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
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
// Global-memory access through address space 1.  Pointers read from session
// tables are generic to the compiler; casting them lets it emit global_load /
// global_store (counted by vmcnt only) instead of flat accesses.
// ---------------------------------------------------------------------------
#define KVQ8_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ldg128(const void* p) {
  return *(const KVQ8_GLOBAL u32x4*)(p);
}
// streaming (non-temporal) 128-bit load: data read once, not kept in the caches
__device__ __forceinline__ u32x4 ldg128_nt(const void* p) {
  return __builtin_nontemporal_load((const KVQ8_GLOBAL u32x4*)(p));
}
__device__ __forceinline__ uint16_t ldg16(const void* p) {
  return *(const KVQ8_GLOBAL uint16_t*)(p);
}
__device__ __forceinline__ void stg128(void* p, u32x4 v) {
  *(KVQ8_GLOBAL u32x4*)(p) = v;
}
__device__ __forceinline__ void stg64(void* p, u32x2 v) {
  *(KVQ8_GLOBAL u32x2*)(p) = v;
}
__device__ __forceinline__ void stg32(void* p, uint32_t v) {
  *(KVQ8_GLOBAL uint32_t*)(p) = v;
}
__device__ __forceinline__ void stg16(void* p, uint16_t v) {
  *(KVQ8_GLOBAL uint16_t*)(p) = v;
}

// Reinterpret a 32-bit word as fp32.  Takes the word by value: applying
// __builtin_bit_cast directly to an ext_vector element (v[i]) reads element 0
// with this compiler, so vector elements must pass through a scalar first.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

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
  if (fmt != KV_FMT_F16) {
    if (s.k_scale == nullptr || s.v_scale == nullptr || (sc & 15)) return KV_DEV_BAD_SESSION;
  } else if (sc != 0) {
    return KV_DEV_BAD_SESSION;
  }
  if (s.cap <= 0 || (s.cap & 63) || s.cap > KV_MAX_CAP) return KV_DEV_BAD_SESSION;
  return 0;
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status != nullptr && bits) atomicOr(status, bits);
}

// ---------------------------------------------------------------------------
// Launchers (validated arguments only; return hipError_t of the launch)
// ---------------------------------------------------------------------------
// d_pages: NULL for contiguous sessions, else the page tables of paged ones
hipError_t launch_append(int fmt, int kvh, const kv_session* d_tab, const int32_t* d_len,
                         int n_sess, int n_tok, const float* d_k, const float* d_v,
                         int32_t* d_status, hipStream_t st, const int32_t* d_pages = nullptr,
                         int page_stride = 0);

// host-side checks shared by the entry points (KV_OK or a negative KV_ERR_*)
int check_shape(const kv_shape* s);
int check_session(const kv_shape* s, const kv_session* e);

// rows of one session into another (kv_copy_rows, with the copy kind given: the
// window also moves pages from pinned host memory)
int copy_rows(const kv_shape* h_shape, const kv_session* h_src, int src_row0,
              const kv_session* h_dst, int dst_row0, int n_rows, void* stream,
              hipMemcpyKind kind);

struct DecodePlan {
  int S;      // splits (workgroups) per (session, kv head): grid x
  size_t ws_o_bytes, ws_lse_bytes;
  // a batch's sessions ranked longest first (0 for one session): the session table,
  // lengths and session indices in that order
  size_t ws_ord_bytes;
  size_t total() const { return ws_o_bytes + ws_lse_bytes + ws_ord_bytes; }
};
// depends on the arguments and on how many split workgroups the current device
// holds at once (queried once per device)
DecodePlan decode_plan(int fmt, int kvh, int nqh, int n_sess, int max_len);
hipError_t launch_decode(int fmt, int kvh, int nqh, const kv_session* d_tab,
                         const int32_t* d_len, int n_sess, int max_len, const float* d_q,
                         float sm_scale, float* d_out, void* d_ws, const DecodePlan& plan,
                         int32_t* d_status, hipStream_t st, const int32_t* d_pages = nullptr,
                         int page_stride = 0);

// kv_decode_attn_static's scratch on the current device (KV_DECODE_STATIC_WS_BYTES
// bytes; its address fetched once per device), or NULL if it cannot be had
void* static_workspace();

hipError_t launch_compact(int fmt, int kvh, const kv_session& sess, int P, uint16_t* d_k16,
                          uint16_t* d_v16, hipStream_t st);

hipError_t launch_prefill(int kvh, int nqh, const uint16_t* k16, const uint16_t* v16,
                          long row_stride, int pos0, int n_tok, const float* d_q,
                          float sm_scale, float* d_out, hipStream_t st);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace kvq8
