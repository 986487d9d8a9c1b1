// The C ABI of libkvq8: argument validation (before any HIP call) and launches.
// Declarations and their contracts are in include/kvq8.h.
#include <cmath>
#include <cstring>

#include "kvq8_internal.h"

using namespace kvq8;

namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
}  // namespace

int kvq8::check_shape(const kv_shape* s) {
  if (s == nullptr) return KV_ERR_ARG;
  if (s->fmt != KV_FMT_F16 && s->fmt != KV_FMT_Q8 && s->fmt != KV_FMT_K8V4) return KV_ERR_FMT;
  if (s->n_kv_heads < 1 || s->n_kv_heads > KV_MAX_KV_HEADS || s->n_q_heads < 1 ||
      s->n_q_heads % s->n_kv_heads != 0)
    return KV_ERR_ARG;
  if (s->head_dim != HD) return KV_ERR_UNSUPPORTED;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KV_ERR_UNSUPPORTED;
  return KV_OK;
}

// host copy of one session entry (prefill / compaction take one on the host)
int kvq8::check_session(const kv_shape* s, const kv_session* e) {
  if (e == nullptr || e->k == nullptr || e->v == nullptr) return KV_ERR_ARG;
  if (s->fmt != KV_FMT_F16) {
    if (e->k_scale == nullptr || e->v_scale == nullptr) return KV_ERR_FMT;
  } else if (e->k_scale != nullptr || e->v_scale != nullptr) {
    return KV_ERR_FMT;
  }
  if (!aligned16(e->k) || !aligned16(e->v) || !aligned16(e->k_scale) || !aligned16(e->v_scale))
    return KV_ERR_ALIGN;
  if (e->cap <= 0 || (e->cap & 63)) return KV_ERR_ALIGN;
  if (e->cap > KV_MAX_CAP) return KV_ERR_RANGE;
  return KV_OK;
}

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? KV_OK : KV_ERR_HIP; }

// The arrays of a session in packed order (K values, K scales, V values, V scales)
// and the bytes of one head row of each (0: the format has no such array).
void row_arrays(int fmt, const kv_session& e, char* ptr[4], size_t rb[4]) {
  ptr[0] = static_cast<char*>(e.k);
  ptr[1] = reinterpret_cast<char*>(e.k_scale);
  ptr[2] = static_cast<char*>(e.v);
  ptr[3] = reinterpret_cast<char*>(e.v_scale);
  const bool f16 = fmt == KV_FMT_F16, k8v4 = fmt == KV_FMT_K8V4;
  rb[0] = f16 ? HD * 2 : HD;
  rb[1] = f16 ? 0 : NGRP * 2;
  rb[2] = f16 ? HD * 2 : k8v4 ? HD / 2 : HD;
  rb[3] = f16 ? 0 : (k8v4 ? NQ4 : NGRP) * 2;
}

// rows [row0, row0 + n) inside the session's capacity
bool rows_fit(const kv_session& e, int row0, int n) {
  return row0 >= 0 && n >= 0 && (long long)row0 + n <= e.cap;
}

// packed block order: K values, K scales, V values, V scales
constexpr int kRowOrder[4] = {0, 1, 2, 3};
// saved image order: the body (K values, V values), then the scales body
constexpr int kImageOrder[4] = {0, 2, 1, 3};

// gather (to_packed) or scatter between rows of a session and a packed block whose
// arrays follow `order`
int move_packed(const kv_shape* h_shape, const kv_session* h_sess, int row0, int n_rows,
                char* packed, bool to_packed, void* stream, const int* order = kRowOrder) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  rc = check_session(h_shape, h_sess);
  if (rc) return rc;
  if (packed == nullptr || n_rows < 0) return KV_ERR_ARG;
  if (!rows_fit(*h_sess, row0, n_rows)) return KV_ERR_RANGE;
  if (n_rows == 0) return KV_OK;
  char* ptr[4];
  size_t rb[4];
  row_arrays(h_shape->fmt, *h_sess, ptr, rb);
  const size_t kvh = (size_t)h_shape->n_kv_heads, cap = (size_t)h_sess->cap;
  hipStream_t st = static_cast<hipStream_t>(stream);
  size_t off = 0;
  for (int i = 0; i < 4; ++i) {
    const int a = order[i];
    if (rb[a] == 0) continue;
    const size_t w = (size_t)n_rows * rb[a];   // one head's rows, packed
    char* rows = ptr[a] + (size_t)row0 * rb[a];
    const hipError_t e =
        to_packed ? hipMemcpy2DAsync(packed + off, w, rows, cap * rb[a], w, kvh, hipMemcpyDefault, st)
                  : hipMemcpy2DAsync(rows, cap * rb[a], packed + off, w, w, kvh, hipMemcpyDefault, st);
    if (e != hipSuccess) return KV_ERR_HIP;
    off += w * kvh;
  }
  return KV_OK;
}

// Saved session image: a 128-byte little-endian header (magic "KVQ8", u32 version,
// fmt, kv heads, head_dim, tokens, u64 body bytes, u64 scales bytes, zeros), the
// token ids as int32, the body, the scales body.
constexpr size_t kImageHeader = 128;
constexpr uint32_t kImageV2 = 2, kImageV3 = 3;

void put_le(unsigned char* p, uint64_t v, int bytes) {
  for (int i = 0; i < bytes; ++i) p[i] = (unsigned char)(v >> (8 * i));
}
uint64_t get_le(const unsigned char* p, int bytes) {
  uint64_t v = 0;
  for (int i = 0; i < bytes; ++i) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

// body and scales-body bytes of n rows of a valid shape
void image_regions(const kv_shape* s, int n, size_t* body, size_t* scales) {
  kv_session none{};
  char* ptr[4];
  size_t rb[4];
  row_arrays(s->fmt, none, ptr, rb);
  const size_t rows = (size_t)s->n_kv_heads * (size_t)n;
  *body = rows * (rb[0] + rb[2]);
  *scales = rows * (rb[1] + rb[3]);
}

// Parse and check a header against the shape and the image size; the token count,
// or a negative KV_ERR_*.
int image_header(const kv_shape* s, const unsigned char* img, size_t image_bytes) {
  if (image_bytes < kImageHeader || img[0] != 'K' || img[1] != 'V' || img[2] != 'Q' ||
      img[3] != '8')
    return KV_ERR_IMAGE;
  const uint64_t version = get_le(img + 4, 4), fmt = get_le(img + 8, 4),
                 kvh = get_le(img + 12, 4), hd = get_le(img + 16, 4), n = get_le(img + 20, 4),
                 body = get_le(img + 24, 8), scales = get_le(img + 32, 8);
  if (fmt != (uint64_t)s->fmt || kvh != (uint64_t)s->n_kv_heads || hd != (uint64_t)s->head_dim)
    return KV_ERR_IMAGE;
  // version 2 carries no scales: loadable for FP16 only
  if (version != kImageV3 && !(version == kImageV2 && s->fmt == KV_FMT_F16)) return KV_ERR_IMAGE;
  if (n > (uint64_t)KV_MAX_CAP) return KV_ERR_IMAGE;
  size_t want_body, want_scales;
  image_regions(s, (int)n, &want_body, &want_scales);
  if (body != want_body || scales != want_scales) return KV_ERR_IMAGE;
  if (image_bytes < kImageHeader + 4 * n + want_body + want_scales) return KV_ERR_IMAGE;
  return (int)n;
}

}  // namespace

extern "C" {

size_t kv_cache_bytes(int fmt, int n_kv_heads, int cap, int head_dim, int part) {
  if ((fmt != KV_FMT_F16 && fmt != KV_FMT_Q8 && fmt != KV_FMT_K8V4) || n_kv_heads < 0 ||
      cap < 0 || head_dim <= 0 || head_dim % KV_GROUP != 0 || part < 0 || part > 3)
    return 0;
  const size_t n = (size_t)n_kv_heads * (size_t)cap * (size_t)head_dim;
  if (fmt == KV_FMT_K8V4 && part >= 2) return part == 2 ? n / 2 : 2 * (n / KV_Q4_BLOCK);
  if ((part & 1) == 0) return fmt == KV_FMT_F16 ? 2 * n : n;
  return fmt == KV_FMT_F16 ? 0 : 2 * (n / KV_GROUP);
}

int kv_append(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_len, int n_sess,
              int n_tok, const float* d_k_new, const float* d_v_new, int32_t* d_status,
              void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if (d_tab == nullptr || d_len == nullptr || d_k_new == nullptr || d_v_new == nullptr)
    return KV_ERR_ARG;
  if (n_sess < 1 || n_sess > 65535 || n_tok < 0) return KV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_tab) & 7) || !aligned4(d_len) || !aligned16(d_k_new) ||
      !aligned16(d_v_new) || !aligned4(d_status))
    return KV_ERR_ALIGN;
  if (n_tok == 0) return KV_OK;
  return hip_status(launch_append(h_shape->fmt, h_shape->n_kv_heads, d_tab, d_len, n_sess, n_tok,
                                  d_k_new, d_v_new, d_status, static_cast<hipStream_t>(stream)));
}

int kv_append_paged(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_pages,
                    int page_stride, const int32_t* d_len, int n_sess, int n_tok,
                    const float* d_k_new, const float* d_v_new, int32_t* d_status, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if (d_tab == nullptr || d_pages == nullptr || d_len == nullptr || d_k_new == nullptr ||
      d_v_new == nullptr)
    return KV_ERR_ARG;
  if (n_sess < 1 || n_sess > 65535 || n_tok < 0 || page_stride < 1 ||
      page_stride > KV_MAX_CAP / KV_PAGE_ROWS)
    return KV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_tab) & 7) || !aligned4(d_pages) || !aligned4(d_len) ||
      !aligned16(d_k_new) || !aligned16(d_v_new) || !aligned4(d_status))
    return KV_ERR_ALIGN;
  if (n_tok == 0) return KV_OK;
  return hip_status(launch_append(h_shape->fmt, h_shape->n_kv_heads, d_tab, d_len, n_sess, n_tok,
                                  d_k_new, d_v_new, d_status, static_cast<hipStream_t>(stream),
                                  d_pages, page_stride));
}

size_t kv_decode_workspace_bytes(const kv_shape* h_shape, int n_sess, int max_len) {
  if (check_shape(h_shape) || n_sess < 1 || n_sess > KV_DEC_MAX_SESS || max_len < 0) return 0;
  const DecodePlan p =
      decode_plan(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, n_sess, max_len);
  return p.total();
}

int kv_decode_attn(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_len,
                   int n_sess, int max_len, const float* d_q, float sm_scale, float* d_out,
                   void* d_ws, size_t ws_bytes, int32_t* d_status, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if (d_tab == nullptr || d_len == nullptr || d_q == nullptr || d_out == nullptr) return KV_ERR_ARG;
  if (n_sess < 1 || n_sess > KV_DEC_MAX_SESS || max_len < 0 || !std::isfinite(sm_scale))
    return KV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_tab) & 7) || !aligned4(d_len) || !aligned16(d_q) ||
      !aligned16(d_out) || !aligned16(d_ws) || !aligned4(d_status))
    return KV_ERR_ALIGN;
  if (d_ws == nullptr) return KV_ERR_WORKSPACE;
  const DecodePlan p =
      decode_plan(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, n_sess, max_len);
  if (ws_bytes < p.total()) return KV_ERR_WORKSPACE;
  return hip_status(launch_decode(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, d_tab,
                                  d_len, n_sess, max_len, d_q, sm_scale, d_out, d_ws, p, d_status,
                                  static_cast<hipStream_t>(stream)));
}

int kv_decode_attn_static(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_len,
                          int n_sess, int max_len, const float* d_q, float sm_scale, float* d_out,
                          int32_t* d_status, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if (d_tab == nullptr || d_len == nullptr || d_q == nullptr || d_out == nullptr) return KV_ERR_ARG;
  if (n_sess < 1 || n_sess > KV_DEC_MAX_SESS || max_len < 0 || !std::isfinite(sm_scale))
    return KV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_tab) & 7) || !aligned4(d_len) || !aligned16(d_q) ||
      !aligned16(d_out) || !aligned4(d_status))
    return KV_ERR_ALIGN;
  const DecodePlan p =
      decode_plan(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, n_sess, max_len);
  if (p.total() > (size_t)KV_DECODE_STATIC_WS_BYTES) return KV_ERR_WORKSPACE;
  void* ws = static_workspace();
  if (ws == nullptr) return KV_ERR_HIP;
  return hip_status(launch_decode(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, d_tab,
                                  d_len, n_sess, max_len, d_q, sm_scale, d_out, ws, p, d_status,
                                  static_cast<hipStream_t>(stream)));
}

int kv_decode_attn_paged(const kv_shape* h_shape, const kv_session* d_tab,
                         const int32_t* d_pages, int page_stride, const int32_t* d_len, int n_sess,
                         int max_len, const float* d_q, float sm_scale, float* d_out, void* d_ws,
                         size_t ws_bytes, int32_t* d_status, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if (d_tab == nullptr || d_pages == nullptr || d_len == nullptr || d_q == nullptr ||
      d_out == nullptr)
    return KV_ERR_ARG;
  if (n_sess < 1 || n_sess > KV_DEC_MAX_SESS || max_len < 0 || !std::isfinite(sm_scale))
    return KV_ERR_ARG;
  // every page of a session of up to max_len cells has a table entry
  if (page_stride < 1 || (long long)page_stride * KV_PAGE_ROWS < (long long)max_len)
    return KV_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_tab) & 7) || !aligned4(d_pages) || !aligned4(d_len) ||
      !aligned16(d_q) || !aligned16(d_out) || !aligned16(d_ws) || !aligned4(d_status))
    return KV_ERR_ALIGN;
  if (d_ws == nullptr) return KV_ERR_WORKSPACE;
  const DecodePlan p =
      decode_plan(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, n_sess, max_len);
  if (ws_bytes < p.total()) return KV_ERR_WORKSPACE;
  return hip_status(launch_decode(h_shape->fmt, h_shape->n_kv_heads, h_shape->n_q_heads, d_tab,
                                  d_len, n_sess, max_len, d_q, sm_scale, d_out, d_ws, p, d_status,
                                  static_cast<hipStream_t>(stream), d_pages, page_stride));
}

int kv_compact_f16(const kv_shape* h_shape, const kv_session* h_sess, int P, uint16_t* d_k16,
                   uint16_t* d_v16, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  rc = check_session(h_shape, h_sess);
  if (rc) return rc;
  if (d_k16 == nullptr || d_v16 == nullptr || P < 1) return KV_ERR_ARG;
  if (!aligned16(d_k16) || !aligned16(d_v16)) return KV_ERR_ALIGN;
  if (P > h_sess->cap) return KV_ERR_RANGE;
  return hip_status(launch_compact(h_shape->fmt, h_shape->n_kv_heads, *h_sess, P, d_k16, d_v16,
                                   static_cast<hipStream_t>(stream)));
}

size_t kv_prefill_workspace_bytes(const kv_shape* h_shape, int P) {
  if (check_shape(h_shape) || P < 0) return 0;
  if (h_shape->fmt == KV_FMT_F16) return 0;
  const size_t half = ((size_t)h_shape->n_kv_heads * (size_t)P * HD * 2 + 255) & ~(size_t)255;
  return 2 * half;
}

int kv_prefill_attn(const kv_shape* h_shape, const kv_session* h_sess, int pos0, int n_tok,
                    const float* d_q, float sm_scale, float* d_out, void* d_ws, size_t ws_bytes,
                    void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  rc = check_session(h_shape, h_sess);
  if (rc) return rc;
  if (d_q == nullptr || d_out == nullptr || pos0 < 0 || n_tok < 0 || !std::isfinite(sm_scale) ||
      !(sm_scale > 0.0f))
    return KV_ERR_ARG;
  if (!aligned16(d_q) || !aligned16(d_out) || !aligned16(d_ws)) return KV_ERR_ALIGN;
  if ((long long)pos0 + n_tok > h_sess->cap) return KV_ERR_RANGE;
  if (n_tok == 0) return KV_OK;
  const int P = pos0 + n_tok;
  const size_t need = kv_prefill_workspace_bytes(h_shape, P);
  if (need > 0 && (d_ws == nullptr || ws_bytes < need)) return KV_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int kvh = h_shape->n_kv_heads;
  const uint16_t *k16, *v16;
  long row_stride;  // rows between kv heads
  if (h_shape->fmt != KV_FMT_F16) {
    uint16_t* wk = static_cast<uint16_t*>(d_ws);
    uint16_t* wv = reinterpret_cast<uint16_t*>(static_cast<char*>(d_ws) + need / 2);
    rc = hip_status(launch_compact(h_shape->fmt, kvh, *h_sess, P, wk, wv, st));
    if (rc) return rc;
    k16 = wk;
    v16 = wv;
    row_stride = P;
  } else {
    // an FP16 cache is already the fp16 [kvh][cap][HD] layout: read it in place
    k16 = static_cast<const uint16_t*>(h_sess->k);
    v16 = static_cast<const uint16_t*>(h_sess->v);
    row_stride = h_sess->cap;
  }
  return hip_status(launch_prefill(kvh, h_shape->n_q_heads, k16, v16, row_stride, pos0, n_tok, d_q,
                                   sm_scale, d_out, st));
}

int kv_probe_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream) {
  if (d_src == nullptr || d_sink == nullptr || (bytes & 15)) return KV_ERR_ARG;
  if (!aligned16(d_src) || !aligned4(d_sink)) return KV_ERR_ALIGN;
  if (bytes == 0) return KV_OK;
  return hip_status(launch_stream_read(d_src, bytes, d_sink, static_cast<hipStream_t>(stream)));
}

size_t kv_rows_bytes(const kv_shape* h_shape, int n_rows) {
  if (check_shape(h_shape) || n_rows < 0) return 0;
  kv_session none{};
  char* ptr[4];
  size_t rb[4];
  row_arrays(h_shape->fmt, none, ptr, rb);
  return (size_t)h_shape->n_kv_heads * (size_t)n_rows * (rb[0] + rb[1] + rb[2] + rb[3]);
}

int kv_copy_rows(const kv_shape* h_shape, const kv_session* h_src, int src_row0,
                 const kv_session* h_dst, int dst_row0, int n_rows, void* stream) {
  return kvq8::copy_rows(h_shape, h_src, src_row0, h_dst, dst_row0, n_rows, stream,
                         hipMemcpyDeviceToDevice);
}

}  // extern "C"

// rows of one session into another, every array of the format; kind says where the
// two live (device to device, or between pinned host memory and the device)
int kvq8::copy_rows(const kv_shape* h_shape, const kv_session* h_src, int src_row0,
                    const kv_session* h_dst, int dst_row0, int n_rows, void* stream,
                    hipMemcpyKind kind) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if ((rc = check_session(h_shape, h_src)) || (rc = check_session(h_shape, h_dst))) return rc;
  if (n_rows < 0) return KV_ERR_ARG;
  if (!rows_fit(*h_src, src_row0, n_rows) || !rows_fit(*h_dst, dst_row0, n_rows))
    return KV_ERR_RANGE;
  if (n_rows == 0) return KV_OK;
  char *ps[4], *pd[4];
  size_t rb[4];
  row_arrays(h_shape->fmt, *h_src, ps, rb);
  row_arrays(h_shape->fmt, *h_dst, pd, rb);
  const size_t kvh = (size_t)h_shape->n_kv_heads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int a = 0; a < 4; ++a) {
    if (rb[a] == 0) continue;
    const hipError_t e = hipMemcpy2DAsync(
        pd[a] + (size_t)dst_row0 * rb[a], (size_t)h_dst->cap * rb[a],
        ps[a] + (size_t)src_row0 * rb[a], (size_t)h_src->cap * rb[a], (size_t)n_rows * rb[a],
        kvh, kind, st);
    if (e != hipSuccess) return KV_ERR_HIP;
  }
  return KV_OK;
}

extern "C" {

int kv_gather_rows(const kv_shape* h_shape, const kv_session* h_sess, int row0, int n_rows,
                   void* d_or_h_dst, void* stream) {
  return move_packed(h_shape, h_sess, row0, n_rows, static_cast<char*>(d_or_h_dst), true, stream);
}

int kv_scatter_rows(const kv_shape* h_shape, const kv_session* h_sess, int row0, int n_rows,
                    const void* d_or_h_src, void* stream) {
  return move_packed(h_shape, h_sess, row0, n_rows,
                     const_cast<char*>(static_cast<const char*>(d_or_h_src)), false, stream);
}

size_t kv_image_bytes(const kv_shape* h_shape, int n_tokens) {
  if (check_shape(h_shape) || n_tokens < 0 || n_tokens > KV_MAX_CAP) return 0;
  size_t body, scales;
  image_regions(h_shape, n_tokens, &body, &scales);
  return kImageHeader + 4 * (size_t)n_tokens + body + scales;
}

int kv_image_save(const kv_shape* h_shape, const kv_session* h_sess, int n_tokens,
                  const int32_t* h_tokens, void* h_image, size_t image_bytes, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if ((rc = check_session(h_shape, h_sess))) return rc;
  if (h_image == nullptr || n_tokens < 0 || (n_tokens > 0 && h_tokens == nullptr))
    return KV_ERR_ARG;
  if (!rows_fit(*h_sess, 0, n_tokens)) return KV_ERR_RANGE;
  if (image_bytes < kv_image_bytes(h_shape, n_tokens)) return KV_ERR_ARG;
  size_t body, scales;
  image_regions(h_shape, n_tokens, &body, &scales);
  unsigned char* img = static_cast<unsigned char*>(h_image);
  memset(img, 0, kImageHeader);
  memcpy(img, "KVQ8", 4);
  put_le(img + 4, h_shape->fmt == KV_FMT_F16 ? kImageV2 : kImageV3, 4);
  put_le(img + 8, (uint32_t)h_shape->fmt, 4);
  put_le(img + 12, (uint32_t)h_shape->n_kv_heads, 4);
  put_le(img + 16, (uint32_t)h_shape->head_dim, 4);
  put_le(img + 20, (uint32_t)n_tokens, 4);
  put_le(img + 24, body, 8);
  put_le(img + 32, scales, 8);
  for (int t = 0; t < n_tokens; ++t) put_le(img + kImageHeader + 4 * (size_t)t, (uint32_t)h_tokens[t], 4);
  return move_packed(h_shape, h_sess, 0, n_tokens,
                     reinterpret_cast<char*>(img + kImageHeader + 4 * (size_t)n_tokens), true,
                     stream, kImageOrder);
}

int kv_image_tokens(const kv_shape* h_shape, const void* h_image, size_t image_bytes) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if (h_image == nullptr) return KV_ERR_ARG;
  return image_header(h_shape, static_cast<const unsigned char*>(h_image), image_bytes);
}

int kv_image_load(const kv_shape* h_shape, const kv_session* h_sess, const void* h_image,
                  size_t image_bytes, int32_t* h_tokens, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if ((rc = check_session(h_shape, h_sess))) return rc;
  if (h_image == nullptr) return KV_ERR_ARG;
  const unsigned char* img = static_cast<const unsigned char*>(h_image);
  const int n = image_header(h_shape, img, image_bytes);
  if (n < 0) return n;
  if (!rows_fit(*h_sess, 0, n)) return KV_ERR_RANGE;
  if (h_tokens != nullptr)
    for (int t = 0; t < n; ++t)
      h_tokens[t] = (int32_t)(uint32_t)get_le(img + kImageHeader + 4 * (size_t)t, 4);
  rc = move_packed(h_shape, h_sess, 0, n,
                   const_cast<char*>(reinterpret_cast<const char*>(img + kImageHeader + 4 * (size_t)n)),
                   false, stream, kImageOrder);
  return rc ? rc : n;
}

const char* kv_status_str(int status) {
  switch (status) {
    case KV_OK: return "ok";
    case KV_ERR_ARG: return "invalid argument (null pointer, size or head counts)";
    case KV_ERR_FMT: return "unknown cache format, or scale pointers inconsistent with it";
    case KV_ERR_ALIGN: return "pointer not 16-byte aligned, or cap not a multiple of 64";
    case KV_ERR_UNSUPPORTED: return "unsupported head_dim or query/kv head ratio";
    case KV_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ERR_RANGE: return "rows outside the session's capacity";
    case KV_ERR_HIP: return "HIP kernel launch or copy failed";
    case KV_ERR_IMAGE: return "saved image refused (magic, version, format, shape or size)";
    case KV_ERR_WINDOW: return "window state missing, too small or not initialised";
    default: return "unknown status";
  }
}

}  // extern "C"
