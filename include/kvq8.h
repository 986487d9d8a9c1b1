/*
 * kvq8.h -- attention over a reduced-precision K/V cache on MI355X (gfx950).
 *
 * C ABI.  Every pointer named d_* is a DEVICE pointer, every h_* a HOST pointer.
 * Every call that takes a `stream` (a hipStream_t passed as void*, NULL for the
 * null stream) only enqueues work on it and returns; nothing allocates, frees or
 * synchronises.  The caller owns every buffer: caches, session tables, lengths,
 * workspaces.  Calls are reentrant and thread-safe.  What the library keeps between
 * calls: per device, the number of decode workgroups that device holds at once
 * (queried on the first decode planning with that device current, then read only),
 * which sets the split count and so the workspace size; and, per device, the fixed
 * scratch array of kv_decode_attn_static.
 *
 * Error behaviour: every argument a host can check is checked before anything is
 * enqueued; on error the call returns a negative KV_ERR_* code and enqueues
 * nothing.  What only the device can see (a session table entry, a length) is
 * checked by the kernels: the offending session is skipped (no byte of its cache
 * is written; its decode output is written as zeros) and a KV_DEV_* bit is OR-ed
 * into *d_status when d_status is not NULL (the caller zeroes it).
 *
 * Sources (web pages, cited by title and section):
 *   [P1] PR #3084 "FP16 K/V cache by default, int8 with --kv-q8 (262144 fits a
 *        16 GiB card)" -- sections Summary, What changed, Extra Notes.
 *   [P2] Issue #67 "Path F format v3: persist per-head INT8 KV scales".
 *   [P3] PR #711 "kv: --kv k8v4 streams with --kv-resident" -- sections What, How.
 */
#ifndef KVQ8_H
#define KVQ8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache formats [P1, Summary]: FP16 values, or int8 codes with one FP16 scale per
 * 64 dims; and [P3, What]'s K8V4: the int8 K with a rotated 4-bit V.  An explicit
 * enum, checked against which scale pointers are present, rather than inferring the
 * format from pointer presence (the silent-skip trap described in [P3, How]). */
typedef enum { KV_FMT_F16 = 0, KV_FMT_Q8 = 1, KV_FMT_K8V4 = 2 } kv_fmt;

#define KV_GROUP 64    /* dims per FP16 scale of the int8 codes [P1, Summary] */
#define KV_PAGE_ROWS 64 /* cells per page of a paged session (kv_decode_attn_paged) */
#define KV_Q4_BLOCK 32 /* values per FP16 scale of the K8V4 V codes [P3, What] */

typedef struct {
  int32_t fmt;        /* kv_fmt */
  int32_t n_kv_heads; /* 1 .. 1024 */
  int32_t n_q_heads;  /* n_kv_heads * G, G in {1, 2, 4, 8}; query head q reads kv head q / G */
  int32_t head_dim;   /* 128 */
} kv_shape;

/* One session's cache for one layer.  Layout [P1, Extra Notes: [kvh][ctx][HD]]:
 *   F16: k, v  = fp16 bits, [n_kv_heads][cap][head_dim]; k_scale = v_scale = NULL.
 *   Q8 : k, v  = int8 codes, [n_kv_heads][cap][head_dim];
 *        k_scale, v_scale = fp16 bits, [n_kv_heads][cap][head_dim / 64]; scale g of
 *        a row covers dims [64g, 64g + 64).  Codes and scales are separate arrays
 *        ([P1, What changed]; separate byte runs in [P3, How]).
 *   K8V4: k, k_scale as Q8.  v = uint8 [n_kv_heads][cap][head_dim / 2]: the V row
 *        rotated, w = H x (H the 128 x 128 Sylvester Hadamard matrix, applied as fp32
 *        butterflies, stages 1, 2, 4, ..., 64), quantised per 32 values as
 *        d = fp16(max|w| / 7), code = clamp(rint(w / d), -7, 7), stored as code + 8,
 *        byte j holding value 2j in its low nibble and 2j + 1 in its high nibble;
 *        v_scale = fp16 bits [n_kv_heads][cap][head_dim / 32].  A read sees
 *        V = H (code * d) / 128: the orthonormal rotation H / sqrt(128), undone.
 * All four pointers 16-byte aligned; cap a multiple of 64 and at most 2^24 (a head's
 * rows are addressed with 32-bit byte offsets).  An array of these
 * lives in device memory for the batched calls. */
typedef struct {
  void* k;
  void* v;
  uint16_t* k_scale;
  uint16_t* v_scale;
  int32_t cap;
  int32_t reserved; /* 0 */
} kv_session;

enum {
  KV_OK = 0,
  KV_ERR_ARG = -1,         /* null pointer, size out of range, n_q_heads % n_kv_heads != 0 */
  KV_ERR_FMT = -2,         /* unknown format, or scale pointers inconsistent with it */
  KV_ERR_ALIGN = -3,       /* pointer not 16-byte aligned, or cap % 64 != 0 */
  KV_ERR_UNSUPPORTED = -4, /* head_dim != 128, or G not in {1, 2, 4, 8} */
  KV_ERR_WORKSPACE = -5,   /* workspace null or smaller than the *_workspace_bytes value */
  KV_ERR_RANGE = -6,       /* rows outside [0, cap), or cap above 2^24 (host-checkable cases) */
  KV_ERR_HIP = -7,         /* a kernel launch or copy failed */
  KV_ERR_IMAGE = -8,       /* a saved image refused: magic, version, format, shape or size */
  KV_ERR_WINDOW = -9       /* window state missing, too small or not initialised */
};

/* bits OR-ed into *d_status by kernels */
enum {
  KV_DEV_RANGE = 1,       /* len < 0, len + n_tok > cap (append), len > max_len or cap (decode) */
  KV_DEV_BAD_SESSION = 2, /* table entry with null/unaligned pointers, scales inconsistent with
                             the format, or cap not a positive multiple of 64 or above 2^24 */
  KV_DEV_BAD_PAGE = 4     /* a page table entry outside the pool (kv_decode_attn_paged) */
};

/* Bytes of one array of one layer: part 0 the K values/codes, part 1 the K scales
 * (0 for F16), parts 2 and 3 the same for V.  Per value: 2 B (F16), or 1 B + 2 B
 * per 64 (Q8, and the K8V4 K), which reproduces the 6.0 / 3.1 GiB at 262144 cells of
 * [P1, Summary]; the K8V4 V: 1/2 B + 2 B per 32, so a K8V4 cell of 512 values per
 * array takes the 816 B of [P3, What].  Returns 0 for invalid arguments. */
size_t kv_cache_bytes(int fmt, int n_kv_heads, int cap, int head_dim, int part);

/* Write n_tok new cells per session: quantise-on-write (Q8) or FP16 store (F16).
 * [P1, What changed]: scale = fp16(max|x| / 127) per 64-dim group of a head row,
 * with IEEE fp32 division and round-to-nearest-even; code = clamp(rint(x / s),
 * -127, 127) dividing (IEEE fp32) by the stored fp16 scale; a zero scale stores
 * code 0.  F16 stores fp16_rne(x).
 *   d_tab   : kv_session [n_sess] (device), 1 <= n_sess <= 65535
 *   d_len   : int32 [n_sess] (device): session b's cells go to rows
 *             [d_len[b], d_len[b] + n_tok).  NOT modified (the caller advances it).
 *   d_k_new, d_v_new : fp32 [n_sess][n_tok][n_kv_heads][head_dim] (device)
 *   d_status: int32 (device) or NULL; KV_DEV_* bits.  A session whose rows do not
 *             fit is skipped whole. */
int kv_append(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_len,
              int n_sess, int n_tok, const float* d_k_new, const float* d_v_new,
              int32_t* d_status, void* stream);

/* kv_append into paged sessions ([P3, How]: the decode and prompt appends write the
 * streamed state's pool): cell c of session b (c in [d_len[b], d_len[b] + n_tok)) goes
 * to row c % 64 of the pool slot d_pages[b * page_stride + c / 64] of d_tab[b] (usually
 * one pool for every session), with the same arithmetic as kv_append.  A session then
 * holds up to 64 page_stride cells: d_len[b] + n_tok above that flags KV_DEV_RANGE and
 * skips the session; a table entry outside [0, cap / 64) flags KV_DEV_BAD_PAGE and
 * skips that row.  d_pages: int32, device, 4-byte aligned; page_stride 1 .. 2^18.
 * Mapping the pages first (kv_window_map) and copying the new rows back to the host
 * store (kv_window_writeback) are the caller's. */
int kv_append_paged(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_pages,
                    int page_stride, const int32_t* d_len, int n_sess, int n_tok,
                    const float* d_k_new, const float* d_v_new, int32_t* d_status, void* stream);

/* Workspace for kv_decode_attn: split-K partials and, for more than one session, the
 * session table, lengths and indices ranked longest first (a batch's long sessions
 * are started first; the outputs do not depend on the order).  Depends on its arguments and on
 * the current HIP device (the split count follows that device's occupancy); query
 * it with the device current that kv_decode_attn will run on.  0 on invalid
 * arguments (n_sess outside 1 .. 65535). */
size_t kv_decode_workspace_bytes(const kv_shape* h_shape, int n_sess, int max_len);

/* Split-K decode attention of one new token per session over the cache, reading
 * the cache format directly ([P1, What changed / Extra Notes]).  For query head q
 * of session b, kv head h = q / G:
 *   out[b][q] = sum_t softmax_t(sm_scale * q . K[h][t]) V[h][t],  t < d_len[b],
 * with K, V the dequantised cache values (code * scale, exact in fp32, or the
 * fp16 values).  Partials of each split of the context are merged by log-sum-exp.
 * Softmax weights come from the hardware fp32 exp2 of the logit (in base 2) minus a
 * running maximum; a weight below 2^-126 of that maximum counts as 0.
 * d_len[b] == 0 gives a zero row.  Arithmetic:
 *   F16: fp16 values widened to fp32; dot products, softmax and sums in fp32.
 *   int8 K (Q8, K8V4): the scaled query is split per 64-dim group into three int8
 *     levels, q = s (a + b/254 + c/254^2) with s = max|q| / 127 over the group
 *     (residual at most s / (2 * 254^2)); each level's dot product with the codes
 *     is an exact integer (matrix cores), combined with the K scales in fp32.
 *   V with G <= 4 (Q8 and K8V4): each softmax weight times its V scale (per 64
 *     dims for Q8, per 32 for K8V4) is carried as two bf16 values, hi + lo, with
 *     |w - hi - lo| <= 2^-16 |w|; codes times hi and lo are summed in fp32 on the
 *     matrix cores.  A Q8 output element then lies within 2^-16 A of the exact
 *     weighted sum, A = sum_t w_t |V_td| / sum_t w_t, plus fp32 rounding.  K8V4 sums
 *     the rotated values u = code * d and applies H / 128 in fp32 after the merge,
 *     so its bound is 2^-16 times the mean over dims of A taken over |u|.
 *   V with G = 8: fp32 vector sums.
 *   d_q   : fp32 [n_sess][n_q_heads][head_dim];  d_out : fp32 [n_sess][n_q_heads][head_dim]
 *   n_sess : 1 .. 65535.
 *   max_len : host upper bound of every d_len[b] (sizes the grid); a session over it
 *             is flagged KV_DEV_RANGE and gets a zero row.
 *   d_ws, ws_bytes : at least kv_decode_workspace_bytes(h_shape, n_sess, max_len).
 * Deterministic: the same inputs on the same device give bitwise the same output. */
int kv_decode_attn(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_len,
                   int n_sess, int max_len, const float* d_q, float sm_scale, float* d_out,
                   void* d_ws, size_t ws_bytes, int32_t* d_status, void* stream);

/* kv_decode_attn without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the split partials go to a fixed scratch array of
 * KV_DECODE_STATIC_WS_BYTES that the library holds on each device it runs on, from
 * its first use until the process ends.  No call allocates or frees anything.
 * Same arguments, plan, kernels and results (bitwise) as kv_decode_attn, without
 * d_ws / ws_bytes; KV_ERR_WORKSPACE when the call's partials
 * (kv_decode_workspace_bytes) exceed the scratch, KV_ERR_HIP if its address cannot
 * be had.  Every call on one device shares that device's scratch: calls that may
 * overlap on a device (on different streams, or from several threads without
 * ordering) race and must not be made; calls in order on one stream are safe. */
#define KV_DECODE_STATIC_WS_BYTES (16u << 20)
int kv_decode_attn_static(const kv_shape* h_shape, const kv_session* d_tab, const int32_t* d_len,
                          int n_sess, int max_len, const float* d_q, float sm_scale, float* d_out,
                          int32_t* d_status, void* stream);

/* Compaction [P1, What changed; Extra Notes]: cache rows [0, P) rewritten as the FP16
 * [kvh][P][HD] array on which prompt-chunk attention runs both of its matrix
 * products.  F16: a copy (stride cap -> P).
 * Q8: fp16_rne(float(code) * float(scale)) -- one rounding of an exact product.
 *   h_sess : one session (host struct holding device pointers), P <= h_sess->cap
 *   d_k16, d_v16 : fp16 bits [n_kv_heads][P][head_dim] (device), 16-byte aligned. */
int kv_compact_f16(const kv_shape* h_shape, const kv_session* h_sess, int P,
                   uint16_t* d_k16, uint16_t* d_v16, void* stream);

/* Workspace for kv_prefill_attn: the compacted copy (Q8), 0 bytes for F16. */
size_t kv_prefill_workspace_bytes(const kv_shape* h_shape, int P);

/* Causal attention of a prompt chunk over the cache, computed on an FP16 copy with
 * fp16 Q and fp32 accumulation on the matrix cores ([P1, Extra Notes]).  The chunk
 * must already be appended at rows [pos0, pos0 + n_tok).  Row i (position pos0 + i)
 * of query head q attends keys [0, pos0 + i] of kv head q / G:
 *   out[i][q] = sum_t softmax_t(sm_scale * fp16(q_i) . K16[t]) V16[t]
 * with each softmax weight carried into the P V product as the sum of two fp16
 * values (about 22 significant bits).
 *   sm_scale : finite and > 0, else KV_ERR_ARG
 *   d_q  : fp32 [n_tok][n_q_heads][head_dim];  d_out : fp32 [n_tok][n_q_heads][head_dim]
 *   d_ws : at least kv_prefill_workspace_bytes(h_shape, pos0 + n_tok) (may be NULL if 0). */
int kv_prefill_attn(const kv_shape* h_shape, const kv_session* h_sess, int pos0, int n_tok,
                    const float* d_q, float sm_scale, float* d_out, void* d_ws, size_t ws_bytes,
                    void* stream);

/* Moving a session's rows, sized by the format ([P1, What changed]: copying a session
 * into a slot counts the format's own element size, and int8 adds a copy of the scale
 * arrays; [P2, Phased plan]: gather to the host and scatter back, the scales beside
 * the KV body).  A packed block of n_rows rows holds, for each array of the
 * format in the order K values, K scales, V values, V scales (absent arrays take no
 * bytes), [n_kv_heads][n_rows][row bytes of that array]: F16 256 / - / 256 / -,
 * Q8 128 / 4 / 128 / 4, K8V4 128 / 4 / 64 / 8 bytes per row of one head.
 * kv_rows_bytes: the size of such a block; 0 on invalid arguments. */
size_t kv_rows_bytes(const kv_shape* h_shape, int n_rows);

/* Device copy of rows [src_row0, src_row0 + n_rows) of every kv head of h_src into rows
 * [dst_row0, dst_row0 + n_rows) of h_dst (host structs holding device pointers), every
 * array of the format.  The two row ranges must not overlap when h_src and h_dst share
 * arrays.  KV_ERR_RANGE if a range leaves its session's capacity; n_rows == 0 is a no-op. */
int kv_copy_rows(const kv_shape* h_shape, const kv_session* h_src, int src_row0,
                 const kv_session* h_dst, int dst_row0, int n_rows, void* stream);

/* Gather rows [row0, row0 + n_rows) of a session into the packed block at d_or_h_dst
 * (device memory, or host memory allocated pinned, kv_rows_bytes(h_shape, n_rows)
 * bytes), and scatter such a block back into rows [row0, row0 + n_rows).  Asynchronous
 * on the stream; a host buffer must stay valid until the stream reaches the call. */
int kv_gather_rows(const kv_shape* h_shape, const kv_session* h_sess, int row0, int n_rows,
                   void* d_or_h_dst, void* stream);
int kv_scatter_rows(const kv_shape* h_shape, const kv_session* h_sess, int row0, int n_rows,
                    const void* d_or_h_src, void* stream);

/* Paged sessions and a streamed window ([P3, What / How]: the K/V of a session live in
 * host memory and move to a device-resident window block by block, each block a list of
 * byte runs, codes and scales alike; attention over the window equals attention over a
 * resident cache bit for bit).  A page holds KV_PAGE_ROWS cells.  A pool is a kv_session
 * whose cap is KV_PAGE_ROWS x slots; slot s holds rows [64 s, 64 s + 64) of each array.
 *
 * kv_decode_attn_paged: kv_decode_attn over sessions whose page p (cells [64 p, 64 p +
 * 64)) lies in slot d_pages[b * page_stride + p] of d_tab[b] (usually one pool for every
 * session).  The same plan, arithmetic and order as kv_decode_attn, so a paged session
 * gives bitwise the output of the resident one.  page_stride >= ceil(max_len / 64), else
 * KV_ERR_ARG; d_pages: int32, device, 4-byte aligned.  A table entry outside [0, cap/64)
 * is read as slot 0 and flags KV_DEV_BAD_PAGE in *d_status.  Workspace as for
 * kv_decode_attn (kv_decode_workspace_bytes). */
int kv_decode_attn_paged(const kv_shape* h_shape, const kv_session* d_tab,
                         const int32_t* d_pages, int page_stride, const int32_t* d_len, int n_sess,
                         int max_len, const float* d_q, float sm_scale, float* d_out, void* d_ws,
                         size_t ws_bytes, int32_t* d_status, void* stream);

/* The window's bookkeeping, in caller-owned host memory of kv_window_bytes(n_slots) bytes
 * (0 for n_slots outside 1 .. 2^18): which (session, page) each pool slot holds, and CLOCK
 * replacement.  kv_window_init marks every slot free (KV_ERR_WINDOW if bytes is short).
 * Calls on one state must not overlap. */
size_t kv_window_bytes(int n_slots);
int kv_window_init(void* h_state, size_t bytes, int n_slots);

/* Make pages [0, n_pages) of session sess_id (a caller-chosen id >= 0) resident, host only:
 * h_pages (host int32 [n_pages], the session's page table from its last call, or -1s) is
 * updated in place; the pages that must be copied are listed in h_missed (host int32
 * [n_pages]), *h_misses of them.  Pages already resident are kept; others take slots by
 * CLOCK, never a slot this call keeps.  KV_ERR_RANGE if n_pages exceeds the slots. */
int kv_window_plan(void* h_state, int sess_id, int n_pages, int32_t* h_pages, int32_t* h_missed,
                   int* h_misses);

/* kv_window_plan, then the copies: each missed page's rows from h_store (a session whose
 * arrays are pinned host memory, cap >= 64 n_pages) into its pool slot of h_pool (device,
 * cap >= 64 x slots), consecutive pages in consecutive slots as one copy per array, and
 * h_pages (pinned) to d_pages (device int32 [n_pages]).  Asynchronous on the stream:
 * h_store must stay valid, and h_pages must be neither freed nor passed to another call
 * (the next kv_window_map of the session rewrites it), until the stream reaches this
 * call -- e.g. record an event after it and wait on that event before the session's next
 * map.  A decode of the session enqueued after it on the stream reads the pages.
 * Every argument (shape, both sessions' format, alignment and capacity, the window
 * state) is checked before the window's state changes.  If a copy cannot be enqueued
 * the call returns KV_ERR_HIP, the pages not yet copied are unmapped (their slots
 * free, their h_pages entries -1, so the next plan lists them as missed); copies of
 * earlier runs of this call may already be enqueued. */
int kv_window_map(const kv_shape* h_shape, void* h_state, const kv_session* h_store, int sess_id,
                  int n_pages, const kv_session* h_pool, int32_t* h_pages, int32_t* h_missed,
                  int32_t* d_pages, int* h_misses, void* stream);

/* Copy rows [row0, row0 + n_rows) of session sess_id from their pool slots back to its
 * host store ([P3, How]: appends write the host copy as well as the pool), one copy per
 * array for each run of consecutive pages in consecutive slots.  h_pages: the session's
 * page table from its last kv_window_map; every page the rows touch must be resident for
 * the session in the slot the table names, else KV_ERR_WINDOW (nothing enqueued).
 * h_store: pinned host arrays, cap >= row0 + n_rows (else KV_ERR_RANGE).  Asynchronous on
 * the stream: the rows reach the store once the stream passes the call; a later map on
 * the same stream that copies them back to the pool reads the new values. */
int kv_window_writeback(const kv_shape* h_shape, void* h_state, const kv_session* h_store,
                        int sess_id, int row0, int n_rows, const kv_session* h_pool,
                        const int32_t* h_pages, void* stream);

/* Saved session image ([P2, Scope]: a header, the token ids, the KV body, then the
 * scales body; [P2, Phased plan]: version 3 carries the scales, and a version-2 image
 * is refused for an int8 cache).  The calls build and read an image in caller-owned
 * host memory; writing it to a file, or reading it back, is the caller's.  Layout:
 *   bytes [0, 128)  header, little-endian: "KVQ8", u32 version (3 when the format has
 *                   scales, else 2), u32 fmt, u32 n_kv_heads, u32 head_dim,
 *                   u32 n_tokens, u64 body bytes, u64 scales bytes, zeros;
 *   then            n_tokens int32 token ids;
 *   then the body   K values, then V values, of rows [0, n_tokens);
 *   then the scales K scales, then V scales (absent for F16);
 * each array's rows as [n_kv_heads][n_tokens][row bytes] (row bytes as for
 * kv_rows_bytes).  The scale arrays are the format's fp16 ones, in place of one
 * fp32 per token, head and K/V.
 * kv_image_bytes: the image size for n_tokens rows; 0 on invalid arguments. */
size_t kv_image_bytes(const kv_shape* h_shape, int n_tokens);

/* Build the image of rows [0, n_tokens) of a session in h_image (host memory
 * allocated pinned, at least kv_image_bytes bytes).  The header and the token ids
 * (h_tokens: host int32 [n_tokens], may be NULL when n_tokens == 0) are written
 * before the call returns; the body and scales are copied asynchronously on the
 * stream, so the image is complete once the stream reaches the call.
 * KV_ERR_RANGE if n_tokens exceeds the capacity, KV_ERR_ARG for a short image. */
int kv_image_save(const kv_shape* h_shape, const kv_session* h_sess, int n_tokens,
                  const int32_t* h_tokens, void* h_image, size_t image_bytes, void* stream);

/* Check an image's header against h_shape and image_bytes; the number of tokens it
 * holds, or KV_ERR_IMAGE (bad magic, version 2 with a format that has scales, an
 * unknown version, another format, n_kv_heads or head_dim, region sizes that do not
 * match them, or an image shorter than its regions).  Host only. */
int kv_image_tokens(const kv_shape* h_shape, const void* h_image, size_t image_bytes);

/* Load an image into rows [0, n) of a session: checks as kv_image_tokens, then
 * KV_ERR_RANGE if n exceeds the capacity; copies the token ids to h_tokens (host,
 * room for n; may be NULL) before returning, and enqueues the copies of the body and
 * scales into the session on the stream (h_image: host memory allocated pinned,
 * valid until the stream reaches the call).  Returns n >= 0 on success.  Rows at and
 * above n are left as they were. */
int kv_image_load(const kv_shape* h_shape, const kv_session* h_sess, const void* h_image,
                  size_t image_bytes, int32_t* h_tokens, void* stream);

/* Static text for a KV_* status code. */
const char* kv_status_str(int status);

/* Measurement aid, not part of the method: reads bytes bytes at d_src once, with
 * the loads a decode makes (128-bit, non-temporal, every CU busy) and no
 * arithmetic, so that its rate is the read bandwidth a decode of the same bytes
 * can be set against.
 *   d_src : device, 16-byte aligned; bytes : a multiple of 16 (0: nothing launched).
 *   d_sink : one device uint32 the kernel may overwrite (it keeps the loads live).
 * KV_ERR_ARG for a null pointer or bytes not a multiple of 16, KV_ERR_ALIGN for a
 * misaligned d_src or d_sink, KV_ERR_HIP if the launch fails. */
int kv_probe_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ8_H */
