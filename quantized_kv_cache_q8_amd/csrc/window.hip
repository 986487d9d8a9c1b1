// Streamed K/V pages (PR #711 "kv: --kv k8v4 streams with --kv-resident", sections
// What and How: a session's K/V live in host memory and move to a device-resident
// window block by block, each block a list of byte runs, codes and scales alike).
//
// Here a block is a page of KV_PAGE_ROWS cells; the host store is a session whose
// arrays lie in pinned host memory, so a page's runs are its rows of each array and
// a run of consecutive pages is one 2-D copy per array.  The window is a pool of
// page slots on the device (a session whose cap is 64 x slots); its bookkeeping lives
// in caller-owned host memory: which (session, page) each slot holds, and CLOCK
// replacement (a reference bit per slot and a sweeping hand).  Host code only.
#include <algorithm>
#include <cstring>

#include "kvq8_internal.h"

using namespace kvq8;

namespace {

constexpr uint32_t kWindowMagic = 0x4B565157u;  // "WQVK"

struct WinHeader {
  uint32_t magic;
  int32_t n_slots;
  int32_t hand;
  int32_t epoch;
};
struct WinSlot {
  int32_t sess;   // -1: free
  int32_t page;
  int32_t stamp;  // the request that last used the slot
  int32_t ref;    // CLOCK reference bit
};

WinHeader* header(void* st) { return static_cast<WinHeader*>(st); }
WinSlot* slots(void* st) { return reinterpret_cast<WinSlot*>(static_cast<char*>(st) + sizeof(WinHeader)); }

bool resident(const WinSlot* sl, int n_slots, int32_t s, int sess, int page) {
  return s >= 0 && s < n_slots && sl[s].sess == sess && sl[s].page == page;
}

}  // namespace

extern "C" {

size_t kv_window_bytes(int n_slots) {
  if (n_slots < 1 || n_slots > KV_MAX_CAP / KV_PAGE_ROWS) return 0;
  return sizeof(WinHeader) + (size_t)n_slots * sizeof(WinSlot);
}

int kv_window_init(void* h_state, size_t bytes, int n_slots) {
  const size_t need = kv_window_bytes(n_slots);
  if (need == 0 || h_state == nullptr) return KV_ERR_ARG;
  if (bytes < need) return KV_ERR_WINDOW;
  WinHeader* hd = header(h_state);
  hd->magic = kWindowMagic;
  hd->n_slots = n_slots;
  hd->hand = 0;
  hd->epoch = 0;
  WinSlot* sl = slots(h_state);
  for (int i = 0; i < n_slots; ++i) sl[i] = WinSlot{-1, -1, -1, 0};
  return KV_OK;
}

int kv_window_plan(void* h_state, int sess_id, int n_pages, int32_t* h_pages,
                   int32_t* h_missed, int* h_misses) {
  if (h_state == nullptr || header(h_state)->magic != kWindowMagic) return KV_ERR_WINDOW;
  WinHeader* hd = header(h_state);
  WinSlot* sl = slots(h_state);
  const int n = hd->n_slots;
  if (sess_id < 0 || n_pages < 0 || h_misses == nullptr) return KV_ERR_ARG;
  if (n_pages > 0 && (h_pages == nullptr || h_missed == nullptr)) return KV_ERR_ARG;
  if (n_pages > n) return KV_ERR_RANGE;  // the request would evict its own pages
  const int32_t epoch = ++hd->epoch;
  // pages already resident are pinned for this request first, so that none of them
  // is evicted to make room for another
  for (int p = 0; p < n_pages; ++p) {
    const int32_t s = h_pages[p];
    if (resident(sl, n, s, sess_id, p)) {
      sl[s].stamp = epoch;
      sl[s].ref = 1;
    }
  }
  int misses = 0;
  for (int p = 0; p < n_pages; ++p) {
    if (resident(sl, n, h_pages[p], sess_id, p) && sl[h_pages[p]].stamp == epoch) continue;
    // CLOCK: skip this request's slots, give referenced slots a second chance; at most
    // n_pages - 1 slots are pinned, so two sweeps find one
    int s;
    for (;;) {
      s = hd->hand;
      hd->hand = (hd->hand + 1) % n;
      if (sl[s].stamp == epoch) continue;
      if (sl[s].ref) {
        sl[s].ref = 0;
        continue;
      }
      break;
    }
    sl[s] = WinSlot{sess_id, p, epoch, 1};
    h_pages[p] = s;
    h_missed[misses++] = p;
  }
  *h_misses = misses;
  return KV_OK;
}

int kv_window_map(const kv_shape* h_shape, void* h_state, const kv_session* h_store, int sess_id,
                  int n_pages, const kv_session* h_pool, int32_t* h_pages, int32_t* h_missed,
                  int32_t* d_pages, int* h_misses, void* stream) {
  // every argument is checked before the plan changes the window's state
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if ((rc = check_session(h_shape, h_store)) || (rc = check_session(h_shape, h_pool))) return rc;
  if (h_state == nullptr || header(h_state)->magic != kWindowMagic) return KV_ERR_WINDOW;
  const int n_slots = header(h_state)->n_slots;
  if ((long long)h_pool->cap < (long long)n_slots * KV_PAGE_ROWS) return KV_ERR_RANGE;
  if ((long long)h_store->cap < (long long)n_pages * KV_PAGE_ROWS) return KV_ERR_RANGE;
  if (n_pages > 0 && d_pages == nullptr) return KV_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_pages) & 3) return KV_ERR_ALIGN;
  rc = kv_window_plan(h_state, sess_id, n_pages, h_pages, h_missed, h_misses);
  if (rc) return rc;
  // copy the missed pages, runs of consecutive pages in consecutive slots at once
  const int m = *h_misses;
  for (int i = 0; i < m;) {
    int j = i + 1;
    while (j < m && h_missed[j] == h_missed[j - 1] + 1 &&
           h_pages[h_missed[j]] == h_pages[h_missed[j - 1]] + 1)
      ++j;
    rc = copy_rows(h_shape, h_store, h_missed[i] * KV_PAGE_ROWS, h_pool,
                   h_pages[h_missed[i]] * KV_PAGE_ROWS, (j - i) * KV_PAGE_ROWS, stream,
                   hipMemcpyHostToDevice);
    if (rc) {
      // the pages from this run on were planned but never copied: their slots are
      // marked free and the pages unmapped, so a later plan lists them as missed
      // (the runs before this one were enqueued and keep their slots)
      WinSlot* sl = slots(h_state);
      for (int k = i; k < m; ++k) {
        const int32_t s = h_pages[h_missed[k]];
        sl[s] = WinSlot{-1, -1, -1, 0};
        h_pages[h_missed[k]] = -1;
      }
      return rc;
    }
    i = j;
  }
  if (n_pages > 0 &&
      hipMemcpyAsync(d_pages, h_pages, (size_t)n_pages * sizeof(int32_t), hipMemcpyHostToDevice,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return KV_ERR_HIP;
  return KV_OK;
}

int kv_window_writeback(const kv_shape* h_shape, void* h_state, const kv_session* h_store,
                        int sess_id, int row0, int n_rows, const kv_session* h_pool,
                        const int32_t* h_pages, void* stream) {
  int rc = check_shape(h_shape);
  if (rc) return rc;
  if ((rc = check_session(h_shape, h_store)) || (rc = check_session(h_shape, h_pool))) return rc;
  if (h_state == nullptr || header(h_state)->magic != kWindowMagic) return KV_ERR_WINDOW;
  if (sess_id < 0 || row0 < 0 || n_rows < 0) return KV_ERR_ARG;
  if (n_rows > 0 && h_pages == nullptr) return KV_ERR_ARG;
  if ((long long)row0 + n_rows > h_store->cap) return KV_ERR_RANGE;
  if (n_rows == 0) return KV_OK;
  const int n_slots = header(h_state)->n_slots;
  if ((long long)h_pool->cap < (long long)n_slots * KV_PAGE_ROWS) return KV_ERR_RANGE;
  const WinSlot* sl = slots(h_state);
  const int p0 = row0 / KV_PAGE_ROWS, p1 = (row0 + n_rows - 1) / KV_PAGE_ROWS;
  // every page the rows touch must be the session's, in the slot its table names
  for (int p = p0; p <= p1; ++p)
    if (!resident(sl, n_slots, h_pages[p], sess_id, p)) return KV_ERR_WINDOW;
  // runs of rows in consecutive pages of consecutive slots, one copy per array each
  int r = row0;
  const int end = row0 + n_rows;
  while (r < end) {
    const int p = r / KV_PAGE_ROWS;
    int q = p;
    while ((q + 1) * KV_PAGE_ROWS < end && h_pages[q + 1] == h_pages[q] + 1) ++q;
    const int r1 = std::min(end, (q + 1) * KV_PAGE_ROWS);
    const int pool_row = h_pages[p] * KV_PAGE_ROWS + (r - p * KV_PAGE_ROWS);
    rc = copy_rows(h_shape, h_pool, pool_row, h_store, r, r1 - r, stream, hipMemcpyDeviceToHost);
    if (rc) return rc;
    r = r1;
  }
  return KV_OK;
}

}  // extern "C"
