// Host-side checks of libkvq8's C ABI under AddressSanitizer and UBSan, on the CPU.
//
// The host translation units of the library (argument validation, the saved-image
// header parser, the streamed window's planner and its copies) are built host-only
// with the sanitizers and linked against this driver.  The kernel launchers, which
// live in the device translation units, are replaced here by counting stubs, so the
// driver can also check that no call launches anything when it refuses its
// arguments.  Copies go to the HIP runtime, which fails them without a GPU: that is
// how the window's rollback after a failed copy is exercised.
//
// Session pointers are fake, aligned values: nothing here dereferences them (a call
// that would enqueue work on them gets a runtime error instead).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <vector>

#include "../../quantized_kv_cache_q8_amd/csrc/kvq8_internal.h"

// ---------------------------------------------------------------------------
// stubs of the device translation units' launchers
// ---------------------------------------------------------------------------
static int g_launches = 0;

namespace kvq8 {
hipError_t launch_append(int, int, const kv_session*, const int32_t*, int, int, const float*,
                         const float*, int32_t*, hipStream_t, const int32_t*, int) {
  ++g_launches;
  return hipSuccess;
}
DecodePlan decode_plan(int, int, int nqh, int n_sess, int) {
  DecodePlan p;
  p.S = 4;
  p.ws_o_bytes = ((size_t)n_sess * nqh * p.S * HD * 4 + 255) & ~(size_t)255;
  p.ws_lse_bytes = ((size_t)n_sess * nqh * p.S * 4 + 255) & ~(size_t)255;
  p.ws_ord_bytes = n_sess > 1 ? ((size_t)n_sess * 48 + 255) & ~(size_t)255 : 0;
  return p;
}
hipError_t launch_decode(int, int, int, const kv_session*, const int32_t*, int, int, const float*,
                         float, float*, void*, const DecodePlan&, int32_t*, hipStream_t,
                         const int32_t*, int) {
  ++g_launches;
  return hipSuccess;
}
void* static_workspace() { return reinterpret_cast<void*>(0x7E0000000000ull); }
hipError_t launch_compact(int, int, const kv_session&, int, uint16_t*, uint16_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill(int, int, const uint16_t*, const uint16_t*, long, int, int, const float*,
                          float, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_stream_read(const void*, size_t, uint32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace kvq8

static int g_fail = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static const uintptr_t A = 0x7F0000000000ull;

static kv_session fake(int fmt, int cap, uintptr_t base = A) {
  kv_session s{};
  s.k = reinterpret_cast<void*>(base);
  s.v = reinterpret_cast<void*>(base + 0x1000000);
  if (fmt != KV_FMT_F16) {
    s.k_scale = reinterpret_cast<uint16_t*>(base + 0x2000000);
    s.v_scale = reinterpret_cast<uint16_t*>(base + 0x3000000);
  }
  s.cap = cap;
  return s;
}

template <class T>
static T* P(uintptr_t off) { return reinterpret_cast<T*>(A + off); }

// ---------------------------------------------------------------------------
// every argument error refuses before any launch
// ---------------------------------------------------------------------------
static void argument_errors() {
  const kv_shape ok{KV_FMT_Q8, 8, 32, 128};
  const kv_shape bad_shapes[] = {
      {7, 8, 32, 128},          {KV_FMT_Q8, 0, 32, 128},  {KV_FMT_Q8, 8, 30, 128},
      {KV_FMT_Q8, 8, 32, 64},   {KV_FMT_Q8, 8, 8 * 16, 128}, {KV_FMT_Q8, 2048, 2048, 128},
      {KV_FMT_F16, -1, 4, 128}, {KV_FMT_K8V4, 8, 0, 128}};
  int32_t* st = P<int32_t>(0x4000000);
  const int before = g_launches;
  for (const kv_shape& b : bad_shapes) {
    CHECK(kv_append(&b, P<kv_session>(0), P<int32_t>(64), 1, 1, P<float>(0x100), P<float>(0x200),
                    st, nullptr) < 0);
    CHECK(kv_decode_workspace_bytes(&b, 1, 100) == 0);
    CHECK(kv_decode_attn(&b, P<kv_session>(0), P<int32_t>(64), 1, 100, P<float>(0x100), 0.1f,
                         P<float>(0x200), P<void>(0x300), 1 << 30, st, nullptr) < 0);
    kv_session s = fake(b.fmt == KV_FMT_F16 ? KV_FMT_F16 : KV_FMT_Q8, 128);
    CHECK(kv_prefill_attn(&b, &s, 0, 1, P<float>(0x100), 0.1f, P<float>(0x200), P<void>(0x300),
                          1 << 30, nullptr) < 0);
    CHECK(kv_compact_f16(&b, &s, 64, P<uint16_t>(0x100), P<uint16_t>(0x200), nullptr) < 0);
    CHECK(kv_rows_bytes(&b, 3) == 0);
    CHECK(kv_image_bytes(&b, 3) == 0);
  }
  CHECK(kv_append(nullptr, P<kv_session>(0), P<int32_t>(64), 1, 1, P<float>(0x100),
                  P<float>(0x200), st, nullptr) == KV_ERR_ARG);
  // append: null pointers, counts, alignment
  CHECK(kv_append(&ok, nullptr, P<int32_t>(64), 1, 1, P<float>(0x100), P<float>(0x200), st,
                  nullptr) == KV_ERR_ARG);
  CHECK(kv_append(&ok, P<kv_session>(0), P<int32_t>(64), 0, 1, P<float>(0x100), P<float>(0x200),
                  st, nullptr) == KV_ERR_ARG);
  CHECK(kv_append(&ok, P<kv_session>(0), P<int32_t>(64), 65536, 1, P<float>(0x100),
                  P<float>(0x200), st, nullptr) == KV_ERR_ARG);
  CHECK(kv_append(&ok, P<kv_session>(0), P<int32_t>(64), 1, -1, P<float>(0x100), P<float>(0x200),
                  st, nullptr) == KV_ERR_ARG);
  CHECK(kv_append(&ok, P<kv_session>(4), P<int32_t>(64), 1, 1, P<float>(0x100), P<float>(0x200),
                  st, nullptr) == KV_ERR_ALIGN);
  CHECK(kv_append(&ok, P<kv_session>(0), P<int32_t>(64), 1, 1, P<float>(0x104), P<float>(0x200),
                  st, nullptr) == KV_ERR_ALIGN);
  CHECK(kv_append(&ok, P<kv_session>(0), P<int32_t>(66), 1, 1, P<float>(0x100), P<float>(0x200),
                  st, nullptr) == KV_ERR_ALIGN);
  // paged append
  CHECK(kv_append_paged(&ok, P<kv_session>(0), nullptr, 4, P<int32_t>(64), 1, 1, P<float>(0x100),
                        P<float>(0x200), st, nullptr) == KV_ERR_ARG);
  CHECK(kv_append_paged(&ok, P<kv_session>(0), P<int32_t>(0x500), 0, P<int32_t>(64), 1, 1,
                        P<float>(0x100), P<float>(0x200), st, nullptr) == KV_ERR_ARG);
  CHECK(kv_append_paged(&ok, P<kv_session>(0), P<int32_t>(0x502), 4, P<int32_t>(64), 1, 1,
                        P<float>(0x100), P<float>(0x200), st, nullptr) == KV_ERR_ALIGN);
  CHECK(kv_append_paged(&ok, P<kv_session>(0), P<int32_t>(0x500), 4, P<int32_t>(64), 1, 1,
                        P<float>(0x108), P<float>(0x200), st, nullptr) == KV_ERR_ALIGN);
  // decode
  CHECK(kv_decode_attn(&ok, P<kv_session>(0), P<int32_t>(64), 1, 100, P<float>(0x100), 0.1f,
                       P<float>(0x200), nullptr, 0, st, nullptr) == KV_ERR_WORKSPACE);
  CHECK(kv_decode_attn(&ok, P<kv_session>(0), P<int32_t>(64), 1, 100, P<float>(0x100), 0.1f,
                       P<float>(0x200), P<void>(0x300), 16, st, nullptr) == KV_ERR_WORKSPACE);
  CHECK(kv_decode_attn(&ok, P<kv_session>(0), P<int32_t>(64), 1, -1, P<float>(0x100), 0.1f,
                       P<float>(0x200), P<void>(0x300), 1 << 30, st, nullptr) == KV_ERR_ARG);
  CHECK(kv_decode_attn(&ok, P<kv_session>(0), P<int32_t>(64), 1, 100, P<float>(0x100), NAN,
                       P<float>(0x200), P<void>(0x300), 1 << 30, st, nullptr) == KV_ERR_ARG);
  CHECK(kv_decode_attn(&ok, P<kv_session>(0), P<int32_t>(64), 1, 100, P<float>(0x104), 0.1f,
                       P<float>(0x200), P<void>(0x300), 1 << 30, st, nullptr) == KV_ERR_ALIGN);
  CHECK(kv_decode_attn_static(&ok, P<kv_session>(0), P<int32_t>(64), 65536, 100, P<float>(0x100),
                              0.1f, P<float>(0x200), st, nullptr) == KV_ERR_ARG);
  CHECK(kv_decode_attn_static(&ok, P<kv_session>(0), P<int32_t>(64), 1, 100, P<float>(0x100),
                              0.1f, P<float>(0x204), st, nullptr) == KV_ERR_ALIGN);
  // the stub plan's partials for 1000 sessions exceed the fixed scratch
  CHECK(kv_decode_attn_static(&ok, P<kv_session>(0), P<int32_t>(64), 1000, 100, P<float>(0x100),
                              0.1f, P<float>(0x200), st, nullptr) == KV_ERR_WORKSPACE);
  CHECK(kv_decode_attn_static(&ok, P<kv_session>(0), P<int32_t>(64), 1, 100, nullptr, 0.1f,
                              P<float>(0x200), st, nullptr) == KV_ERR_ARG);
  CHECK(kv_decode_attn_paged(&ok, P<kv_session>(0), P<int32_t>(0x500), 1, P<int32_t>(64), 1, 100,
                             P<float>(0x100), 0.1f, P<float>(0x200), P<void>(0x300), 1 << 30, st,
                             nullptr) == KV_ERR_ARG);   // page_stride * 64 < max_len
  CHECK(kv_decode_attn_paged(&ok, P<kv_session>(0), nullptr, 2, P<int32_t>(64), 1, 100,
                             P<float>(0x100), 0.1f, P<float>(0x200), P<void>(0x300), 1 << 30, st,
                             nullptr) == KV_ERR_ARG);
  // sessions handed over on the host: format, alignment, capacity
  kv_session s = fake(KV_FMT_Q8, 128);
  kv_session f16 = fake(KV_FMT_F16, 128);
  CHECK(kv_compact_f16(&ok, &f16, 64, P<uint16_t>(0x100), P<uint16_t>(0x200), nullptr) ==
        KV_ERR_FMT);
  kv_session mis = s;
  mis.v_scale = P<uint16_t>(0x3000002);
  CHECK(kv_compact_f16(&ok, &mis, 64, P<uint16_t>(0x100), P<uint16_t>(0x200), nullptr) ==
        KV_ERR_ALIGN);
  kv_session odd = s;
  odd.cap = 100;
  CHECK(kv_compact_f16(&ok, &odd, 64, P<uint16_t>(0x100), P<uint16_t>(0x200), nullptr) ==
        KV_ERR_ALIGN);
  kv_session huge = s;
  huge.cap = (1 << 24) + 64;
  CHECK(kv_compact_f16(&ok, &huge, 64, P<uint16_t>(0x100), P<uint16_t>(0x200), nullptr) ==
        KV_ERR_RANGE);
  CHECK(kv_compact_f16(&ok, &s, 129, P<uint16_t>(0x100), P<uint16_t>(0x200), nullptr) ==
        KV_ERR_RANGE);
  CHECK(kv_prefill_attn(&ok, &s, 100, 29, P<float>(0x100), 0.1f, P<float>(0x200),
                        P<void>(0x300), 1 << 30, nullptr) == KV_ERR_RANGE);
  CHECK(kv_prefill_attn(&ok, &s, 0, 1, P<float>(0x100), -1.f, P<float>(0x200), P<void>(0x300),
                        1 << 30, nullptr) == KV_ERR_ARG);
  CHECK(kv_prefill_attn(&ok, &s, 0, 64, P<float>(0x100), 0.1f, P<float>(0x200), P<void>(0x300),
                        100, nullptr) == KV_ERR_WORKSPACE);
  // row moves
  CHECK(kv_copy_rows(&ok, &s, 0, &s, 64, 65, nullptr) == KV_ERR_RANGE);
  CHECK(kv_copy_rows(&ok, &s, -1, &s, 64, 1, nullptr) == KV_ERR_RANGE);
  CHECK(kv_copy_rows(&ok, &s, 0, &f16, 0, 1, nullptr) == KV_ERR_FMT);
  CHECK(kv_gather_rows(&ok, &s, 0, 129, P<void>(0x100), nullptr) == KV_ERR_RANGE);
  CHECK(kv_scatter_rows(&ok, &s, 0, 1, nullptr, nullptr) == KV_ERR_ARG);
  CHECK(kv_probe_stream_read(P<void>(0x100), 15, P<uint32_t>(0x200), nullptr) == KV_ERR_ARG);
  CHECK(kv_probe_stream_read(P<void>(0x108), 16, P<uint32_t>(0x200), nullptr) == KV_ERR_ALIGN);
  CHECK(g_launches == before);
}

// ---------------------------------------------------------------------------
// saved image: truncated and corrupted headers never read past the image
// ---------------------------------------------------------------------------
static void image_fuzz() {
  const kv_shape shapes[] = {{KV_FMT_F16, 3, 3, 128}, {KV_FMT_Q8, 3, 12, 128},
                             {KV_FMT_K8V4, 2, 8, 128}};
  std::mt19937_64 rng(20240611);
  for (const kv_shape& sh : shapes) {
    const int n = 5;
    const size_t full = kv_image_bytes(&sh, n);
    CHECK(full > 128);
    // a well-formed header written by the library for a session of fake pointers;
    // the body copy fails without a GPU (or succeeds on one), the header is complete
    std::vector<unsigned char> good(full, 0);
    kv_session s = fake(sh.fmt, 128);
    int32_t toks[n] = {1, -2, 3, 2147483647, 0};
    const int rc = kv_image_save(&sh, &s, n, toks, good.data(), full, nullptr);
    CHECK(rc == KV_OK || rc == KV_ERR_HIP);
    // every prefix length: exactly sized heap copies, so a read past the end is caught
    for (size_t len = 0; len <= full; ++len) {
      unsigned char* img = static_cast<unsigned char*>(std::malloc(len ? len : 1));
      std::memcpy(img, good.data(), len);
      const int t = kv_image_tokens(&sh, img, len);
      CHECK(len == full ? t == n : t == KV_ERR_IMAGE);
      std::free(img);
    }
    // random corruptions of header bytes, and of the size fields with extreme values
    int accepted = 0;
    for (int it = 0; it < 20000; ++it) {
      std::vector<unsigned char> v(good);
      const int nflip = 1 + (int)(rng() % 4);
      for (int k = 0; k < nflip; ++k) v[rng() % 40] ^= (unsigned char)(1u << (rng() % 8));
      if (it % 4 == 0) {
        const int field = (int)(rng() % 3);
        const uint64_t big = rng();
        const int off = field == 0 ? 20 : field == 1 ? 24 : 32;
        const int nb = field == 0 ? 4 : 8;
        for (int b = 0; b < nb; ++b) v[off + b] = (unsigned char)(big >> (8 * b));
      }
      const size_t len = it % 3 == 0 ? full : (size_t)(rng() % (full + 64));
      unsigned char* img = static_cast<unsigned char*>(std::malloc(len ? len : 1));
      std::memcpy(img, v.data(), std::min(len, v.size()));
      const int t = kv_image_tokens(&sh, img, len);
      CHECK(t == KV_ERR_IMAGE || (t >= 0 && (size_t)t <= (1u << 24)));
      if (t >= 0) {
        ++accepted;
        // an accepted header describes regions inside the image
        CHECK(kv_image_bytes(&sh, t) <= len);
        std::vector<int32_t> tk((size_t)t + 1);
        kv_session big = fake(sh.fmt, 1 << 24);
        const int l = kv_image_load(&sh, &big, img, len, tk.data(), nullptr);
        CHECK(l == t || l == KV_ERR_HIP);
      }
      std::free(img);
    }
    std::printf("image fmt=%d: %d of 20000 corrupted images accepted (bit flips that keep a "
                "consistent header)\n", sh.fmt, accepted);
    // version 2 with scales refused, for the int8 formats
    if (sh.fmt != KV_FMT_F16) {
      std::vector<unsigned char> v(good);
      v[4] = 2;
      CHECK(kv_image_tokens(&sh, v.data(), v.size()) == KV_ERR_IMAGE);
    }
  }
}

// ---------------------------------------------------------------------------
// the window's planner: random requests, garbage page tables
// ---------------------------------------------------------------------------
static void window_plan_fuzz() {
  std::mt19937_64 rng(7);
  for (int n_slots : {1, 2, 7, 64, 300}) {
    std::vector<unsigned char> state(kv_window_bytes(n_slots));
    CHECK(kv_window_init(state.data(), state.size(), n_slots) == KV_OK);
    CHECK(kv_window_init(state.data(), state.size() - 1, n_slots) == KV_ERR_WINDOW);
    const int n_sess = 5;
    std::vector<std::vector<int32_t>> tables(n_sess, std::vector<int32_t>(2 * n_slots + 3, -1));
    std::vector<int32_t> missed(2 * n_slots + 3);
    for (int it = 0; it < 4000; ++it) {
      const int sid = (int)(rng() % n_sess);
      std::vector<int32_t>& t = tables[sid];
      const int np = (int)(rng() % (n_slots + 3));
      if (it % 97 == 0)   // garbage entries: read as not resident, never indexed
        for (auto& e : t) e = (int32_t)rng();
      int misses = -1;
      const int rc = kv_window_plan(state.data(), sid, np, t.data(), missed.data(), &misses);
      if (np > n_slots) {
        CHECK(rc == KV_ERR_RANGE);
        continue;
      }
      CHECK(rc == KV_OK);
      CHECK(misses >= 0 && misses <= np);
      // the request's pages are in distinct slots of the window
      std::set<int32_t> used;
      for (int p = 0; p < np; ++p) {
        CHECK(t[p] >= 0 && t[p] < n_slots);
        used.insert(t[p]);
      }
      CHECK((int)used.size() == np);
      // the same request again: nothing to copy
      int again = -1;
      CHECK(kv_window_plan(state.data(), sid, np, t.data(), missed.data(), &again) == KV_OK);
      CHECK(again == 0);
    }
    int m = 0;
    CHECK(kv_window_plan(state.data(), -1, 1, tables[0].data(), missed.data(), &m) == KV_ERR_ARG);
    CHECK(kv_window_plan(nullptr, 0, 1, tables[0].data(), missed.data(), &m) == KV_ERR_WINDOW);
  }
}

// ---------------------------------------------------------------------------
// kv_window_map: refused arguments leave the window unchanged; a failed copy
// unmaps the pages it did not copy
// ---------------------------------------------------------------------------
static void window_map_errors() {
  const kv_shape sh{KV_FMT_Q8, 2, 8, 128};
  const int n_slots = 16, np = 6;
  std::vector<unsigned char> state(kv_window_bytes(n_slots));
  CHECK(kv_window_init(state.data(), state.size(), n_slots) == KV_OK);
  kv_session store = fake(KV_FMT_Q8, 64 * 8, A);
  kv_session pool = fake(KV_FMT_Q8, 64 * n_slots, A + 0x10000000);
  std::vector<int32_t> pages(np, -1), missed(np);
  int32_t* d_pages = P<int32_t>(0x5000000);
  int misses = -1;
  // misaligned store, a store of another format, a short pool: refused, state unchanged
  kv_session mis = store;
  mis.k_scale = P<uint16_t>(0x2000002);
  CHECK(kv_window_map(&sh, state.data(), &mis, 0, np, &pool, pages.data(), missed.data(), d_pages,
                      &misses, nullptr) == KV_ERR_ALIGN);
  kv_session f16 = fake(KV_FMT_F16, 64 * 8, A);
  CHECK(kv_window_map(&sh, state.data(), &f16, 0, np, &pool, pages.data(), missed.data(), d_pages,
                      &misses, nullptr) == KV_ERR_FMT);
  kv_session small = pool;
  small.cap = 64 * (n_slots - 1);
  CHECK(kv_window_map(&sh, state.data(), &store, 0, np, &small, pages.data(), missed.data(),
                      d_pages, &misses, nullptr) == KV_ERR_RANGE);
  for (int p = 0; p < np; ++p) CHECK(pages[p] == -1);
  std::vector<int32_t> probe(np, -1);
  CHECK(kv_window_plan(state.data(), 0, np, probe.data(), missed.data(), &misses) == KV_OK);
  CHECK(misses == np);
  // a map whose copies cannot be enqueued (no GPU here): the pages stay unmapped
  CHECK(kv_window_init(state.data(), state.size(), n_slots) == KV_OK);
  const int rc = kv_window_map(&sh, state.data(), &store, 0, np, &pool, pages.data(),
                               missed.data(), d_pages, &misses, nullptr);
  if (rc == KV_ERR_HIP) {
    for (int p = 0; p < np; ++p) CHECK(pages[p] == -1);
    std::vector<int32_t> again(np, -1);
    CHECK(kv_window_plan(state.data(), 0, np, again.data(), missed.data(), &misses) == KV_OK);
    CHECK(misses == np);
    std::printf("window map: failed copy rolled back\n");
  } else {
    CHECK(rc == KV_OK);   // a machine with a GPU and these fake pointers would not get here
  }
}

// kv_window_writeback: pages not resident for the session, or rows beyond the store,
// are refused before anything is enqueued
static void window_writeback_errors() {
  const kv_shape sh{KV_FMT_Q8, 2, 8, 128};
  const int n_slots = 8;
  std::vector<unsigned char> state(kv_window_bytes(n_slots));
  CHECK(kv_window_init(state.data(), state.size(), n_slots) == KV_OK);
  kv_session store = fake(KV_FMT_Q8, 64 * 4, A);
  kv_session pool = fake(KV_FMT_Q8, 64 * n_slots, A + 0x10000000);
  std::vector<int32_t> pages(4, -1), missed(4);
  int misses = -1;
  CHECK(kv_window_plan(state.data(), 3, 2, pages.data(), missed.data(), &misses) == KV_OK);
  CHECK(misses == 2);
  // page 2 not mapped; another session's id; rows past the store; a null table
  CHECK(kv_window_writeback(&sh, state.data(), &store, 3, 100, 40, &pool, pages.data(), nullptr) ==
        KV_ERR_WINDOW);
  CHECK(kv_window_writeback(&sh, state.data(), &store, 4, 0, 1, &pool, pages.data(), nullptr) ==
        KV_ERR_WINDOW);
  CHECK(kv_window_writeback(&sh, state.data(), &store, 3, 250, 7, &pool, pages.data(), nullptr) ==
        KV_ERR_RANGE);
  CHECK(kv_window_writeback(&sh, state.data(), &store, 3, 0, 1, &pool, nullptr, nullptr) ==
        KV_ERR_ARG);
  std::vector<int32_t> garbage = {1 << 30, -5, 7, 0};
  CHECK(kv_window_writeback(&sh, state.data(), &store, 3, 0, 70, &pool, garbage.data(), nullptr) ==
        KV_ERR_WINDOW);
  CHECK(kv_window_writeback(&sh, state.data(), &store, 3, 5, 0, &pool, pages.data(), nullptr) ==
        KV_OK);
  // mapped rows: the copy itself fails without a GPU
  const int rc = kv_window_writeback(&sh, state.data(), &store, 3, 60, 10, &pool, pages.data(),
                                     nullptr);
  CHECK(rc == KV_ERR_HIP || rc == KV_OK);
}

int main() {
  // Fake pointers reach the runtime's copy calls; with a GPU present a copy could be
  // enqueued on them, so this driver runs on machines without one only.
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0) {
    std::printf("GPU visible: host checks not run\n");
    return 3;
  }
  argument_errors();
  image_fuzz();
  window_plan_fuzz();
  window_map_errors();
  window_writeback_errors();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
