"""Paged sessions on the CPU: the oracle's page view against an independent scatter,
and the window's bookkeeping (kv_window_plan, host code of the library) against a
separate model of CLOCK replacement and its invariants."""
import numpy as np
import pytest

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from oracle import kvq8_oracle as o


def test_page_view_round_trip():
    r = np.random.default_rng(11)
    for fmt in (o.FMT_F16, o.FMT_Q8, o.FMT_K8V4):
        n = 300
        c = oracle.Cache(fmt, 2, 320, 128)
        assert c.append(0, kvsynth.kv_tokens(3, 0, n, 2, 128, "K", True),
                        kvsynth.kv_tokens(3, 0, n, 2, 128, "V", True))
        n_pages = 5
        pages = r.permutation(9)[:n_pages]
        pool = oracle.Cache(fmt, 2, 9 * 64, 128)
        for name in o.ROW_ARRAYS:           # scatter written here, not with the oracle
            a = getattr(c, name)
            if a is not None:
                dst = getattr(pool, name)
                for p, s in enumerate(pages):
                    dst[:, s * 64:(s + 1) * 64] = a[:, p * 64:(p + 1) * 64]
        v = o.paged_cache(pool, pages, n)
        for name in o.ROW_ARRAYS:
            if getattr(c, name) is not None:
                assert np.array_equal(getattr(v, name)[:, :n], getattr(c, name)[:, :n]), (fmt, name)
        # identity pages of a pool that is the session itself
        w = o.paged_cache(c, np.arange(n_pages), n)
        assert np.array_equal(w.k[:, :n], c.k[:, :n])


class ClockModel:
    """CLOCK with pinning of the request's resident pages, written from its definition."""

    def __init__(self, n):
        self.n, self.hand = n, 0
        self.owner = [None] * n
        self.ref = [0] * n

    def request(self, sess, pages):
        keep = {p for p, s in enumerate(pages) if 0 <= s < self.n and self.owner[s] == (sess, p)}
        pinned = {pages[p] for p in keep}
        for s in pinned:
            self.ref[s] = 1
        missed = []
        for p in range(len(pages)):
            if p in keep:
                continue
            while True:
                s = self.hand
                self.hand = (self.hand + 1) % self.n
                if s in pinned:
                    continue
                if self.ref[s]:
                    self.ref[s] = 0
                    continue
                break
            self.owner[s] = (sess, p)
            self.ref[s] = 1
            pinned.add(s)
            pages[p] = s
            missed.append(p)
        return missed


def test_window_plan_matches_clock_model_and_invariants():
    r = np.random.default_rng(12)
    n_slots = 24
    w = kq.Window(n_slots)
    model = ClockModel(n_slots)
    tables = {s: np.full(20, -1, np.int32) for s in range(5)}
    model_tables = {s: [-1] * 20 for s in range(5)}
    for step in range(200):
        sess = int(r.integers(0, 5))
        n = int(r.integers(0, 21))
        got = w.plan(sess, tables[sess][:n] if n else np.zeros(0, np.int32))
        if n:
            t = model_tables[sess][:n]
            want = model.request(sess, t)
            model_tables[sess][:n] = t
            assert list(got) == want, step
            assert list(tables[sess][:n]) == t, step
            # every page resident, in distinct slots
            assert len(set(tables[sess][:n].tolist())) == n
            assert all(0 <= s < n_slots for s in tables[sess][:n])


def test_window_keeps_resident_pages_and_refuses_oversize():
    w = kq.Window(8)
    a = np.full(6, -1, np.int32)
    assert list(w.plan(1, a)) == [0, 1, 2, 3, 4, 5]
    a_before = a.copy()
    b = np.full(5, -1, np.int32)
    w.plan(2, b)                      # evicts some of session 1's pages
    missed = w.plan(1, a)
    # pages of session 1 that kept their slot were not copied again
    for p in range(6):
        if p not in missed:
            assert a[p] == a_before[p]
    with pytest.raises(kq.KvError) as e:
        w.plan(3, np.full(9, -1, np.int32))
    assert e.value.status == kq.KV_ERR_RANGE


def test_window_and_paged_decode_validation():
    import ctypes
    L = kq.raw_lib()
    assert L.kv_window_bytes(0) == 0 and L.kv_window_bytes(1) > 0
    buf = ctypes.create_string_buffer(16)
    assert L.kv_window_init(buf, 16, 4) == kq.KV_ERR_WINDOW
    n = ctypes.c_int(0)
    assert L.kv_window_plan(ctypes.create_string_buffer(64), 0, 0, None, None, ctypes.byref(n)) == kq.KV_ERR_WINDOW
    sh = kq.make_shape(kq.KV_FMT_Q8, 8, 32)
    A = 0x7F0000000000
    dec = lambda pages, stride, max_len: L.kv_decode_attn_paged(  # noqa: E731
        ctypes.byref(sh), A, pages, stride, A, 1, max_len, A, ctypes.c_float(0.1), A, A, 1 << 30,
        None, None)
    assert dec(None, 4, 256) == kq.KV_ERR_ARG          # no page table
    assert dec(A, 3, 256) == kq.KV_ERR_ARG             # 3 pages cannot hold 256 cells
    assert dec(A, 0, 0) == kq.KV_ERR_ARG
    assert dec(A + 2, 4, 256) == kq.KV_ERR_ALIGN
