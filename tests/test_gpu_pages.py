"""Paged sessions and the streamed window on the GPU: a decode over pages scattered
through a pool, or streamed into a window from a pinned host store, equals the decode
over the resident session bit for bit (PR #711 "kv: --kv k8v4 streams with
--kv-resident", section Tests: the streamed decode must match the resident one bit
for bit)."""
import numpy as np
import pytest
import torch

import kvsynth
import quantized_kv_cache_q8_amd as kq
from gpu_util import DEV, append_bulk, check_close, oracle_cache, say, shape, sm_scale
from oracle import kvq8_oracle as o

pytestmark = pytest.mark.gpu
P = kq.KV_PAGE_ROWS


def filled(fmt, kvh, cap, n, seed):
    xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True)
    s = kq.Session(fmt, kvh, cap, fill=0)
    assert append_bulk(shape(fmt, kvh, kvh), [s], [0], xk[None], xv[None]) == 0
    return s, xk, xv


def copy_pages(src, dst, pages, n_pages):
    """Rows of page p of src into slot pages[p] of dst (torch copies)."""
    for a, b in zip(src.tensors(), dst.tensors()):
        for p in range(n_pages):
            s = int(pages[p])
            b[:, s * P:(s + 1) * P].copy_(a[:, p * P:(p + 1) * P])


def decode(sh, sessions, lens, q, max_len, pages=None, stride=0, status=None):
    n = len(sessions)
    tab = kq.session_table([s.entry() for s in sessions])
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = torch.empty((n, sh.n_q_heads, 128), device=DEV)
    ws = torch.zeros(kq.kv_decode_workspace_bytes(sh, n, max_len), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    if pages is None:
        kq.kv_decode_attn(sh, tab, ln, n, max_len, qd, sm_scale(), out, ws, status)
    else:
        kq.kv_decode_attn_paged(sh, tab, pages, stride, ln, n, max_len, qd, sm_scale(), out, ws, status)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fmt,G", [(0, 4), (1, 4), (2, 4), (1, 1), (1, 8), (0, 2)])
def test_paged_decode_equals_resident(fmt, G):
    kvh, n = 4, 3001
    say(f"paged fmt={fmt} G={G}")
    sess, xk, xv = filled(fmt, kvh, 3072, n, 31)
    sh = shape(fmt, kvh, G * kvh)
    q = kvsynth.queries(31, 0, 1, G * kvh, 128)
    y_res = decode(sh, [sess], [n], q, n)
    n_pages = (n + P - 1) // P
    n_slots = 80
    perm = np.random.default_rng(fmt * 10 + G).permutation(n_slots)[:n_pages].astype(np.int32)
    # 0xFF bytes: NaN fp16 values and scales wherever the pool was not written, so a
    # read of a row past the session's end (0 weight or not) would show in the output
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)
    copy_pages(sess, pool, perm, n_pages)
    pages = torch.from_numpy(perm).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y_pag = decode(sh, [pool], [n], q, n, pages, n_pages, status)
    assert int(status.item()) == 0
    assert np.array_equal(y_pag, y_res)
    # and the oracle's decode over the oracle's view of the pool
    ref = oracle_cache(fmt, kvh, 3072, 128, xk, xv)
    view = o.paged_cache(ref, np.arange(n_pages), n)
    want = o.decode_attn(q[0], view.dequant("k", n), view.dequant("v", n), n, sm_scale())
    check_close(y_pag[0], want, f"paged fmt={fmt} G={G}")


@pytest.mark.parametrize("fmt", [kq.KV_FMT_Q8, kq.KV_FMT_K8V4])
def test_paged_long_batch_equals_resident(fmt):
    """8 sessions of up to 65536 cells over 8 kv heads: the grid then gives a pair
    more than 128 steps, which takes the wider page map."""
    kvh, G, n = 8, 4, 65536
    say(f"paged long batch fmt={fmt}")
    lens = [65536, 41000, 65533, 12345, 65536, 300, 50001, 64]
    sh = shape(fmt, kvh, G * kvh)
    master = filled(fmt, kvh, n, n, 61)[0]
    q = kvsynth.queries(62, 0, len(lens), G * kvh, 128)
    # the split count from the workspace size: per split, nqh rows of HD + 1 floats
    splits = kq.kv_decode_workspace_bytes(sh, len(lens), n) // (len(lens) * G * kvh * 129 * 4)
    J = n // 8
    assert -(-J // (4 * splits)) > 128, splits
    y_res = decode(sh, [master] * len(lens), lens, q, n)
    stride = n // P
    n_pg = [(m + P - 1) // P for m in lens]
    n_slots = sum(n_pg) + 5
    perm = np.random.default_rng(63).permutation(n_slots).astype(np.int32)
    table = np.zeros((len(lens), stride), np.int32)
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)   # NaN where not written
    k = 0
    for b, npg in enumerate(n_pg):
        table[b, :npg] = perm[k:k + npg]
        k += npg
        idx = torch.from_numpy(table[b, :npg].astype(np.int64)).to(DEV)
        for a, d in zip(master.tensors(), pool.tensors()):
            d.view(kvh, n_slots, -1)[:, idx] = a.view(kvh, n // P, -1)[:, :npg]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y_pag = decode(sh, [pool] * len(lens), lens, q, n, torch.from_numpy(table).to(DEV), stride,
                   status)
    assert int(status.item()) == 0
    assert np.array_equal(y_pag, y_res)


@pytest.mark.slow
def test_paged_single_session_wide_map():
    """One session whose pairs hold more than 128 steps each: the one-session int8
    launch with the 4-register page map and units of four steps, paged against resident,
    bit for bit."""
    fmt, kvh, G, n = kq.KV_FMT_Q8, 32, 4, 131072
    say("paged single session, wide page map")
    sh = shape(fmt, kvh, G * kvh)
    # 8192 seeded cells, tiled over the session on the device (the comparison is of
    # two decodes of the same cache)
    master = filled(fmt, kvh, n, 8192, 71)[0]
    for t in master.tensors():
        t.view(kvh, n // 8192, 8192, -1)[:, 1:] = t.view(kvh, n // 8192, 8192, -1)[:, :1]
    q = kvsynth.queries(72, 0, 1, G * kvh, 128)
    splits = kq.kv_decode_workspace_bytes(sh, 1, n) // (G * kvh * 129 * 4)
    assert -(-(n // 8) // (4 * splits)) > 128, splits
    y_res = decode(sh, [master], [n], q, n)
    n_pg = n // P
    n_slots = n_pg + 3
    perm = np.random.default_rng(73).permutation(n_slots)[:n_pg].astype(np.int32)
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)   # NaN where not written
    idx = torch.from_numpy(perm.astype(np.int64)).to(DEV)
    for a, d in zip(master.tensors(), pool.tensors()):
        d.view(kvh, n_slots, -1)[:, idx] = a.view(kvh, n_pg, -1)
    del master
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y_pag = decode(sh, [pool], [n], q, n, torch.from_numpy(perm).to(DEV), n_pg, status)
    assert int(status.item()) == 0
    assert np.array_equal(y_pag, y_res)


def test_paged_batch_and_bad_page():
    fmt, kvh, G = kq.KV_FMT_Q8, 8, 4
    say("paged batch")
    lens = [700, 2500, 64, 1999]
    sh = shape(fmt, kvh, G * kvh)
    sessions = [filled(fmt, kvh, 2560, n, 40 + i)[0] for i, n in enumerate(lens)]
    q = kvsynth.queries(41, 0, len(lens), G * kvh, 128)
    max_len = max(lens)
    y_res = decode(sh, sessions, lens, q, max_len)
    stride = (max_len + P - 1) // P
    n_slots = sum((n + P - 1) // P for n in lens) + 7
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)   # NaN where not written
    perm = np.random.default_rng(5).permutation(n_slots).astype(np.int32)
    table = np.zeros((len(lens), stride), np.int32)
    k = 0
    for b, (s, n) in enumerate(zip(sessions, lens)):
        npg = (n + P - 1) // P
        table[b, :npg] = perm[k:k + npg]
        k += npg
        copy_pages(s, pool, table[b], npg)
    pages = torch.from_numpy(table).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    y_pag = decode(sh, [pool] * len(lens), lens, q, max_len, pages, stride, status)
    assert int(status.item()) == 0
    assert np.array_equal(y_pag, y_res)
    # a page outside the pool: flagged, read as slot 0 (in bounds), the others intact
    bad = table.copy()
    bad[1, 3] = n_slots + 5
    status.zero_()
    y_bad = decode(sh, [pool] * len(lens), lens, q, max_len, torch.from_numpy(bad).to(DEV), stride,
                   status)
    assert int(status.item()) & kq.KV_DEV_BAD_PAGE
    assert np.array_equal(y_bad[[0, 2, 3]], y_res[[0, 2, 3]])


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_streamed_window_equals_resident(fmt):
    kvh, G = 4, 4
    say(f"window fmt={fmt}")
    sh = shape(fmt, kvh, G * kvh)
    lens = {0: 2000, 1: 3001, 2: 1300}
    res = {s: filled(fmt, kvh, 3072, n, 50 + s)[0] for s, n in lens.items()}
    # host stores: pinned copies of the sessions
    store = {}
    for s, sess in res.items():
        st = kq.Session(fmt, kvh, 3072, pinned=True)
        for a, b in zip(sess.tensors(), st.tensors()):
            b.copy_(a.cpu())
        store[s] = st
    n_slots = 64                      # fewer than the 32 + 47 + 21 pages of the three
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)   # NaN where not written
    win = kq.Window(n_slots)
    model = kq.Window(n_slots)        # the same plan, host only, to predict the copies
    h_pages = {s: torch.full((48,), -1, dtype=torch.int32).pin_memory() for s in lens}
    m_pages = {s: np.full(48, -1, np.int32) for s in lens}
    d_pages = torch.zeros(48, dtype=torch.int32, device=DEV)
    q = kvsynth.queries(52, 0, 1, G * kvh, 128)
    for s in (0, 1, 0, 2, 1, 1, 0):
        n = lens[s]
        npg = (n + P - 1) // P
        copied = win.map(sh, store[s], s, npg, pool, h_pages[s], d_pages)
        want_missed = model.plan(s, m_pages[s][:npg])
        assert copied == len(want_missed)
        y_win = decode(sh, [pool], [n], q, n, d_pages[:npg].contiguous(), npg)
        y_res = decode(sh, [res[s]], [n], q, n)
        assert np.array_equal(y_win, y_res), s


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_streamed_window_interleaved_without_sync(fmt):
    """Map/decode pairs of three sessions enqueued back to back on one stream, with no
    synchronisation between them: each session's page table is rewritten by its next
    map while earlier copies from it may still be queued (the binding waits for the
    copy that read the table before the table is rewritten).  Every output equals the
    resident decode bit for bit."""
    kvh, G = 4, 4
    say(f"window no-sync fmt={fmt}")
    sh = shape(fmt, kvh, G * kvh)
    lens = {0: 2000, 1: 3001, 2: 1300}
    res = {s: filled(fmt, kvh, 3072, n, 150 + s)[0] for s, n in lens.items()}
    store = {}
    for s, sess in res.items():
        st = kq.Session(fmt, kvh, 3072, pinned=True)
        for a, b in zip(sess.tensors(), st.tensors()):
            b.copy_(a.cpu())
        store[s] = st
    n_slots = 64
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)
    win = kq.Window(n_slots)
    h_pages = {s: torch.full((48,), -1, dtype=torch.int32).pin_memory() for s in lens}
    d_pages = {s: torch.zeros(48, dtype=torch.int32, device=DEV) for s in lens}
    q = kvsynth.queries(152, 0, 1, G * kvh, 128)
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    order = (0, 1, 0, 2, 1, 1, 0, 2, 2, 0, 1)
    max_len = max(lens.values())
    ws = torch.zeros(kq.kv_decode_workspace_bytes(sh, 1, max_len), dtype=torch.uint8, device=DEV)
    tab = kq.session_table([pool.entry()])
    outs = []
    for s in order:
        n = lens[s]
        npg = (n + P - 1) // P
        win.map(sh, store[s], s, npg, pool, h_pages[s], d_pages[s])
        out = torch.empty((1, G * kvh, 128), device=DEV)
        ln = torch.tensor([n], dtype=torch.int32, device=DEV)
        kq.kv_decode_attn_paged(sh, tab, d_pages[s], 48, ln, 1, max_len, qd, sm_scale(), out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    for s, out in zip(order, outs):
        n = lens[s]
        y_res = decode(sh, [res[s]], [n], q, max_len)
        assert np.array_equal(out.cpu().numpy(), y_res), s


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_paged_append_equals_resident(fmt):
    """kv_append_paged writes exactly the rows kv_append writes, into the slots the page
    tables name: three sessions in one call, appends that start mid-page and cross pages,
    every other pool row left as it was; a table entry outside the pool skips its rows
    (flagged), and a session whose pages cannot hold the append is skipped (flagged)."""
    kvh, n_tok = 4, 150
    lens = [0, 100, 1000]
    stride = 20                          # 1280 cells per session
    sh = shape(fmt, kvh, kvh)
    n_slots = 3 * stride + 4
    perm = np.random.default_rng(90 + fmt).permutation(n_slots).astype(np.int32)
    table = perm[:3 * stride].reshape(3, stride).copy()
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0x5A)
    res = [kq.Session(fmt, kvh, stride * P, fill=0x5A) for _ in lens]
    xk = kvsynth.kv_tokens(91, 0, 3 * n_tok, kvh, 128, "K", True).reshape(3, n_tok, kvh, 128)
    xv = kvsynth.kv_tokens(91, 0, 3 * n_tok, kvh, 128, "V", True).reshape(3, n_tok, kvh, 128)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dk = torch.from_numpy(np.ascontiguousarray(xk)).to(DEV)
    dv = torch.from_numpy(np.ascontiguousarray(xv)).to(DEV)
    kq.kv_append_paged(sh, kq.session_table([pool.entry()] * 3), torch.from_numpy(table).to(DEV),
                       stride, ln, 3, n_tok, dk, dv, status)
    kq.kv_append(sh, kq.session_table([s.entry() for s in res]), ln, 3, n_tok, dk, dv, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    touched = np.zeros(n_slots * P, bool)
    for b, n in enumerate(lens):
        for c in range(n, n + n_tok):
            prow = int(table[b, c // P]) * P + c % P
            touched[prow] = True
            for a, d in zip(res[b].tensors(), pool.tensors()):
                assert torch.equal(a[:, c], d[:, prow]), (b, c)
    untouched = torch.from_numpy(np.flatnonzero(~touched)).to(DEV)
    for d in pool.tensors():
        assert bool((d.view(torch.uint8).view(kvh, n_slots * P, -1)[:, untouched] == 0x5A).all())
    # a page outside the pool: its rows skipped and flagged, the other rows written
    bad = table.copy()
    bad[1, 2] = n_slots + 9                     # cells 128 .. 191 of session 1
    pool2 = kq.Session(fmt, kvh, n_slots * P, fill=0x5A)
    status.zero_()
    kq.kv_append_paged(sh, kq.session_table([pool2.entry()] * 3), torch.from_numpy(bad).to(DEV),
                       stride, ln, 3, n_tok, dk, dv, status)
    torch.cuda.synchronize()
    assert int(status.item()) == kq.KV_DEV_BAD_PAGE
    for a, d in zip(pool.tensors(), pool2.tensors()):
        row = int(table[1, 1]) * P + 100 % P    # cell 100 of session 1, a good page
        assert torch.equal(a[:, row], d[:, row])
    # more cells than the pages hold: the session is skipped whole
    status.zero_()
    pool3 = kq.Session(fmt, kvh, n_slots * P, fill=0x5A)
    ln3 = torch.tensor([stride * P - 10], dtype=torch.int32, device=DEV)
    kq.kv_append_paged(sh, kq.session_table([pool3.entry()]), torch.from_numpy(table[:1].copy()).to(DEV),
                       stride, ln3, 1, 11, dk[:1, :11].contiguous(), dv[:1, :11].contiguous(), status)
    torch.cuda.synchronize()
    assert int(status.item()) == kq.KV_DEV_RANGE
    for d in pool3.tensors():
        assert bool((d.view(torch.uint8) == 0x5A).all())
