"""Streamed sessions that grow (PR #711 "kv: --kv k8v4 streams with --kv-resident":
section How, the decode appends write the streamed state's pool and host copy; section
Tests, streamed and resident attention bitwise equal over many batches, with block
lookups and misses counted).

Five sessions live in pinned host stores behind a window smaller than their sum.  Each
of several hundred steps picks one session, maps its pages (kv_window_map), appends one
token into its pool slot (kv_append_paged), writes the new row back to the host store
(kv_window_writeback) and decodes over the pages (kv_decode_attn_paged); a resident
twin of the session gets the same append (kv_append) and decode (kv_decode_attn).  Every
decode must equal its twin's bit for bit; the test stops at the first that does not.
At the end every host store must equal its resident twin byte for byte."""
import numpy as np
import pytest
import torch

import kvsynth
import quantized_kv_cache_q8_amd as kq
from gpu_util import DEV, append_bulk, say, shape, sm_scale

pytestmark = pytest.mark.gpu
P = kq.KV_PAGE_ROWS


@pytest.mark.parametrize("fmt", [kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4])
def test_streamed_sessions_grow_bitwise(fmt):
    kvh, G, n_sess, steps = 4, 4, 5, 300
    sh = shape(fmt, kvh, G * kvh)
    r = np.random.default_rng(200 + fmt)
    lens = [int(x) for x in r.integers(2500, 9000, size=n_sess)]
    cap = kvsynth.round_up(max(lens) + steps, P)
    stride = cap // P
    res, store = [], []
    for s in range(n_sess):
        xk = kvsynth.kv_tokens(210 + s, 0, lens[s], kvh, 128, "K", outliers=True)
        xv = kvsynth.kv_tokens(210 + s, 0, lens[s], kvh, 128, "V", outliers=True)
        ses = kq.Session(fmt, kvh, cap, fill=0)
        assert append_bulk(shape(fmt, kvh, kvh), [ses], [0], xk[None], xv[None]) == 0
        st = kq.Session(fmt, kvh, cap, pinned=True)
        for a, b in zip(ses.tensors(), st.tensors()):
            b.copy_(a.cpu())
        res.append(ses)
        store.append(st)
    total_pages = sum((n + steps + P - 1) // P for n in lens)
    max_pages = max((n + steps + P - 1) // P for n in lens)
    n_slots = max(max_pages + 8, 3 * total_pages // 4)   # room for any one session, not all
    assert n_slots < total_pages
    say(f"stream grow fmt={fmt}: {n_sess} sessions, lengths {lens}, {total_pages} pages, "
        f"{n_slots} slots")
    pool = kq.Session(fmt, kvh, n_slots * P, fill=0xFF)   # NaN where not written
    win = kq.Window(n_slots)
    h_pages = [torch.full((stride,), -1, dtype=torch.int32).pin_memory() for _ in range(n_sess)]
    d_pages = [torch.zeros(stride, dtype=torch.int32, device=DEV) for _ in range(n_sess)]
    tab_pool = kq.session_table([pool.entry()])
    tab_res = [kq.session_table([s.entry()]) for s in res]
    ws_p = torch.zeros(kq.kv_decode_workspace_bytes(sh, 1, cap), dtype=torch.uint8, device=DEV)
    ws_r = torch.zeros_like(ws_p)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    lookups = misses = 0
    for step in range(steps):
        s = int(r.integers(0, n_sess))
        n = lens[s]
        npg = (n + 1 + P - 1) // P
        misses += win.map(sh, store[s], s, npg, pool, h_pages[s], d_pages[s])
        lookups += npg
        xk = torch.from_numpy(kvsynth.kv_tokens(220 + s, 0, 1, kvh, 128, "K", True,
                                                stream=kvsynth.S_K_NEW, sub=step)[None]).to(DEV)
        xv = torch.from_numpy(kvsynth.kv_tokens(220 + s, 0, 1, kvh, 128, "V", True,
                                                stream=kvsynth.S_V_NEW, sub=step)[None]).to(DEV)
        ln = torch.tensor([n], dtype=torch.int32, device=DEV)
        kq.kv_append_paged(sh, tab_pool, d_pages[s], stride, ln, 1, 1, xk, xv, status)
        win.writeback(sh, store[s], s, n, 1, pool, h_pages[s])
        kq.kv_append(sh, tab_res[s], ln, 1, 1, xk, xv, status)
        q = torch.from_numpy(kvsynth.queries(230 + s, 0, 1, G * kvh, 128, sub=step)).to(DEV)
        ln1 = torch.tensor([n + 1], dtype=torch.int32, device=DEV)
        y_p = torch.empty((1, G * kvh, 128), device=DEV)
        y_r = torch.empty_like(y_p)
        kq.kv_decode_attn_paged(sh, tab_pool, d_pages[s], stride, ln1, 1, cap, q, sm_scale(), y_p,
                                ws_p, status)
        kq.kv_decode_attn(sh, tab_res[s], ln1, 1, cap, q, sm_scale(), y_r, ws_r, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"step {step}: status {int(status.item())}"
        assert torch.equal(y_p, y_r), f"step {step}: session {s} at {n + 1} cells differs"
        lens[s] = n + 1
    say(f"  {steps} decodes bitwise equal; {lookups} page lookups, {misses} misses "
        f"({misses / lookups:.1%})")
    assert 0 < misses < lookups
    # the host stores kept every appended row: equal to the resident twins
    torch.cuda.synchronize()
    for s in range(n_sess):
        for a, b in zip(res[s].tensors(), store[s].tensors()):
            assert torch.equal(a[:, :lens[s]].cpu(), b[:, :lens[s]]), f"store of session {s}"
