"""The calls inside a captured HIP graph: a decode step (one-token append, then
decode, for two layers of each format) captured once and replayed several times,
with eager work and synchronisation between replays; every replay must equal the
same step run eagerly, bit for bit.  (The calls allocate and clear nothing, so they
capture as plain kernel nodes.)"""
import numpy as np
import pytest
import torch

import kvsynth
import quantized_kv_cache_q8_amd as kq
from gpu_util import DEV, append_bulk, say, shape, sm_scale

pytestmark = pytest.mark.gpu


def make(fmt, kvh, nqh, cap, n, seed):
    xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True)
    s = kq.Session(fmt, kvh, cap)
    assert append_bulk(shape(fmt, kvh, nqh), [s], [0], xk[None], xv[None]) == 0
    return s


def test_step_graph_replays_equal_eager():
    kvh, nqh, n, steps = 2, 8, 3000, 3
    cap = kvsynth.round_up(n + steps + 8, 64)
    fmts = [kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4]
    layers = [(fmt, li) for fmt in fmts for li in range(2)]
    graph_s = {k: make(k[0], kvh, nqh, cap, n, 70 + 10 * k[0] + k[1]) for k in layers}
    eager_s = {k: make(k[0], kvh, nqh, cap, n, 70 + 10 * k[0] + k[1]) for k in layers}
    q = {k: torch.from_numpy(kvsynth.queries(71 + k[1], 0, 1, nqh, 128)).to(DEV) for k in layers}
    xk = torch.from_numpy(kvsynth.kv_tokens(72, 0, steps, kvh, 128, "K", True)).to(DEV)
    xv = torch.from_numpy(kvsynth.kv_tokens(72, 0, steps, kvh, 128, "V", True)).to(DEV)
    max_len = cap
    ws = {k: kq.kv_decode_workspace(shape(k[0], kvh, nqh), 1, max_len, DEV) for k in layers}

    def step(sess, tabs, lens_w, lens_d, xk1, xv1, outs):
        for k in layers:
            sh = shape(k[0], kvh, nqh)
            kq.kv_append(sh, tabs[k], lens_w, 1, 1, xk1, xv1)
            kq.kv_decode_attn(sh, tabs[k], lens_d, 1, max_len, q[k], sm_scale(), outs[k], ws[k])
        lens_w += 1
        lens_d += 1

    g_tabs = {k: kq.session_table([graph_s[k].entry()]) for k in layers}
    e_tabs = {k: kq.session_table([eager_s[k].entry()]) for k in layers}
    g_lw = torch.full((1,), n, dtype=torch.int32, device=DEV)
    g_ld = g_lw + 1
    g_out = {k: torch.zeros((1, nqh, 128), device=DEV) for k in layers}
    g_xk = torch.empty((1, 1, kvh, 128), device=DEV)
    g_xv = torch.empty_like(g_xk)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            step(graph_s, g_tabs, g_lw, g_ld, g_xk, g_xv, g_out)
    torch.cuda.synchronize()
    # capture runs nothing: the cells and the lengths are as before
    assert g_lw.item() == n
    e_lw = torch.full((1,), n, dtype=torch.int32, device=DEV)
    e_ld = e_lw + 1
    e_out = {k: torch.zeros((1, nqh, 128), device=DEV) for k in layers}
    for t in range(steps):
        say(f"graph replay {t}")
        g_xk.copy_(xk[t].view(1, 1, kvh, 128))
        g_xv.copy_(xv[t].view(1, 1, kvh, 128))
        graph.replay()
        torch.cuda.synchronize()
        step(eager_s, e_tabs, e_lw, e_ld, xk[t].view(1, 1, kvh, 128).contiguous(),
             xv[t].view(1, 1, kvh, 128).contiguous(), e_out)
        torch.cuda.synchronize()
        assert g_lw.item() == e_lw.item() == n + t + 1
        for k in layers:
            assert torch.equal(g_out[k], e_out[k]), (k, t)
            assert torch.isfinite(g_out[k]).all()
    for k in layers:
        for a, b in zip(graph_s[k].tensors(), eager_s[k].tensors()):
            assert torch.equal(a, b), k
