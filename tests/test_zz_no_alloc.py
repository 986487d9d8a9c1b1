"""kv_decode_attn_static (the decode with the library's fixed per-device scratch,
for callers that cannot allocate) against kv_decode_attn with a caller workspace:
bitwise equal outputs on two calls in a row, the second smaller than the first,
and a call whose partials exceed the scratch refused with KV_ERR_WORKSPACE."""
import numpy as np
import pytest
import torch

import kvsynth
import quantized_kv_cache_q8_amd as kq
from gpu_util import DEV, append_bulk, say, shape, sm_scale, to_dev

pytestmark = pytest.mark.gpu


def session(fmt, kvh, cap, n, seed):
    xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True)
    s = kq.Session(fmt, kvh, cap)
    assert append_bulk(shape(fmt, kvh, kvh), [s], [0], xk[None], xv[None], chunk=65536) == 0
    return s


def both(sh, sessions, lens, q):
    n = len(sessions)
    tab = kq.session_table([s.entry() for s in sessions])
    ln = to_dev(np.asarray(lens, np.int32))
    max_len = int(max(lens))
    qd = to_dev(q)
    ref = torch.full((n, sh.n_q_heads, 128), float("nan"), device=DEV)
    got = torch.full((n, sh.n_q_heads, 128), float("nan"), device=DEV)
    ws = torch.empty(kq.kv_decode_workspace_bytes(sh, n, max_len), dtype=torch.uint8, device=DEV)
    assert ws.numel() <= kq.KV_DECODE_STATIC_WS_BYTES
    st_ref = torch.zeros(1, dtype=torch.int32, device=DEV)
    st_got = torch.zeros(1, dtype=torch.int32, device=DEV)
    kq.kv_decode_attn(sh, tab, ln, n, max_len, qd, sm_scale(), ref, ws, st_ref)
    kq.kv_decode_attn_static(sh, tab, ln, n, max_len, qd, sm_scale(), got, st_got)
    torch.cuda.synchronize()
    assert int(st_ref.item()) == int(st_got.item()) == 0
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("fmt", [kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4])
def test_static_scratch_decode_equals_workspace_decode(fmt):
    kvh, G = 8, 4
    sh = shape(fmt, kvh, kvh * G)
    say(f"static scratch fmt={fmt}: first call, 16 sessions up to 32768 cells")
    big = session(fmt, kvh, 32768, 32768, 91)
    lens = [32768, 30000, 1, 65, 12345, 32767, 64, 20000, 32768, 9, 4096, 777, 31000, 2, 16000, 8]
    q1 = kvsynth.queries(92, 0, len(lens), kvh * G, 128)
    ref, got = both(sh, [big] * len(lens), lens, q1)
    assert np.array_equal(got, ref)
    say(f"static scratch fmt={fmt}: second call, 2 sessions of at most 3000 cells")
    small = session(fmt, kvh, 3008, 3000, 93)
    q2 = kvsynth.queries(94, 0, 2, kvh * G, 128)
    ref2, got2 = both(sh, [small, big], [3000, 2999], q2)
    assert np.array_equal(got2, ref2)


def test_static_scratch_too_small_is_refused():
    kvh, G = 8, 4
    sh = shape(kq.KV_FMT_Q8, kvh, kvh * G)
    n_sess, max_len = 4096, 65536
    assert kq.kv_decode_workspace_bytes(sh, n_sess, max_len) > kq.KV_DECODE_STATIC_WS_BYTES
    s = kq.Session(kq.KV_FMT_Q8, kvh, 64)
    tab = kq.session_table([s.entry()] * n_sess)
    ln = torch.zeros(n_sess, dtype=torch.int32, device=DEV)
    q = torch.zeros((n_sess, kvh * G, 128), device=DEV)
    out = torch.full((n_sess, kvh * G, 128), 5.0, device=DEV)
    with pytest.raises(kq.KvError) as e:
        kq.kv_decode_attn_static(sh, tab, ln, n_sess, max_len, q, sm_scale(), out)
    assert e.value.status == kq.KV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())     # nothing was enqueued
