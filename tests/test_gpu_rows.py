"""Moving a session's rows on the GPU: gather to device and pinned host memory,
scatter back, copy between sessions; bytes equal the oracle's packed block, rows
outside the range untouched, and a decode over moved rows equals one over the
originals bit for bit."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from oracle import kvq8_oracle as o
from gpu_util import (DEV, append_bulk, assert_cache_equal, decode_gpu, download, oracle_cache,
                      say, shape, sm_scale)

pytestmark = pytest.mark.gpu
FMTS = [kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4]


def filled(fmt, kvh, cap, n, seed):
    xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True)
    s = kq.Session(fmt, kvh, cap, fill=0)
    assert append_bulk(shape(fmt, kvh, kvh), [s], [0], xk[None], xv[None]) == 0
    return s, oracle_cache(fmt, kvh, cap, 128, xk, xv)


@pytest.mark.parametrize("fmt", FMTS)
def test_gather_scatter_copy(fmt):
    kvh, cap, n = 4, 1024, 1000
    say(f"rows fmt={fmt}")
    s, ref = filled(fmt, kvh, cap, n, 91)
    sh = shape(fmt, kvh, 4 * kvh)
    row0, m = 137, 600
    nbytes = kq.kv_rows_bytes(sh, m)
    want = o.pack_rows(ref, row0, m)
    assert nbytes == want.size
    # gather to device memory and to pinned host memory
    dbuf = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    kq.kv_gather_rows(sh, s.entry(), row0, m, dbuf)
    hbuf = torch.full((nbytes,), 0xA5, dtype=torch.uint8).pin_memory()
    kq.kv_gather_rows(sh, s.entry(), row0, m, hbuf)
    torch.cuda.synchronize()
    assert np.array_equal(dbuf.cpu().numpy(), want)
    assert np.array_equal(hbuf.numpy(), want)
    # scatter the host block into another session (other capacity), at another row
    t = kq.Session(fmt, kvh, 2048, fill=0x5A)
    before = download(t)
    kq.kv_scatter_rows(sh, t.entry(), 1400, m, hbuf)
    torch.cuda.synchronize()
    exp = oracle.Cache(fmt, kvh, 2048, 128)
    o.unpack_rows(exp, 1400, m, want)
    assert_cache_equal(t, exp, rows=slice(1400, 1400 + m))
    after = download(t)
    for name in after:
        for rows in (slice(0, 1400), slice(1400 + m, 2048)):
            assert np.array_equal(after[name][:, rows], before[name][:, rows]), name
    # device copy of the whole filled range into a third session; a decode over it
    # equals the decode over the original, bit for bit
    u = kq.Session(fmt, kvh, 1024, fill=0x33)
    kq.kv_copy_rows(sh, s.entry(), 0, u.entry(), 0, n)
    torch.cuda.synchronize()
    assert_cache_equal(u, ref, rows=slice(0, n))
    q = kvsynth.queries(91, 0, 1, 4 * kvh, 128)
    a = decode_gpu(sh, [s], [n], q, sm_scale())
    b = decode_gpu(sh, [u], [n], q, sm_scale())
    assert np.array_equal(a, b)
