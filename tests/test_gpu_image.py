"""Saved session images on the GPU: the image built from a GPU cache equals the
oracle's image byte for byte; an oracle image loaded into a fresh session gives the
oracle's rows and leaves the rest untouched; and a second turn that continues a
loaded session (append, then decode) equals one that never left the GPU, bit for bit
(the warm-turn check of the Path F v3 issue, section Phased plan)."""
import numpy as np
import pytest
import torch

import kvsynth
from oracle import kvq8_oracle as o
import quantized_kv_cache_q8_amd as kq
from gpu_util import (append_bulk, assert_cache_equal, decode_gpu, download, oracle_cache, say,
                      shape, sm_scale)

pytestmark = pytest.mark.gpu
FMTS = [kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4]


def tokens_k(seed, n, kvh):
    return (kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True),
            kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True))


@pytest.mark.parametrize("fmt", FMTS)
def test_image_save_load(fmt):
    kvh, cap, n_fill, n = 4, 1024, 1000, 777
    say(f"image fmt={fmt}")
    xk, xv = tokens_k(67, n_fill, kvh)
    s = kq.Session(fmt, kvh, cap, fill=0)
    sh = shape(fmt, kvh, 2 * kvh)
    assert append_bulk(sh, [s], [0], xk[None], xv[None]) == 0
    ref = oracle_cache(fmt, kvh, cap, 128, xk, xv)
    toks = np.random.default_rng(3).integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    want = o.save_image(ref, n, toks)
    size = kq.kv_image_bytes(sh, n)
    assert size == len(want)
    img = torch.full((size + 64,), 0xA5, dtype=torch.uint8).pin_memory()
    kq.kv_image_save(sh, s.entry(), n, torch.from_numpy(toks), img)
    torch.cuda.synchronize()
    got = img.numpy()
    assert got[:size].tobytes() == want
    assert (got[size:] == 0xA5).all()
    # load the oracle's image into a fresh, larger session
    src = torch.frombuffer(bytearray(want), dtype=torch.uint8).pin_memory()
    t = kq.Session(fmt, kvh, 2048, fill=0x5A)
    before = download(t)
    out = torch.zeros(n, dtype=torch.int32)
    assert kq.kv_image_load(sh, t.entry(), src, out) == n
    torch.cuda.synchronize()
    assert np.array_equal(out.numpy(), toks)
    assert_cache_equal(t, ref, rows=slice(0, n))
    after = download(t)
    for name in after:
        assert np.array_equal(after[name][:, n:], before[name][:, n:]), name
    # an image of another format is refused, and nothing is copied
    other = shape((fmt + 1) % 3, kvh, 2 * kvh)
    with pytest.raises(kq.KvError):
        kq.kv_image_tokens(other, src)


@pytest.mark.parametrize("fmt", FMTS)
def test_second_turn_from_an_image(fmt):
    kvh, cap, n1, n2 = 8, 4096, 2500, 300
    say(f"image second turn fmt={fmt}")
    sh = shape(fmt, kvh, 8 * kvh)
    xk1, xv1 = tokens_k(68, n1, kvh)
    xk2, xv2 = tokens_k(69, n2, kvh)
    # the session that stays on the GPU
    a = kq.Session(fmt, kvh, cap, fill=0)
    assert append_bulk(sh, [a], [0], xk1[None], xv1[None]) == 0
    img = torch.empty(kq.kv_image_bytes(sh, n1), dtype=torch.uint8).pin_memory()
    kq.kv_image_save(sh, a.entry(), n1, torch.arange(n1, dtype=torch.int32), img)
    torch.cuda.synchronize()
    # turn 2: a fresh session hydrated from the image, then both continue
    b = kq.Session(fmt, kvh, cap, fill=0x77)
    assert kq.kv_image_load(sh, b.entry(), img) == n1
    assert append_bulk(sh, [a], [n1], xk2[None], xv2[None]) == 0
    assert append_bulk(sh, [b], [n1], xk2[None], xv2[None]) == 0
    torch.cuda.synchronize()
    da, db = download(a), download(b)
    for name in da:
        assert np.array_equal(da[name][:, :n1 + n2], db[name][:, :n1 + n2]), name
    q = kvsynth.queries(68, 0, 1, 8 * kvh, 128)
    ya = decode_gpu(sh, [a], [n1 + n2], q, sm_scale())
    yb = decode_gpu(sh, [b], [n1 + n2], q, sm_scale())
    assert np.array_equal(ya, yb)
