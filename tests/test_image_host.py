"""The saved-image calls of the C ABI on the host, against the oracle's images.

Header checks, sizes and refusals need no GPU: kv_image_tokens reads only the host
image, and kv_image_save / kv_image_load with zero tokens, or with arguments they
refuse, return before any copy is enqueued.  Session pointers are fake and aligned.
"""
import ctypes

import numpy as np

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from oracle import kvq8_oracle as o

L = kq.raw_lib()
A = 0x7F0000000000
FMTS = (o.FMT_F16, o.FMT_Q8, o.FMT_K8V4)


def filled(fmt, kvh=3, cap=128, n=45, seed=67):
    c = oracle.Cache(fmt, kvh, cap, 128)
    if n:
        assert c.append(0, kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True),
                        kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True))
    return c


def fake_sess(fmt, cap=128):
    sc = fmt != o.FMT_F16
    return kq.kv_session(A, A + 0x100000, A + 0x200000 if sc else None,
                         A + 0x300000 if sc else None, cap, 0)


def buf(b):
    return ctypes.create_string_buffer(bytes(b), len(b))


def tokens_of(img, shape):
    b = buf(img)
    return L.kv_image_tokens(ctypes.byref(shape), b, len(img))


def test_image_bytes_match_oracle():
    for fmt in FMTS:
        sh = kq.make_shape(fmt, 3, 6)
        for n in (0, 1, 45, 128):
            c = filled(fmt, n=n)
            assert kq.kv_image_bytes(sh, n) == len(o.save_image(c, n, np.arange(n))), (fmt, n)
    assert kq.kv_image_bytes(kq.make_shape(7, 3, 6), 4) == 0
    assert kq.kv_image_bytes(kq.make_shape(o.FMT_Q8, 3, 6), -1) == 0


def test_header_reading_accepts_oracle_images_and_refuses_the_rest():
    r = np.random.default_rng(5)
    for fmt in FMTS:
        sh = kq.make_shape(fmt, 3, 6)
        c = filled(fmt)
        img = o.save_image(c, 45, r.integers(0, 1 << 20, 45))
        assert tokens_of(img, sh) == 45
        assert tokens_of(img + b"\0" * 7, sh) == 45          # a longer buffer is fine
        E = kq.KV_ERR_IMAGE
        assert tokens_of(img[:-1], sh) == E                    # short
        assert tokens_of(img[:100], sh) == E                   # shorter than a header
        assert tokens_of(b"KVQ9" + img[4:], sh) == E           # magic
        v2 = img[:4] + (2).to_bytes(4, "little") + img[8:]
        assert tokens_of(v2, sh) == (45 if fmt == o.FMT_F16 else E)   # v2: FP16 only
        v4 = img[:4] + (4).to_bytes(4, "little") + img[8:]
        assert tokens_of(v4, sh) == E                          # unknown version
        assert tokens_of(img, kq.make_shape((fmt + 1) % 3, 3, 6)) == E
        assert tokens_of(img, kq.make_shape(fmt, 1, 2)) == E   # other kv heads
        bad_body = img[:24] + (1).to_bytes(8, "little") + img[32:]
        assert tokens_of(bad_body, sh) == E                    # sizes do not match the shape
    assert L.kv_image_tokens(ctypes.byref(kq.make_shape(o.FMT_Q8, 3, 6)), None, 128) == kq.KV_ERR_ARG


def test_empty_save_writes_the_oracle_header():
    for fmt in FMTS:
        sh = kq.make_shape(fmt, 3, 6)
        want = o.save_image(filled(fmt, n=0), 0, np.zeros(0, np.int32))
        b = ctypes.create_string_buffer(b"\xAA" * 200, 200)
        s = fake_sess(fmt)
        assert L.kv_image_save(ctypes.byref(sh), ctypes.byref(s), 0, None, b, 200, None) == kq.KV_OK
        assert b.raw[:128] == want and b.raw[128:] == b"\xAA" * 72, fmt


def test_save_and_load_validation():
    sh = kq.make_shape(o.FMT_Q8, 3, 6)
    s = fake_sess(o.FMT_Q8)
    img = o.save_image(filled(o.FMT_Q8), 45, np.arange(45))
    b = buf(img)
    tok = (ctypes.c_int32 * 45)()
    save = lambda n, size, t=tok, e=s, sh=sh: L.kv_image_save(  # noqa: E731
        ctypes.byref(sh), ctypes.byref(e), n, t, b, size, None)
    load = lambda im, size, e=s, sh=sh: L.kv_image_load(  # noqa: E731
        ctypes.byref(sh), ctypes.byref(e), im, size, tok, None)
    assert save(45, len(img) - 1) == kq.KV_ERR_ARG          # image too small
    assert save(129, 1 << 20) == kq.KV_ERR_RANGE            # past the capacity
    assert save(-1, len(img)) == kq.KV_ERR_ARG
    assert save(45, len(img), t=None) == kq.KV_ERR_ARG      # tokens missing
    assert save(1, len(img), e=fake_sess(o.FMT_F16)) == kq.KV_ERR_FMT
    assert L.kv_image_save(ctypes.byref(sh), ctypes.byref(s), 0, None, None, 128, None) == kq.KV_ERR_ARG
    assert load(buf(img[:-1]), len(img) - 1) == kq.KV_ERR_IMAGE
    v2 = img[:4] + (2).to_bytes(4, "little") + img[8:]
    assert load(buf(v2), len(img)) == kq.KV_ERR_IMAGE              # int8 cache from a v2 image
    big = o.save_image(filled(o.FMT_Q8, cap=192, n=130), 130, np.arange(130))
    assert load(buf(big), len(big)) == kq.KV_ERR_RANGE             # 130 tokens, capacity 128
    assert load(None, len(img)) == kq.KV_ERR_ARG
    empty = o.save_image(filled(o.FMT_Q8, n=0), 0, [])
    assert load(buf(empty), len(empty)) == 0                        # nothing to copy
