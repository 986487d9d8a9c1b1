"""The packed row block of the oracle (moving a session's rows) against the byte
accounting pinned to the pages, a round trip, and the C library's block size."""
import numpy as np

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from oracle import kvq8_oracle as o

FMTS = (o.FMT_F16, o.FMT_Q8, o.FMT_K8V4)


def filled(fmt, kvh=3, cap=128, n=100, seed=90):
    c = oracle.Cache(fmt, kvh, cap, 128)
    xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True)
    assert c.append(0, xk, xv)
    return c


def test_block_size_is_the_byte_accounting():
    # n rows of a session are n cells: the block holds exactly the arrays' bytes for
    # a cache of n cells (the accounting the pages' GiB figures pin), nothing sized in
    # fp32 elements and no array left out
    for fmt in FMTS:
        c = filled(fmt)
        for row0, n in ((0, 1), (7, 33), (0, 100)):
            blk = o.pack_rows(c, row0, n)
            assert blk.size == sum(o.cache_bytes(fmt, 3, n, 128, p) for p in range(4)), fmt


def test_round_trip_and_order():
    for fmt in FMTS:
        c = filled(fmt)
        blk = o.pack_rows(c, 20, 50)
        d = oracle.Cache(fmt, 3, 256, 128)
        o.unpack_rows(d, 100, 50, blk)
        for a in o.ROW_ARRAYS:
            if getattr(c, a) is not None:
                assert np.array_equal(getattr(d, a)[:, 100:150], getattr(c, a)[:, 20:70]), (fmt, a)
                assert not getattr(d, a)[:, :100].any() and not getattr(d, a)[:, 150:].any()
        # K values come first, one head's rows after another
        assert np.array_equal(blk[:c.k[0, 20:70].nbytes], c.k[0, 20:70].view(np.uint8).reshape(-1))


def test_library_block_size_matches():
    for fmt in FMTS:
        c = filled(fmt)
        sh = kq.make_shape(fmt, 3, 12, 128)
        for n in (0, 1, 33):
            assert kq.kv_rows_bytes(sh, n) == o.pack_rows(c, 0, n).size
