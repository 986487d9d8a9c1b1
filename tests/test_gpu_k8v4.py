"""The K8V4 format (int8 K, Walsh-Hadamard-rotated 4-bit V) written and read on the
GPU against the oracle: codes, nibbles and scales bit for bit, nothing outside the
written rows touched; decode over a deep cache and a batch within
|gpu - ref| <= 2e-3 + 1e-3 |ref|.  (Every head ratio, compaction and the prompt chunk
run in test_gpu_decode.py and test_gpu_prefill.py with the other formats.)"""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from gpu_util import (append_bulk, assert_cache_equal, check_close, decode_gpu, download,
                      oracle_cache, say, shape, sm_scale)
from test_gpu_decode import oracle_decode

pytestmark = pytest.mark.gpu
K4 = kq.KV_FMT_K8V4


def inputs(seed, n, kvh):
    xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", outliers=True)
    xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", outliers=True)
    xv[5] *= np.float32(1e-6)      # tiny rows: subnormal fp16 scales after the rotation
    xk[7] *= np.float32(1e-6)
    xv[6] = 0                      # an all-zero row: zero scales, code 0
    xv[9, :, 17] = np.float32(3e4)  # one large value: its block clamps nothing, others shrink
    return xk, xv


def test_append_bitexact_bulk_and_token_by_token():
    kvh, n, cap = 8, 3000, 3072
    say(f"k8v4 append kvh={kvh} n={n}")
    xk, xv = inputs(61, n, kvh)
    ref = oracle_cache(K4, kvh, cap, 128, xk, xv)
    sh = shape(K4, kvh, 32)
    s1 = kq.Session(K4, kvh, cap, fill=0)
    assert append_bulk(sh, [s1], [0], xk[None], xv[None]) == 0
    assert_cache_equal(s1, ref)
    s2 = kq.Session(K4, kvh, cap, fill=0)
    assert append_bulk(sh, [s2], [0], xk[None, :150], xv[None, :150], chunk=1) == 0
    assert_cache_equal(s2, ref, rows=slice(0, 150))


def test_append_at_an_offset_touches_only_its_rows():
    kvh, cap, pos, n = 2, 256, 100, 37
    xk, xv = inputs(63, n, kvh)
    s = kq.Session(K4, kvh, cap, fill=0x5A)
    before = download(s)
    assert append_bulk(shape(K4, kvh, 8), [s], [pos], xk[None], xv[None]) == 0
    ref = oracle.Cache(K4, kvh, cap, 128)
    assert ref.append(pos, xk, xv)
    assert_cache_equal(s, ref, rows=slice(pos, pos + n))
    after = download(s)
    for name in after:
        for rows in (slice(0, pos), slice(pos + n, cap)):
            assert np.array_equal(after[name][:, rows], before[name][:, rows]), name


def test_decode_32768_cells_and_a_batch():
    kvh, nqh = 8, 32
    n = 32768
    say("k8v4 decode 32768 cells: fill")
    xk, xv = inputs(64, n, kvh)
    ref = oracle_cache(K4, kvh, n, 128, xk, xv)
    s = kq.Session(K4, kvh, n)
    assert append_bulk(shape(K4, kvh, nqh), [s], [0], xk[None], xv[None], chunk=8192) == 0
    q = kvsynth.queries(64, 0, 3, nqh, 128)
    lens = [n, 1, 20000]
    say("k8v4 decode 32768 cells: batch of 3 lengths")
    got = decode_gpu(shape(K4, kvh, nqh), [s, s, s], lens, q, sm_scale())
    for b, length in enumerate(lens):
        check_close(got[b], oracle_decode(ref, q[b], length, sm_scale()), f"len={length}")
