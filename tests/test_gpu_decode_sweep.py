"""A seeded sweep of decode configurations against the fp64 oracle: every format, 1, 2,
4 or 8 query heads per kv head, 1 to 4 kv heads, batches of 1 to 4 sessions with
ragged lengths (empty, one cell, ends inside a step, a split and a chunk, several
thousand cells), each output within 2e-3 + 1e-3 |ref| and within the fidelity gate."""
import numpy as np
import pytest

import kvsynth
import quantized_kv_cache_q8_amd as kq
from gpu_util import check_close, check_fidelity, decode_gpu, say, shape, sm_scale
from test_gpu_decode import filled, oracle_decode

pytestmark = pytest.mark.gpu
F16, Q8, K4 = kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4


def _configs(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = (F16, Q8, K4)[i % 3]
        G = (1, 2, 4, 8)[(i // 3) % 4]
        kvh = int(rng.choice([1, 2, 4]))
        n_sess = int(rng.integers(1, 5))
        lens = []
        for _ in range(n_sess):
            kind = rng.integers(0, 6)
            if kind == 0:
                lens.append(int(rng.choice([0, 1, 7, 8, 9])))
            elif kind == 1:
                lens.append(int(rng.integers(10, 600)))
            else:
                lens.append(int(rng.integers(600, 6000)))
        out.append((fmt, G, kvh, lens))
    return out


@pytest.mark.parametrize("idx,cfg", list(enumerate(_configs(24))))
def test_decode_sweep(idx, cfg):
    fmt, G, kvh, lens = cfg
    nqh = kvh * G
    cap = max(64, (max(lens) + 63) // 64 * 64)
    say(f"sweep {idx}: fmt={fmt} G={G} kvh={kvh} lens={lens}")
    sess, refs = [], []
    for b, n in enumerate(lens):
        s, ref = filled(fmt, kvh, cap, max(n, 1), 900 + idx, outliers=bool(b % 2), layer=b)
        sess.append(s)
        refs.append(ref)
    q = kvsynth.queries(900 + idx, 0, len(lens), nqh, 128)
    got = decode_gpu(shape(fmt, kvh, nqh), sess, lens, q, sm_scale())
    for b, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(got[b], np.zeros_like(got[b])), "an empty session decodes to 0"
            continue
        want, absv = oracle_decode(refs[b], q[b], n, sm_scale(), with_abs=True)
        check_close(got[b], want, f"session {b} len={n}")
        check_fidelity(got[b], want, absv, f"session {b} len={n}")
