"""A seeded sweep of prompt-chunk configurations against the oracle: every format,
1, 2, 4 or 8 query heads per kv head, chunks from 1 to ~700 tokens at positions from 0
to ~3000 (ragged query blocks and key tiles), within 2e-3 + 1e-3 |ref|."""
import numpy as np
import pytest

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from gpu_util import check_close, say, sm_scale
from test_gpu_prefill import build, run_prefill

pytestmark = pytest.mark.gpu
F16, Q8, K4 = kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4


def _configs(n, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = (F16, Q8, K4)[i % 3]
        G = (1, 2, 4, 8)[(i // 3) % 4]
        kvh = int(rng.choice([1, 2]))
        pos0 = int(rng.choice([0, int(rng.integers(1, 64)), int(rng.integers(64, 3000))]))
        n_tok = int(rng.choice([1, int(rng.integers(2, 65)), int(rng.integers(65, 700))]))
        out.append((fmt, G, kvh, pos0, n_tok))
    return out


@pytest.mark.parametrize("idx,cfg", list(enumerate(_configs(12))))
def test_prefill_sweep(idx, cfg):
    fmt, G, kvh, pos0, n_tok = cfg
    nqh = kvh * G
    P = pos0 + n_tok
    say(f"prefill sweep {idx}: fmt={fmt} G={G} kvh={kvh} pos0={pos0} n_tok={n_tok}")
    s, ref = build(fmt, kvh, P, kvsynth.round_up(P + 1, 64), 700 + idx, outliers=bool(idx % 2))
    q = kvsynth.queries(700 + idx, 0, n_tok, nqh, 128, stream=kvsynth.S_Q_PREFILL)
    got = run_prefill(fmt, s, kvh, nqh, pos0, n_tok, q, sm_scale())
    k16, v16 = oracle.compact_f16(ref, P)
    want = oracle.prefill_attn(q, k16, v16, pos0, sm_scale())
    check_close(got, want, "prefill")
