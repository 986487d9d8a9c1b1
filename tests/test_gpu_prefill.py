"""kv_compact_f16 (bit-exact) and kv_prefill_attn (MFMA) on the GPU against the
oracle: compaction bit for bit, prompt-chunk attention within 2e-3 + 1e-3 |ref|."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from gpu_util import DEV, append_bulk, check_close, oracle_cache, say, shape, sm_scale, to_dev

pytestmark = pytest.mark.gpu
F16, Q8, K4 = kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4


def build(fmt, kvh, P, cap, seed, outliers=True):
    xk = kvsynth.kv_tokens(seed, 0, P, kvh, 128, "K", outliers=outliers)
    xv = kvsynth.kv_tokens(seed, 0, P, kvh, 128, "V", outliers=outliers)
    s = kq.Session(fmt, kvh, cap, fill=0x5A)
    assert append_bulk(shape(fmt, kvh, kvh), [s], [0], xk[None], xv[None], chunk=65536) == 0
    return s, oracle_cache(fmt, kvh, cap, 128, xk, xv)


@pytest.mark.parametrize("fmt", [F16, Q8, K4])
@pytest.mark.parametrize("P", [1, 63, 200, 1000])
def test_compaction_bitexact(fmt, P):
    kvh = 3
    s, ref = build(fmt, kvh, P, kvsynth.round_up(P + 17, 64), 31 + P)
    k16 = torch.full((kvh, P, 128), 0x5A5A, dtype=torch.int16, device=DEV)
    v16 = torch.full((kvh, P, 128), 0x5A5A, dtype=torch.int16, device=DEV)
    kq.kv_compact_f16(shape(fmt, kvh, kvh), s.entry(), P, k16, v16)
    torch.cuda.synchronize()
    rk, rv = oracle.compact_f16(ref, P)
    assert np.array_equal(k16.cpu().numpy().view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(v16.cpu().numpy().view(np.uint16), rv.view(np.uint16))


def run_prefill(fmt, s, kvh, nqh, pos0, n_tok, q, sm):
    sh = shape(fmt, kvh, nqh)
    P = pos0 + n_tok
    nbytes = kq.kv_prefill_workspace_bytes(sh, P)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV) if nbytes else None
    out = torch.full((n_tok, nqh, 128), float("nan"), device=DEV)
    kq.kv_prefill_attn(sh, s.entry(), pos0, n_tok, to_dev(q), sm, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", [F16, Q8, K4])
@pytest.mark.parametrize("kvh,nqh,pos0,n_tok", [
    (2, 8, 100, 70),      # G=4, ragged chunk and key tail, several key tiles
    (2, 8, 0, 130),       # pure causal prompt from position 0
    (1, 1, 37, 300),      # G=1: 256-query blocks, two of them
    (2, 4, 64, 129),      # G=2
    (1, 8, 250, 45),      # G=8: 32-query blocks
    (2, 8, 500, 1),       # one-token chunk
])
def test_prefill_small(fmt, kvh, nqh, pos0, n_tok):
    P = pos0 + n_tok
    say(f"prefill fmt={fmt} kvh={kvh} nqh={nqh} pos0={pos0} n_tok={n_tok}")
    s, ref = build(fmt, kvh, P, kvsynth.round_up(P + 5, 64), 40 + P)
    q = kvsynth.queries(40 + P, 0, n_tok, nqh, 128, stream=kvsynth.S_Q_PREFILL)
    got = run_prefill(fmt, s, kvh, nqh, pos0, n_tok, q, sm_scale())
    k16, v16 = oracle.compact_f16(ref, P)
    want = oracle.prefill_attn(q, k16, v16, pos0, sm_scale())
    check_close(got, want, "prefill")


def test_prefill_single_token_equals_decode_definition():
    """A one-token chunk at position p attends keys [0, p], as decode over p+1
    cells does (on the fp16 copy, with the query rounded to fp16)."""
    kvh, nqh, pos0 = 2, 8, 777
    s, ref = build(Q8, kvh, pos0 + 1, 832, 9)
    q = kvsynth.queries(9, 0, 1, nqh, 128, stream=kvsynth.S_Q_PREFILL)
    got = run_prefill(Q8, s, kvh, nqh, pos0, 1, q, sm_scale())[0]
    k16, v16 = oracle.compact_f16(ref, pos0 + 1)
    q16 = q[0].astype(np.float16).astype(np.float32)
    want = oracle.decode_attn(q16, k16.astype(np.float64), v16.astype(np.float64), pos0 + 1, sm_scale())
    check_close(got, want, "one-token chunk")


@pytest.mark.slow
def test_prefill_chunk4096_at131072_sampled_rows():
    """The 4096-token prompt chunk at position 131072 of an int8 cache (8 kv heads,
    32 query heads); 72 sampled rows (all heads) against the oracle, rows 0 and
    n_tok - 1 among them."""
    w = kvsynth.WORKLOADS["prefill4096_at131072"]
    kvh, nqh, pos0, n_tok, seed = w["kvh"], w["nqh"], w["pos0"], w["n_tok"], w["seed"]
    P = pos0 + n_tok
    say("prefill 4096@131072: fill")
    s, ref = build(Q8, kvh, P, P, seed)
    q = kvsynth.queries(seed, 0, n_tok, nqh, 128, stream=kvsynth.S_Q_PREFILL)
    say("prefill 4096@131072: run")
    got = run_prefill(Q8, s, kvh, nqh, pos0, n_tok, q, sm_scale())
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 255, 256, 2047, 4094, 4095],
                                     np.random.default_rng(seed).choice(n_tok, 63, replace=False)]))
    assert rows.size >= 64 and rows[0] == 0 and rows[-1] == n_tok - 1
    k16, v16 = oracle.compact_f16(ref, P)
    say("prefill 4096@131072: oracle")
    want = oracle.prefill_attn(q, k16, v16, pos0, sm_scale(), rows=rows)
    check_close(got[rows], want, "prefill chunk rows")
    assert np.isfinite(got).all()
