"""kv_append on the GPU against the oracle: int8 codes, fp16 scales and fp16 values
must match bit for bit; nothing outside the written rows may change."""
import json
import os

import numpy as np
import pytest
import torch

import kvsynth
import oracle
import pins
import quantized_kv_cache_q8_amd as kq
from gpu_util import DEV, append_bulk, assert_cache_equal, download, oracle_cache, say, shape

pytestmark = pytest.mark.gpu
F16, Q8 = kq.KV_FMT_F16, kq.KV_FMT_Q8


def test_tiny_q8_bulk_equals_oracle_and_single_token_appends():
    w = kvsynth.WORKLOADS["tiny_q8_ctx1024"]
    kvh, hd, n = w["kvh"], w["hd"], w["ctx"]
    say(f"tiny q8 append: kvh={kvh} n={n}")
    xk = kvsynth.kv_tokens(w["seed"], 0, n, kvh, hd, "K", outliers=False)
    xv = kvsynth.kv_tokens(w["seed"], 0, n, kvh, hd, "V", outliers=False)
    ref = oracle_cache(Q8, kvh, n, hd, xk, xv)
    sh = shape(Q8, kvh, w["nqh"])
    s1 = kq.Session(Q8, kvh, n, fill=0x5A)
    assert append_bulk(sh, [s1], [0], xk[None], xv[None]) == 0
    assert_cache_equal(s1, ref)
    s2 = kq.Session(Q8, kvh, n, fill=0x5A)
    assert append_bulk(sh, [s2], [0], xk[None], xv[None], chunk=1) == 0   # 1024 one-token appends
    for a, b in zip(s1.tensors(), s2.tensors()):
        assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", [F16, Q8])
def test_outlier_rows_bitexact(fmt):
    kvh, hd, n, cap = 8, 128, 3000, 3072
    say(f"append fmt={fmt} kvh={kvh} n={n}")
    xk = kvsynth.kv_tokens(22, 0, n, kvh, hd, "K", outliers=True)
    xv = kvsynth.kv_tokens(22, 0, n, kvh, hd, "V", outliers=True)
    ref = oracle_cache(fmt, kvh, cap, hd, xk, xv)
    s = kq.Session(fmt, kvh, cap, fill=0)
    assert append_bulk(shape(fmt, kvh, 32), [s], [0], xk[None], xv[None]) == 0
    assert_cache_equal(s, ref)


def test_worked_examples_and_every_fp16_scale():
    """The hand-derived groups, the reciprocal-trap groups and the sweep over every
    positive finite fp16 scale, quantised by the GPU."""
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "quant_worked_examples.json")))
    groups = []
    for g in gold["groups"]:
        x = np.zeros(64, np.float32)
        x[: len(g["x"])] = g["x"]
        groups.append(x)
    traps = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "recip_trap_cases.json")))
    for g in traps["groups_f32_bits"]:
        groups.append(np.array([int(b, 16) for b in g], np.uint32).view(np.float32))
    sweep = pins.scale_sweep_groups()
    allg = np.concatenate([np.stack(groups), sweep])
    if len(allg) % 2:
        allg = np.concatenate([allg, np.zeros((1, 64), np.float32)])
    rows = allg.reshape(-1, 1, 128)                 # n_tok rows of one kv head, two groups each
    n = rows.shape[0]
    cap = (n + 63) // 64 * 64
    say(f"sweep append rows={n}")
    s = kq.Session(Q8, 1, cap, fill=0x5A)
    assert append_bulk(shape(Q8, 1, 1), [s], [0], rows[None], rows[None]) == 0
    got = download(s)
    codes = got["k"][0, :n].reshape(-1, 64)
    scales = got["k_scale"][0, :n].reshape(-1).view(np.uint16)
    # the hand-derived worked examples, against their printed values
    for i, g in enumerate(gold["groups"]):
        want = np.zeros(64, np.int8)
        want[: len(g["codes"])] = g["codes"]
        assert int(scales[i]) == int(g["scale_bits"], 16), g["label"]
        assert np.array_equal(codes[i], want), g["label"]
    # everything against the oracle
    oc, os_ = oracle.quantize_q8(allg)
    assert np.array_equal(codes, oc)
    assert np.array_equal(scales, os_.reshape(-1).view(np.uint16))
    assert np.array_equal(got["v"][0, :n], got["k"][0, :n])


@pytest.mark.parametrize("fmt", [F16, Q8])
def test_sentinels_ranges_and_batched_sessions(fmt):
    kvh, hd = 3, 128
    sh = shape(fmt, kvh, kvh)
    caps = [128, 64, 192, 128]
    lens = [13, 60, 0, 125]          # session 1 and 3 do not fit 7 tokens
    n_tok = 7
    sessions = [kq.Session(fmt, kvh, c, fill=0x5A) for c in caps]
    r = np.random.default_rng(9)
    xk = r.standard_normal((4, n_tok, kvh, hd), dtype=np.float32) * np.float32(3)
    xv = r.standard_normal((4, n_tok, kvh, hd), dtype=np.float32)
    st = append_bulk(sh, sessions, lens, xk, xv)
    assert st == kq.KV_DEV_RANGE
    for b, s in enumerate(sessions):
        got = download(s)
        fits = lens[b] + n_tok <= caps[b]
        for name, arr in got.items():
            u8 = arr.view(np.uint8).reshape(kvh, caps[b], -1)
            mask = np.ones(caps[b], bool)
            if fits:
                mask[lens[b]:lens[b] + n_tok] = False
            assert (u8[:, mask] == 0x5A).all(), (b, name)
        if fits:
            ref = oracle_cache(fmt, kvh, caps[b], hd, xk[b], xv[b], pos=lens[b])
            assert_cache_equal(s, ref, rows=slice(lens[b], lens[b] + n_tok))


def test_bad_session_entries_are_skipped_and_flagged():
    kvh, hd = 2, 128
    sh = shape(Q8, kvh, 4)
    good = kq.Session(Q8, kvh, 64, fill=0x5A)
    other = kq.Session(Q8, kvh, 64, fill=0x5A)
    e_bad = other.entry()
    e_bad.k_scale = None                      # int8 format without a K scale array
    tab = kq.session_table([good.entry(), e_bad])
    x = np.ones((2, 1, kvh, hd), np.float32)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    lens = torch.zeros(2, dtype=torch.int32, device=DEV)
    kq.kv_append(sh, tab, lens, 2, 1, torch.from_numpy(x).to(DEV), torch.from_numpy(x).to(DEV), status)
    torch.cuda.synchronize()
    assert status.item() == kq.KV_DEV_BAD_SESSION
    for t in other.tensors():
        assert (t.view(torch.uint8) == 0x5A).all()
    assert (good.k[:, 0] == 127).all() and (good.k[:, 1:].view(torch.uint8) == 0x5A).all()
    # a capacity beyond 2^24 cells is refused on the device as well (nothing is touched)
    e_big = other.entry()
    e_big.cap = (1 << 24) + 64
    status.zero_()
    tab = kq.session_table([e_big])
    kq.kv_append(sh, tab, lens[:1], 1, 1, torch.from_numpy(x[:1]).to(DEV),
                 torch.from_numpy(x[:1]).to(DEV), status)
    torch.cuda.synchronize()
    assert status.item() == kq.KV_DEV_BAD_SESSION
    for t in other.tensors():
        assert (t.view(torch.uint8) == 0x5A).all()
