"""kv_decode_attn on the GPU against the fp64 oracle on the same dequantised cache
(|gpu - ref| <= 2e-3 + 1e-3 |ref| elementwise), plus exact cases, determinism,
variable-length batches and device-side range checks."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
import quantized_kv_cache_q8_amd as kq
from gpu_util import (DEV, append_bulk, assert_cache_equal, check_close, check_fidelity,
                      decode_gpu, oracle_cache, say, shape, sm_scale, to_dev)

pytestmark = pytest.mark.gpu
F16, Q8, K4 = kq.KV_FMT_F16, kq.KV_FMT_Q8, kq.KV_FMT_K8V4


def oracle_decode(cache: oracle.Cache, q, length, sm, with_abs=False):
    """fp64 decode one kv head at a time (bounded memory at long contexts).
    with_abs: also the fidelity gate's A: the attention of the same weights over |V|
    (K8V4: over the rotated values |code * d|, averaged over the dims)."""
    nqh = q.shape[0]
    G = nqh // cache.kvh
    out = np.zeros((nqh, cache.hd))
    absv = np.zeros((nqh, cache.hd))
    for h in range(cache.kvh):
        sub = oracle.Cache(cache.fmt, 1, cache.cap, cache.hd)
        sub.k, sub.v = cache.k[h:h + 1], cache.v[h:h + 1]
        if cache.fmt != F16:
            sub.k_scale, sub.v_scale = cache.k_scale[h:h + 1], cache.v_scale[h:h + 1]
        K = sub.dequant("k", length)
        V = sub.dequant("v", length)
        out[h * G:(h + 1) * G] = oracle.decode_attn(q[h * G:(h + 1) * G], K, V, length, sm)
        if with_abs and cache.fmt == K4:
            # the V sums run over the rotated values and H / HD takes them back, so an
            # output element's error is at most the mean over dims of theirs
            u = np.abs(sub.v_rotated(length))
            a = oracle.decode_attn(q[h * G:(h + 1) * G], K, u, length, sm)
            absv[h * G:(h + 1) * G] = a.mean(axis=-1, keepdims=True)
        elif with_abs:
            absv[h * G:(h + 1) * G] = oracle.decode_attn(q[h * G:(h + 1) * G], K, np.abs(V),
                                                         length, sm)
    return (out, absv) if with_abs else out


def filled(fmt, kvh, cap, n, seed, outliers, layer=0):
    xk = kvsynth.kv_tokens(seed, layer, n, kvh, 128, "K", outliers=outliers)
    xv = kvsynth.kv_tokens(seed, layer, n, kvh, 128, "V", outliers=outliers)
    s = kq.Session(fmt, kvh, cap)
    assert append_bulk(shape(fmt, kvh, kvh), [s], [0], xk[None], xv[None], chunk=65536) == 0
    ref = oracle_cache(fmt, kvh, cap, 128, xk, xv)
    return s, ref


def test_tiny_q8_decode_ragged_lengths():
    w = kvsynth.WORKLOADS["tiny_q8_ctx1024"]
    kvh, nqh, n = w["kvh"], w["nqh"], w["ctx"]
    s, ref = filled(Q8, kvh, n, n, w["seed"], outliers=False)
    q = kvsynth.queries(w["seed"], 0, 1, nqh, 128)[0]
    sh = shape(Q8, kvh, nqh)
    for length in (1, 7, 63, 64, 65, 255, 256, 257, 1000, 1024):
        say(f"tiny q8 decode len={length}")
        got = decode_gpu(sh, [s], [length], q[None], sm_scale())[0]
        check_close(got, oracle_decode(ref, q, length, sm_scale()), f"len={length}")


@pytest.mark.parametrize("fmt", [F16, Q8])
def test_single_cell_is_exactly_the_value_row(fmt):
    s, ref = filled(fmt, 2, 64, 5, 3, outliers=True)
    q = kvsynth.queries(3, 0, 1, 8, 128)[0]
    got = decode_gpu(shape(fmt, 2, 8), [s], [1], q[None], 0.3)[0]
    want = np.repeat(ref.dequant("v", 1)[:, 0], 4, axis=0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [F16, Q8, K4])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_every_head_ratio(fmt, G):
    """Each supported query heads per kv head (the K-pass reduction and the logit
    layout depend on it), at lengths that end inside a step, a split and a chunk."""
    kvh = 2
    s, ref = filled(fmt, kvh, 4096, 3001, 20 + G, outliers=True)
    q = kvsynth.queries(20 + G, 0, 1, kvh * G, 128)[0]
    sh = shape(fmt, kvh, kvh * G)
    for length in (1, 9, 777, 3001):
        say(f"decode fmt={fmt} G={G} len={length}")
        got = decode_gpu(sh, [s], [length], q[None], sm_scale())[0]
        want, absv = oracle_decode(ref, q, length, sm_scale(), with_abs=True)
        check_close(got, want, f"G={G} len={length}")
        check_fidelity(got, want, absv, f"G={G} len={length}")


def test_empty_session_gives_zeros_and_determinism():
    s, ref = filled(Q8, 2, 4096, 4000, 5, outliers=True)
    q = kvsynth.queries(5, 0, 3, 8, 128)
    sh = shape(Q8, 2, 8)
    a = decode_gpu(sh, [s, s, s], [0, 4000, 2500], q, sm_scale())
    b = decode_gpu(sh, [s, s, s], [0, 4000, 2500], q, sm_scale())
    assert not a[0].any()
    assert np.array_equal(a, b)                      # bitwise run-to-run
    check_close(a[1], oracle_decode(ref, q[1], 4000, sm_scale()), "len=4000")
    check_close(a[2], oracle_decode(ref, q[2], 2500, sm_scale()), "len=2500")


def test_f16_ctx32768_steps():
    """FP16 cache at 32768 context with outlier channels; each step appends one
    token (FP16 store) and decodes."""
    w = kvsynth.WORKLOADS["f16_ctx32768"]
    kvh, nqh, ctx, seed = w["kvh"], w["nqh"], w["ctx"], w["seed"]
    steps = 3
    cap = kvsynth.round_up(ctx + steps, 64)
    say("f16 ctx32768: fill")
    s, ref = filled(F16, kvh, cap, ctx - steps, seed, outliers=True)
    sh = shape(F16, kvh, nqh)
    tab = kq.session_table([s.entry()])
    for step in range(steps):
        length = ctx - steps + step
        xk = kvsynth.kv_tokens(seed, 0, 1, kvh, 128, "K", True, stream=kvsynth.S_K_NEW, sub=step)
        xv = kvsynth.kv_tokens(seed, 0, 1, kvh, 128, "V", True, stream=kvsynth.S_V_NEW, sub=step)
        kq.kv_append(sh, tab, to_dev(np.array([length], np.int32)), 1, 1, to_dev(xk[None]),
                     to_dev(xv[None]))
        assert ref.append(length, xk, xv)
        q = kvsynth.queries(seed, 0, 1, nqh, 128, sub=step, half_grid=True)[0]
        got = decode_gpu(sh, [s], [length + 1], q[None], sm_scale())[0]
        want, absv = oracle_decode(ref, q, length + 1, sm_scale(), with_abs=True)
        check_close(got, want, f"f16 step {step}")
        check_fidelity(got, want, absv, f"f16 step {step}")
    assert_cache_equal(s, ref)


def test_q8_ctx131072_steps():
    w = kvsynth.WORKLOADS["q8_ctx131072"]
    kvh, nqh, ctx, seed = w["kvh"], w["nqh"], w["ctx"], w["seed"]
    steps = 2
    cap = kvsynth.round_up(ctx + steps, 64)
    say("q8 ctx131072: fill")
    s, ref = filled(Q8, kvh, cap, ctx, seed, outliers=True)
    say("q8 ctx131072: codes and scales of the seeded fill, bit for bit")
    assert_cache_equal(s, ref)
    sh = shape(Q8, kvh, nqh)
    tab = kq.session_table([s.entry()])
    for step in range(steps):
        length = ctx + step
        xk = kvsynth.kv_tokens(seed, 0, 1, kvh, 128, "K", True, stream=kvsynth.S_K_NEW, sub=step)
        xv = kvsynth.kv_tokens(seed, 0, 1, kvh, 128, "V", True, stream=kvsynth.S_V_NEW, sub=step)
        kq.kv_append(sh, tab, to_dev(np.array([length], np.int32)), 1, 1, to_dev(xk[None]),
                     to_dev(xv[None]))
        assert ref.append(length, xk, xv)
        q = kvsynth.queries(seed, 0, 1, nqh, 128, sub=step)[0]
        got = decode_gpu(sh, [s], [length + 1], q[None], sm_scale())[0]
        want, absv = oracle_decode(ref, q, length + 1, sm_scale(), with_abs=True)
        check_close(got, want, f"q8 step {step}")
        check_fidelity(got, want, absv, f"q8 step {step}")
    say("q8 ctx131072: the appended rows too")
    assert_cache_equal(s, ref)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [F16, Q8])
def test_full_context_262144_layer(fmt):
    """One layer of the full-context workload (8 kv heads, 32 query heads, 262144
    cells, outlier channels), in the launch configuration the benchmark times."""
    w = kvsynth.WORKLOADS["full_ctx262144_48l"]
    kvh, nqh, ctx, seed = w["kvh"], w["nqh"], w["ctx"], w["seed"]
    say(f"full ctx fmt={fmt}: fill")
    s, ref = filled(fmt, kvh, ctx, ctx, seed, outliers=True)
    say(f"full ctx fmt={fmt}: cache of the seeded fill, bit for bit")
    assert_cache_equal(s, ref)
    q = kvsynth.queries(seed, 0, 1, nqh, 128)[0]
    say("full ctx: decode")
    got = decode_gpu(shape(fmt, kvh, nqh), [s], [ctx], q[None], sm_scale())[0]
    want, absv = oracle_decode(ref, q, ctx, sm_scale(), with_abs=True)
    check_close(got, want, f"full ctx fmt={fmt}")
    check_fidelity(got, want, absv, f"full ctx fmt={fmt}")


def test_batched_variable_lengths_small():
    """64 sessions of different lengths and capacities in one session table."""
    kvh, nqh, n_sess = 2, 8, 64
    r = np.random.default_rng(77)
    lens = r.integers(1, 3000, size=n_sess)
    lens[:3] = [1, 64, 2999]
    sessions, refs = [], []
    for b in range(n_sess):
        cap = kvsynth.round_up(lens[b] + int(r.integers(0, 100)), 64)
        s, ref = filled(Q8, kvh, cap, int(lens[b]), 1000 + b, outliers=True)
        sessions.append(s)
        refs.append(ref)
    q = kvsynth.queries(77, 0, n_sess, nqh, 128)
    got = decode_gpu(shape(Q8, kvh, nqh), sessions, lens, q, sm_scale())
    for b in range(n_sess):
        check_close(got[b], oracle_decode(refs[b], q[b], int(lens[b]), sm_scale()), f"session {b}")


@pytest.mark.slow
def test_batched64_full_lengths_sampled():
    """64 int8 sessions with lengths uniform on [1024, 65536]; every session is
    decoded in one launch, the oracle checks 6 of them (shortest, longest, others)."""
    w = kvsynth.WORKLOADS["batched64_q8"]
    kvh, nqh, seed = w["kvh"], w["nqh"], w["seed"]
    lens = kvsynth.session_lengths(seed, w["batch"], w["lo"], w["hi"])
    check = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, 40, 63})
    sessions, refs = [], {}
    sh = shape(Q8, kvh, nqh)
    for b in range(w["batch"]):
        n = int(lens[b])
        s = kq.Session(Q8, kvh, kvsynth.round_up(n + 1, 64))
        xk = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "K", True, sub=b)
        xv = kvsynth.kv_tokens(seed, 0, n, kvh, 128, "V", True, sub=b)
        assert append_bulk(sh, [s], [0], xk[None], xv[None], chunk=65536) == 0
        if b in check:
            refs[b] = oracle_cache(Q8, kvh, s.cap, 128, xk, xv)
        sessions.append(s)
    say("batched64: decode")
    q = kvsynth.queries(seed, 0, w["batch"], nqh, 128)
    got = decode_gpu(sh, sessions, lens, q, sm_scale())
    for b in check:
        check_close(got[b], oracle_decode(refs[b], q[b], int(lens[b]), sm_scale()), f"session {b}")


def test_workspace_reused_across_shapes():
    """One workspace for calls of different session counts and lengths (so of
    different split counts and partial layouts), each checked against the oracle."""
    kvh, nqh = 2, 8
    sh = shape(Q8, kvh, nqh)
    s, ref = filled(Q8, kvh, 8192, 8000, 31, outliers=True)
    calls = ((1, 8000, [8000]), (9, 300, [300, 1, 0, 299, 64, 65, 7, 200, 300]),
             (3, 8000, [5000, 8000, 17]), (1, 1, [1]))
    nbytes = max(kq.kv_decode_workspace_bytes(sh, n, m) for n, m, _ in calls)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for n_sess, max_len, lens in calls:
        q = kvsynth.queries(31, 0, n_sess, nqh, 128, sub=n_sess)
        say(f"reuse n_sess={n_sess} max_len={max_len}")
        got = decode_gpu(sh, [s] * n_sess, lens, q, sm_scale(), max_len=max_len, ws=ws)
        for b in range(n_sess):
            if lens[b] == 0:
                assert not got[b].any()
            else:
                check_close(got[b], oracle_decode(ref, q[b], lens[b], sm_scale()), f"b={b}")


def test_device_side_range_checks():
    s, ref = filled(Q8, 2, 128, 100, 8, outliers=False)
    q = kvsynth.queries(8, 0, 2, 4, 128)
    sh = shape(Q8, 2, 4)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    # max_len smaller than a session's length: that session is flagged and zeroed
    got = decode_gpu(sh, [s, s], [100, 50], q, sm_scale(), max_len=64, status=status)
    assert status.item() == kq.KV_DEV_RANGE
    assert not got[0].any()
    check_close(got[1], oracle_decode(ref, q[1], 50, sm_scale()), "len=50")
    # a length beyond the capacity, a negative length, a bad table entry
    status.zero_()
    bad = s.entry()
    bad.v_scale = None
    sess_entries = [s.entry(), s.entry(), bad]
    tab = kq.session_table(sess_entries)
    lens = to_dev(np.array([129, -1, 10], np.int32))
    ws = kq.kv_decode_workspace(sh, 3, 200, DEV)
    out = torch.full((3, 4, 128), 7.0, device=DEV)
    kq.kv_decode_attn(sh, tab, lens, 3, 200, to_dev(np.zeros((3, 4, 128), np.float32)), 0.1, out,
                      ws, status)
    torch.cuda.synchronize()
    assert status.item() == kq.KV_DEV_RANGE | kq.KV_DEV_BAD_SESSION
    assert not out.any()


@pytest.mark.parametrize("fmt", [F16, Q8, K4])
def test_batch_composition_bitwise(fmt):
    """A session's decode does not depend on its place in a batch or on what the other
    sessions hold: permuting the batch, or replacing every other session's cache and
    query, gives it bitwise the same output (the split count and step unit depend only
    on the call's session count and max_len, and each session's arithmetic only on
    its own length).  A one-session call plans its own split count and step unit, so a
    session decoded alone and in a batch take different summation orders; both are
    checked against the oracle, with the fidelity gate."""
    kvh, G = 2, 4
    nqh = kvh * G
    sh = shape(fmt, kvh, nqh)
    lens = [3000, 1, 2999, 64, 1500, 3000]
    a = [filled(fmt, kvh, 3008, n, 700 + i, outliers=True) for i, n in enumerate(lens)]
    b = [filled(fmt, kvh, 3008, n, 800 + i, outliers=True) for i, n in enumerate(lens)]
    q = kvsynth.queries(90, 0, len(lens), nqh, 128)
    q2 = kvsynth.queries(91, 0, len(lens), nqh, 128)
    base = decode_gpu(sh, [s for s, _ in a], lens, q, sm_scale())
    perm = [4, 2, 0, 5, 3, 1]
    got = decode_gpu(sh, [a[i][0] for i in perm], [lens[i] for i in perm], q[perm], sm_scale())
    for k, i in enumerate(perm):
        assert np.array_equal(got[k], base[i]), f"permuted batch, session {i}"
    # session 0 and 4 kept, the others replaced by other caches and queries
    keep = (0, 4)
    mixed = [a[i][0] if i in keep else b[i][0] for i in range(len(lens))]
    qm = np.stack([q[i] if i in keep else q2[i] for i in range(len(lens))])
    got = decode_gpu(sh, mixed, lens, qm, sm_scale())
    for i in keep:
        assert np.array_equal(got[i], base[i]), f"neighbours changed, session {i}"
    for i in range(len(lens)):
        single = decode_gpu(sh, [a[i][0]], [lens[i]], q[i][None], sm_scale())[0]
        want, absv = oracle_decode(a[i][1], q[i], lens[i], sm_scale(), with_abs=True)
        check_close(base[i], want, f"batched session {i}")
        check_close(single, want, f"single session {i}")
        check_fidelity(base[i], want, absv, f"batched session {i}")
        check_fidelity(single, want, absv, f"single session {i}")


@pytest.mark.parametrize("fmt", [F16, Q8])
def test_many_sessions_ranked(fmt):
    """1500 sessions in one call, more than the 1024 threads of the workgroup that ranks
    a batch by length (its loops take two passes), with many equal lengths: views into
    one pool of 128-cell slots, lengths 1 .. 128.  Each session's output is bitwise the
    same with the table in reverse order, and sampled sessions match the oracle."""
    kvh, nqh, n, slot = 1, 4, 1500, 128
    r = np.random.default_rng(123)
    lens = r.integers(1, slot + 1, size=n)
    lens[:4] = [1, slot, slot, 1]
    say(f"many sessions fmt={fmt}: fill {n * slot} cells")
    pool, ref = filled(fmt, kvh, n * slot, n * slot, 4242, outliers=True)
    row_bytes = 2 * 128 if fmt == F16 else 128
    sc_bytes = 0 if fmt == F16 else 2 * (128 // 64)

    def view(b):
        o = int(b) * slot
        k, v = pool.k.data_ptr() + o * row_bytes, pool.v.data_ptr() + o * row_bytes
        ks = None if fmt == F16 else pool.k_scale.data_ptr() + o * sc_bytes
        vs = None if fmt == F16 else pool.v_scale.data_ptr() + o * sc_bytes
        return kq.kv_session(k, v, ks, vs, slot, 0)

    sh = shape(fmt, kvh, nqh)
    q = kvsynth.queries(124, 0, n, nqh, 128)

    def run(order):
        tab = kq.session_table([view(b) for b in order])
        lt = to_dev(lens[order].astype(np.int32))
        ws = kq.kv_decode_workspace(sh, n, slot, DEV)
        out = torch.full((n, nqh, 128), float("nan"), device=DEV)
        kq.kv_decode_attn(sh, tab, lt, n, slot, to_dev(q[order].astype(np.float32)), sm_scale(),
                          out, ws)
        torch.cuda.synchronize()
        res = np.empty((n, nqh, 128))
        res[order] = out.cpu().numpy()
        return res

    say("many sessions: decode, then the table reversed")
    got = run(np.arange(n))
    rev = run(np.arange(n)[::-1].copy())
    assert np.array_equal(got, rev), "a session's output depends on its place in the table"
    for b in sorted({0, 1, 2, 3, 700, 1024, 1499} | set(r.integers(0, n, size=5).tolist())):
        sub = oracle.Cache(fmt, kvh, slot, 128)
        sub.k, sub.v = ref.k[:, b * slot:(b + 1) * slot], ref.v[:, b * slot:(b + 1) * slot]
        if fmt != F16:
            sub.k_scale = ref.k_scale[:, b * slot:(b + 1) * slot]
            sub.v_scale = ref.v_scale[:, b * slot:(b + 1) * slot]
        want, absv = oracle_decode(sub, q[b], int(lens[b]), sm_scale(), with_abs=True)
        check_close(got[b], want, f"session {b} (len {lens[b]})")
        check_fidelity(got[b], want, absv, f"session {b}")
