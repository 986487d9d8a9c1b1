"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` takes the oracle function(s) under test as arguments and raises
AssertionError on a mismatch, so that the same pins run against the oracle
(tests/test_oracle_*.py) and against planted mistakes
(tests/test_oracle_mutations.py), which must each fail at least one pin.

What pins what:
  * quantiser: hand-derived worked examples; brute force with exact rational
    arithmetic (fp32 division and fp16 rounding written from the IEEE
    definition); |code| <= 127 and max |code| = 127 for normal scales; the
    reconstruction bound |code*s - x| <= s*(1/2 + 2^-17); sign symmetry;
    power-of-two scaling; an exhaustive sweep over every positive finite fp16
    scale; stored cases where a reciprocal multiply differs.
  * byte accounting: the 12.0 / 6.0 / 3.1 GiB of PR #3084, section Summary.
  * decode: torch's CPU scaled_dot_product_attention in float64 (a library
    routine); len = 1, q = 0, constant V, V*2, token permutation; scalar brute
    force; the FP16 cache equals fp32 attention on fp16-rounded K/V.
  * split-K: the log-sum-exp merge equals single-pass softmax for any split
    size, with and without padded empty splits.
  * prefill: torch's causal SDPA over the whole sequence (rows pos0..);
    a one-token chunk equals decode; future keys do not affect a row; brute force.
  * compaction: the exact rational product rounded once to fp16.
  * K8V4: the rotation against SciPy's Hadamard matrix (a library routine), its
    involution H H = 128 I and a rounding bound, and the per-operation fp32
    rounding written out in fractions; the 4-bit quantiser by hand-worked
    examples, brute force and invariants; the nibble layout; the read-back
    against SciPy's matrix and a closed-form error bound; the compacted V exact
    on dyadic inputs and per row against the fraction butterflies; the byte
    count against the 816 B per cell of PR #711, section What.
  * saved image: the layout of Issue #67, section Scope (128-byte header, 4 bytes
    per token, body, scales body; 8 scale bytes per token and kv head for q8 at
    head_dim 128), the version rule of its Phased plan, the header read at its
    stated offsets, the body read back against the inputs within the quantiser
    bound, a round trip, and each refusal.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

from _exact import f16, fwht_f32_exact, quant_block_exact, quant_group_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _group(vals):
    x = np.zeros(64, np.float32)
    x[: len(vals)] = np.asarray(vals, np.float32)
    return x


# ----------------------------------------------------------------------------
# quantiser
# ----------------------------------------------------------------------------
def pin_quant_worked_examples(quant):
    gold = _load("quant_worked_examples.json")
    x = np.stack([_group(g["x"]) for g in gold["groups"]])      # [n][64], one group each
    codes, scales = quant(x)
    for i, g in enumerate(gold["groups"]):
        want = np.zeros(64, np.int8)
        want[: len(g["codes"])] = g["codes"]
        assert int(scales[i].view(np.uint16)[0]) == int(g["scale_bits"], 16), g["label"]
        assert np.array_equal(codes[i], want), g["label"]
    # two groups in one head row keep separate scales (group = 64 contiguous dims)
    row = np.concatenate([_group(gold["groups"][0]["x"]), _group(gold["groups"][1]["x"])])
    c, s = quant(row[None])
    assert s.shape[-1] == 2
    assert [int(b) for b in s.view(np.uint16)[0]] == [0x3C00, 0x4000]
    assert np.array_equal(c[0, :64], codes[0]) and np.array_equal(c[0, 64:], codes[1])


def _random_groups(seed, n):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, 64), dtype=np.float32)
    x *= np.exp2(r.integers(-20, 12, size=(n, 1))).astype(np.float32)   # normal and subnormal scales
    x[r.random((n, 64)) < 0.05] *= np.float32(20)                        # outliers
    x[:3] = 0
    x[1, 5] = np.float32(-1e-30)       # scale underflows to 0
    x[2, :] = np.float32(7.0)          # constant group
    return x


def pin_quant_brute_force(quant, n=300, n_exhaustive=8):
    x = _random_groups(1, n)
    codes, scales = quant(x)
    for i in range(n):
        s, c = quant_group_exact(x[i], brute=(i < n_exhaustive))
        assert Fraction(float(scales[i, 0])) == s, (i, float(scales[i, 0]), float(s))
        assert codes[i].tolist() == c, i


def pin_quant_invariants(quant):
    x = _random_groups(2, 4000)
    codes, scales = quant(x)
    c = codes.astype(np.int32)
    s = scales[:, 0].astype(np.float64)
    assert np.abs(c).max() <= 127
    normal = s >= 2.0 ** -14
    assert normal.sum() > 1000
    assert (np.abs(c[normal]).max(-1) == 127).all()
    err = np.abs(c * s[:, None] - x.astype(np.float64))
    assert (err[normal] <= s[normal, None] * (0.5 + 2.0 ** -17)).all()
    # sign symmetry
    cn, sn = quant(-x)
    assert np.array_equal(cn, -codes) and np.array_equal(sn.view(np.uint16), scales.view(np.uint16))
    # power-of-two scaling while the scale stays a normal fp16 value
    sel = (s >= 2.0 ** -12) & (s <= 2.0 ** 10)
    c2, s2 = quant(x[sel] * np.float32(4))
    assert np.array_equal(c2, codes[sel])
    assert np.array_equal(s2.astype(np.float64), 4 * scales[sel].astype(np.float64))


def scale_sweep_groups():
    """Every positive finite fp16 value h: groups with amax = fl32(127 h) and its
    fp32 neighbours, holding +amax, -amax, amax/3 and a small value.  [n][64]"""
    h = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    h = h[:-1]                                      # fp32 neighbours of 127*65504 would overflow fp16
    amax = (h * np.float32(127)).astype(np.float32)
    amaxes = np.concatenate([amax, np.nextafter(amax, np.float32(np.inf)),
                             np.nextafter(amax, np.float32(0))])
    x = np.zeros((amaxes.size, 64), np.float32)
    x[:, 0] = amaxes
    x[:, 1] = -amaxes
    x[:, 2] = amaxes / np.float32(3)
    x[:, 3] = amaxes * np.float32(0.0123)
    return x


def pin_quant_scale_sweep(quant):
    x = scale_sweep_groups()
    amaxes = x[:, 0]
    codes, scales = quant(x)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    s = scales[:, 0].astype(np.float64)
    normal = s >= 2.0 ** -14
    assert (codes[normal, 0] == 127).all() and (codes[normal, 1] == -127).all()
    # exact check of the scale and the four codes on a strided subset of the sweep
    for i in range(0, amaxes.size, 41):
        se, ce = quant_group_exact(x[i, :4].tolist() + [0.0])
        assert Fraction(float(scales[i, 0])) == se, i
        assert codes[i, :4].tolist() == ce[:4], i


def pin_quant_recip_traps(quant):
    gold = _load("recip_trap_cases.json")
    x = np.array([[int(b, 16) for b in g] for g in gold["groups_f32_bits"]], np.uint32).view(np.float32)
    assert len(x) >= 4
    codes, scales = quant(x)
    for i in range(len(x)):
        s, c = quant_group_exact(x[i])
        assert Fraction(float(scales[i, 0])) == s
        assert codes[i].tolist() == c, i


QUANT_PINS = [pin_quant_worked_examples, pin_quant_brute_force, pin_quant_invariants,
              pin_quant_scale_sweep, pin_quant_recip_traps]


# ----------------------------------------------------------------------------
# byte accounting
# ----------------------------------------------------------------------------
def pin_cache_bytes_pages(cache_bytes, FMT_F16, FMT_Q8):
    gold = _load("cache_bytes_pr3084.json")
    cells = gold["cells"]
    gib = float(2 ** 30)
    # 12.0 GiB of fp32 at 262144 cells fixes the values per cell: 12288
    vals_per_cell = round(gold["gib_fp32"] * gib / cells / 4)
    assert vals_per_cell * cells * 4 == gold["gib_fp32"] * gib
    # any factorisation layers * 2 (K, V) * kvh * hd of that count; here 6 * 2 * 8 * 128
    layers, kvh, hd = 6, 8, 128
    assert layers * 2 * kvh * hd == vals_per_cell

    def total(fmt):
        return layers * 2 * (cache_bytes(fmt, kvh, cells, hd, 0) + cache_bytes(fmt, kvh, cells, hd, 1))

    assert total(FMT_F16) == gold["gib_fp16"] * gib
    assert round(total(FMT_Q8) / gib, gold["printed_decimals"]) == gold["gib_q8"]
    assert cache_bytes(FMT_F16, kvh, cells, hd, 1) == 0


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def _sdpa_decode(q, K, V, length, sm_scale, dtype=torch.float64):
    """torch's CPU SDPA, one query position, GQA by kv-head repetition."""
    if length == 0:
        return np.zeros(q.shape)
    qt = torch.from_numpy(np.asarray(q, np.float64)).to(dtype)[None, :, None, :]     # [1][nqh][1][hd]
    kt = torch.from_numpy(np.asarray(K[:, :length], np.float64)).to(dtype)[None]      # [1][kvh][L][hd]
    vt = torch.from_numpy(np.asarray(V[:, :length], np.float64)).to(dtype)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=float(np.float32(sm_scale)), enable_gqa=True)
    return o[0, :, 0, :].double().numpy()


def _decode_case(seed, kvh, G, hd, L, outliers=True):
    r = np.random.default_rng(seed)
    K = r.standard_normal((kvh, L, hd))
    V = r.standard_normal((kvh, L, hd))
    if outliers:
        K[:, :, 3] *= 20
        V[:, :, 7] *= 20
    q = r.standard_normal((kvh * G, hd)).astype(np.float32)
    return q, K, V


def pin_decode_sdpa(decode):
    for seed, (kvh, G, hd, L, length) in enumerate(
            [(2, 2, 128, 70, 70), (1, 4, 64, 33, 17), (3, 1, 128, 9, 9), (2, 4, 128, 300, 257)]):
        q, K, V = _decode_case(seed, kvh, G, hd, L)
        sm = 1 / math.sqrt(hd)
        got = decode(q, K, V, length, sm)
        ref = _sdpa_decode(q, K, V, length, sm)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()


def pin_decode_closed_forms(decode):
    q, K, V = _decode_case(10, 2, 2, 128, 40)
    sm = 0.125
    # one cached cell: the output is that cell's V row, exactly
    out = decode(q, K, V, 1, sm)
    assert np.array_equal(out, np.repeat(V[:, 0], 2, axis=0))
    # zero query: uniform weights, the mean of the V rows
    out = decode(np.zeros_like(q), K, V, 40, sm)
    assert np.allclose(out, np.repeat(V.mean(axis=1), 2, axis=0), rtol=1e-13, atol=1e-13)
    # constant V
    Vc = np.full_like(V, 3.25)
    assert np.allclose(decode(q, K, Vc, 40, sm), 3.25, rtol=1e-14, atol=0)
    # V * 2 => out * 2 (exact in binary arithmetic)
    assert np.array_equal(decode(q, K, 2 * V, 40, sm), 2 * decode(q, K, V, 40, sm))
    # token permutation invariance
    perm = np.random.default_rng(3).permutation(40)
    a = decode(q, K, V, 40, sm)
    b = decode(q, K[:, perm], V[:, perm], 40, sm)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    # empty cache gives zeros
    assert not decode(q, K, V, 0, sm).any()
    # cells beyond length are ignored
    K2, V2 = K.copy(), V.copy()
    K2[:, 30:] = 1e3
    V2[:, 30:] = -1e3
    assert np.array_equal(decode(q, K, V, 30, sm), decode(q, K2, V2, 30, sm))


def pin_decode_brute(decode, brute_row):
    q, K, V = _decode_case(20, 2, 2, 8, 12)
    sm = 0.3
    for length in (1, 5, 12):
        out = decode(q, K, V, length, sm)
        for qh in range(4):
            h = qh // 2
            ref = brute_row(q[qh], K[h, :length], V[h, :length], sm)
            assert np.allclose(out[qh], ref, rtol=1e-12, atol=1e-12)


def pin_f16_cache_equals_fp32_attention(decode, Cache, FMT_F16):
    """An FP16 cache gives the attention that fp32 arithmetic gives on K/V
    rounded to fp16 (torch CPU SDPA in float32)."""
    kvh, G, hd, L = 2, 4, 128, 500
    r = np.random.default_rng(30)
    xk = r.standard_normal((L, kvh, hd), dtype=np.float32)
    xv = r.standard_normal((L, kvh, hd), dtype=np.float32)
    xk[:, :, 11] *= 20
    cache = Cache(FMT_F16, kvh, 512, hd)
    assert cache.append(0, xk, xv)
    q = r.standard_normal((kvh * G, hd), dtype=np.float32)
    got = decode(q, cache.dequant("k", L), cache.dequant("v", L), L, 1 / math.sqrt(hd))
    k16 = np.transpose(xk.astype(np.float16), (1, 0, 2))
    v16 = np.transpose(xv.astype(np.float16), (1, 0, 2))
    ref = _sdpa_decode(q, k16.astype(np.float32), v16.astype(np.float32), L, 1 / math.sqrt(hd),
                       dtype=torch.float32)
    assert np.allclose(got, ref, rtol=2e-5, atol=2e-5), np.abs(got - ref).max()


DECODE_PINS = [pin_decode_sdpa, pin_decode_closed_forms]


# ----------------------------------------------------------------------------
# split-K + merge
# ----------------------------------------------------------------------------
def pin_splitk_identity(decode, partials, merge):
    q, K, V = _decode_case(40, 2, 4, 64, 97)
    sm = 0.2
    ref = decode(q, K, V, 97, sm)
    for T in (1, 3, 16, 32, 96, 97, 200):
        o, lse = partials(q, K, V, 97, sm, T)
        assert o.shape[1] == -(-97 // T)
        got = merge(o, lse)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), T
    # padded empty splits (lse = -inf, o = 0) weigh nothing
    o, lse = partials(q, K, V, 97, sm, 16)
    pad = 5
    o2 = np.concatenate([o, np.zeros((o.shape[0], pad, o.shape[2]))], axis=1)
    l2 = np.concatenate([lse, np.full((lse.shape[0], pad), -np.inf)], axis=1)
    assert np.allclose(merge(o2, l2), ref, rtol=1e-12, atol=1e-12)
    # a merge of a single split is that split's partial
    o, lse = partials(q, K, V, 97, sm, 97)
    assert np.allclose(merge(o, lse), o[:, 0], rtol=1e-14, atol=1e-14)
    # partial lse is the log of the split's softmax denominator
    o, lse = partials(q, K, V, 10, sm, 10)
    for qh in range(o.shape[0]):
        z = float(np.float32(sm)) * (K[qh // 4, :10] @ q[qh].astype(np.float64))
        assert abs(lse[qh, 0] - math.log(math.fsum(math.exp(t) for t in z))) < 1e-12


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------
def _prefill_case(seed, kvh, G, hd, pos0, n_tok):
    r = np.random.default_rng(seed)
    P = pos0 + n_tok
    K16 = r.standard_normal((kvh, P, hd)).astype(np.float16)
    V16 = r.standard_normal((kvh, P, hd)).astype(np.float16)
    K16[:, :, 5] *= 8
    q = r.standard_normal((n_tok, kvh * G, hd)).astype(np.float32)
    return q, K16, V16


def pin_prefill_sdpa_causal(prefill):
    """Full-sequence causal SDPA (top-left aligned, no hand-made mask) with the
    chunk's queries at positions pos0..P-1; the rows before pos0 are fillers."""
    for seed, (kvh, G, hd, pos0, n_tok) in enumerate([(2, 2, 64, 37, 11), (1, 4, 128, 0, 9),
                                                      (2, 1, 128, 64, 64)]):
        q, K16, V16 = _prefill_case(seed, kvh, G, hd, pos0, n_tok)
        sm = 1 / math.sqrt(hd)
        got = prefill(q, K16, V16, pos0, sm)
        P = pos0 + n_tok
        Qfull = np.zeros((P, kvh * G, hd))
        Qfull[pos0:] = q.astype(np.float16).astype(np.float64)
        qt = torch.from_numpy(np.transpose(Qfull, (1, 0, 2)))[None]
        kt = torch.from_numpy(K16.astype(np.float64))[None]
        vt = torch.from_numpy(V16.astype(np.float64))[None]
        o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=float(np.float32(sm)),
                                           enable_gqa=True)
        ref = np.transpose(o[0].numpy(), (1, 0, 2))[pos0:]
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), np.abs(got - ref).max()


def pin_prefill_invariants(prefill, decode):
    kvh, G, hd, pos0, n_tok = 2, 2, 64, 20, 6
    q, K16, V16 = _prefill_case(50, kvh, G, hd, pos0, n_tok)
    sm = 0.125
    full = prefill(q, K16, V16, pos0, sm)
    # each row equals decode of the fp16-rounded query over keys [0, pos0 + i]
    for i in range(n_tok):
        q16 = q[i].astype(np.float16).astype(np.float32)
        d = decode(q16, K16.astype(np.float64), V16.astype(np.float64), pos0 + i + 1, sm)
        assert np.allclose(full[i], d, rtol=1e-12, atol=1e-12), i
    # future keys do not move a row
    i = 2
    K2, V2 = K16.copy(), V16.copy()
    K2[:, pos0 + i + 1:] = 100
    V2[:, pos0 + i + 1:] = -100
    # (to rounding: a product over a different set of rows may sum in another order)
    assert np.allclose(prefill(q, K2, V2, pos0, sm, rows=[i]), full[[i]], rtol=1e-13, atol=1e-13)
    # a row subset equals the same rows of the full result
    assert np.allclose(prefill(q, K16, V16, pos0, sm, rows=[0, 5]), full[[0, 5]], rtol=1e-13,
                       atol=1e-13)


def pin_prefill_brute(prefill, brute_row):
    kvh, G, hd, pos0, n_tok = 1, 2, 8, 3, 4
    q, K16, V16 = _prefill_case(60, kvh, G, hd, pos0, n_tok)
    sm = 0.4
    out = prefill(q, K16, V16, pos0, sm)
    q16 = q.astype(np.float16).astype(np.float64)
    for i in range(n_tok):
        for qh in range(2):
            n = pos0 + i + 1
            ref = brute_row(q16[i, qh], K16[0, :n].astype(np.float64), V16[0, :n].astype(np.float64), sm)
            assert np.allclose(out[i, qh], ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# compaction
# ----------------------------------------------------------------------------
def pin_compact_exact(compact, Cache, FMT_F16, FMT_Q8):
    kvh, hd, cap, n = 2, 128, 64, 40
    r = np.random.default_rng(70)
    xk = r.standard_normal((n, kvh, hd), dtype=np.float32) * np.float32(30)
    xv = r.standard_normal((n, kvh, hd), dtype=np.float32) * np.float32(1e-3)
    for fmt in (FMT_F16, FMT_Q8):
        c = Cache(fmt, kvh, cap, hd)
        assert c.append(0, xk, xv)
        k16, v16 = compact(c, n)
        assert k16.shape == (kvh, n, hd) and k16.dtype == np.float16
        if fmt == FMT_F16:
            assert np.array_equal(k16.view(np.uint16), c.k[:, :n].view(np.uint16))
            assert np.array_equal(v16.view(np.uint16), c.v[:, :n].view(np.uint16))
            continue
        for which, out in (("k", k16), ("v", v16)):
            codes = getattr(c, which)
            sc = getattr(c, which + "_scale")
            for (h, t, d) in [(0, 0, 0), (1, 39, 127), (0, 17, 64), (1, 3, 63), (0, 25, 100)] + \
                    [tuple(r.integers(0, m) for m in (kvh, n, hd)) for _ in range(200)]:
                exact = Fraction(int(codes[h, t, d])) * Fraction(float(sc[h, t, d // 64]))
                assert Fraction(float(out[h, t, d])) == f16(exact), (which, h, t, d)


# ----------------------------------------------------------------------------
# K8V4: rotation, 4-bit quantiser, nibble layout, read-back, byte count
# ----------------------------------------------------------------------------
def _hadamard(n):
    from scipy.linalg import hadamard
    return hadamard(n).astype(np.float64)


def pin_fwht(fwht):
    H = _hadamard(128)
    r = np.random.default_rng(80)
    xi = r.integers(-1000, 1001, size=(20, 128)).astype(np.float32)   # integer rows: exact
    assert np.array_equal(fwht(xi).astype(np.float64), xi.astype(np.float64) @ H.T)
    assert np.array_equal(fwht(fwht(xi)), xi * np.float32(128))        # H H = 128 I
    x = r.standard_normal((50, 128)).astype(np.float32)
    err = np.abs(fwht(x).astype(np.float64) - x.astype(np.float64) @ H.T)
    # seven stages, each rounding a partial sum bounded by the sum of |x|
    assert (err <= 7 * 2.0 ** -24 * np.abs(x).astype(np.float64).sum(-1, keepdims=True)).all()
    for row in r.standard_normal((12, 8)).astype(np.float32):         # order-8 rows, in fractions
        assert [Fraction(float(v)) for v in fwht(row[None])[0]] == fwht_f32_exact(row)
    for row in x[:3]:
        assert [Fraction(float(v)) for v in fwht(row[None])[0]] == fwht_f32_exact(row)


def _q4_block(vals):
    x = np.zeros(32, np.float32)
    x[: len(vals)] = np.asarray(vals, np.float32)
    return x


def pin_q4_worked_examples(quant4):
    # amax 7 -> d = 7/7 = 1 exactly: codes are rint(x), ties to even; -3.5 -> -4
    a = _q4_block([7, -3.5, 0.5, 1.5, 2.5, -7, 0, 6.49])
    # amax 14 -> d = 2: x / 2 = 7, 0.5 -> 0, 1.5 -> 2, -2.5 -> -2, 3.25 -> 3
    b = _q4_block([14, 1, 3, -5, 6.5])
    z = _q4_block([])                              # all zero: d = 0, codes 0
    # amax 0.7 -> d = fp16(0.1) = 0x2E66 = 0.0999755859375; 0.7 / d = 7.0017 -> 7,
    # -0.35 / d = -3.5009 -> -4 (not a tie), 0.05 / d = 0.5001 -> 1
    t = _q4_block([0.7, -0.35, 0.05])
    codes, d = quant4(np.stack([a, b, z, t]))
    bits = [int(v) for v in d.view(np.uint16)[:, 0]]
    assert bits == [0x3C00, 0x4000, 0x0000, 0x2E66], [hex(v) for v in bits]
    assert codes[0, :8].tolist() == [7, -4, 0, 2, 2, -7, 0, 6]
    assert codes[1, :5].tolist() == [7, 0, 2, -2, 3]
    assert not codes[2].any()
    assert codes[3, :3].tolist() == [7, -4, 1]
    # four blocks per 128-dim row, each with its own scale
    row = np.concatenate([a, b, z, t])
    c, s = quant4(row[None])
    assert s.shape == (1, 4) and np.array_equal(c[0], codes.reshape(-1))


def _random_blocks(seed, n):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, 32), dtype=np.float32)
    x *= np.exp2(r.integers(-20, 12, size=(n, 1))).astype(np.float32)
    x[r.random((n, 32)) < 0.05] *= np.float32(20)
    x[:2] = 0
    x[1, 3] = np.float32(-1e-30)
    return x


def pin_q4_brute_force(quant4, n=300):
    x = _random_blocks(81, n)
    codes, d = quant4(x)
    for i in range(n):
        s, c = quant_block_exact(x[i], 7, -7, 7, brute=(i < 8))
        assert Fraction(float(d[i, 0])) == s, i
        assert codes[i].tolist() == c, i


def pin_q4_invariants(quant4):
    x = _random_blocks(82, 4000)
    codes, d = quant4(x)
    c = codes.astype(np.int32)
    s = d[:, 0].astype(np.float64)
    assert np.abs(c).max() <= 7
    normal = s >= 2.0 ** -14
    assert normal.sum() > 1000
    assert (np.abs(c[normal]).max(-1) == 7).all()
    err = np.abs(c * s[:, None] - x.astype(np.float64))
    assert (err[normal] <= s[normal, None] * (0.5 + 2.0 ** -8)).all()
    cn, dn = quant4(-x)
    assert np.array_equal(cn, -codes) and np.array_equal(dn.view(np.uint16), d.view(np.uint16))


def pin_nibbles(pack, unpack):
    # byte j: code 2j + 8 in the low nibble, code 2j + 1 + 8 in the high nibble
    assert pack(np.array([[-8, 7, 0, -1]], np.int8)).tolist() == [[0xF0, 0x78]]
    c = np.random.default_rng(83).integers(-8, 8, size=(7, 128)).astype(np.int8)
    b = pack(c)
    assert b.shape == (7, 64) and b.dtype == np.uint8
    assert np.array_equal(unpack(b), c)
    assert np.array_equal(b & 0x0F, (c[:, 0::2] + 8).astype(np.uint8))


def pin_k8v4_read(Cache, FMT_K8V4, unpack):
    kvh, hd, cap, n = 2, 128, 64, 24
    r = np.random.default_rng(84)
    xk = r.standard_normal((n, kvh, hd), dtype=np.float32)
    xv = r.standard_normal((n, kvh, hd), dtype=np.float32)
    xv[:, :, 5] *= np.float32(20)                                    # an outlier channel
    c = Cache(FMT_K8V4, kvh, cap, hd)
    assert c.append(0, xk, xv)
    assert c.v.shape == (kvh, cap, hd // 2) and c.v_scale.shape == (kvh, cap, hd // 32)
    codes = unpack(c.v[:, :n]).astype(np.float64)
    d = np.repeat(c.v_scale[:, :n].astype(np.float64), 32, axis=-1)
    want = (codes * d) @ _hadamard(hd).T / hd                         # H (code d) / hd
    got = c.dequant("v", n)
    assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
    # error bound: the rotated error is at most d/2 per value, and H / sqrt(hd) is
    # orthonormal, so |V - x|_2 <= sqrt(sum of (d/2)^2 over the row) / sqrt(hd) * sqrt(hd)
    xr = np.transpose(xv, (1, 0, 2)).astype(np.float64)
    row_err = np.sqrt(((got - xr) ** 2).sum(-1))
    bound = np.sqrt(((d / 2 * (1 + 2.0 ** -7)) ** 2).sum(-1)) / np.sqrt(hd)
    assert (row_err <= bound).all()
    assert row_err.max() > 0
    # K is stored exactly as in the int8 format
    assert c.k.dtype == np.int8 and c.k_scale.shape == (kvh, cap, hd // 64)


def pin_k8v4_compact(compact, Cache, FMT_K8V4):
    kvh, hd, cap = 1, 128, 64
    H = _hadamard(hd)
    r = np.random.default_rng(85)
    # dyadic rows: y integer with block maxima 7 * 2^k, x = H y / 128 exactly; then the
    # rotated row is y, d = 2^k, code = y / 2^k, and the compacted V is fp16(x)
    y = r.integers(-7, 8, size=(6, hd)).astype(np.float64)
    y[:, 0::32] = 7
    y *= np.repeat(np.exp2(r.integers(-3, 3, size=(6, hd // 32))), 32, axis=-1)
    x = (y @ H.T) / hd
    xv = x.astype(np.float32)[:, None, :]
    assert np.array_equal(xv[:, 0].astype(np.float64), x)
    c = Cache(FMT_K8V4, kvh, cap, hd)
    assert c.append(0, xv, xv)
    _, v16 = compact(c, 6)
    assert np.array_equal(v16[0].astype(np.float64), np.vectorize(lambda t: float(f16(Fraction(t))))(x))
    # random rows: fp16 of the fraction butterflies of code * d, times 2^-7
    xr = r.standard_normal((5, 1, hd), dtype=np.float32)
    c = Cache(FMT_K8V4, kvh, cap, hd)
    assert c.append(0, xr, xr)
    _, v16 = compact(c, 5)
    u = c.v_rotated(5)[0]
    for t in range(5):
        want = [f16(v / hd) for v in fwht_f32_exact(u[t].astype(np.float32))]
        assert [Fraction(float(v)) for v in v16[0, t]] == want, t


def pin_cache_bytes_k8v4(cache_bytes, FMT_K8V4):
    gold = _load("k8v4_pages.json")
    # any kvh * hd = 512 (e.g. 2 heads of 256): K codes + K scales + V nibbles + V scales
    for kvh, hd in ((2, 256), (4, 128)):
        per_cell = sum(cache_bytes(FMT_K8V4, kvh, 1, hd, p) for p in range(4))
        assert per_cell == gold["bytes_per_cell"], (kvh, hd, per_cell)
    assert cache_bytes(FMT_K8V4, 8, 1, 128, 2) == 8 * 64
    assert cache_bytes(FMT_K8V4, 8, 1, 128, 3) == 8 * 4 * 2


# ----------------------------------------------------------------------------
# saved session image
# ----------------------------------------------------------------------------
def _image_fields(img):
    """The header read field by field at its stated offsets (independent of the
    oracle's parser): version, fmt, kvh, hd, n, body bytes, scales bytes."""
    assert img[:4] == b"KVQ8"
    u32 = [int.from_bytes(img[4 + 4 * i:8 + 4 * i], "little") for i in range(5)]
    u64 = [int.from_bytes(img[24 + 8 * i:32 + 8 * i], "little") for i in range(2)]
    return (*u32, *u64)


def pin_image(save, load, Cache, cache_bytes, FMT_F16, FMT_Q8, FMT_K8V4):
    gold = _load("image_pages.json")
    H, T = gold["header_bytes"], gold["token_bytes"]
    r = np.random.default_rng(67)
    kvh, cap, hd, n = 3, 128, 128, 37
    xk = (r.standard_normal((n, kvh, hd)) * 2).astype(np.float32)
    xv = (r.standard_normal((n, kvh, hd)) * 0.5 + 1).astype(np.float32)
    tokens = r.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    for fmt in (FMT_F16, FMT_Q8, FMT_K8V4):
        c = Cache(fmt, kvh, cap, hd)
        assert c.append(0, xk, xv)
        img = save(c, n, tokens)
        version, f, h, d, nn, body, scales = _image_fields(img)
        assert (f, h, d, nn) == (fmt, kvh, hd, n), fmt
        # version 3 exactly when the cache has scales; the header is 128 bytes, then
        # 4 bytes per token, the body and the scales, sized by the pinned accounting
        assert version == (gold["version_f16"] if fmt == FMT_F16 else gold["version_int8"])
        assert not any(img[40:H])
        parts = [cache_bytes(fmt, kvh, n, hd, p) for p in range(4)]
        assert body == parts[0] + parts[2] and scales == parts[1] + parts[3], fmt
        assert len(img) == H + T * n + body + scales
        assert np.array_equal(np.frombuffer(img[H:H + T * n], "<i4"), tokens)
        # the regions read back as the inputs: K then V in the body, K scales then V
        # scales in the scales body, each [kvh][n][row]
        b0, s0 = H + T * n, H + T * n + body
        kx = np.transpose(xk, (1, 0, 2))
        vx = np.transpose(xv, (1, 0, 2))
        if fmt == FMT_F16:
            assert scales == 0
            k = np.frombuffer(img[b0:b0 + parts[0]], "<f2").reshape(kvh, n, hd)
            v = np.frombuffer(img[b0 + parts[0]:s0], "<f2").reshape(kvh, n, hd)
            assert np.array_equal(k, kx.astype(np.float16)) and np.array_equal(v, vx.astype(np.float16))
        else:
            k = np.frombuffer(img[b0:b0 + parts[0]], np.int8).reshape(kvh, n, hd // 64, 64)
            ks = np.frombuffer(img[s0:s0 + parts[1]], "<f2").reshape(kvh, n, hd // 64, 1).astype(np.float64)
            err = np.abs(k * ks - kx.reshape(k.shape))
            assert np.all(err <= ks * (0.5 + 2.0**-16)), fmt
            assert np.all(np.abs(k).max(-1) == 127), fmt
            if fmt == FMT_Q8:
                # the pages' scales body: 2 x 4 bytes per token and kv head at hd 128
                assert scales == gold["scales_bytes_per_token_head"] * n * kvh
                v = np.frombuffer(img[b0 + parts[0]:s0], np.int8).reshape(kvh, n, hd // 64, 64)
                vs = np.frombuffer(img[s0 + parts[1]:], "<f2").reshape(kvh, n, hd // 64, 1).astype(np.float64)
                assert np.all(np.abs(v * vs - vx.reshape(v.shape)) <= vs * (0.5 + 2.0**-16))
        # a round trip rebuilds rows [0, n) and leaves the rest zero
        d, m, toks = load(img, fmt, kvh, cap, hd)
        assert m == n and np.array_equal(toks, tokens)
        for a in ("k", "v", "k_scale", "v_scale"):
            if getattr(c, a) is not None:
                assert np.array_equal(getattr(d, a), getattr(c, a)), (fmt, a)
        # refusals: a version-2 image of an int8 cache, another format or shape, a
        # short image, a bad magic, more tokens than the capacity
        def refused(b, f=fmt, h=kvh, cp=cap):
            try:
                load(b, f, h, cp, hd)
            except ValueError:
                return True
            return False
        v2 = img[:4] + (2).to_bytes(4, "little") + img[8:]
        assert refused(v2) == (fmt != FMT_F16), fmt
        if fmt != FMT_F16:
            assert not refused(img)
        assert refused(img, f=(fmt + 1) % 3) and refused(img, h=kvh + 1)
        assert refused(img[:-1]) and refused(b"KVQ9" + img[4:])
        assert refused(img, cp=32)
    # an empty image: header only, its version still set by the format, and loadable
    for fmt in (FMT_F16, FMT_Q8, FMT_K8V4):
        c = Cache(fmt, kvh, cap, hd)
        img = save(c, 0, np.zeros(0, np.int32))
        fields = _image_fields(img)
        assert len(img) == H and fields[4:] == (0, 0, 0)
        assert fields[0] == (gold["version_f16"] if fmt == FMT_F16 else gold["version_int8"])
        assert load(img, fmt, kvh, cap, hd)[1] == 0
