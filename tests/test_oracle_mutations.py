"""Planted mistakes in copies of the oracle's functions must each fail a pin.

This shows the pins are strong enough: a dropped term, a wrong sign, index,
rounding mode or operand in the oracle would not go unnoticed.  Mistakes are
planted only here, in CPU code.
"""
import math

import numpy as np
import pytest

import oracle
import pins


def _fails(pin, *args):
    try:
        pin(*args)
    except AssertionError:
        return True
    return False


# ----------------------------------------------------------------------------
# quantiser mutants
# ----------------------------------------------------------------------------
def _quant_template(x, amax_fn=None, divisor=127.0, scale_dtype=np.float16, divide="div",
                    rounding="rint", lo=-127, hi=127, group=64, trunc_scale=False):
    x = np.asarray(x, np.float32)
    g = x.reshape(*x.shape[:-1], x.shape[-1] // group, group)
    amax = amax_fn(g) if amax_fn else np.abs(g).max(-1)
    s = amax / np.float32(divisor)
    if trunc_scale:   # truncate toward zero to fp16 instead of rounding to nearest even
        bits = s.astype(np.float32).view(np.uint32)
        s16 = np.where(s >= 2.0 ** -14, (bits & np.uint32(0xFFFFE000)).view(np.float32), s).astype(np.float16)
    else:
        s16 = s.astype(scale_dtype)
    sw = (s16.astype(np.float32) if scale_dtype == np.float16 else s.astype(np.float32))[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = g * (np.float32(1) / sw) if divide == "recip" else g / sw
    r = np.where(sw == 0, np.float32(0), r)
    if rounding == "rint":
        q = np.rint(r)
    elif rounding == "half_away":
        q = np.sign(r) * np.floor(np.abs(r) + np.float32(0.5))
    else:
        q = np.trunc(r)
    codes = np.clip(q, lo, hi).astype(np.int8)
    s_out = s16 if scale_dtype == np.float16 else s.astype(np.float16)
    return codes.reshape(x.shape), s_out.reshape(*x.shape[:-1], x.shape[-1] // group)


QUANT_MUTANTS = {
    "divide by 128": dict(divisor=128.0),
    "reciprocal multiply": dict(divide="recip"),
    "round half away from zero": dict(rounding="half_away"),
    "truncate instead of round": dict(rounding="trunc"),
    "divide by unrounded fp32 scale": dict(scale_dtype=np.float32),
    "signed max instead of max abs": dict(amax_fn=lambda g: g.max(-1)),
    "clamp to -128": dict(lo=-128),
    "scale truncated to fp16": dict(trunc_scale=True),
    "group of 32": dict(group=32),
}


@pytest.mark.parametrize("name", list(QUANT_MUTANTS))
def test_quant_mutant_is_caught(name):
    kw = QUANT_MUTANTS[name]
    mutant = lambda x: _quant_template(x, **kw)  # noqa: E731
    caught = []
    for pin in pins.QUANT_PINS:
        try:
            if _fails(pin, mutant):
                caught.append(pin.__name__)
        except Exception:           # shape errors count as caught too
            caught.append(pin.__name__ + " (error)")
    assert caught, name


def test_unmutated_template_passes_all_pins():
    for pin in pins.QUANT_PINS:
        pin(lambda x: _quant_template(x))


def test_cache_bytes_mutants_caught():
    def fp32_scales(fmt, kvh, cap, hd, part):
        return oracle.cache_bytes(fmt, kvh, cap, hd, part) * (2 if part == 1 else 1)

    def group_32(fmt, kvh, cap, hd, part):
        return oracle.cache_bytes(fmt, kvh, cap, hd, part) * (2 if part == 1 else 1)

    def f16_one_byte(fmt, kvh, cap, hd, part):
        return kvh * cap * hd if part == 0 else oracle.cache_bytes(fmt, kvh, cap, hd, part)

    for m in (fp32_scales, group_32, f16_one_byte):
        assert _fails(pins.pin_cache_bytes_pages, m, oracle.FMT_F16, oracle.FMT_Q8), m.__name__


# ----------------------------------------------------------------------------
# decode / split-K mutants
# ----------------------------------------------------------------------------
def _decode_template(q, K, V, length, sm_scale, head_map="div", use_scale=True, norm="sum",
                     off=0):
    nqh, hd = q.shape
    kvh = K.shape[0]
    G = nqh // kvh
    out = np.zeros((nqh, hd))
    if length == 0:
        return out
    sm = float(np.float32(sm_scale)) if use_scale else 1.0
    n = length + off
    for qh in range(nqh):
        h = qh // G if head_map == "div" else qh % kvh
        z = sm * (K[h, :n] @ q[qh].astype(np.float64))
        w = np.exp(z - z.max())
        den = w.sum() if norm == "sum" else n
        out[qh] = (w @ V[h, :n]) / den
    return out


DECODE_MUTANTS = {
    "kv head q % kvh": dict(head_map="mod"),
    "softmax scale dropped": dict(use_scale=False),
    "normalise by length": dict(norm="len"),
    "one cell too many": dict(off=1),
}


@pytest.mark.parametrize("name", list(DECODE_MUTANTS))
def test_decode_mutant_is_caught(name):
    kw = DECODE_MUTANTS[name]
    mutant = lambda *a: _decode_template(*a, **kw)  # noqa: E731
    caught = [p.__name__ for p in pins.DECODE_PINS if _fails(p, mutant)]
    caught += ["brute"] if _fails(pins.pin_decode_brute, mutant, oracle.brute_attention_row) else []
    assert caught, name


def test_unmutated_decode_template_passes():
    for p in pins.DECODE_PINS:
        p(_decode_template)


def _merge_mutant_no_shift(o, lse):
    nqh, S, hd = o.shape
    out = np.zeros((nqh, hd))
    for qh in range(nqh):
        w = np.exp(lse[qh])                  # forgets to divide by the total
        out[qh] = (w[:, None] * o[qh]).sum(0)
    return out


def _merge_mutant_uniform(o, lse):
    return o.mean(axis=1)


def _partials_mutant_unnormalised(q, K, V, length, sm_scale, T):
    o, lse = oracle.decode_partials(q, K, V, length, sm_scale, T)
    # returns o scaled by l_j (forgets the per-split normalisation)
    return o * np.exp(lse - lse.max(axis=1, keepdims=True))[:, :, None], lse


def test_splitk_mutants_caught():
    for merge in (_merge_mutant_no_shift, _merge_mutant_uniform):
        assert _fails(pins.pin_splitk_identity, oracle.decode_attn, oracle.decode_partials, merge)
    assert _fails(pins.pin_splitk_identity, oracle.decode_attn, _partials_mutant_unnormalised,
                  oracle.merge_partials)


# ----------------------------------------------------------------------------
# prefill / compaction mutants
# ----------------------------------------------------------------------------
def _prefill_template(q, K16, V16, pos0, sm_scale, rows=None, mask="ok", round_q=True):
    n_tok, nqh, hd = q.shape
    kvh = K16.shape[0]
    G = nqh // kvh
    rows = np.arange(n_tok) if rows is None else np.asarray(rows)
    sm = float(np.float32(sm_scale))
    Q = np.asarray(q, np.float32)
    Q = Q.astype(np.float16).astype(np.float64) if round_q else Q.astype(np.float64)
    out = np.zeros((len(rows), nqh, hd))
    for qh in range(nqh):
        h = qh // G
        for r, i in enumerate(rows):
            n_keys = {"ok": pos0 + i + 1, "excl_self": pos0 + i, "no_pos0": i + 1,
                      "none": K16.shape[1]}[mask]
            n_keys = max(n_keys, 1)
            z = sm * (K16[h, :n_keys].astype(np.float64) @ Q[i, qh])
            w = np.exp(z - z.max())
            out[r, qh] = (w @ V16[h, :n_keys].astype(np.float64)) / w.sum()
    return out


@pytest.mark.parametrize("kw", [dict(mask="excl_self"), dict(mask="no_pos0"), dict(mask="none"),
                                dict(round_q=False)])
def test_prefill_mutant_is_caught(kw):
    mutant = lambda *a, **k: _prefill_template(*a, **k, **kw)  # noqa: E731
    assert (_fails(pins.pin_prefill_sdpa_causal, mutant)
            or _fails(pins.pin_prefill_invariants, mutant, oracle.decode_attn)
            or _fails(pins.pin_prefill_brute, mutant, oracle.brute_attention_row)), kw


def test_unmutated_prefill_template_passes():
    pins.pin_prefill_sdpa_causal(_prefill_template)
    pins.pin_prefill_invariants(_prefill_template, oracle.decode_attn)


def test_compaction_mutants_caught():
    def codes_only(cache, P):
        k, v = oracle.compact_f16(cache, P)
        if cache.fmt == oracle.FMT_Q8:
            return cache.k[:, :P].astype(np.float16), cache.v[:, :P].astype(np.float16)
        return k, v

    def wrong_group(cache, P):
        if cache.fmt != oracle.FMT_Q8:
            return oracle.compact_f16(cache, P)
        out = []
        for which in ("k", "v"):
            sc = getattr(cache, which + "_scale")[:, :P].astype(np.float32)
            sc = np.tile(sc, (1, 1, 64))        # interleaves groups instead of repeating
            out.append((getattr(cache, which)[:, :P].astype(np.float32) * sc).astype(np.float16))
        return tuple(out)

    def truncating(cache, P):
        k, v = oracle.compact_f16(cache, P)
        if cache.fmt != oracle.FMT_Q8:
            return k, v
        out = []
        for which in ("k", "v"):
            sc = getattr(cache, which + "_scale")[:, :P].astype(np.float32)
            prod = getattr(cache, which)[:, :P].astype(np.float32) * np.repeat(sc, 64, -1)
            bits = prod.view(np.uint32) & np.uint32(0xFFFFE000)
            out.append(bits.view(np.float32).astype(np.float16))
        return tuple(out)

    for m in (codes_only, wrong_group, truncating):
        assert _fails(pins.pin_compact_exact, m, oracle.Cache, oracle.FMT_F16, oracle.FMT_Q8), \
            m.__name__
    assert math.isfinite(1.0)


# ----------------------------------------------------------------------------
# K8V4 mutants: rotation, 4-bit quantiser, nibble layout, read-back, bytes
# ----------------------------------------------------------------------------
from oracle import kvq8_oracle as _o  # noqa: E402


def _fwht_template(x, sign="ab", stages=None):
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    lead = y.shape[:-1]
    h, k = 1, 0
    while h < n and (stages is None or k < stages):
        z = y.reshape(*lead, n // (2 * h), 2, h)
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b if sign == "ab" else b - a], axis=-2).reshape(*lead, n)
        h *= 2
        k += 1
    return y


@pytest.mark.parametrize("kw", [dict(sign="ba"), dict(stages=6)])
def test_fwht_mutant_is_caught(kw):
    assert _fails(pins.pin_fwht, lambda x: _fwht_template(x, **kw)), kw


def test_unmutated_fwht_template_passes():
    pins.pin_fwht(_fwht_template)


def _q4_template(w, divisor=7.0, lo=-7, hi=7, rounding="rint"):
    w = np.asarray(w, np.float32)
    g = w.reshape(*w.shape[:-1], w.shape[-1] // 32, 32)
    d16 = (np.abs(g).max(-1) / np.float32(divisor)).astype(np.float16)
    d32 = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d32 == 0, np.float32(0), g / d32)
    q = np.rint(r) if rounding == "rint" else np.trunc(r)
    return np.clip(q, lo, hi).astype(np.int8).reshape(w.shape), d16


Q4_MUTANTS = {"divide by 8": dict(divisor=8.0), "clamp to -8": dict(lo=-8),
              "truncate": dict(rounding="trunc")}


@pytest.mark.parametrize("name", list(Q4_MUTANTS))
def test_q4_mutant_is_caught(name):
    mutant = lambda w: _q4_template(w, **Q4_MUTANTS[name])  # noqa: E731
    caught = [p.__name__ for p in (pins.pin_q4_worked_examples, pins.pin_q4_brute_force,
                                   pins.pin_q4_invariants) if _fails(p, mutant)]
    assert caught, name


def test_unmutated_q4_template_passes():
    for p in (pins.pin_q4_worked_examples, pins.pin_q4_brute_force, pins.pin_q4_invariants):
        p(_q4_template)


def test_nibble_order_mutant_is_caught():
    def pack_high_first(c):
        u = (np.asarray(c, np.int16) + 8).astype(np.uint8)
        return ((u[..., 0::2] << 4) | u[..., 1::2]).astype(np.uint8)

    def unpack_high_first(b):
        out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
        out[..., 0::2] = (b >> 4).astype(np.int8) - 8
        out[..., 1::2] = (b & 0x0F).astype(np.int8) - 8
        return out

    assert _fails(pins.pin_nibbles, pack_high_first, unpack_high_first)


def test_k8v4_read_mutants_caught():
    class NoInverseScale(oracle.Cache):      # forgets the 1/HD of the inverse rotation
        def dequant(self, which, length):
            out = super().dequant(which, length)
            return out * self.hd if which == "v" and self.fmt == _o.FMT_K8V4 else out

    class NotRotatedBack(oracle.Cache):      # returns the rotated V as if it were V
        def dequant(self, which, length):
            if which == "v" and self.fmt == _o.FMT_K8V4:
                return self.v_rotated(length)
            return super().dequant(which, length)

    for m in (NoInverseScale, NotRotatedBack):
        assert _fails(pins.pin_k8v4_read, m, _o.FMT_K8V4, _o.unpack_nibbles), m.__name__


def test_k8v4_bytes_mutant_caught():
    def v_scales_per_64(fmt, kvh, cap, hd, part):
        if fmt == _o.FMT_K8V4 and part == 3:
            return 2 * (kvh * cap * hd // 64)
        return oracle.cache_bytes(fmt, kvh, cap, hd, part)

    assert _fails(pins.pin_cache_bytes_k8v4, v_scales_per_64, _o.FMT_K8V4)


# ----------------------------------------------------------------------------
# saved image mutants: region order, scale interleave, version rule, token width
# ----------------------------------------------------------------------------
def _save_template(cache, n, tokens, order=("k", "v"), sc_order=("k_scale", "v_scale"),
                   interleave=False, always_v3=False, tok_dtype="<i4", version_from_bytes=False):
    def rows(name):
        a = getattr(cache, name)
        return b"" if a is None else np.ascontiguousarray(a[:, :n]).tobytes()
    body = b"".join(rows(a) for a in order)
    if interleave and cache.k_scale is not None:
        scales = b"".join(np.ascontiguousarray(getattr(cache, a)[h, :n]).tobytes()
                          for h in range(cache.kvh) for a in sc_order)
    else:
        scales = b"".join(rows(a) for a in sc_order)
    version = 3 if (cache.fmt != oracle.FMT_F16 or always_v3) else 2
    if version_from_bytes:
        version = 3 if scales else 2
    head = (b"KVQ8" + np.array([version, cache.fmt, cache.kvh, cache.hd, n], "<u4").tobytes()
            + np.array([len(body), len(scales)], "<u8").tobytes())
    head += bytes(128 - len(head))
    return head + np.asarray(tokens, tok_dtype).tobytes() + body + scales


def _pin_image_with(save=None, load=None):
    return _fails(pins.pin_image, save or oracle.save_image, load or oracle.load_image,
                  oracle.Cache, oracle.cache_bytes, oracle.FMT_F16, oracle.FMT_Q8,
                  oracle.FMT_K8V4)


IMAGE_MUTANTS = {
    "V body before K": dict(order=("v", "k")),
    "V scales before K scales": dict(sc_order=("v_scale", "k_scale")),
    "scales interleaved per head": dict(interleave=True),
    "version 3 for FP16": dict(always_v3=True),
    "8-byte token ids": dict(tok_dtype="<i8"),
    "version from the scale bytes": dict(version_from_bytes=True),
}


@pytest.mark.parametrize("name", sorted(IMAGE_MUTANTS))
def test_image_save_mutant_is_caught(name):
    kw = IMAGE_MUTANTS[name]
    assert _pin_image_with(save=lambda c, n, t: _save_template(c, n, t, **kw)), name


def test_unmutated_image_template_passes():
    assert not _pin_image_with(save=_save_template)


def test_image_load_accepting_v2_for_int8_is_caught():
    def lenient(img, fmt, kvh, cap, hd):
        b = bytearray(img)
        if int.from_bytes(b[4:8], "little") == 2:
            b[4:8] = (3).to_bytes(4, "little")
        return oracle.load_image(bytes(b), fmt, kvh, cap, hd)
    assert _pin_image_with(load=lenient)
