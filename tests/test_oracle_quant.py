"""Oracle quantiser, FP16 store, byte accounting and cache bookkeeping against their pins."""
import numpy as np

import oracle
import pins


def test_worked_examples():
    pins.pin_quant_worked_examples(oracle.quantize_q8)


def test_brute_force_exact_rational():
    pins.pin_quant_brute_force(oracle.quantize_q8)


def test_invariants():
    pins.pin_quant_invariants(oracle.quantize_q8)


def test_every_fp16_scale():
    pins.pin_quant_scale_sweep(oracle.quantize_q8)


def test_reciprocal_trap_cases():
    pins.pin_quant_recip_traps(oracle.quantize_q8)


def test_cache_bytes_match_pages():
    pins.pin_cache_bytes_pages(oracle.cache_bytes, oracle.FMT_F16, oracle.FMT_Q8)


def test_cache_bytes_full_context_layer():
    # one layer of 8 kv heads x 128 dims at 262144 cells: 1 GiB (FP16) or 0.515625 GiB (q8), K+V
    f16 = 2 * sum(oracle.cache_bytes(oracle.FMT_F16, 8, 262144, 128, p) for p in (0, 1))
    q8 = 2 * sum(oracle.cache_bytes(oracle.FMT_Q8, 8, 262144, 128, p) for p in (0, 1))
    assert f16 == 1073741824 and q8 == 553648128


def test_store_f16_is_ieee_rne():
    # 1 + 2^-11 is a tie between 1 and 1 + 2^-10: even significand wins (1.0);
    # 1 + 3*2^-11 ties between 1+2^-10 and 1+2^-9: goes to 1 + 2^-9
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26], np.float32)
    got = oracle.store_f16(x).astype(np.float64)
    assert got.tolist() == [1.0, 1 + 2.0 ** -9, 65504.0, 2.0 ** -24, 0.0, 2.0 ** -24]


def _naive_append_reference(fmt, kvh, cap, hd, pos, xk):
    """Element loops: where row (token t, head h) of the input must land."""
    c = oracle.Cache(fmt, kvh, cap, hd)
    n = xk.shape[0]
    for t in range(n):
        for h in range(kvh):
            if fmt == oracle.FMT_F16:
                c.k[h, pos + t] = oracle.store_f16(xk[t, h])
            else:
                codes, s = oracle.quantize_q8(xk[t, h])
                c.k[h, pos + t] = codes
                c.k_scale[h, pos + t] = s
    return c


def test_append_layout_and_bounds():
    r = np.random.default_rng(5)
    kvh, cap, hd, pos, n = 3, 64, 128, 13, 7
    xk = r.standard_normal((n, kvh, hd), dtype=np.float32)
    xv = r.standard_normal((n, kvh, hd), dtype=np.float32)
    for fmt in (oracle.FMT_F16, oracle.FMT_Q8):
        c = oracle.Cache(fmt, kvh, cap, hd)
        assert c.append(pos, xk, xv)
        ref = _naive_append_reference(fmt, kvh, cap, hd, pos, xk)
        assert np.array_equal(c.k, ref.k)
        if fmt == oracle.FMT_Q8:
            assert np.array_equal(c.k_scale.view(np.uint16), ref.k_scale.view(np.uint16))
        # rows outside [pos, pos+n) untouched
        assert not c.k[:, :pos].any() and not c.k[:, pos + n:].any()
        # does not fit: nothing written
        c2 = oracle.Cache(fmt, kvh, cap, hd)
        assert not c2.append(cap - n + 1, xk, xv)
        assert not c2.k.any()
    # dequant of q8 is code * scale, exactly
    c = oracle.Cache(oracle.FMT_Q8, kvh, cap, hd)
    c.append(0, xk, xv)
    d = c.dequant("v", n)
    assert d[1, 2, 70] == float(c.v[1, 2, 70]) * float(c.v_scale[1, 2, 1])
