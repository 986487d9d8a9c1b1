"""The K8V4 parts of the oracle (rotated 4-bit V) against their pins."""
import oracle
import pins
from oracle import kvq8_oracle as o


def test_fwht():
    pins.pin_fwht(o.fwht_f32)


def test_q4_worked_examples():
    pins.pin_q4_worked_examples(o.quantize_q4)


def test_q4_brute_force():
    pins.pin_q4_brute_force(o.quantize_q4)


def test_q4_invariants():
    pins.pin_q4_invariants(o.quantize_q4)


def test_nibbles():
    pins.pin_nibbles(o.pack_nibbles, o.unpack_nibbles)


def test_k8v4_read():
    pins.pin_k8v4_read(oracle.Cache, o.FMT_K8V4, o.unpack_nibbles)


def test_k8v4_compact():
    pins.pin_k8v4_compact(oracle.compact_f16, oracle.Cache, o.FMT_K8V4)


def test_cache_bytes_k8v4():
    pins.pin_cache_bytes_k8v4(oracle.cache_bytes, o.FMT_K8V4)
