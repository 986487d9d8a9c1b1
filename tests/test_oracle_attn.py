"""Oracle decode, split-K merge, prefill and compaction against their pins."""
import oracle
import pins


def test_decode_matches_library_sdpa():
    pins.pin_decode_sdpa(oracle.decode_attn)


def test_decode_closed_forms():
    pins.pin_decode_closed_forms(oracle.decode_attn)


def test_decode_brute_force():
    pins.pin_decode_brute(oracle.decode_attn, oracle.brute_attention_row)


def test_f16_cache_equals_fp32_attention_on_rounded_kv():
    pins.pin_f16_cache_equals_fp32_attention(oracle.decode_attn, oracle.Cache, oracle.FMT_F16)


def test_splitk_merge_equals_single_pass():
    pins.pin_splitk_identity(oracle.decode_attn, oracle.decode_partials, oracle.merge_partials)


def test_prefill_matches_library_causal_sdpa():
    pins.pin_prefill_sdpa_causal(oracle.prefill_attn)


def test_prefill_invariants():
    pins.pin_prefill_invariants(oracle.prefill_attn, oracle.decode_attn)


def test_prefill_brute_force():
    pins.pin_prefill_brute(oracle.prefill_attn, oracle.brute_attention_row)


def test_compaction_exact():
    pins.pin_compact_exact(oracle.compact_f16, oracle.Cache, oracle.FMT_F16, oracle.FMT_Q8)
