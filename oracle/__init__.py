"""CPU oracle (test infrastructure only; see kvq8_oracle.py)."""
from .kvq8_oracle import *  # noqa: F401,F403
from .kvq8_oracle import (GROUP, QMAX, FMT_F16, FMT_Q8, Cache, cache_bytes, quantize_q8,  # noqa: F401
                          store_f16, compact_f16, decode_attn, decode_partials, merge_partials,
                          decode_attn_splitk, prefill_attn, brute_attention_row)
