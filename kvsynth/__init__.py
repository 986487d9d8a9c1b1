"""Seeded synthetic inputs for the reduced-precision K/V-cache attention path.

This module is the only code shared by the CPU oracle's tests and the GPU path's
tests and benchmark.  It draws random numbers and lays them out; it holds none of
the method's arithmetic (no quantisation, no rounding to the cache format, no
attention).

Every stream is ``numpy.random.default_rng([seed, layer, stream, sub])`` so that
each purpose (K, V, Q, outlier channels, new tokens, session lengths, prefill Q)
draws from its own reproducible generator, independent of call order.

Value model (stand-in for a model's K/V activations, which need trained weights):
values are standard normal float32; optionally 4 distinct channels per
(layer, kv head) are scaled by 20, fixed across tokens, separately for K and V.
"""
from __future__ import annotations

import numpy as np

# stream ids
S_K, S_V, S_Q, S_K_OUT, S_V_OUT, S_K_NEW, S_V_NEW, S_LENS, S_Q_PREFILL = range(9)

N_OUTLIERS = 4
OUTLIER_GAIN = np.float32(20.0)


def rng(seed: int, layer: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(layer), int(stream), int(sub)])


def outlier_channels(seed: int, layer: int, kvh: int, hd: int, which: str) -> np.ndarray:
    """int64 [kvh][4]: the outlier channel indices of each kv head (``which`` is 'K' or 'V')."""
    stream = S_K_OUT if which == "K" else S_V_OUT
    r = rng(seed, layer, stream)
    return np.stack([r.choice(hd, N_OUTLIERS, replace=False) for _ in range(kvh)])


def kv_tokens(seed: int, layer: int, n_tok: int, kvh: int, hd: int, which: str,
              outliers: bool, stream: int | None = None, sub: int = 0) -> np.ndarray:
    """float32 [n_tok][kvh][hd]: K or V rows of ``n_tok`` consecutive token positions.

    ``stream`` defaults to the cache-fill stream of ``which`` (K or V); the per-step
    new-token streams are S_K_NEW / S_V_NEW.  ``sub`` separates sessions or steps.
    """
    if stream is None:
        stream = S_K if which == "K" else S_V
    x = rng(seed, layer, stream, sub).standard_normal((n_tok, kvh, hd), dtype=np.float32)
    if outliers:
        ch = outlier_channels(seed, layer, kvh, hd, which)
        for h in range(kvh):
            x[:, h, ch[h]] *= OUTLIER_GAIN
    return x


def queries(seed: int, layer: int, n: int, nqh: int, hd: int, stream: int = S_Q,
            sub: int = 0, half_grid: bool = False) -> np.ndarray:
    """float32 [n][nqh][hd] standard-normal queries.

    ``half_grid`` snaps the draws onto values representable in IEEE binary16, for
    workloads whose queries arrive as fp16 activations.
    """
    x = rng(seed, layer, stream, sub).standard_normal((n, nqh, hd), dtype=np.float32)
    if half_grid:
        x = x.astype(np.float16).astype(np.float32)
    return x


def session_lengths(seed: int, n_sess: int, lo: int, hi: int) -> np.ndarray:
    """int64 [n_sess], uniform on the closed range [lo, hi]."""
    return rng(seed, 0, S_LENS).integers(lo, hi, size=n_sess, endpoint=True)


def round_up(x: int, m: int) -> int:
    return (int(x) + m - 1) // m * m


# Named workloads (shapes of the pages' workloads; synthetic values).
WORKLOADS = {
    # tiny int8 cache, no outliers: parity case the oracle finishes in well under a second
    "tiny_q8_ctx1024": dict(seed=11, layers=1, kvh=2, nqh=4, hd=128, ctx=1024, batch=1,
                            fmt="q8", outliers=False),
    # FP16 cache at 32768 context, outlier channels, fp16-grid queries
    "f16_ctx32768": dict(seed=22, layers=1, kvh=8, nqh=32, hd=128, ctx=32768, batch=1,
                         fmt="f16", outliers=True),
    # int8 cache at 131072 context, quantised on write
    "q8_ctx131072": dict(seed=33, layers=1, kvh=8, nqh=32, hd=128, ctx=131072, batch=1,
                         fmt="q8", outliers=True),
    # full 262144 context, 48 layers, both formats
    "full_ctx262144_48l": dict(seed=44, layers=48, kvh=8, nqh=32, hd=128, ctx=262144, batch=1,
                               fmt="both", outliers=True),
    # 64 sessions with lengths uniform on [1024, 65536] in one int8 session table
    "batched64_q8": dict(seed=55, layers=1, kvh=8, nqh=32, hd=128, lo=1024, hi=65536,
                         batch=64, fmt="q8", outliers=True),
    # one 4096-token prompt chunk at position 131072 of an int8 cache
    "prefill4096_at131072": dict(seed=55, layers=1, kvh=8, nqh=32, hd=128, pos0=131072,
                                 n_tok=4096, fmt="q8", outliers=True),
}
