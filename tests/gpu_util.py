"""Helpers for the GPU parity tests: device buffers in, numpy out.

Inputs come from kvsynth (seeded, host side); expected values come from the CPU
oracle run on those same host inputs.  Nothing read back from the GPU is fed to
the oracle.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import quantized_kv_cache_q8_amd as kq

DEV = "cuda"
ATOL, RTOL = 2e-3, 1e-3   # attention outputs vs the fp64 oracle (allclose form)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def shape(fmt, kvh, nqh, hd=128):
    return kq.make_shape(fmt, kvh, nqh, hd)


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def append_bulk(sh, sessions, lens, xk, xv, chunk=None):
    """Append xk/xv (fp32 [n_sess][n_tok][kvh][hd]) at rows lens[b].. of each
    session with kv_append; returns the device status word."""
    tab = kq.session_table([s.entry() for s in sessions])
    n_sess, n_tok = xk.shape[0], xk.shape[1]
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    chunk = chunk or n_tok
    for t0 in range(0, n_tok, chunk):
        t1 = min(n_tok, t0 + chunk)
        lt = to_dev(np.asarray(lens, np.int32) + t0)
        kq.kv_append(sh, tab, lt, n_sess, t1 - t0, to_dev(xk[:, t0:t1]), to_dev(xv[:, t0:t1]), status)
    torch.cuda.synchronize()
    return int(status.item())


def download(sess: kq.Session):
    out = {}
    for name in ("k", "v", "k_scale", "v_scale"):
        t = getattr(sess, name)
        if t is not None:
            out[name] = t.cpu().numpy()
    return out


def assert_cache_equal(sess: kq.Session, ref: oracle.Cache, rows=None):
    """Bit-exact comparison of codes/values and scales (as integer bit patterns)."""
    got = download(sess)
    sl = slice(None) if rows is None else rows
    if sess.fmt == kq.KV_FMT_F16:
        for w in ("k", "v"):
            a = got[w][:, sl].view(np.uint16)
            b = getattr(ref, w)[:, sl].view(np.uint16)
            assert np.array_equal(a, b), f"{w}: {np.count_nonzero(a != b)} fp16 values differ"
    else:
        for w in ("k", "v"):
            a, b = got[w][:, sl], getattr(ref, w)[:, sl]
            assert np.array_equal(a, b), f"{w}: {np.count_nonzero(a != b)} codes differ"
            a = got[w + "_scale"][:, sl].view(np.uint16)
            b = getattr(ref, w + "_scale")[:, sl].view(np.uint16)
            assert np.array_equal(a, b), f"{w}_scale: {np.count_nonzero(a != b)} scales differ"


def oracle_cache(fmt, kvh, cap, hd, xk_rows, xv_rows, pos=0):
    """Oracle cache for one session from fp32 [n][kvh][hd] rows written at pos."""
    c = oracle.Cache(fmt, kvh, cap, hd)
    assert c.append(pos, xk_rows, xv_rows)
    return c


def decode_gpu(sh, sessions, lens, q, sm_scale, max_len=None, status=None, ws=None):
    n_sess = len(sessions)
    tab = kq.session_table([s.entry() for s in sessions])
    lt = to_dev(np.asarray(lens, np.int32))
    max_len = int(max(lens)) if max_len is None else max_len
    if ws is None:
        ws = kq.kv_decode_workspace(sh, n_sess, max_len, DEV)
    out = torch.full((n_sess, sh.n_q_heads, sh.head_dim), float("nan"), device=DEV)
    qd = to_dev(q.astype(np.float32))
    kq.kv_decode_attn(sh, tab, lt, n_sess, max_len, qd, sm_scale, out, ws, status)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check_close(got, ref, what, atol=ATOL, rtol=RTOL):
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    say(f"  {what}: max_abs={err.max():.3e} max_rel(|ref|>1e-2)="
        f"{rel[np.abs(ref) > 1e-2].max() if (np.abs(ref) > 1e-2).any() else 0:.3e} "
        f"worst_ratio={np.max(err / bound):.3f}")
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside atol={atol} rtol={rtol}"


def sm_scale(hd=128):
    return float(np.float32(1.0 / math.sqrt(hd)))


# Fidelity gate of the decode, tighter than the tolerance: every output element
# within FID_C * A_d + FID_ABS of the fp64 reference, where A_d = sum_t w_t |V_td| /
# sum_t w_t is the attention of the same weights over |V| (computed by the oracle).
# The int8 decode carries each weight p * s_v as two bf16 values with
# |w - hi - lo| <= 2^-16 |w|, which moves an output by at most 2^-16 A_d; the
# three-level int8 split of the query leaves a residual of about 2^-24 of each
# group's largest query value, and the rest is fp32 rounding of products and sums
# (together measured under 0.5 x 2^-16 A_d on every decode test).  FID_C = 2^-14
# leaves 4x the weight-split term; a two-level query split or a single bf16 weight
# (2^-8 A_d) lands far outside.  K8V4 sums the rotated values u = code * d with the
# same weight split and applies H / 128 after the merge, which averages the rotated
# sums' errors over the dims: its A_d is the mean over dims of the attention over |u|.
FID_C = 2.0 ** -14
FID_ABS = 1e-6


def check_fidelity(got, ref, absref, what):
    err = np.abs(got - ref)
    bound = FID_C * absref + FID_ABS
    ratio = err / (2.0 ** -16 * absref + FID_ABS)
    say(f"  {what} fidelity: max_abs={err.max():.3e} worst err/(2^-16 A + 1e-6)={ratio.max():.3f} "
        f"worst err/bound={np.max(err / bound):.3f}")
    assert (err <= bound).all(), f"{what}: {(err > bound).sum()} of {err.size} outside the fidelity gate"
