"""CPU oracle for attention over a reduced-precision (FP16 or int8 "q8") K/V cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product
path (``quantized_kv_cache_q8_amd`` and its HIP library) never does, and this
module imports nothing from it.

Plain, slow, obviously correct NumPy.  Attention is computed in float64 on the
dequantised cache values; the quantiser is computed in float32 (the precision in
which the GPU kernel takes the same integer decisions).

Sources (web pages; cited by title and section):
  [P1] PR #3084 "FP16 K/V cache by default, int8 with --kv-q8 (262144 fits a
       16 GiB card)": sections Summary, What changed, Extra Notes.
  [P2] Issue #67 "Path F format v3: persist per-head INT8 KV scales": sections
       Scope, Phased plan, Not in scope.
  [P3] PR #711 "kv: --kv k8v4 streams with --kv-resident": sections What, How.

Readings where the pages are silent:
  * K8V4 ([P3, What]: int8 K with a rotated 4-bit V): K is the q8 K; V is rotated by
    the orthonormal Walsh-Hadamard matrix H/sqrt(HD) (H the Sylvester Hadamard
    matrix), computed as the unnormalised transform w = H x in fp32 butterflies
    (stages h = 1, 2, 4, ..., HD/2), then quantised per 32-value block with the
    int8 rule with 7 for 127: d = fp16(max|w| / 7), code = clamp(rint(w / d), -7, 7),
    stored as code + 8 in nibbles (byte j: value 2j low, 2j+1 high).  The V a
    read sees is H (code * d) / HD, i.e. H/sqrt(HD) applied to code * d / sqrt(HD)
    ... = the orthonormal rotation undone.  Which rotation and which 4-bit
    rounding the pages' kernels use is not on the pages: those two are readings,
    pinned here to mathematics, not to the pages.
  * fp16(.) is IEEE round-to-nearest-even; rint is round-half-to-even.
  * ``x / scale`` divides by the *stored* fp16 scale widened to fp32, with a
    true IEEE fp32 division (not a reciprocal multiply).
  * a group whose scale is zero stores code 0 (x/0 is otherwise undefined).
  * group g of a head row holds dims [64g, 64g+64) of one token, K and V separately.
  * query head q reads kv head q // G, G = n_q_heads / n_kv_heads.
  * the prompt chunk rounds its queries to fp16 before Q K^T, as the GEMMs read
    halves; row i of a chunk at position pos0 attends keys [0, pos0 + i].
  * saved image ([P2]): the header's fields are not on the pages, so they are this
    module's own (magic, version, format, shape, token count, region sizes); the
    scales body holds the fp16 scale arrays of the format in place of one fp32 per
    token, head and K/V; the version is 3 for every format with scales (also with
    zero tokens) and 2 for FP16.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force with exact rational arithmetic and
independent library routines (torch's CPU scaled-dot-product attention).  No
function here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 64          # dims per fp16 scale  [P1, Summary]
QMAX = 127          # symmetric int8 range [P1, What changed]
Q4_BLOCK = 32       # values per fp16 scale of the 4-bit V (Q4_0 blocks) [P3, What]
Q4_MAX = 7          # symmetric 4-bit range (codes -7 .. 7, stored + 8 in a nibble)
FMT_F16, FMT_Q8, FMT_K8V4 = 0, 1, 2


# ----------------------------------------------------------------------------
# Storage cost
# ----------------------------------------------------------------------------
def cache_bytes(fmt: int, kvh: int, cap: int, hd: int, part: int) -> int:
    """Bytes of one array of one layer.

    part 0: K values (fp16, 2 B each) or int8 codes (1 B each); part 1: the fp16
    K scales of the q8 and K8V4 formats (one 2-B scale per 64 values, [P1,
    Summary]); the FP16 format has no scales.  parts 2 and 3: the same for V, which
    differs only for K8V4 (4-bit codes, 2 per byte, and one fp16 scale per 32
    values [P3, What]).
    """
    n = kvh * cap * hd
    if part in (2, 3) and fmt == FMT_K8V4:
        return n // 2 if part == 2 else 2 * (n // Q4_BLOCK)
    part = part - 2 if part in (2, 3) else part
    if part == 0:
        return 2 * n if fmt == FMT_F16 else n
    return 0 if fmt == FMT_F16 else 2 * (n // GROUP)


# ----------------------------------------------------------------------------
# O1 / O2: writing a cell (quantise-on-write, FP16 store)
# ----------------------------------------------------------------------------
def quantize_q8(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise-on-write of [P1, What changed]: per 64-dim group of a head row,
    scale = fp16(max|x| / 127) and code = clamp(rint(x / scale), -127, 127).

    x: float32 [..., HD], HD a multiple of 64.
    returns (codes int8 [..., HD], scales float16 [..., HD // 64]).
    """
    x = np.asarray(x, dtype=np.float32)
    hd = x.shape[-1]
    assert hd % GROUP == 0
    g = x.reshape(*x.shape[:-1], hd // GROUP, GROUP)
    amax = np.abs(g).max(axis=-1)                        # exact in float32
    s16 = (amax / np.float32(QMAX)).astype(np.float16)   # fp32 division, then RNE to fp16
    s32 = s16.astype(np.float32)[..., None]              # the stored scale, widened
    with np.errstate(divide="ignore", invalid="ignore"):
        r = g / s32                                      # IEEE fp32 division
    r = np.where(s32 == 0, np.float32(0), r)             # all-zero (or underflowed) group
    codes = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)
    return codes.reshape(x.shape), s16


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform over the last axis (length a power of
    two), H x with H the Sylvester Hadamard matrix, as fp32 butterflies: stage h
    (h = 1, 2, 4, ...) maps each pair (i, i + h) inside blocks of 2h to (a + b,
    a - b).  Every output of a stage is one IEEE fp32 addition or subtraction, so
    the result does not depend on the order pairs are visited in."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    assert n & (n - 1) == 0
    lead = y.shape[:-1]
    h = 1
    while h < n:
        z = y.reshape(*lead, n // (2 * h), 2, h)
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(*lead, n)
        h *= 2
    return y


def quantize_q4(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """4-bit quantisation of the rotated V, per 32-value block (the int8 rule with
    7 for 127): d = fp16(max|w| / 7), code = clamp(rint(w / d), -7, 7), a zero scale
    giving code 0.  w: float32 [..., HD].  Returns (codes int8 in -7..7 [..., HD],
    scales float16 [..., HD // 32])."""
    w = np.asarray(w, dtype=np.float32)
    hd = w.shape[-1]
    assert hd % Q4_BLOCK == 0
    g = w.reshape(*w.shape[:-1], hd // Q4_BLOCK, Q4_BLOCK)
    amax = np.abs(g).max(axis=-1)
    d16 = (amax / np.float32(Q4_MAX)).astype(np.float16)
    d32 = d16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = g / d32
    r = np.where(d32 == 0, np.float32(0), r)
    codes = np.clip(np.rint(r), -Q4_MAX, Q4_MAX).astype(np.int8)
    return codes.reshape(w.shape), d16


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """codes int8 -8..7 [..., HD] -> uint8 [..., HD // 2]: byte j holds code 2j + 8
    in its low nibble and code 2j + 1 + 8 in its high nibble."""
    u = (np.asarray(codes, np.int16) + 8).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """The inverse of pack_nibbles: uint8 [..., HD // 2] -> int8 -8..7 [..., HD]."""
    b = np.asarray(b, np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = (b & 0x0F).astype(np.int8) - 8
    out[..., 1::2] = (b >> 4).astype(np.int8) - 8
    return out


def store_f16(x: np.ndarray) -> np.ndarray:
    """FP16 cache write of [P1, Summary]: IEEE round-to-nearest-even to binary16."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


# ----------------------------------------------------------------------------
# Cache (one layer, one session): the data structure of [P1, Summary / What changed]
# ----------------------------------------------------------------------------
class Cache:
    """One session's cache for one layer.

    F16: k, v float16 [kvh][cap][hd].
    Q8 : k, v int8 [kvh][cap][hd] plus k_scale, v_scale float16 [kvh][cap][hd/64]
         (scale arrays kept beside the code arrays, [P1, What changed]; codes and
         scales are separate runs of bytes, [P3, How]).
    K8V4: k, k_scale as Q8; v uint8 [kvh][cap][hd/2] (4-bit codes of the rotated
         row, pack_nibbles), v_scale float16 [kvh][cap][hd/32].
    """

    def __init__(self, fmt: int, kvh: int, cap: int, hd: int):
        self.fmt, self.kvh, self.cap, self.hd = fmt, kvh, cap, hd
        if fmt == FMT_F16:
            self.k = np.zeros((kvh, cap, hd), np.float16)
            self.v = np.zeros((kvh, cap, hd), np.float16)
            self.k_scale = self.v_scale = None
        elif fmt == FMT_K8V4:
            self.k = np.zeros((kvh, cap, hd), np.int8)
            self.k_scale = np.zeros((kvh, cap, hd // GROUP), np.float16)
            self.v = np.zeros((kvh, cap, hd // 2), np.uint8)
            self.v_scale = np.zeros((kvh, cap, hd // Q4_BLOCK), np.float16)
        else:
            self.k = np.zeros((kvh, cap, hd), np.int8)
            self.v = np.zeros((kvh, cap, hd), np.int8)
            self.k_scale = np.zeros((kvh, cap, hd // GROUP), np.float16)
            self.v_scale = np.zeros((kvh, cap, hd // GROUP), np.float16)

    def append(self, pos: int, xk: np.ndarray, xv: np.ndarray) -> bool:
        """Write n_tok new cells at rows [pos, pos + n_tok).  xk, xv: float32
        [n_tok][kvh][hd].  Returns False, writing nothing, when the rows do not fit."""
        n = xk.shape[0]
        if pos < 0 or pos + n > self.cap:
            return False
        for src, dst, dsc in ((xk, "k", "k_scale"), (xv, "v", "v_scale")):
            rows = np.transpose(np.asarray(src, np.float32), (1, 0, 2))  # [kvh][n][hd]
            if self.fmt == FMT_F16:
                getattr(self, dst)[:, pos:pos + n] = store_f16(rows)
            elif self.fmt == FMT_K8V4 and dst == "v":
                c, s = quantize_q4(fwht_f32(rows))
                self.v[:, pos:pos + n] = pack_nibbles(c)
                self.v_scale[:, pos:pos + n] = s
            else:
                c, s = quantize_q8(rows)
                getattr(self, dst)[:, pos:pos + n] = c
                getattr(self, dsc)[:, pos:pos + n] = s
        return True

    # O3: what the decode reads -- exact dequantised values in float64
    def dequant(self, which: str, length: int) -> np.ndarray:
        """float64 [kvh][length][hd].  q8: code * scale, which is exact (a 7-bit
        integer times an 11-bit significand); F16: the stored halves."""
        vals = getattr(self, which)[:, :length]
        if self.fmt == FMT_F16:
            return vals.astype(np.float64)
        sc = getattr(self, which + "_scale")[:, :length].astype(np.float64)
        if self.fmt == FMT_K8V4 and which == "v":
            # the rotation undone: H (code * d) / HD, exact in float64 up to the sum
            rot = self.v_rotated(length)
            return rot @ hadamard_f64(self.hd).T / self.hd
        return vals.astype(np.float64) * np.repeat(sc, GROUP, axis=-1)

    def v_rotated(self, length: int) -> np.ndarray:
        """K8V4: the dequantised rotated V, code * d (exact), float64 [kvh][length][hd]."""
        assert self.fmt == FMT_K8V4
        codes = unpack_nibbles(self.v[:, :length]).astype(np.float64)
        d = self.v_scale[:, :length].astype(np.float64)
        return codes * np.repeat(d, Q4_BLOCK, axis=-1)


# ----------------------------------------------------------------------------
# Moving a session's rows: the packed block of [P1, What changed] (the session-to-slot
# copy sized in the format's elements, with the scales) and [P2, Phased plan]
# (gather to the host, scatter back, the scales beside the KV body)
# ----------------------------------------------------------------------------
ROW_ARRAYS = ("k", "k_scale", "v", "v_scale")


def pack_rows(cache: Cache, row0: int, n: int) -> np.ndarray:
    """uint8: for each array of the format in the order K values, K scales, V values,
    V scales (absent arrays skipped), its rows [row0, row0 + n) of every head as
    [kvh][n][row bytes]."""
    parts = [np.ascontiguousarray(getattr(cache, a)[:, row0:row0 + n]).view(np.uint8).reshape(-1)
             for a in ROW_ARRAYS if getattr(cache, a) is not None]
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)


def unpack_rows(cache: Cache, row0: int, n: int, buf: np.ndarray) -> None:
    """The inverse of pack_rows: write a packed block into rows [row0, row0 + n)."""
    buf = np.asarray(buf, np.uint8)
    off = 0
    for a in ROW_ARRAYS:
        arr = getattr(cache, a)
        if arr is None:
            continue
        dst = arr[:, row0:row0 + n]
        nb = dst.nbytes
        dst[...] = buf[off:off + nb].view(arr.dtype).reshape(dst.shape)
        off += nb
    assert off == buf.size


# ----------------------------------------------------------------------------
# Paged sessions ([P3, How]: a session's K/V move block by block; attention over the
# blocks in a window equals attention over the resident cache).  A page holds 64
# cells; page p (cells 64p .. 64p + 63) lies in slot pages[p] of a pool, rows
# 64 s .. 64 s + 63 of each array.  The session the pool holds is its pages read back
# in order; decode over it is the decode above.
# ----------------------------------------------------------------------------
PAGE_ROWS = 64


def paged_cache(pool: Cache, pages, length: int) -> Cache:
    """The session of `length` cells that page table `pages` describes in `pool`."""
    n_pages = (length + PAGE_ROWS - 1) // PAGE_ROWS
    c = Cache(pool.fmt, pool.kvh, max(PAGE_ROWS, n_pages * PAGE_ROWS), pool.hd)
    for p in range(n_pages):
        s = int(pages[p])
        for name in ROW_ARRAYS:
            a = getattr(pool, name)
            if a is not None:
                getattr(c, name)[:, p * PAGE_ROWS:(p + 1) * PAGE_ROWS] = a[:, s * PAGE_ROWS:(s + 1) * PAGE_ROWS]
    return c


# ----------------------------------------------------------------------------
# A saved session image: [P2, Scope] lays a saved KV file out as a 128-byte header,
# the token ids (4 B each), the KV body and then, new in its version 3, a scales body;
# version 3 is written only when the cache has scales, and version-2 files (no
# scales) stay loadable for FP16 but are refused for an int8 cache [P2, Phased plan
# and Not in scope].  Here the scales body holds the format's fp16 scale arrays
# rather than one fp32 per token, head and K/V.  Header (little-endian): magic
# b"KVQ8", u32 version, u32 format, u32 kv heads, u32 head_dim, u32 tokens, u64 body
# bytes, u64 scales bytes, zeros to 128 bytes.  Body: K values then V values; scales
# body: K scales then V scales; each array's rows [0, n) as [kvh][n][row bytes].
# ----------------------------------------------------------------------------
IMAGE_MAGIC = b"KVQ8"
IMAGE_VERSION = 3
IMAGE_HEADER = 128


def save_image(cache: Cache, n: int, tokens) -> bytes:
    def rows(name):
        a = getattr(cache, name)
        return b"" if a is None else np.ascontiguousarray(a[:, :n]).tobytes()
    body = rows("k") + rows("v")
    scales = rows("k_scale") + rows("v_scale")
    version = 2 if cache.fmt == FMT_F16 else IMAGE_VERSION
    head = (IMAGE_MAGIC + np.array([version, cache.fmt, cache.kvh, cache.hd, n], "<u4").tobytes()
            + np.array([len(body), len(scales)], "<u8").tobytes())
    head += bytes(IMAGE_HEADER - len(head))
    return head + np.asarray(tokens, "<i4").tobytes() + body + scales


def load_image(image: bytes, fmt: int, kvh: int, cap: int, hd: int):
    """Parse an image written by save_image into a fresh Cache; returns (cache, n,
    tokens), or raises ValueError for a wrong magic, version, format or shape, a
    version-2 image (no scales body) of a format with scales, or a short image."""
    b = bytes(image)
    if len(b) < IMAGE_HEADER or b[:4] != IMAGE_MAGIC:
        raise ValueError("not an image")
    version, f, h, d, n = np.frombuffer(b[4:24], "<u4").tolist()
    body_bytes, scale_bytes = np.frombuffer(b[24:40], "<u8").tolist()
    if (f, h, d) != (fmt, kvh, hd):
        raise ValueError("format or shape differs")
    if version not in (2, IMAGE_VERSION) or (version == 2 and fmt != FMT_F16):
        raise ValueError(f"version {version} cannot hold this format")
    if n > cap:
        raise ValueError("more tokens than the capacity")
    c = Cache(fmt, kvh, cap, hd)
    want_body = sum(getattr(c, a)[:, :n].nbytes for a in ("k", "v"))
    want_sc = sum(getattr(c, a)[:, :n].nbytes for a in ("k_scale", "v_scale")
                  if getattr(c, a) is not None)
    if body_bytes != want_body or scale_bytes != want_sc or \
            len(b) < IMAGE_HEADER + 4 * n + want_body + want_sc:
        raise ValueError("sizes differ")
    off = IMAGE_HEADER
    tokens = np.frombuffer(b[off:off + 4 * n], "<i4").copy()
    off += 4 * n
    for name in ("k", "v", "k_scale", "v_scale"):
        a = getattr(c, name)
        if a is None:
            continue
        dst = a[:, :n]
        dst[...] = np.frombuffer(b[off:off + dst.nbytes], a.dtype).reshape(dst.shape)
        off += dst.nbytes
    return c, n, tokens


# ----------------------------------------------------------------------------
# O4: compaction to the FP16 [kvh][P][HD] copy the prompt GEMMs read
# ----------------------------------------------------------------------------
def hadamard_f64(n: int) -> np.ndarray:
    """The Sylvester Hadamard matrix of order n (a power of two), float64."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def compact_f16(cache: Cache, P: int) -> tuple[np.ndarray, np.ndarray]:
    """[P1, Extra Notes]: the prompt chunk's GEMMs read an FP16 [kvh][P][HD] copy
    of the cache.  F16: rows 0..P-1 copied (a stride change only).  q8:
    fp16(float(code) * float(scale)), one rounding of an exact fp32 product.
    K8V4 V: the rotation undone in fp32 -- u = code * d (exact), then
    fp16(fwht_f32(u) * 2^-log2(HD)) (the power of two is exact)."""
    out = []
    for which in ("k", "v"):
        vals = getattr(cache, which)[:, :P]
        if cache.fmt == FMT_K8V4 and which == "v":
            u = cache.v_rotated(P).astype(np.float32)          # exact in fp32
            out.append((fwht_f32(u) * np.float32(1.0 / cache.hd)).astype(np.float16))
        elif cache.fmt == FMT_F16:
            out.append(vals.copy())
        else:
            sc = getattr(cache, which + "_scale")[:, :P].astype(np.float32)
            prod = vals.astype(np.float32) * np.repeat(sc, GROUP, axis=-1)
            out.append(prod.astype(np.float16))
    return out[0], out[1]


# ----------------------------------------------------------------------------
# O5: decode attention, the plain definition
# ----------------------------------------------------------------------------
def decode_attn(q: np.ndarray, K: np.ndarray, V: np.ndarray, length: int,
                sm_scale: float) -> np.ndarray:
    """Attention of one new token over the first ``length`` cached cells.

    q: [nqh][hd] (float32 values); K, V: float64 [kvh][>=length][hd] dequantised
    cache; returns float64 [nqh][hd].  length == 0 returns zeros.
    """
    nqh, hd = q.shape
    kvh = K.shape[0]
    G = nqh // kvh
    out = np.zeros((nqh, hd))
    if length == 0:
        return out
    sm = float(np.float32(sm_scale))
    for qh in range(nqh):
        h = qh // G
        z = sm * (K[h, :length] @ q[qh].astype(np.float64))
        w = np.exp(z - z.max())
        out[qh] = (w @ V[h, :length]) / w.sum()
    return out


# ----------------------------------------------------------------------------
# O6: the same result by split-K partials and a log-sum-exp merge
# ----------------------------------------------------------------------------
def decode_partials(q, K, V, length, sm_scale, T):
    """Per split j (tokens [jT, min((j+1)T, length))): normalised partial output
    o_j and lse_j = m_j + ln(l_j).  An empty split has lse = -inf and o = 0.
    Returns (o float64 [nqh][S][hd], lse float64 [nqh][S]), S = ceil(length / T)."""
    nqh, hd = q.shape
    kvh = K.shape[0]
    G = nqh // kvh
    S = max(1, -(-length // T))
    o = np.zeros((nqh, S, hd))
    lse = np.full((nqh, S), -np.inf)
    sm = float(np.float32(sm_scale))
    for qh in range(nqh):
        h = qh // G
        for j in range(S):
            a, b = j * T, min((j + 1) * T, length)
            if a >= b:
                continue
            z = sm * (K[h, a:b] @ q[qh].astype(np.float64))
            m = z.max()
            w = np.exp(z - m)
            l = w.sum()
            o[qh, j] = (w @ V[h, a:b]) / l
            lse[qh, j] = m + math.log(l)
    return o, lse


def merge_partials(o: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """out = sum_j exp(lse_j - L) o_j with L = log sum_j exp(lse_j); empty splits
    (lse = -inf) weigh zero; all-empty gives zeros."""
    nqh, S, hd = o.shape
    out = np.zeros((nqh, hd))
    for qh in range(nqh):
        m = lse[qh].max()
        if m == -np.inf:
            continue
        w = np.exp(lse[qh] - m)
        L = m + math.log(w.sum())
        out[qh] = (np.exp(lse[qh] - L)[:, None] * o[qh]).sum(axis=0)
    return out


def decode_attn_splitk(q, K, V, length, sm_scale, T):
    return merge_partials(*decode_partials(q, K, V, length, sm_scale, T))


# ----------------------------------------------------------------------------
# O7: prompt-chunk attention, the plain definition
# ----------------------------------------------------------------------------
def prefill_attn(q: np.ndarray, K16: np.ndarray, V16: np.ndarray, pos0: int,
                 sm_scale: float, rows=None) -> np.ndarray:
    """Causal attention of a prompt chunk over the FP16 compacted copy.

    q: float32 [n_tok][nqh][hd] (rounded to fp16 here, as the GEMMs read halves);
    K16, V16: float16 [kvh][P][hd] with P >= pos0 + n_tok.  Row i (absolute
    position pos0 + i) attends keys [0, pos0 + i].  ``rows`` selects a subset of
    chunk rows (all by default).  Returns float64 [len(rows)][nqh][hd].
    """
    n_tok, nqh, hd = q.shape
    kvh = K16.shape[0]
    G = nqh // kvh
    rows = np.arange(n_tok) if rows is None else np.asarray(rows)
    sm = float(np.float32(sm_scale))
    Q16 = np.asarray(q, np.float32).astype(np.float16).astype(np.float64)
    n_max = pos0 + int(rows.max()) + 1
    keys = np.arange(n_max)
    allowed = keys[None, :] <= (pos0 + rows)[:, None]          # row i attends keys [0, pos0 + i]
    out = np.zeros((len(rows), nqh, hd))
    for h in range(kvh):
        Kh = K16[h, :n_max].astype(np.float64)
        Vh = V16[h, :n_max].astype(np.float64)
        for qh in range(h * G, (h + 1) * G):
            Z = sm * (Q16[rows, qh] @ Kh.T)                      # [rows][keys]
            Z = np.where(allowed, Z, -np.inf)
            W = np.exp(Z - Z.max(axis=1, keepdims=True))
            out[:, qh] = (W @ Vh) / W.sum(axis=1, keepdims=True)
    return out


# ----------------------------------------------------------------------------
# O8: brute force on tiny inputs (scalar loops, math.exp / math.fsum)
# ----------------------------------------------------------------------------
def brute_attention_row(qv, Krows, Vrows, sm_scale):
    """One query vector against explicit key/value row lists, scalar Python."""
    sm = float(np.float32(sm_scale))
    z = [sm * math.fsum(float(a) * float(b) for a, b in zip(qv, kr)) for kr in Krows]
    m = max(z)
    w = [math.exp(t - m) for t in z]
    l = math.fsum(w)
    hd = len(Vrows[0])
    return [math.fsum(w[t] * float(Vrows[t][d]) for t in range(len(w))) / l for d in range(hd)]
