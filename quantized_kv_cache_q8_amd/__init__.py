"""Python binding of libkvq8 (reduced-precision K/V-cache attention, MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP library; these
wrappers check dtypes, contiguity and devices of torch tensors, pass their device
pointers and the current HIP stream, and raise KvError on a negative status.
The names are those of the C ABI in include/kvq8.h.

If libkvq8.so is not built, importing this package raises ImportError: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq8.so")

KV_FMT_F16, KV_FMT_Q8, KV_FMT_K8V4 = 0, 1, 2
KV_GROUP = 64
KV_Q4_BLOCK = 32
KV_OK, KV_ERR_ARG, KV_ERR_FMT, KV_ERR_ALIGN, KV_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
KV_ERR_WORKSPACE, KV_ERR_RANGE, KV_ERR_HIP, KV_ERR_IMAGE, KV_ERR_WINDOW = -5, -6, -7, -8, -9
KV_DEV_RANGE, KV_DEV_BAD_SESSION, KV_DEV_BAD_PAGE = 1, 2, 4
KV_PAGE_ROWS = 64
KV_DECODE_STATIC_WS_BYTES = 16 << 20

EXPORTED = ["kv_cache_bytes", "kv_append", "kv_decode_workspace_bytes", "kv_decode_attn",
            "kv_compact_f16", "kv_prefill_workspace_bytes", "kv_prefill_attn", "kv_status_str",
            "kv_probe_stream_read", "kv_rows_bytes", "kv_copy_rows", "kv_gather_rows",
            "kv_scatter_rows", "kv_image_bytes", "kv_image_save", "kv_image_tokens",
            "kv_image_load", "kv_decode_attn_paged", "kv_window_bytes", "kv_window_init",
            "kv_window_plan", "kv_window_map", "kv_decode_attn_static", "kv_append_paged",
            "kv_window_writeback"]

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run quantized_kv_cache_q8_amd.build.build() "
                      "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)


class kv_shape(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class kv_session(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("cap", ctypes.c_int32), ("reserved", ctypes.c_int32)]


assert ctypes.sizeof(kv_session) == 40

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_sig = {
    "kv_cache_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "kv_append": (_I, [ctypes.POINTER(kv_shape), _P, _P, _I, _I, _P, _P, _P, _P]),
    "kv_decode_workspace_bytes": (_SZ, [ctypes.POINTER(kv_shape), _I, _I]),
    "kv_decode_attn": (_I, [ctypes.POINTER(kv_shape), _P, _P, _I, _I, _P, ctypes.c_float, _P, _P,
                            _SZ, _P, _P]),
    "kv_compact_f16": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _I, _P, _P, _P]),
    "kv_prefill_workspace_bytes": (_SZ, [ctypes.POINTER(kv_shape), _I]),
    "kv_prefill_attn": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _I, _I, _P,
                             ctypes.c_float, _P, _P, _SZ, _P]),
    "kv_status_str": (ctypes.c_char_p, [_I]),
    "kv_probe_stream_read": (_I, [_P, _SZ, _P, _P]),
    "kv_rows_bytes": (_SZ, [ctypes.POINTER(kv_shape), _I]),
    "kv_copy_rows": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _I,
                          ctypes.POINTER(kv_session), _I, _I, _P]),
    "kv_gather_rows": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _I, _I, _P, _P]),
    "kv_scatter_rows": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _I, _I, _P, _P]),
    "kv_image_bytes": (_SZ, [ctypes.POINTER(kv_shape), _I]),
    "kv_image_save": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _I, _P, _P, _SZ,
                           _P]),
    "kv_image_tokens": (_I, [ctypes.POINTER(kv_shape), _P, _SZ]),
    "kv_image_load": (_I, [ctypes.POINTER(kv_shape), ctypes.POINTER(kv_session), _P, _SZ, _P, _P]),
    "kv_decode_attn_paged": (_I, [ctypes.POINTER(kv_shape), _P, _P, _I, _P, _I, _I, _P,
                                  ctypes.c_float, _P, _P, _SZ, _P, _P]),
    "kv_decode_attn_static": (_I, [ctypes.POINTER(kv_shape), _P, _P, _I, _I, _P, ctypes.c_float,
                                   _P, _P, _P]),
    "kv_append_paged": (_I, [ctypes.POINTER(kv_shape), _P, _P, _I, _P, _I, _I, _P, _P, _P, _P]),
    "kv_window_writeback": (_I, [ctypes.POINTER(kv_shape), _P, ctypes.POINTER(kv_session), _I, _I,
                                 _I, ctypes.POINTER(kv_session), _P, _P]),
    "kv_window_bytes": (_SZ, [_I]),
    "kv_window_init": (_I, [_P, _SZ, _I]),
    "kv_window_plan": (_I, [_P, _I, _I, _P, _P, _P]),
    "kv_window_map": (_I, [ctypes.POINTER(kv_shape), _P, ctypes.POINTER(kv_session), _I, _I,
                           ctypes.POINTER(kv_session), _P, _P, _P, _P, _P]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class KvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status} ({kv_status_str(status)})")
        self.status = status


def kv_status_str(status: int) -> str:
    return _lib.kv_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != KV_OK:
        raise KvError(status, where)


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_shape(fmt: int, n_kv_heads: int, n_q_heads: int, head_dim: int = 128) -> kv_shape:
    return kv_shape(int(fmt), int(n_kv_heads), int(n_q_heads), int(head_dim))


def kv_cache_bytes(fmt: int, n_kv_heads: int, cap: int, head_dim: int, part: int) -> int:
    return int(_lib.kv_cache_bytes(fmt, n_kv_heads, cap, head_dim, part))


# ----------------------------------------------------------------------------
# caller-owned buffers (torch device memory)
# ----------------------------------------------------------------------------
class Session:
    """One session's cache arrays for one layer, allocated with torch.

    F16: k, v int16 tensors holding fp16 bits [kvh][cap][hd]; Q8: k, v int8 codes
    [kvh][cap][hd] and k_scale, v_scale int16 (fp16 bits) [kvh][cap][hd/64];
    K8V4: k, k_scale as Q8, v uint8 nibble pairs [kvh][cap][hd/2] and v_scale int16
    (fp16 bits) [kvh][cap][hd/32]."""

    def __init__(self, fmt: int, n_kv_heads: int, cap: int, head_dim: int = 128,
                 device="cuda", fill: int | None = None, pinned: bool = False):
        """pinned: the arrays in pinned host memory (a window's host store)."""
        self.fmt, self.kvh, self.cap, self.hd = fmt, n_kv_heads, cap, head_dim
        self.pinned = pinned
        if pinned:
            device = "cpu"
        shp = (n_kv_heads, cap, head_dim)
        if fmt == KV_FMT_F16:
            self.k = torch.empty(shp, dtype=torch.int16, device=device)
            self.v = torch.empty(shp, dtype=torch.int16, device=device)
            self.k_scale = self.v_scale = None
        elif fmt == KV_FMT_K8V4:
            self.k = torch.empty(shp, dtype=torch.int8, device=device)
            self.v = torch.empty((n_kv_heads, cap, head_dim // 2), dtype=torch.uint8, device=device)
            self.k_scale = torch.empty((n_kv_heads, cap, head_dim // KV_GROUP), dtype=torch.int16,
                                       device=device)
            self.v_scale = torch.empty((n_kv_heads, cap, head_dim // KV_Q4_BLOCK), dtype=torch.int16,
                                       device=device)
        else:
            self.k = torch.empty(shp, dtype=torch.int8, device=device)
            self.v = torch.empty(shp, dtype=torch.int8, device=device)
            sshp = (n_kv_heads, cap, head_dim // KV_GROUP)
            self.k_scale = torch.empty(sshp, dtype=torch.int16, device=device)
            self.v_scale = torch.empty(sshp, dtype=torch.int16, device=device)
        if pinned:
            for name in ("k", "v", "k_scale", "v_scale"):
                t = getattr(self, name)
                if t is not None:
                    setattr(self, name, t.pin_memory())
        for t in self.tensors():
            if fill is None:
                t.zero_()
            else:
                t.view(torch.uint8).fill_(fill)

    def tensors(self):
        return [t for t in (self.k, self.v, self.k_scale, self.v_scale) if t is not None]

    def entry(self) -> kv_session:
        ptr = (lambda t: None if t is None else _ptr_dev_or_pinned(t, "array")) if self.pinned else _ptr
        return kv_session(ptr(self.k), ptr(self.v), ptr(self.k_scale), ptr(self.v_scale),
                          self.cap, 0)


def session_table(entries, device="cuda") -> torch.Tensor:
    """Device array of kv_session structs (a uint8 tensor of 40 * n bytes)."""
    n = len(entries)
    arr = (kv_session * n)(*entries)
    host = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return host.to(device)


# ----------------------------------------------------------------------------
# the C ABI, tensor in / tensor out
# ----------------------------------------------------------------------------
def kv_append(shape: kv_shape, tab: torch.Tensor, lens: torch.Tensor, n_sess: int, n_tok: int,
              k_new: torch.Tensor, v_new: torch.Tensor, status: torch.Tensor | None = None,
              stream=None) -> None:
    _check(_lib.kv_append(ctypes.byref(shape), _ptr(tab, torch.uint8, "tab"),
                          _ptr(lens, torch.int32, "lens"), n_sess, n_tok,
                          _ptr(k_new, torch.float32, "k_new"), _ptr(v_new, torch.float32, "v_new"),
                          _ptr(status, torch.int32, "status"), _stream(stream)), "kv_append")


def kv_append_paged(shape: kv_shape, tab: torch.Tensor, pages: torch.Tensor, page_stride: int,
                    lens: torch.Tensor, n_sess: int, n_tok: int, k_new: torch.Tensor,
                    v_new: torch.Tensor, status: torch.Tensor | None = None, stream=None) -> None:
    """kv_append into paged sessions: pages int32 [n_sess][page_stride] (device)."""
    _check(_lib.kv_append_paged(ctypes.byref(shape), _ptr(tab, torch.uint8, "tab"),
                                _ptr(pages, torch.int32, "pages"), page_stride,
                                _ptr(lens, torch.int32, "lens"), n_sess, n_tok,
                                _ptr(k_new, torch.float32, "k_new"),
                                _ptr(v_new, torch.float32, "v_new"),
                                _ptr(status, torch.int32, "status"), _stream(stream)),
           "kv_append_paged")


def kv_decode_workspace_bytes(shape: kv_shape, n_sess: int, max_len: int) -> int:
    return int(_lib.kv_decode_workspace_bytes(ctypes.byref(shape), n_sess, max_len))


def kv_decode_workspace(shape: kv_shape, n_sess: int, max_len: int, device="cuda") -> torch.Tensor:
    """A decode workspace on `device` (zero-filled; kv_decode_attn overwrites what it
    reads)."""
    return torch.zeros(max(kv_decode_workspace_bytes(shape, n_sess, max_len), 256),
                       dtype=torch.uint8, device=device)


def kv_decode_attn(shape: kv_shape, tab: torch.Tensor, lens: torch.Tensor, n_sess: int,
                   max_len: int, q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                   ws: torch.Tensor, status: torch.Tensor | None = None, stream=None) -> None:
    _check(_lib.kv_decode_attn(ctypes.byref(shape), _ptr(tab, torch.uint8, "tab"),
                               _ptr(lens, torch.int32, "lens"), n_sess, max_len,
                               _ptr(q, torch.float32, "q"), float(sm_scale),
                               _ptr(out, torch.float32, "out"), _ptr(ws, None, "ws"),
                               ws.numel() * ws.element_size(), _ptr(status, torch.int32, "status"),
                               _stream(stream)), "kv_decode_attn")


def kv_decode_attn_static(shape: kv_shape, tab: torch.Tensor, lens: torch.Tensor, n_sess: int,
                          max_len: int, q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                          status: torch.Tensor | None = None, stream=None) -> None:
    """kv_decode_attn with the library's fixed per-device scratch (no workspace)."""
    _check(_lib.kv_decode_attn_static(ctypes.byref(shape), _ptr(tab, torch.uint8, "tab"),
                                      _ptr(lens, torch.int32, "lens"), n_sess, max_len,
                                      _ptr(q, torch.float32, "q"), float(sm_scale),
                                      _ptr(out, torch.float32, "out"),
                                      _ptr(status, torch.int32, "status"), _stream(stream)),
           "kv_decode_attn_static")


def kv_decode_attn_paged(shape: kv_shape, tab: torch.Tensor, pages: torch.Tensor, page_stride: int,
                         lens: torch.Tensor, n_sess: int, max_len: int, q: torch.Tensor,
                         sm_scale: float, out: torch.Tensor, ws: torch.Tensor,
                         status: torch.Tensor | None = None, stream=None) -> None:
    """kv_decode_attn over paged sessions: pages int32 [n_sess][page_stride] (device)."""
    _check(_lib.kv_decode_attn_paged(ctypes.byref(shape), _ptr(tab, torch.uint8, "tab"),
                                     _ptr(pages, torch.int32, "pages"), page_stride,
                                     _ptr(lens, torch.int32, "lens"), n_sess, max_len,
                                     _ptr(q, torch.float32, "q"), float(sm_scale),
                                     _ptr(out, torch.float32, "out"), _ptr(ws, None, "ws"),
                                     ws.numel() * ws.element_size(),
                                     _ptr(status, torch.int32, "status"), _stream(stream)),
           "kv_decode_attn_paged")


class Window:
    """A streamed window's host-side state (kv_window_*): n_slots pool slots."""

    def __init__(self, n_slots: int):
        nb = int(_lib.kv_window_bytes(n_slots))
        if nb == 0:
            raise ValueError("kv_window_bytes: n_slots out of range")
        self.n_slots = n_slots
        self.state = ctypes.create_string_buffer(nb)
        # per page-table buffer (by address): the event recorded after the map that
        # last enqueued a copy from it; the next map of that table waits for it
        self._table_events = {}
        _check(_lib.kv_window_init(self.state, nb, n_slots), "kv_window_init")

    def plan(self, sess_id: int, pages: "np.ndarray"):
        """Host-only planning: updates pages (int32 numpy array) in place; returns the
        missed pages."""
        import numpy as np
        assert pages.dtype == np.int32 and pages.flags.c_contiguous
        missed = np.zeros(max(1, pages.size), np.int32)
        n = ctypes.c_int(0)
        _check(_lib.kv_window_plan(self.state, sess_id, pages.size, pages.ctypes.data,
                                   missed.ctypes.data, ctypes.byref(n)), "kv_window_plan")
        return missed[:n.value].copy()

    def map(self, shape: kv_shape, store: "Session", sess_id: int, n_pages: int, pool: "Session",
            h_pages: torch.Tensor, d_pages: torch.Tensor, stream=None) -> int:
        """Make pages [0, n_pages) resident, copying the missed ones from the pinned host
        store; h_pages: pinned int32 [>= n_pages] (kept per session), d_pages: device
        int32 row of the page table.  Returns the number of pages copied."""
        if not store.pinned:
            raise ValueError("store: must be a pinned Session")
        if h_pages.dtype != torch.int32 or not h_pages.is_pinned() or h_pages.numel() < n_pages:
            raise ValueError("h_pages: expected a pinned int32 tensor of at least n_pages entries")
        missed = torch.zeros(max(1, n_pages), dtype=torch.int32)
        n = ctypes.c_int(0)
        # the previous map's copy from this table must have run before the table is
        # rewritten (the copy reads h_pages when the stream reaches it)
        ev = self._table_events.pop(h_pages.data_ptr(), None)
        if ev is not None:
            ev.synchronize()
        _check(_lib.kv_window_map(ctypes.byref(shape), self.state, ctypes.byref(store.entry()),
                                  sess_id, n_pages, ctypes.byref(pool.entry()), h_pages.data_ptr(),
                                  missed.data_ptr(), _ptr(d_pages, torch.int32, "d_pages"),
                                  ctypes.byref(n), _stream(stream)), "kv_window_map")
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream() if stream is None else stream)
        self._table_events[h_pages.data_ptr()] = ev
        return n.value


def _window_writeback(self, shape: kv_shape, store: "Session", sess_id: int, row0: int,
                      n_rows: int, pool: "Session", h_pages: torch.Tensor, stream=None) -> None:
    """Rows [row0, row0 + n_rows) of the session from their pool slots back to its pinned
    host store (kv_window_writeback); h_pages: the table of the session's last map."""
    if not store.pinned:
        raise ValueError("store: must be a pinned Session")
    if h_pages.dtype != torch.int32 or h_pages.device.type != "cpu" or not h_pages.is_contiguous():
        raise ValueError("h_pages: expected a contiguous int32 host tensor")
    _check(_lib.kv_window_writeback(ctypes.byref(shape), self.state, ctypes.byref(store.entry()),
                                    sess_id, row0, n_rows, ctypes.byref(pool.entry()),
                                    h_pages.data_ptr(), _stream(stream)), "kv_window_writeback")


Window.writeback = _window_writeback


def kv_compact_f16(shape: kv_shape, sess: kv_session, P: int, k16: torch.Tensor,
                   v16: torch.Tensor, stream=None) -> None:
    _check(_lib.kv_compact_f16(ctypes.byref(shape), ctypes.byref(sess), P,
                               _ptr(k16, torch.int16, "k16"), _ptr(v16, torch.int16, "v16"),
                               _stream(stream)), "kv_compact_f16")


def kv_prefill_workspace_bytes(shape: kv_shape, P: int) -> int:
    return int(_lib.kv_prefill_workspace_bytes(ctypes.byref(shape), P))


def kv_prefill_attn(shape: kv_shape, sess: kv_session, pos0: int, n_tok: int, q: torch.Tensor,
                    sm_scale: float, out: torch.Tensor, ws: torch.Tensor | None,
                    stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.kv_prefill_attn(ctypes.byref(shape), ctypes.byref(sess), pos0, n_tok,
                                _ptr(q, torch.float32, "q"), float(sm_scale),
                                _ptr(out, torch.float32, "out"), _ptr(ws, None, "ws"), nbytes,
                                _stream(stream)), "kv_prefill_attn")


def kv_probe_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement aid: one plain read of all of src (see include/kvq8.h)."""
    _check(_lib.kv_probe_stream_read(_ptr(src, None, "src"), src.numel() * src.element_size(),
                                     _ptr(sink, torch.int32, "sink"), _stream(stream)),
           "kv_probe_stream_read")


def _ptr_dev_or_pinned(t, name):
    """Pointer of a contiguous GPU tensor or pinned host tensor."""
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous torch.Tensor")
    if t.device.type != "cuda" and not t.is_pinned():
        raise ValueError(f"{name}: must be a GPU tensor or pinned host memory")
    return t.data_ptr()


def kv_rows_bytes(shape: kv_shape, n_rows: int) -> int:
    return int(_lib.kv_rows_bytes(ctypes.byref(shape), n_rows))


def kv_copy_rows(shape: kv_shape, src: kv_session, src_row0: int, dst: kv_session, dst_row0: int,
                 n_rows: int, stream=None) -> None:
    _check(_lib.kv_copy_rows(ctypes.byref(shape), ctypes.byref(src), src_row0, ctypes.byref(dst),
                             dst_row0, n_rows, _stream(stream)), "kv_copy_rows")


def kv_gather_rows(shape: kv_shape, sess: kv_session, row0: int, n_rows: int, dst: torch.Tensor,
                   stream=None) -> None:
    if dst.numel() * dst.element_size() < kv_rows_bytes(shape, n_rows):
        raise ValueError("kv_gather_rows: destination smaller than kv_rows_bytes")
    _check(_lib.kv_gather_rows(ctypes.byref(shape), ctypes.byref(sess), row0, n_rows,
                               _ptr_dev_or_pinned(dst, "dst"), _stream(stream)), "kv_gather_rows")


def kv_scatter_rows(shape: kv_shape, sess: kv_session, row0: int, n_rows: int, src: torch.Tensor,
                    stream=None) -> None:
    if src.numel() * src.element_size() < kv_rows_bytes(shape, n_rows):
        raise ValueError("kv_scatter_rows: source smaller than kv_rows_bytes")
    _check(_lib.kv_scatter_rows(ctypes.byref(shape), ctypes.byref(sess), row0, n_rows,
                                _ptr_dev_or_pinned(src, "src"), _stream(stream)), "kv_scatter_rows")


def _host_u8(t, name, pinned):
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or not t.is_contiguous() \
            or t.dtype != torch.uint8:
        raise ValueError(f"{name}: expected a contiguous uint8 host tensor")
    if pinned and not t.is_pinned():
        raise ValueError(f"{name}: must be pinned host memory")
    return t.data_ptr()


def _host_i32(t, n, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or not t.is_contiguous() \
            or t.dtype != torch.int32 or t.numel() < n:
        raise ValueError(f"{name}: expected a contiguous int32 host tensor of at least {n} entries")
    return t.data_ptr()


def kv_image_bytes(shape: kv_shape, n_tokens: int) -> int:
    return int(_lib.kv_image_bytes(ctypes.byref(shape), n_tokens))


def kv_image_save(shape: kv_shape, sess: kv_session, n_tokens: int, tokens, image: torch.Tensor,
                  stream=None) -> None:
    """Saved image of rows [0, n_tokens) into a pinned uint8 host tensor; complete once
    the stream reaches the call."""
    _check(_lib.kv_image_save(ctypes.byref(shape), ctypes.byref(sess), n_tokens,
                              _host_i32(tokens, n_tokens, "tokens"),
                              _host_u8(image, "image", True), image.numel(), _stream(stream)),
           "kv_image_save")


def kv_image_tokens(shape: kv_shape, image: torch.Tensor) -> int:
    n = _lib.kv_image_tokens(ctypes.byref(shape), _host_u8(image, "image", False), image.numel())
    _check(min(n, 0), "kv_image_tokens")
    return n


def kv_image_load(shape: kv_shape, sess: kv_session, image: torch.Tensor, tokens=None,
                  stream=None) -> int:
    """Load a saved image (pinned uint8 host tensor) into rows [0, n); returns n."""
    need = kv_image_tokens(shape, image) if tokens is not None else 0
    n = _lib.kv_image_load(ctypes.byref(shape), ctypes.byref(sess), _host_u8(image, "image", True),
                           image.numel(), _host_i32(tokens, need, "tokens"), _stream(stream))
    _check(min(n, 0), "kv_image_load")
    return n


def raw_lib() -> ctypes.CDLL:
    """The loaded C library (for calls with raw pointers)."""
    return _lib
