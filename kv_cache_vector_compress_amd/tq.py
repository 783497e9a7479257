"""Thin Python binding of libtq.so (the C ABI in include/tq.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  PyTorch supplies device memory (tensors) and the current HIP
stream.  There is no fallback: if libtq.so is missing or fails to load, every
call raises.

Names follow the C ABI, which mirrors the pages' interface (nav.superapi.store
"turboquant-pytorch", 核心 API: build_lloyd_max_codebook,
TurboQuantKVCache.append_key / append_value / attention_scores, and the
softmax-weighted sum over decompressed values of 常见使用模式).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK = 0
STATUS = {0: "TQ_OK", -1: "TQ_EINVAL", -2: "TQ_ECAPACITY", -3: "TQ_ENOCODEBOOK", -4: "TQ_ENOMEM",
          -5: "TQ_EDEVICE", -6: "TQ_EUNSUPPORTED", -7: "TQ_EWORKSPACE"}
TQ_F16, TQ_F32 = 1, 2
BLOCK_TOKENS = 128


class TQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("proj_dim", ctypes.c_int32),
                ("key_bits", ctypes.c_int32), ("value_bits", ctypes.c_int32)]


class CacheView(ctypes.Structure):
    _fields_ = [("key_records", ctypes.c_void_p), ("value_blocks", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("n_seq", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libtq.so (built in place by kv_cache_vector_compress_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not built: run `python -m kv_cache_vector_compress_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double)
    CFG = ctypes.POINTER(Config)
    VIEW = ctypes.POINTER(CacheView)
    sig = {
        "tq_lloyd_max_codebook": (ctypes.c_int, [I32, I32, D, D]),
        "tq_config_key_record_bytes": (SZ, [CFG]),
        "tq_key_record_bytes": (SZ, [P]),
        "tq_value_record_bytes": (SZ, [P]),
        "tq_attend_workspace_bytes": (SZ, [P, I32, I32, I64]),
        "tq_value_block_bytes": (SZ, [CFG]),
        "tq_cache_key_bytes": (SZ, [CFG, I32, I64]),
        "tq_cache_value_bytes": (SZ, [CFG, I32, I64]),
        "tq_workspace_bytes": (SZ, [CFG, I32, I32, I64]),
        "tq_last_error": (ctypes.c_char_p, []),
        "tq_create": (ctypes.c_int, [CFG, D, D, ctypes.POINTER(P)]),
        "tq_destroy": (ctypes.c_int, [P]),
        "tq_codebook_load": (ctypes.c_int, [P, I32, D, D]),
        "tq_append_key": (ctypes.c_int, [P, VIEW, P, I32, I64, I64, P]),
        "tq_append_value": (ctypes.c_int, [P, VIEW, P, I32, I64, I64, P]),
        "tq_append_workspace_bytes": (SZ, [P, I32, I64]),
        "tq_append_key_ws": (ctypes.c_int, [P, VIEW, P, I32, I64, I64, P, SZ, P]),
        "tq_append_value_ws": (ctypes.c_int, [P, VIEW, P, I32, I64, I64, P, SZ, P]),
        "tq_attention_scores": (ctypes.c_int, [P, VIEW, P, I32, I32, I64, P, P, SZ, P]),
        "tq_attend": (ctypes.c_int, [P, VIEW, P, I32, I32, I64, ctypes.c_float, P, P, SZ, P]),
        "tq_topk_workspace_bytes": (SZ, [CFG, I32, I32, I64, I32]),
        "tq_topk_scores": (ctypes.c_int, [P, VIEW, P, I32, I32, I64, I32, P, P, P, SZ, P]),
        "tq_get_values": (ctypes.c_int, [P, VIEW, I64, I64, P, P]),
        "tq_get_keys": (ctypes.c_int, [P, VIEW, I64, I64, P, P]),
        "tq_hbm_stream": (ctypes.c_int, [P, SZ, P, SZ, P, I32, I32, P]),
        "tq_attend_noalloc": (ctypes.c_int, [P, VIEW, P, I32, I32, I64, ctypes.c_float, P, P]),
        "tq_decode_step": (ctypes.c_int, [P, VIEW, P, P, I32, I64, I64, P, I32, ctypes.c_float, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return (lib().tq_last_error() or b"").decode()


def _check(rc: int) -> None:
    if rc != TQ_OK:
        raise TQError(rc, last_error())


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


# ---- host helpers -------------------------------------------------------------

def lloyd_max_codebook(head_dim: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """(centroids, boundaries) of the Lloyd-Max quantiser of N(0, 1/head_dim),
    computed by the library on the host."""
    L = 1 << bits
    c = np.zeros(L)
    b = np.zeros(max(L - 1, 1))
    _check(lib().tq_lloyd_max_codebook(head_dim, bits, _dptr(c), _dptr(b)))
    return c, b[:L - 1]


def key_record_bytes(cfg: Config) -> int:
    return lib().tq_config_key_record_bytes(ctypes.byref(cfg))


def value_block_bytes(cfg: Config) -> int:
    return lib().tq_value_block_bytes(ctypes.byref(cfg))


def cache_key_bytes(cfg: Config, n_seq: int, capacity: int) -> int:
    return lib().tq_cache_key_bytes(ctypes.byref(cfg), n_seq, capacity)


def cache_value_bytes(cfg: Config, n_seq: int, capacity: int) -> int:
    return lib().tq_cache_value_bytes(ctypes.byref(cfg), n_seq, capacity)


def workspace_bytes(cfg: Config, n_seq: int, G: int, n_tokens: int) -> int:
    return lib().tq_workspace_bytes(ctypes.byref(cfg), n_seq, G, n_tokens)


# ---- device side ----------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return TQ_F16
    if t.dtype == torch.float32:
        return TQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use float16 or float32")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class Context:
    """A tq_ctx: the rotation R, the QJL matrix S and the loaded codebooks on
    the current device."""

    def __init__(self, head_dim: int, proj_dim: int, key_bits: int, value_bits: int,
                 R: np.ndarray, S: np.ndarray, load_codebooks: bool = True):
        self.cfg = Config(head_dim, proj_dim, key_bits, value_bits)
        R = np.ascontiguousarray(R, dtype=np.float64)
        S = np.ascontiguousarray(S, dtype=np.float64)
        if R.shape != (head_dim, head_dim) or S.shape != (proj_dim, head_dim):
            raise ValueError("R must be (d, d) and S (m, d)")
        h = ctypes.c_void_p()
        _check(lib().tq_create(ctypes.byref(self.cfg), _dptr(R), _dptr(S), ctypes.byref(h)))
        self._h = h
        if load_codebooks:
            for b in sorted({key_bits, value_bits}):
                self.codebook_load(b)

    @property
    def handle(self):
        return self._h

    def key_record_bytes(self) -> int:
        """tq_key_record_bytes: bytes of one token's key record."""
        return lib().tq_key_record_bytes(self._h)

    def value_record_bytes(self) -> int:
        """tq_value_record_bytes: one token's share of a 128-token value block."""
        return lib().tq_value_record_bytes(self._h)

    def attend_workspace_bytes(self, n_seq: int, G: int, n_tokens: int) -> int:
        """tq_attend_workspace_bytes: workspace of the score / attend calls."""
        return lib().tq_attend_workspace_bytes(self._h, n_seq, G, n_tokens)

    def append_workspace_bytes(self, n_seq: int, n_new: int) -> int:
        """tq_append_workspace_bytes: workspace of tq_append_key_ws /
        tq_append_value_ws (0: the append uses none)."""
        return lib().tq_append_workspace_bytes(self._h, n_seq, n_new)

    def codebook_load(self, bits: int, centroids: Optional[np.ndarray] = None,
                      boundaries: Optional[np.ndarray] = None) -> None:
        """Load a codebook; by default the library's own Lloyd-Max codebook."""
        if centroids is None:
            centroids, boundaries = lloyd_max_codebook(self.cfg.head_dim, bits)
        c = np.ascontiguousarray(centroids, dtype=np.float64)
        b = np.ascontiguousarray(boundaries, dtype=np.float64)
        if c.size != 1 << bits or b.size != (1 << bits) - 1:
            raise ValueError("codebook sizes do not match bits")
        _check(lib().tq_codebook_load(self._h, bits, _dptr(c), _dptr(b if b.size else np.zeros(1))))

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().tq_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVCache:
    """Caller-owned packed cache (tq_cache_view) backed by torch device memory."""

    def __init__(self, ctx: Context, n_seq: int, capacity: int, device="cuda"):
        torch = _torch()
        if capacity % BLOCK_TOKENS:
            raise ValueError("capacity must be a multiple of 128")
        self.ctx, self.n_seq, self.capacity = ctx, n_seq, capacity
        kb = cache_key_bytes(ctx.cfg, n_seq, capacity)
        vb = cache_value_bytes(ctx.cfg, n_seq, capacity)
        if kb == 0 or vb == 0:
            raise TQError(-1, last_error())
        self.key_records = torch.zeros(kb // 4, dtype=torch.int32, device=device)
        self.value_blocks = torch.zeros(vb // 4, dtype=torch.int32, device=device)
        self.view = CacheView(self.key_records.data_ptr(), self.value_blocks.data_ptr(), capacity, n_seq)
        self._ws = {}   # one attention workspace per stream: calls on different streams never share one
        self._aws = {}  # the same for the appends' workspace (general-path bulk appends)
        self._aws_need = {}  # its size per append length (n_seq is fixed)
        self._ws_need = (None, 0)  # the last attention workspace size query and its answer

    def workspace(self, G: int, n_tokens: int, stream=None):
        """The attention workspace of the given stream (torch's current
        stream by default), grown to tq_attend_workspace_bytes."""
        torch = _torch()
        if self._ws_need[0] == (G, n_tokens):  # (the last size query, kept: decode loops repeat it)
            need = self._ws_need[1]
        else:
            need = self.ctx.attend_workspace_bytes(self.n_seq, G, n_tokens)
            self._ws_need = ((G, n_tokens), need)
        if need == 0:
            raise TQError(-1, f"tq_attend_workspace_bytes: invalid arguments (n_seq {self.n_seq}, G {G}, "
                              f"n_tokens {n_tokens})")
        key = _stream_ptr(stream).value
        ws = self._ws.get(key)
        if ws is None or ws.numel() < need:
            ws = self._ws[key] = torch.empty(need, dtype=torch.uint8, device=self.key_records.device)
        return ws

    # shape checks: the C ABI receives raw pointers and cannot see tensor
    # sizes, so every tensor is checked here against the cache's shape
    def _rows(self, t, name: str) -> int:
        """t must be (n_seq, n, head_dim) on the cache's device; returns n."""
        if t.dim() != 3 or t.shape[0] != self.n_seq or t.shape[2] != self.ctx.cfg.head_dim:
            raise ValueError(f"{name} must have shape (n_seq={self.n_seq}, n, head_dim={self.ctx.cfg.head_dim}), "
                             f"got {tuple(t.shape)}")
        if t.device != self.key_records.device:
            raise ValueError(f"{name} is on {t.device}, the cache on {self.key_records.device}")
        return int(t.shape[1])

    def _out(self, out, shape, name: str):
        torch = _torch()
        if out is None:
            return torch.empty(shape, dtype=torch.float32, device=self.key_records.device)
        if out.dtype != torch.float32 or tuple(out.shape) != tuple(shape) or not out.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}, "
                             f"got {out.dtype} {tuple(out.shape)}")
        if out.device != self.key_records.device:
            raise ValueError(f"{name} is on {out.device}, the cache on {self.key_records.device}")
        return out

    def append_workspace(self, n_new: int, stream=None):
        """The appends' workspace of the given stream, grown to
        tq_append_workspace_bytes, or None when the append uses none."""
        torch = _torch()
        need = self._aws_need.get(n_new)
        if need is None:  # (a host-only size query, remembered per append length)
            need = self._aws_need[n_new] = self.ctx.append_workspace_bytes(self.n_seq, n_new)
        if need == 0:
            return None
        key = _stream_ptr(stream).value
        ws = self._aws.get(key)
        if ws is None or ws.numel() < need:
            ws = self._aws[key] = torch.empty(need, dtype=torch.uint8, device=self.key_records.device)
        return ws

    # hot path ---------------------------------------------------------------
    # The appends go through tq_append_key_ws / tq_append_value_ws with a
    # workspace per stream, so that appends on different streams never share
    # the context's scratch.
    def append_key(self, k, pos: int, stream=None) -> None:
        """k: (n_seq, n_new, d) fp16/fp32 device tensor."""
        n_new = self._rows(k, "k")
        ws = self.append_workspace(n_new, stream)
        _check(lib().tq_append_key_ws(self.ctx.handle, ctypes.byref(self.view), _dev(k, "k"), _dtype_code(k),
                                      pos, n_new, ctypes.c_void_p(ws.data_ptr() if ws is not None else None),
                                      ws.numel() if ws is not None else 0, _stream_ptr(stream)))

    def append_value(self, v, pos: int, stream=None) -> None:
        n_new = self._rows(v, "v")
        ws = self.append_workspace(n_new, stream)
        _check(lib().tq_append_value_ws(self.ctx.handle, ctypes.byref(self.view), _dev(v, "v"), _dtype_code(v),
                                        pos, n_new, ctypes.c_void_p(ws.data_ptr() if ws is not None else None),
                                        ws.numel() if ws is not None else 0, _stream_ptr(stream)))

    def append_key_ctx_scratch(self, k, pos: int, stream=None) -> None:
        """tq_append_key: the same append with the context's scratch buffer
        (calls of one context must then be ordered)."""
        n_new = self._rows(k, "k")
        _check(lib().tq_append_key(self.ctx.handle, ctypes.byref(self.view), _dev(k, "k"), _dtype_code(k),
                                   pos, n_new, _stream_ptr(stream)))

    def append_value_ctx_scratch(self, v, pos: int, stream=None) -> None:
        """tq_append_value with the context's scratch buffer."""
        n_new = self._rows(v, "v")
        _check(lib().tq_append_value(self.ctx.handle, ctypes.byref(self.view), _dev(v, "v"), _dtype_code(v),
                                     pos, n_new, _stream_ptr(stream)))

    def attention_scores(self, q, n_tokens: int, out=None, stream=None):
        """q: (n_seq, G, d).  Returns fp32 (n_seq, G, n_tokens) unscaled estimates."""
        G = self._rows(q, "q")
        out = self._out(out, (self.n_seq, G, n_tokens), "scores")
        ws = self.workspace(G, n_tokens, stream)
        _check(lib().tq_attention_scores(self.ctx.handle, ctypes.byref(self.view), _dev(q, "q"), _dtype_code(q),
                                         G, n_tokens, _dev(out, "scores"), ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel(), _stream_ptr(stream)))
        return out

    def attend(self, q, n_tokens: int, scale: float = 0.0, out=None, stream=None):
        """softmax(scale * est) . V^ over the first n_tokens; fp32 (n_seq, G, d)."""
        G = self._rows(q, "q")
        out = self._out(out, (self.n_seq, G, self.ctx.cfg.head_dim), "out")
        ws = self.workspace(G, n_tokens, stream)
        _check(lib().tq_attend(self.ctx.handle, ctypes.byref(self.view), _dev(q, "q"), _dtype_code(q), G,
                               n_tokens, float(scale), _dev(out, "out"), ctypes.c_void_p(ws.data_ptr()),
                               ws.numel(), _stream_ptr(stream)))
        return out

    def attend_noalloc(self, q, n_tokens: int, scale: float = 0.0, out=None, stream=None):
        """tq_attend_noalloc: attend with the library's static device scratch
        instead of a workspace (no device allocation by the library; pass
        `out` to allocate nothing here either).  Calls on one GPU must not
        overlap."""
        G = self._rows(q, "q")
        out = self._out(out, (self.n_seq, G, self.ctx.cfg.head_dim), "out")
        _check(lib().tq_attend_noalloc(self.ctx.handle, ctypes.byref(self.view), _dev(q, "q"), _dtype_code(q), G,
                                       n_tokens, float(scale), _dev(out, "out"), _stream_ptr(stream)))
        return out

    def decode_step(self, k, v, q, pos: int, scale: float = 0.0, out=None, stream=None):
        """Append k, v (n_seq, n_new, d) at token pos and attend with q over the
        first pos + n_new tokens (tq_decode_step); fp32 (n_seq, G, d)."""
        if k.dtype != v.dtype or k.dtype != q.dtype:
            raise TypeError("k, v and q must share one dtype")
        n_new = self._rows(k, "k")
        if tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"v must have the shape of k {tuple(k.shape)}, got {tuple(v.shape)}")
        self._rows(v, "v")
        G = self._rows(q, "q")
        out = self._out(out, (self.n_seq, G, self.ctx.cfg.head_dim), "out")
        ws = self.workspace(G, pos + n_new, stream)
        _check(lib().tq_decode_step(self.ctx.handle, ctypes.byref(self.view), _dev(k, "k"), _dev(v, "v"),
                                    _dtype_code(k), pos, n_new, _dev(q, "q"), G, float(scale), _dev(out, "out"),
                                    ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream_ptr(stream)))
        return out

    def topk(self, q, n_tokens: int, k: int = 10, stream=None):
        """The k best tokens per query by the score estimate (no score matrix):
        (scores fp32 (n_seq, G, k), indices int32 (n_seq, G, k))."""
        torch = _torch()
        G = self._rows(q, "q")
        need = lib().tq_topk_workspace_bytes(ctypes.byref(self.ctx.cfg), self.n_seq, G, n_tokens, k)
        if need == 0:
            raise TQError(-1, "tq_topk_workspace_bytes: invalid arguments")
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        top_s = torch.empty((self.n_seq, G, k), dtype=torch.float32, device=q.device)
        top_i = torch.empty((self.n_seq, G, k), dtype=torch.int32, device=q.device)
        _check(lib().tq_topk_scores(self.ctx.handle, ctypes.byref(self.view), _dev(q, "q"), _dtype_code(q), G,
                                    n_tokens, k, _dev(top_s, "top_scores"), _dev(top_i, "top_index"),
                                    ctypes.c_void_p(ws.data_ptr()), need, _stream_ptr(stream)))
        return top_s, top_i

    # reconstruction ------------------------------------------------------------
    def get_values(self, pos: int, n_tokens: int, out=None, stream=None):
        """Dequantised values ||v|| R^T c[idx] of tokens [pos, pos + n_tokens): fp32 (n_seq, n_tokens, d)."""
        return self._get(lib().tq_get_values, pos, n_tokens, out, stream)

    def get_keys(self, pos: int, n_tokens: int, out=None, stream=None):
        """Stage-1 (MSE) reconstruction of the keys, ||k|| R^T c[idx]: fp32 (n_seq, n_tokens, d)."""
        return self._get(lib().tq_get_keys, pos, n_tokens, out, stream)

    def _get(self, fn, pos, n_tokens, out, stream):
        out = self._out(out, (self.n_seq, n_tokens, self.ctx.cfg.head_dim), "out")
        _check(fn(self.ctx.handle, ctypes.byref(self.view), pos, n_tokens,
                  _dev(out, "out") if n_tokens > 0 else None, _stream_ptr(stream)))
        return out

    # raw views for inspection ------------------------------------------------
    def key_words(self):
        """(n_seq, capacity, record_words) uint32 numpy copy of the key records."""
        w = self.key_records.cpu().numpy().view(np.uint32)
        return w.reshape(self.n_seq, self.capacity, -1)

    def value_words(self):
        w = self.value_blocks.cpu().numpy().view(np.uint32)
        return w.reshape(self.n_seq, self.capacity // BLOCK_TOKENS, -1)


# ---- measurement -------------------------------------------------------------

STREAM_NONTEMPORAL = 1


def hbm_stream(src, dst=None, sink=None, waves_per_cu: int = 0, loads_in_flight: int = 4,
               nontemporal: bool = False, stream=None) -> None:
    """Stream all of `src` (a contiguous device tensor) and, if `dst` is given,
    write all of `dst` interleaved with the reads (tq_hbm_stream), on a grid
    of `waves_per_cu` waves per compute unit (0: the library's default),
    each lane keeping `loads_in_flight` 16-byte loads (4, 8 or 16) in flight,
    with nontemporal loads and stores if asked.  `sink` is a one-element
    int32 device tensor that receives the XOR of the words read (XOR-ed into
    its current value)."""
    torch = _torch()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    nr = src.numel() * src.element_size()
    nw = 0 if dst is None else dst.numel() * dst.element_size()
    flags = (loads_in_flight << 8) | (STREAM_NONTEMPORAL if nontemporal else 0)
    _check(lib().tq_hbm_stream(_dev(src, "src"), nr, _dev(dst, "dst") if dst is not None else None, nw,
                               _dev(sink, "sink"), waves_per_cu, flags, _stream_ptr(stream)))
    return sink
