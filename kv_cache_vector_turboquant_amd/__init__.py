"""Python binding of libtq, the MI355X TurboQuant library.

Argument marshalling only: every step of the hot path runs in the HIP kernels
of libtq.so, reached through its C ABI (include/tq.h). torch supplies device
memory and the current HIP stream. There is no CPU fallback: importing this
package fails if libtq.so has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python kv_cache_vector_turboquant_amd/build.py` "
        "(or __graft_entry__.build()); there is no CPU fallback")

# torch ships its own HIP runtime. Loading torch first makes libtq.so bind to
# that already-loaded runtime, so the process has exactly one HIP runtime and
# torch-allocated pointers and streams are valid in libtq's kernels. (Loading
# libtq.so first would bring in a second runtime that cannot open the device.)
try:
    import torch as _torch_mod  # noqa: F401
except ImportError:  # pure C-ABI use without torch
    _torch_mod = None

_lib = ctypes.CDLL(LIB_PATH)

TQ_OK, TQ_ERR_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP, TQ_ERR_NOMEM = range(6)
TQ_F32, TQ_BF16 = 0, 1
_c_i32, _c_i64, _c_f32, _c_vp, _c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class TQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"tq status {status}: {msg}")
        self.status = status


class CCodebook(ctypes.Structure):
    _fields_ = [("d", _c_i32), ("bits", _c_i32), ("centroid", ctypes.c_float * 16),
                ("boundary", ctypes.c_float * 15), ("walsh", ctypes.c_float * 8), ("distortion", ctypes.c_double)]


class CAngleCodebook(ctypes.Structure):
    _fields_ = [("level", _c_i32), ("bits", _c_i32), ("centroid", ctypes.c_double * 16),
                ("boundary", ctypes.c_float * 15), ("cos_c", ctypes.c_float * 16), ("sin_c", ctypes.c_float * 16)]


class CPolarPacked(ctypes.Structure):
    _fields_ = [("bits", _c_vp), ("norms", _c_vp), ("n", _c_i64), ("b1", _c_i32), ("b2", _c_i32)]


class CPacked(ctypes.Structure):
    _fields_ = [("bits", _c_vp), ("norms", _c_vp), ("n", _c_i64), ("mse_bits", _c_i32), ("is_key", _c_i32),
                ("qjl", _c_i32), ("norm_f16", _c_i32)]


class CCache(ctypes.Structure):
    _fields_ = [("k", CPacked), ("v", CPacked), ("batch", _c_i32), ("kv_heads", _c_i32), ("capacity", _c_i32),
                ("d_seq_len", _c_vp), ("host_max_len", _c_i32), ("d_block_table", _c_vp), ("page_tokens", _c_i32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("tq_last_error", ctypes.c_char_p, [])
_sig("tq_codebook_build", _c_i32, [_c_i32, _c_i32, ctypes.POINTER(CCodebook)])
_sig("tq_rotation_build", _c_i32, [_c_i32, _c_vp, _c_vp])
_sig("tq_ctx_create", _c_i32, [_c_i32, _c_vp, _c_vp, ctypes.POINTER(_c_vp)])
_sig("tq_ctx_create_seeded", _c_i32, [_c_i32, ctypes.c_uint64, ctypes.POINTER(_c_vp)])
_sig("tq_gaussian_matrix", _c_i32, [ctypes.c_uint64, ctypes.c_uint32, _c_i32, _c_i32, _c_vp])
_sig("tq_format_version", _c_i32, [])
_sig("tq_ctx_destroy", _c_i32, [_c_vp])
_sig("tq_ctx_dim", _c_i32, [_c_vp])
_sig("tq_ctx_export", _c_i32, [_c_vp, _c_vp, _c_vp])
_sig("tq_ctx_codebook", _c_i32, [_c_vp, _c_i32, ctypes.POINTER(CCodebook)])
_sig("tq_quantize_ws_bytes", _c_sz, [_c_vp, _c_i64, _c_i64, _c_i32])
_sig("tq_quantize_kv", _c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(CPacked),
                                _c_i64, _c_i64, _c_vp, _c_sz, _c_vp])
_sig("tq_angle_codebook_build", _c_i32, [_c_i32, _c_i32, ctypes.POINTER(CAngleCodebook)])
_sig("tq_polar_quantize_ws_bytes", _c_sz, [_c_vp, _c_i64])
_sig("tq_polar_quantize", _c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i64, ctypes.POINTER(CPolarPacked), _c_i64,
                                   _c_i64, _c_vp, _c_sz, _c_vp])
_sig("tq_polar_attention_decode_ws_bytes", _c_sz, [_c_vp, ctypes.POINTER(CCache), _c_i32])
_sig("tq_polar_attention_decode", _c_i32, [_c_vp, ctypes.POINTER(CPolarPacked), ctypes.POINTER(CCache), _c_vp, _c_i32,
                                           _c_i32, _c_f32, _c_vp, _c_vp, _c_sz, _c_vp])
_sig("tq_polar_scores_ws_bytes", _c_sz, [_c_vp, _c_i64, _c_i64])
_sig("tq_polar_scores", _c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, ctypes.POINTER(CPolarPacked), _c_vp, _c_vp, _c_sz,
                                 _c_vp])
_sig("tq_append_token", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_vp, _c_i32, _c_vp])
_sig("tq_cache_write", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_vp, _c_i32, _c_i64, _c_i64, _c_i64, _c_i64,
                                _c_vp, _c_sz, _c_vp])
_sig("tq_attention_decode_ws_bytes", _c_sz, [_c_vp, ctypes.POINTER(CCache), _c_i32])
_sig("tq_decode_step_ws_bytes", _c_sz, [_c_vp, ctypes.POINTER(CCache), _c_i32])
_sig("tq_decode_step", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_f32, _c_vp,
                                _c_vp, _c_sz, _c_vp])
_sig("tq_attention_decode", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_i32, _c_i32, _c_f32, _c_vp, _c_vp,
                                     _c_sz, _c_vp])
_sig("tq_attention_decode_noalloc", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_i32, _c_i32, _c_f32, _c_vp,
                                             _c_vp])
_sig("tq_decode_logits", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_i32, _c_i32, _c_f32, _c_vp, _c_vp, _c_sz,
                                  _c_vp])
_sig("tq_attention_prefill_ws_bytes", _c_sz, [_c_vp, ctypes.POINTER(CCache), _c_i32, _c_i32])
_sig("tq_attention_prefill", _c_i32, [_c_vp, ctypes.POINTER(CCache), _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                      _c_vp, _c_vp, _c_sz, _c_vp])
_sig("tq_time_next_decode", _c_i32, [_c_vp, _c_vp])
_sig("tq_read_probe", _c_i32, [_c_vp, _c_sz, _c_i32, _c_vp, _c_vp])
_sig("tq_scores_ws_bytes", _c_sz, [_c_vp, _c_i64, _c_i64, _c_i32, _c_i32])
_sig("tq_scores", _c_i32, [_c_vp, _c_vp, _c_i32, _c_i64, ctypes.POINTER(CPacked), _c_vp, _c_i32, _c_vp, _c_vp,
                           _c_vp, _c_sz, _c_vp])

EXPORTED_SYMBOLS = [
    "tq_format_version", "tq_gaussian_matrix", "tq_ctx_create_seeded",
    "tq_codebook_build", "tq_angle_codebook_build", "tq_rotation_build", "tq_ctx_create", "tq_ctx_destroy", "tq_ctx_dim", "tq_ctx_export", "tq_ctx_codebook",
    "tq_quantize_ws_bytes", "tq_quantize_kv", "tq_cache_write", "tq_append_token", "tq_attention_decode_ws_bytes",
    "tq_attention_decode", "tq_attention_decode_noalloc", "tq_decode_logits", "tq_attention_prefill_ws_bytes", "tq_attention_prefill", "tq_decode_step_ws_bytes",
    "tq_decode_step", "tq_time_next_decode", "tq_read_probe",
    "tq_scores_ws_bytes", "tq_scores", "tq_polar_quantize_ws_bytes", "tq_polar_quantize", "tq_polar_scores_ws_bytes",
    "tq_polar_scores", "tq_polar_attention_decode_ws_bytes", "tq_polar_attention_decode", "tq_last_error",
]


def last_error() -> str:
    return (_lib.tq_last_error() or b"").decode()


def _check(status: int):
    if status != TQ_OK:
        raise TQError(status, last_error())


def lib():
    """The loaded ctypes library (for tests of the raw C ABI)."""
    return _lib


def read_probe(src, grid, sink):
    """Stream all of `src` (a device tensor, 16-byte aligned, size a multiple of 16
    bytes) with the read-bandwidth probe kernel on the current stream; `sink` is a
    device int32/uint32 tensor of at least grid * 256 elements."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() < grid * 256 or sink.element_size() != 4:
        raise ValueError("read_probe: sink needs grid * 256 four-byte elements")
    _check(_lib.tq_read_probe(src.data_ptr(), nbytes, grid, sink.data_ptr(), _stream_ptr()))


def time_next_decode(start=None, stop=None):
    """Arm this thread's next decode call (KVCache.decode / decode_step) to record
    `start` and `stop` (torch.cuda.Event(enable_timing=True)) around its
    score/attention kernel, on that call's stream; no arguments disarm. An event
    that was never recorded has no device handle yet, so each one is recorded once
    here first (on the current stream) to create it."""
    if (start is None) != (stop is None):
        raise ValueError("time_next_decode: pass both events or neither")
    if start is None:
        _check(_lib.tq_time_next_decode(None, None))
        return
    for ev in (start, stop):
        if not ev.cuda_event:
            ev.record()
    _check(_lib.tq_time_next_decode(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)))


# ---------------------------------------------------------------------------
# Host-only calls
# ---------------------------------------------------------------------------

@dataclass
class Codebook:
    d: int
    bits: int
    centroids: np.ndarray
    boundaries: np.ndarray
    walsh: np.ndarray
    distortion: float


def _cb_from_c(c: CCodebook) -> Codebook:
    L = 1 << c.bits
    return Codebook(c.d, c.bits, np.array(c.centroid[:L], np.float32), np.array(c.boundary[:L - 1], np.float32),
                    np.array(c.walsh[:L // 2], np.float32), c.distortion)


def codebook_build(d: int, bits: int) -> Codebook:
    c = CCodebook()
    _check(_lib.tq_codebook_build(d, bits, ctypes.byref(c)))
    return _cb_from_c(c)


def angle_codebook_build(level: int, bits: int) -> dict:
    """PolarQuant angle codebook of one level (host only): fp64 centroids, fp32
    boundaries, cos and sin of the centroids."""
    c = CAngleCodebook()
    _check(_lib.tq_angle_codebook_build(level, bits, ctypes.byref(c)))
    L = 1 << bits
    return {"centroids": np.array(c.centroid[:L]), "boundaries": np.array(c.boundary[:L - 1], dtype=np.float32),
            "cos": np.array(c.cos_c[:L], dtype=np.float32), "sin": np.array(c.sin_c[:L], dtype=np.float32)}


TQ_STREAM_ROTATION, TQ_STREAM_SKETCH = 1, 2
FORMAT_VERSION = 1  # TQ_FORMAT_VERSION of include/tq.h


def format_version() -> int:
    """Version of the packed record formats the loaded library implements."""
    return int(_lib.tq_format_version())


def gaussian_matrix(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """Host-only: the library's seeded N(0,1) draws (float64, row-major)."""
    out = np.empty((rows, cols), np.float64)
    _check(_lib.tq_gaussian_matrix(seed, stream, rows, cols, out.ctypes.data))
    return out


def rotation_build(g: np.ndarray) -> np.ndarray:
    """Host-only: the fp32 rotation the library derives from Gaussian matrix g."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    d = g.shape[0]
    out = np.empty((d, d), np.float32)
    _check(_lib.tq_rotation_build(d, g.ctypes.data, out.ctypes.data))
    return out


# ---------------------------------------------------------------------------
# Context and packed arrays
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


class Context:
    """Rotation, sketch and codebooks on the current device.

    The Gaussian matrices the method draws come from `g_rot` / `g_sketch`
    (float64 d x d host arrays); by default they are drawn from the seeded
    generator in `synth` so that the CPU oracle can receive the same draws.
    """

    def __init__(self, d: int, seed: int = 0, g_rot: np.ndarray | None = None, g_sketch: np.ndarray | None = None):
        if g_rot is None or g_sketch is None:
            import synth
            g_rot = synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d) if g_rot is None else g_rot
            g_sketch = synth.gaussian_matrix(seed, synth.TAG_SKETCH, d, d) if g_sketch is None else g_sketch
        gr = np.ascontiguousarray(g_rot, dtype=np.float64)
        gs = np.ascontiguousarray(g_sketch, dtype=np.float64)
        if gr.shape != (d, d) or gs.shape != (d, d):
            raise ValueError("Gaussian matrices must be d x d")
        h = _c_vp()
        _check(_lib.tq_ctx_create(d, gr.ctypes.data, gs.ctypes.data, ctypes.byref(h)))
        self._h = h
        self.d = d

    @classmethod
    def from_seed(cls, d: int, seed: int) -> "Context":
        """A context built by the library from the seed alone (tq_ctx_create_seeded:
        its own counter-based Gaussian draws for the rotation and the sketch)."""
        self = cls.__new__(cls)
        h = _c_vp()
        _check(_lib.tq_ctx_create_seeded(d, seed, ctypes.byref(h)))
        self._h = h
        self.d = d
        return self

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            _lib.tq_ctx_destroy(self._h)
            self._h = _c_vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def export(self):
        rot = np.empty((self.d, self.d), np.float32)
        sk = np.empty((self.d, self.d), np.float32)
        _check(_lib.tq_ctx_export(self._h, rot.ctypes.data, sk.ctypes.data))
        return rot, sk

    def codebook(self, bits: int) -> Codebook:
        c = CCodebook()
        _check(_lib.tq_ctx_codebook(self._h, bits, ctypes.byref(c)))
        return _cb_from_c(c)


class Packed:
    """Device arrays of packed key or value records (format in include/tq.h)."""

    def __init__(self, n: int, d: int, bits: int, is_key: bool, device="cuda", qjl: bool = True,
                 norm_f16: bool = False):
        """Keys: bits = B MSE bits, qjl = the QJL sign word and |r| (False: MSE-only
        keys; bits = 0 with qjl: pure QJL keys). Values: bits = B, qjl ignored.
        norm_f16: compact records with fp16 norms."""
        torch = _torch()
        if not is_key and n % 32:
            raise ValueError("value capacity must be a multiple of 32")
        W = d // 32
        self.qjl = bool(qjl) and is_key
        self.n, self.d, self.bits, self.is_key = n, d, bits, is_key
        self.norm_f16 = bool(norm_f16)
        ndt = torch.float16 if self.norm_f16 else torch.float32
        if is_key:
            q = int(self.qjl)
            self.words = torch.zeros((n, W, bits + q), dtype=torch.int32, device=device)
            self.norms = torch.zeros((n, 1 + q), dtype=ndt, device=device)
        else:
            self.words = torch.zeros((n // 32, d, bits), dtype=torch.int32, device=device)
            self.norms = torch.zeros((n,), dtype=ndt, device=device)

    def c(self) -> CPacked:
        return CPacked(self.words.data_ptr(), self.norms.data_ptr(), self.n, self.bits, 1 if self.is_key else 0,
                       1 if self.qjl else 0, 1 if self.norm_f16 else 0)

    def host(self):
        """(uint32 words, norms: float32, or float16 when compact) copied to host numpy arrays."""
        return self.words.cpu().numpy().view(np.uint32), self.norms.cpu().numpy()


def quantize_ws_bytes(ctx: Context, n_streams: int, n_tokens: int, is_key: bool) -> int:
    return int(_lib.tq_quantize_ws_bytes(ctx.handle, n_streams, n_tokens, 1 if is_key else 0))


def quantize_kv(ctx: Context, x, out: Packed, n_streams: int | None = None, n_tokens: int | None = None,
                x_stream_stride: int | None = None, x_token_stride: int | None = None,
                out_stream_stride: int = 0, out_offset: int = 0, work=None):
    """Quantize x into `out`. x is [n, d] (one stream) or [streams, tokens, d]
    (any strides with d contiguous)."""
    torch = _torch()
    if x.dim() == 2:
        x3 = x.unsqueeze(0)
    else:
        x3 = x
    S = x3.shape[0] if n_streams is None else n_streams
    T = x3.shape[1] if n_tokens is None else n_tokens
    xs = x3.stride(0) if x_stream_stride is None else x_stream_stride
    xt = x3.stride(1) if x_token_stride is None else x_token_stride
    if x3.stride(-1) != 1:
        raise ValueError("the last dimension of x must be contiguous")
    if out_stream_stride == 0:
        out_stream_stride = T
    ws = None
    nbytes = 0
    if out.is_key:
        nbytes = quantize_ws_bytes(ctx, S, T, True)
        ws = work if work is not None else torch.empty(max(nbytes, 4), dtype=torch.uint8, device=x.device)
    cp = out.c()
    _check(_lib.tq_quantize_kv(ctx.handle, x.data_ptr(), _dtype_code(x), S, T, xs, xt, ctypes.byref(cp),
                               out_stream_stride, out_offset, ws.data_ptr() if ws is not None else None,
                               ws.numel() if ws is not None else 0, _stream_ptr()))


class KVCache:
    """Packed KV cache. Contiguous: records of stream (b, h) at
    (b*kv_heads + h)*capacity + t. Paged (page_tokens set): a pool of n_pages
    pages of page_tokens tokens per KV head, and block_table [batch,
    capacity/page_tokens] (device int32) names the page of each span of
    page_tokens positions of a sequence (token t of stream (b, h) is record
    (table[b, t // P]*kv_heads + h)*P + t % P)."""

    def __init__(self, batch: int, kv_heads: int, capacity: int, d: int, key_bits: int, value_bits: int,
                 device="cuda", key_qjl: bool = True, page_tokens: int | None = None, n_pages: int | None = None,
                 block_table=None, norm_f16: bool = False):
        """key_bits = B MSE bits of the keys; key_qjl = False stores MSE-only keys,
        key_bits = 0 with key_qjl stores pure QJL keys. page_tokens (a multiple of
        256 dividing capacity) selects the paged layout: n_pages defaults to
        batch*capacity/page_tokens, block_table to sequence b owning pages
        b*cols .. b*cols + cols - 1 (cols = capacity/page_tokens). norm_f16 stores
        every norm as fp16 (compact records)."""
        torch = _torch()
        if capacity % 32:
            raise ValueError("capacity must be a multiple of 32")
        self.page_tokens = page_tokens
        if page_tokens:
            if page_tokens % 256 or capacity % page_tokens:
                raise ValueError("page_tokens must be a multiple of 256 dividing capacity")
            cols = capacity // page_tokens
            self.n_pages = n_pages if n_pages is not None else batch * cols
            n = self.n_pages * kv_heads * page_tokens
            if block_table is None:
                block_table = torch.arange(batch * cols, dtype=torch.int32, device=device).view(batch, cols)
            assert block_table.dtype == torch.int32 and tuple(block_table.shape) == (batch, cols)
            self.block_table = block_table.contiguous()
        else:
            n = batch * kv_heads * capacity
            self.n_pages = 0
            self.block_table = None
        self.k = Packed(n, d, key_bits, True, device, qjl=key_qjl, norm_f16=norm_f16)
        self.v = Packed(n, d, value_bits, False, device, norm_f16=norm_f16)
        self.seq_len = torch.zeros((batch,), dtype=torch.int32, device=device)
        self.batch, self.kv_heads, self.capacity, self.d = batch, kv_heads, capacity, d
        self.host_max_len = 0

    def c(self) -> CCache:
        bt = self.block_table.data_ptr() if self.block_table is not None else None
        return CCache(self.k.c(), self.v.c(), self.batch, self.kv_heads, self.capacity, self.seq_len.data_ptr(),
                      self.host_max_len, bt, self.page_tokens or 0)

    def record_index(self, b: int, h: int, t: int) -> int:
        """Record of token t of stream (b, h) (host copy of the table for paged caches)."""
        if self.block_table is None:
            return (b * self.kv_heads + h) * self.capacity + t
        P = self.page_tokens
        page = int(self.block_table[b, t // P])
        return (page * self.kv_heads + h) * P + t % P

    def write(self, ctx: Context, k, v, pos0: int, work=None):
        """tq_cache_write: k, v [batch, kv_heads, tokens, d] (d contiguous, same
        strides) become positions pos0 .. pos0 + tokens - 1 of every stream.
        Lengths are not changed."""
        torch = _torch()
        B, H, T, d = k.shape
        assert (B, H) == (self.batch, self.kv_heads) and d == self.d and tuple(v.shape) == tuple(k.shape)
        assert k.stride() == v.stride() and k.stride(3) == 1 and k.stride(0) == H * k.stride(1)
        need = quantize_ws_bytes(ctx, B * H, T, True)
        if work is None or work.numel() < need:
            work = torch.empty(max(need, 4), dtype=torch.uint8, device=k.device)
        cc = self.c()
        _check(_lib.tq_cache_write(ctx.handle, ctypes.byref(cc), k.data_ptr(), v.data_ptr(), _dtype_code(k), T,
                                   k.stride(1), k.stride(2), pos0, work.data_ptr(), work.numel(), _stream_ptr()))

    def prefill(self, ctx: Context, k, v, work=None):
        """k, v: [batch, kv_heads, tokens, d] (d contiguous). Quantizes all tokens
        to positions 0..tokens-1 and sets every sequence length to `tokens`."""
        T = k.shape[2]
        assert T <= self.capacity
        self.write(ctx, k, v, 0, work)
        self.seq_len.fill_(T)
        self.host_max_len = T

    def extend(self, ctx: Context, k, v, work=None):
        """k, v: [batch, kv_heads, tokens, d]: a chunk of new tokens written after
        the current contents. Every sequence must hold host_max_len tokens, a
        multiple of 32 (value records are written in whole 32-token blocks); all
        lengths grow by `tokens`."""
        L0, T = self.host_max_len, k.shape[2]
        assert L0 % 32 == 0, "extend writes after a multiple of 32 tokens"
        assert L0 + T <= self.capacity
        self.write(ctx, k, v, L0, work)
        self.seq_len.fill_(L0 + T)
        self.host_max_len = L0 + T

    def append(self, ctx: Context, k, v):
        """k, v: [batch, kv_heads, d] contiguous, one new token per sequence."""
        assert k.is_contiguous() and v.is_contiguous() and k.dtype == v.dtype
        cc = self.c()
        _check(_lib.tq_append_token(ctx.handle, ctypes.byref(cc), k.data_ptr(), v.data_ptr(), _dtype_code(k),
                                    _stream_ptr()))
        self.host_max_len = cc.host_max_len

    def decode_ws_bytes(self, ctx: Context, q_heads: int) -> int:
        cc = self.c()
        return int(_lib.tq_attention_decode_ws_bytes(ctx.handle, ctypes.byref(cc), q_heads))

    def decode(self, ctx: Context, q, scale: float | None = None, out=None, ws=None):
        """q: [batch, q_heads, d] contiguous. Returns fp32 [batch, q_heads, d]."""
        torch = _torch()
        assert q.is_contiguous()
        B, Hq, d = q.shape
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        need = self.decode_ws_bytes(ctx, Hq)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
        cc = self.c()
        _check(_lib.tq_attention_decode(ctx.handle, ctypes.byref(cc), q.data_ptr(), _dtype_code(q), Hq,
                                        float(scale), out.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr()))
        return out

    def decode_logits(self, ctx: Context, q, scale: float | None = None, ws=None, out=None):
        """Measurement: the decode kernels' logits scale * s_t, fp32 [batch, q_heads,
        capacity] (entries past each sequence's length are NaN; with a caller's out,
        they keep what out held)."""
        torch = _torch()
        assert q.is_contiguous()
        B, Hq, d = q.shape
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.full((B, Hq, self.capacity), float("nan"), dtype=torch.float32, device=q.device)
        assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, Hq, self.capacity)
        need = self.decode_ws_bytes(ctx, Hq)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
        cc = self.c()
        _check(_lib.tq_decode_logits(ctx.handle, ctypes.byref(cc), q.data_ptr(), _dtype_code(q), Hq, float(scale),
                                     out.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr()))
        return out

    def prefill_ws_bytes(self, ctx: Context, n_q: int, q_heads: int) -> int:
        cc = self.c()
        return int(_lib.tq_attention_prefill_ws_bytes(ctx.handle, ctypes.byref(cc), n_q, q_heads))

    def attend(self, ctx: Context, q, causal: bool = True, scale: float | None = None, out=None, ws=None):
        """Many query positions per sequence over the cache: q [batch, n_q, q_heads, d]
        contiguous; causal: position i sees t < seq_len - n_q + i + 1. Returns fp32
        [batch, n_q, q_heads, d]."""
        torch = _torch()
        assert q.is_contiguous() and q.dim() == 4
        B, NQ, Hq, d = q.shape
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.empty((B, NQ, Hq, d), dtype=torch.float32, device=q.device)
        need = self.prefill_ws_bytes(ctx, NQ, Hq)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
        cc = self.c()
        _check(_lib.tq_attention_prefill(ctx.handle, ctypes.byref(cc), q.data_ptr(), _dtype_code(q), NQ, Hq,
                                         1 if causal else 0, float(scale), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                         _stream_ptr()))
        return out

    def decode_step_ws_bytes(self, ctx: Context, q_heads: int) -> int:
        cc = self.c()
        return int(_lib.tq_decode_step_ws_bytes(ctx.handle, ctypes.byref(cc), q_heads))

    def decode_step(self, ctx: Context, k, v, q, scale: float | None = None, out=None, ws=None):
        """Fused serving step: append k, v ([batch, kv_heads, d]) then decode q
        ([batch, q_heads, d]) with the new token attended. Returns fp32 [batch, q_heads, d]."""
        torch = _torch()
        assert k.is_contiguous() and v.is_contiguous() and q.is_contiguous()
        assert k.dtype == v.dtype == q.dtype
        B, Hq, d = q.shape
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        need = self.decode_step_ws_bytes(ctx, Hq)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
        cc = self.c()
        _check(_lib.tq_decode_step(ctx.handle, ctypes.byref(cc), k.data_ptr(), v.data_ptr(), q.data_ptr(),
                                   _dtype_code(q), Hq, float(scale), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream_ptr()))
        self.host_max_len = cc.host_max_len
        return out


def scores_ws_bytes(ctx: Context, nq: int, n: int, topk: int, want_scores: bool) -> int:
    return int(_lib.tq_scores_ws_bytes(ctx.handle, nq, n, topk, 1 if want_scores else 0))


def scores(ctx: Context, q, keys: Packed, want_scores: bool = True, topk: int = 0, ws=None):
    """q: [nq, d] contiguous. Returns (scores [nq, n] or None, top_idx, top_val)."""
    torch = _torch()
    assert q.is_contiguous() and keys.is_key
    nq = q.shape[0]
    sc = torch.empty((nq, keys.n), dtype=torch.float32, device=q.device) if want_scores else None
    ti = torch.empty((nq, max(topk, 1)), dtype=torch.int32, device=q.device) if topk else None
    tv = torch.empty((nq, max(topk, 1)), dtype=torch.float32, device=q.device) if topk else None
    need = scores_ws_bytes(ctx, nq, keys.n, topk, want_scores)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    kp = keys.c()
    _check(_lib.tq_scores(ctx.handle, q.data_ptr(), _dtype_code(q), nq, ctypes.byref(kp),
                          sc.data_ptr() if sc is not None else None, topk,
                          ti.data_ptr() if ti is not None else None, tv.data_ptr() if tv is not None else None,
                          ws.data_ptr(), ws.numel(), _stream_ptr()))
    return sc, ti, tv


class PolarPacked:
    """Device arrays of PolarQuant key records (d = 128; format in include/tq.h)."""

    def __init__(self, n: int, b1: int = 4, b2: int = 3, device="cuda"):
        torch = _torch()
        self.n, self.b1, self.b2 = n, b1, b2
        self.w1, self.w2 = (b1 * 64 + 31) // 32, (b2 * 63 + 31) // 32
        self.words = torch.zeros((n, self.w1 + self.w2), dtype=torch.int32, device=device)
        self.norms = torch.zeros((n,), dtype=torch.float32, device=device)

    def c(self) -> CPolarPacked:
        return CPolarPacked(self.words.data_ptr(), self.norms.data_ptr(), self.n, self.b1, self.b2)

    def host(self):
        return self.words.cpu().numpy().view(np.uint32), self.norms.cpu().numpy()


def polar_quantize(ctx: Context, x, out: PolarPacked, out_offset: int = 0, n_streams: int = 1,
                   out_stream_stride: int = 0, ws=None):
    """x: [rows, 128] (row stride a multiple of 8, 16-byte aligned), rows =
    n_streams x tokens stream-major -> record s * out_stream_stride +
    out_offset + t of `out`."""
    torch = _torch()
    rows = x.shape[0]
    assert rows % n_streams == 0
    T = rows // n_streams
    need = int(_lib.tq_polar_quantize_ws_bytes(ctx.handle, rows))
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    cp = out.c()
    _check(_lib.tq_polar_quantize(ctx.handle, x.data_ptr(), _dtype_code(x), n_streams, T, x.stride(0),
                                  ctypes.byref(cp), out_stream_stride, out_offset, ws.data_ptr(), ws.numel(),
                                  _stream_ptr()))


def polar_scores(ctx: Context, q, keys: PolarPacked, out=None, ws=None):
    """q: [nq, 128] contiguous -> fp32 scores [nq, keys.n]."""
    torch = _torch()
    assert q.is_contiguous()
    nq = q.shape[0]
    if out is None:
        out = torch.empty((nq, keys.n), dtype=torch.float32, device=q.device)
    need = int(_lib.tq_polar_scores_ws_bytes(ctx.handle, nq, keys.n))
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    kp = keys.c()
    _check(_lib.tq_polar_scores(ctx.handle, q.data_ptr(), _dtype_code(q), nq, ctypes.byref(kp), out.data_ptr(),
                                ws.data_ptr(), ws.numel(), _stream_ptr()))
    return out


class PolarKVCache:
    """PolarQuant keys with stage-1 values: key records of stream (b, h) at
    (b*kv_heads + h)*capacity + t in a PolarPacked array, values in the
    TurboQuant value format (the `values` cache's key array is unused)."""

    def __init__(self, batch: int, kv_heads: int, capacity: int, value_bits: int = 3, b1: int = 4, b2: int = 3,
                 device="cuda"):
        self.keys = PolarPacked(batch * kv_heads * capacity, b1, b2, device)
        self.values = KVCache(batch, kv_heads, capacity, 128, 1, value_bits, device)
        self.values.k = Packed(32, 128, 1, True, device)  # placeholder: the polar keys live in self.keys
        self.batch, self.kv_heads, self.capacity = batch, kv_heads, capacity
        self.seq_len = self.values.seq_len

    @property
    def host_max_len(self):
        return self.values.host_max_len

    @host_max_len.setter
    def host_max_len(self, v):
        self.values.host_max_len = v

    def prefill(self, ctx: Context, k, v):
        """k, v: [batch, kv_heads, tokens, 128] contiguous."""
        B, H, T, d = k.shape
        assert k.is_contiguous() and (B, H) == (self.batch, self.kv_heads) and T <= self.capacity
        polar_quantize(ctx, k.reshape(B * H * T, d), self.keys, 0, B * H, self.capacity)
        quantize_kv(ctx, v.reshape(B * H, T, d), self.values.v, n_streams=B * H, n_tokens=T,
                    out_stream_stride=self.capacity, out_offset=0)
        self.seq_len.fill_(T)
        self.values.host_max_len = T

    def decode_ws_bytes(self, ctx: Context, q_heads: int) -> int:
        cc = self.values.c()
        return int(_lib.tq_polar_attention_decode_ws_bytes(ctx.handle, ctypes.byref(cc), q_heads))

    def decode(self, ctx: Context, q, scale: float | None = None, out=None, ws=None):
        """q: [batch, q_heads, 128] contiguous -> fp32 [batch, q_heads, 128]."""
        torch = _torch()
        assert q.is_contiguous()
        B, Hq, d = q.shape
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        cc = self.values.c()
        need = self.decode_ws_bytes(ctx, Hq)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
        kp = self.keys.c()
        _check(_lib.tq_polar_attention_decode(ctx.handle, ctypes.byref(kp), ctypes.byref(cc), q.data_ptr(),
                                              _dtype_code(q), Hq, float(scale), out.data_ptr(), ws.data_ptr(),
                                              ws.numel(), _stream_ptr()))
        return out
