"""ctypes binding over libla_decode.so (include/la_decode.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library. There
is no fallback: if the library is not built, every call raises.

torch is imported before the library is loaded so that the process holds one
HIP runtime (torch's), which the library then shares.
"""
from __future__ import annotations

import array
import ctypes
import math
import os
import threading

import numpy as np

__all__ = [
    "LaError", "LA_F16", "LA_BF16", "LA_KIND_LEAN", "LA_KIND_FIXED_SPLIT", "LA_KIND_PER_HEAD",
    "LA_KIND_AUTO", "LA_KIND_PULL", "LA_KIND_CHUNKS", "lib", "la_decode", "la_decode_bf16", "la_decode_f16", "la_decode_ex",
    "la_decode_noalloc",
    "la_select", "la_select_for", "la_schedule",
    "la_schedule_dims", "la_default_tile", "la_max_grid", "la_max_grid_grouped", "la_default_grid",
    "la_sync_check",
    "la_last_error",
    "la_shutdown", "la_set_wait_limit_us", "la_stream_read", "decode_attention", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libla_decode.so")

LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EHIP, LA_ETIMEOUT, LA_ENOMEM = range(6)
LA_F16, LA_BF16 = 0, 1
LA_KIND_LEAN, LA_KIND_FIXED_SPLIT, LA_KIND_PER_HEAD, LA_KIND_AUTO = 0, 1, 2, 3
LA_KIND_PULL, LA_KIND_CHUNKS = 4, 5
_STATUS = {0: "LA_OK", 1: "LA_EINVAL", 2: "LA_EUNSUPPORTED", 3: "LA_EHIP", 4: "LA_ETIMEOUT",
           5: "LA_ENOMEM"}
_KINDS = {"lean": LA_KIND_LEAN, "fixed_split": LA_KIND_FIXED_SPLIT, "per_head": LA_KIND_PER_HEAD,
          "auto": LA_KIND_AUTO, "pull": LA_KIND_PULL, "chunks": LA_KIND_CHUNKS}
KIND_NAMES = {v: k for k, v in _KINDS.items()}


class LaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class LaOpts(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("kind", ctypes.c_int),
        ("tile_tokens", ctypes.c_int),
        ("grid", ctypes.c_int),
        ("num_splits", ctypes.c_int),
        ("cooperative", ctypes.c_int),
        ("m_out", ctypes.c_void_p),
        ("l_out", ctypes.c_void_p),
        ("tile_owner", ctypes.c_void_p),
        ("cta_timestamps", ctypes.c_void_p),
        ("ev_start", ctypes.c_void_p),
        ("ev_stop", ctypes.c_void_p),
        ("kv_heads", ctypes.c_int),
        ("q_tokens", ctypes.c_int),
        ("chunk_tiles", ctypes.c_int),
        ("host_tables", ctypes.c_int),
        ("kv_stride", ctypes.c_int),
        ("ctx_lens_device", ctypes.c_void_p),
        ("shared_gpu", ctypes.c_int),
    ]


_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_I32P = ctypes.POINTER(ctypes.c_int32)
_SIG = {
    "la_decode_bf16": (_I, [_P, _P, _P, _I32P, _I, _I, _I, ctypes.c_float, _P, _P]),
    "la_decode_f16": (_I, [_P, _P, _P, _I32P, _I, _I, _I, ctypes.c_float, _P, _P]),
    "la_decode": (_I, [_P, _P, _P, _I32P, _I, _I, _I, ctypes.c_float, _P, _P, _I]),
    "la_opts_init": (None, [ctypes.POINTER(LaOpts)]),
    "la_decode_ex": (_I, [_P, _P, _P, _I32P, _I, _I, _I, ctypes.c_float, _P, _P,
                          ctypes.POINTER(LaOpts)]),
    "la_decode_noalloc": (_I, [_P, _P, _P, _I32P, _I, _I, _I, ctypes.c_float, _P, _P,
                               ctypes.POINTER(LaOpts)]),
    "la_schedule_dims": (_I, [_I32P, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_int64),
                              ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "la_schedule": (_I, [_I32P, _I, _I, _I, _I, _I32P, _I32P, _I32P, _I, ctypes.POINTER(_I),
                         _I32P, _I32P]),
    "la_select_for": (_I, [_I32P, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I),
                           ctypes.POINTER(_I)]),
    "la_select": (_I, [_I32P, _I, _I, _I, ctypes.POINTER(LaOpts), ctypes.POINTER(_I),
                       ctypes.POINTER(_I)]),
    "la_default_tile": (_I, [_I]),
    "la_max_grid": (_I, [_I, _I]),
    "la_max_grid_grouped": (_I, [_I, _I]),
    "la_default_grid": (_I, [_I, _I]),
    "la_sync_check": (_I, [_P]),
    "la_last_error": (ctypes.c_char_p, []),
    "la_shutdown": (None, []),
    "la_set_wait_limit_us": (None, [ctypes.c_uint32]),
    "la_stream_read": (_I, [_P, ctypes.c_size_t, _I, _P, _P, ctypes.POINTER(ctypes.c_size_t)]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            import torch  # noqa: F401  (one HIP runtime per process: torch's)
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m decode_phase_attention_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIG.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
    return _lib


def la_last_error() -> str:
    return (lib().la_last_error() or b"").decode()


def _check(st: int):
    if st != LA_OK:
        raise LaError(st, la_last_error())


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if isinstance(x, torch.Tensor):
        if not x.is_cuda:
            raise ValueError("device tensors expected")
        if not x.is_contiguous():
            raise ValueError("contiguous tensors expected")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x).__name__} as a device pointer")


_I32_MIN, _I32_MAX = -(1 << 31), (1 << 31) - 1


if array.array("i").itemsize != 4:      # the fast path below hands the buffer over as int32
    raise ImportError("array typecode 'i' is not 32-bit on this platform")


def _lens(ctx_lens):
    """ctx_lens as a contiguous int32 array: (owner, pointer). The owner keeps
    the memory alive and supports len() and sum()."""
    if isinstance(ctx_lens, array.array) and ctx_lens.typecode == "i":
        a = ctx_lens
    elif isinstance(ctx_lens, (list, tuple)):
        # the common case, a list of integers: array.array converts and range-
        # checks in C (several times faster than a ctypes constructor)
        try:
            a = array.array("i", ctx_lens)
        except OverflowError:
            raise ValueError("ctx_lens entries must fit in int32") from None
        except TypeError:
            a = None              # not integers: let numpy convert (or reject) them
    else:
        a = None
    if a is not None:
        if len(a) == 0:
            return a, None
        return a, ctypes.cast(a.buffer_info()[0], _I32P)
    arr = np.ascontiguousarray(np.asarray(ctx_lens, dtype=np.int64))
    if arr.ndim != 1:
        raise ValueError("ctx_lens must be one-dimensional")
    if arr.size and (arr.min() < np.iinfo(np.int32).min or arr.max() > np.iinfo(np.int32).max):
        raise ValueError("ctx_lens entries must fit in int32")
    a32 = arr.astype(np.int32)
    return a32, a32.ctypes.data_as(_I32P)


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_torch_mod = None
_TORCH_DTYPES = {}          # LA_F16 / LA_BF16 -> torch dtype, filled with torch


def _torch():
    global _torch_mod
    if _torch_mod is None:
        import torch
        _TORCH_DTYPES.update({LA_F16: torch.float16, LA_BF16: torch.bfloat16})
        _torch_mod = torch
    return _torch_mod


def _check_sizes(q, k_cache, v_cache, out, ctx_lens, B, H, d, kv_heads=0, q_tokens=0,
                 m_out=None, l_out=None, kv_stride=0, dtype=None):
    """For torch tensors, reject a call that would read or write past them, or
    whose q, K and V are not all of the call's input type (the library sees
    only pointers and cannot check)."""
    Tensor = _torch().Tensor
    ins = [t for t in (q, k_cache, v_cache) if isinstance(t, Tensor)]
    if ins:
        want = ins[0].dtype if dtype is None else _TORCH_DTYPES.get(int(dtype))
        for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
            if isinstance(t, Tensor) and want is not None and t.dtype != want:
                raise ValueError(f"{name} is {t.dtype}; this call reads {want}")
    rows = int(B) * int(q_tokens or 1) * int(H)
    Hk = int(kv_heads or H)
    if kv_stride:
        kv = int(B) * Hk * int(kv_stride) * int(d)
    else:
        total = (int(ctx_lens.sum(dtype=np.int64)) if isinstance(ctx_lens, np.ndarray)
                 else sum(ctx_lens))
        kv = Hk * total * int(d)
    for name, t, need, size in (("q", q, rows * int(d), 2), ("k_cache", k_cache, kv, 2),
                                ("v_cache", v_cache, kv, 2), ("out", out, rows * int(d), 4),
                                ("m_out", m_out, rows, 4), ("l_out", l_out, rows, 4)):
        if t is not None and isinstance(t, Tensor):
            if t.element_size() != size:
                raise ValueError(f"{name}: {size}-byte elements expected, got {t.dtype}")
            if t.numel() < need:
                raise ValueError(f"{name} holds {t.numel()} elements; this call uses {need}")


def _dtype_of(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return LA_F16
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise ValueError(f"fp16 or bf16 expected, got {t.dtype}")


def la_decode(q, k_cache, v_cache, ctx_lens, B, H, d, scale, out, stream=None, dtype=None):
    """la_decode(q, k_cache, v_cache, ctx_lens, B, H, d, scale, out, stream, dtype)."""
    if dtype is None:
        dtype = _dtype_of(q)
    arr, p = _lens(ctx_lens)
    _check_sizes(q, k_cache, v_cache, out, arr, B, H, d, dtype=dtype)
    _check(lib().la_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), p, int(B), int(H), int(d),
                           float(scale), _ptr(out), _stream(stream), int(dtype)))


def la_decode_bf16(q, k_cache, v_cache, ctx_lens, B, H, d, scale, out, stream=None):
    arr, p = _lens(ctx_lens)
    _check_sizes(q, k_cache, v_cache, out, arr, B, H, d, dtype=LA_BF16)
    _check(lib().la_decode_bf16(_ptr(q), _ptr(k_cache), _ptr(v_cache), p, int(B), int(H), int(d),
                                float(scale), _ptr(out), _stream(stream)))


def la_decode_f16(q, k_cache, v_cache, ctx_lens, B, H, d, scale, out, stream=None):
    arr, p = _lens(ctx_lens)
    _check_sizes(q, k_cache, v_cache, out, arr, B, H, d, dtype=LA_F16)
    _check(lib().la_decode_f16(_ptr(q), _ptr(k_cache), _ptr(v_cache), p, int(B), int(H), int(d),
                               float(scale), _ptr(out), _stream(stream)))


def _marshal(q, k_cache, v_cache, ctx_lens, B, H, d, out, *, dtype, kind, tile_tokens, grid,
             num_splits, cooperative, m_out, l_out, tile_owner, cta_timestamps, ev_start, ev_stop,
             kv_heads, q_tokens, chunk_tiles, host_tables, kv_stride, ctx_lens_device,
             shared_gpu=False):
    """The la_opts of a call and its lengths pointer, after the size checks."""
    o = LaOpts()              # ctypes zero-fills it: the same as la_opts_init
    o.dtype = _dtype_of(q) if dtype is None else int(dtype)
    o.kind = _KINDS[kind] if isinstance(kind, str) else int(kind)
    # only the fields that differ from zero (each ctypes field store costs)
    if tile_tokens:
        o.tile_tokens = int(tile_tokens)
    if grid:
        o.grid = int(grid)
    if num_splits:
        o.num_splits = int(num_splits)
    if cooperative:
        o.cooperative = 1
    if m_out is not None:
        o.m_out = _ptr(m_out)
    if l_out is not None:
        o.l_out = _ptr(l_out)
    if tile_owner is not None:
        o.tile_owner = _ptr(tile_owner)
    if cta_timestamps is not None:
        o.cta_timestamps = _ptr(cta_timestamps)
    if ev_start is not None:
        o.ev_start = ev_start
    if ev_stop is not None:
        o.ev_stop = ev_stop
    if kv_heads:
        o.kv_heads = int(kv_heads)
    if q_tokens:
        o.q_tokens = int(q_tokens)
    if chunk_tiles:
        o.chunk_tiles = int(chunk_tiles)
    if host_tables:
        o.host_tables = 1
    if kv_stride:
        o.kv_stride = int(kv_stride)
    if shared_gpu:
        o.shared_gpu = 1
    if ctx_lens_device is not None:
        import torch
        if (isinstance(ctx_lens_device, torch.Tensor) and
                (ctx_lens_device.dtype != torch.int32 or ctx_lens_device.numel() < int(B) or
                 not ctx_lens_device.is_cuda or not ctx_lens_device.is_contiguous())):
            raise ValueError("ctx_lens_device must be a contiguous int32 device tensor of at "
                             "least B entries")
        o.ctx_lens_device = _ptr(ctx_lens_device)
        if not kv_stride:
            raise ValueError("ctx_lens_device needs kv_stride (a [B, Hk, S, d] cache)")
        arr, p = [], None
    else:
        arr, p = _lens(ctx_lens)
    _check_sizes(q, k_cache, v_cache, out, arr, B, H, d, kv_heads, q_tokens, m_out, l_out,
                 kv_stride, o.dtype)
    # keep the lengths array alive with the options until the call returns
    return o, arr, p


def la_decode_ex(q, k_cache, v_cache, ctx_lens, B, H, d, scale, out, stream=None, *, dtype=None,
                 kind="lean", tile_tokens=0, grid=0, num_splits=0, cooperative=False,
                 m_out=None, l_out=None, tile_owner=None, cta_timestamps=None, ev_start=None,
                 ev_stop=None, kv_heads=0, q_tokens=0, chunk_tiles=0, host_tables=False,
                 kv_stride=0, ctx_lens_device=None, shared_gpu=False):
    """la_decode_ex with the options as keywords. With ctx_lens_device (a
    device int32 tensor of B lengths), ctx_lens may be None."""
    o, arr, p = _marshal(q, k_cache, v_cache, ctx_lens, B, H, d, out, dtype=dtype, kind=kind,
                         tile_tokens=tile_tokens, grid=grid, num_splits=num_splits,
                         cooperative=cooperative, m_out=m_out, l_out=l_out, tile_owner=tile_owner,
                         cta_timestamps=cta_timestamps, ev_start=ev_start, ev_stop=ev_stop,
                         kv_heads=kv_heads, q_tokens=q_tokens, chunk_tiles=chunk_tiles,
                         host_tables=host_tables, kv_stride=kv_stride,
                         ctx_lens_device=ctx_lens_device, shared_gpu=shared_gpu)
    _check(lib().la_decode_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), p, int(B), int(H), int(d),
                              float(scale), _ptr(out), _stream(stream), ctypes.byref(o)))


def la_decode_noalloc(q, k_cache, v_cache, ctx_lens, B, H, d, scale, out, stream=None, *,
                      dtype=None, kind="lean", tile_tokens=0, grid=0, cooperative=False,
                      m_out=None, l_out=None, tile_owner=None, cta_timestamps=None,
                      ev_start=None, ev_stop=None, kv_heads=0, q_tokens=0, kv_stride=0,
                      ctx_lens_device=None):
    """la_decode_noalloc (the lean kind without any allocation) with the
    options as keywords, as la_decode_ex."""
    o, arr, p = _marshal(q, k_cache, v_cache, ctx_lens, B, H, d, out, dtype=dtype, kind=kind,
                         tile_tokens=tile_tokens, grid=grid, num_splits=0,
                         cooperative=cooperative, m_out=m_out, l_out=l_out, tile_owner=tile_owner,
                         cta_timestamps=cta_timestamps, ev_start=ev_start, ev_stop=ev_stop,
                         kv_heads=kv_heads, q_tokens=q_tokens, chunk_tiles=0, host_tables=False,
                         kv_stride=kv_stride, ctx_lens_device=ctx_lens_device)
    _check(lib().la_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), p, int(B), int(H),
                                   int(d), float(scale), _ptr(out), _stream(stream),
                                   ctypes.byref(o)))


def la_schedule_dims(ctx_lens, H, tile_tokens, grid):
    arr, p = _lens(ctx_lens)
    I = ctypes.c_int64()
    G = ctypes.c_int()
    rows = ctypes.c_int()
    _check(lib().la_schedule_dims(p, len(arr), int(H), int(tile_tokens), int(grid),
                                  ctypes.byref(I), ctypes.byref(G), ctypes.byref(rows)))
    return I.value, G.value, rows.value


def la_schedule(ctx_lens, H, tile_tokens, grid) -> dict:
    """Host scheduler tables as numpy arrays (keys as in the C header)."""
    arr, p = _lens(ctx_lens)
    I, G, rows = la_schedule_dims(arr, H, tile_tokens, grid)
    B = len(arr)
    cta_begin = np.zeros(G + 1, np.int32)
    cta_seg = np.zeros(G + 1, np.int32)
    seg = np.zeros((rows, 6), np.int32)
    host = np.zeros(B * H, np.int32)
    last = np.zeros(B * H, np.int32)
    n = ctypes.c_int()
    _check(lib().la_schedule(p, B, int(H), int(tile_tokens), int(grid),
                             cta_begin.ctypes.data_as(_I32P), cta_seg.ctypes.data_as(_I32P),
                             seg.ctypes.data_as(_I32P), rows, ctypes.byref(n),
                             host.ctypes.data_as(_I32P), last.ctypes.data_as(_I32P)))
    return {"I": I, "G": G, "cta_begin": cta_begin, "cta_seg": cta_seg, "seg": seg[:n.value],
            "host_cta": host, "last_cta": last}


def la_select_for(ctx_lens, H, d, cus, coresident, kv_heads=0, q_tokens=0, tile_tokens=0):
    """(kind name, grid) that kind="auto" picks on a device of this size (host only)."""
    arr, p = _lens(ctx_lens)
    kind, grid = ctypes.c_int(), ctypes.c_int()
    _check(lib().la_select_for(p, len(arr), int(H), int(d), int(kv_heads), int(q_tokens),
                               int(tile_tokens), int(cus), int(coresident), ctypes.byref(kind),
                               ctypes.byref(grid)))
    return KIND_NAMES[kind.value], grid.value


def la_select(ctx_lens, H, d, dtype, kv_heads=0, q_tokens=0, tile_tokens=0, shared_gpu=False):
    """(kind name, grid) that kind="auto" picks on the current device."""
    arr, p = _lens(ctx_lens)
    o = LaOpts()
    lib().la_opts_init(ctypes.byref(o))
    o.dtype = int(dtype)
    o.kv_heads = int(kv_heads)
    o.q_tokens = int(q_tokens)
    o.tile_tokens = int(tile_tokens)
    o.shared_gpu = 1 if shared_gpu else 0
    kind, grid = ctypes.c_int(), ctypes.c_int()
    _check(lib().la_select(p, len(arr), int(H), int(d), ctypes.byref(o), ctypes.byref(kind),
                           ctypes.byref(grid)))
    return KIND_NAMES[kind.value], grid.value


def la_default_tile(d: int) -> int:
    return int(lib().la_default_tile(int(d)))


def la_max_grid(d: int, dtype: int) -> int:
    g = int(lib().la_max_grid(int(d), int(dtype)))
    if g <= 0:
        raise LaError(LA_EHIP, la_last_error())
    return g


def la_stream_read(src, sink, grid=0, stream=None) -> int:
    """Read the device tensor `src` once with the attention kernels' access
    pattern and nothing else (a bandwidth measurement aid); `sink` is a device
    int32/uint32 tensor of at least one element. Returns the bytes read."""
    if src.element_size() * src.numel() < 1 or sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("src must be non-empty and sink a 4-byte device tensor")
    n = ctypes.c_size_t()
    _check(lib().la_stream_read(_ptr(src), src.element_size() * src.numel(), int(grid),
                                _ptr(sink), _stream(stream), ctypes.byref(n)))
    return int(n.value)


def la_max_grid_grouped(d: int, dtype: int) -> int:
    g = int(lib().la_max_grid_grouped(int(d), int(dtype)))
    if g <= 0:
        raise LaError(LA_EHIP, la_last_error())
    return g


def la_default_grid(d: int, dtype: int) -> int:
    g = int(lib().la_default_grid(int(d), int(dtype)))
    if g <= 0:
        raise LaError(LA_EHIP, la_last_error())
    return g


def la_sync_check(stream=None):
    _check(lib().la_sync_check(_stream(stream)))


def la_shutdown():
    lib().la_shutdown()


def la_set_wait_limit_us(us: int):
    lib().la_set_wait_limit_us(int(us))


def decode_attention(q, k_cache, v_cache, ctx_lens, scale=None, kind="lean", out=None,
                     stream=None, **opts):
    """Convenience wrapper: shapes from the tensors, fp32 output allocated if
    not given. q is [B, H, d], or [B, Nq, H, d] for Nq new tokens per request;
    k_cache/v_cache are packed [kv_heads * sum(n_b), d], or a cache
    [B, kv_heads, S, d] of S >= max(n_b) rows per head (kv_heads and kv_stride
    then come from its shape). ctx_lens is a host sequence, or -- with such a
    cache -- an int32 device tensor that the kernel reads in the launch (lean
    kind; the call can then be captured into a graph)."""
    import torch
    dev_lens = isinstance(ctx_lens, torch.Tensor) and ctx_lens.is_cuda
    if dev_lens:
        if k_cache.dim() != 4:
            raise ValueError("lengths on the device need a [B, kv_heads, S, d] cache")
        opts["ctx_lens_device"] = ctx_lens
    if q.dim() == 4:
        B, Nq, H, d = q.shape
        opts["q_tokens"] = Nq
    else:
        B, H, d = q.shape
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if len(ctx_lens) != B:
        raise ValueError("ctx_lens must have B entries")
    if k_cache.dim() == 4:
        Bk, Hk, S, dk = k_cache.shape
        if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("a [B, kv_heads, S, d] cache must match q in B and d, and V must match K")
        opts["kv_heads"], opts["kv_stride"] = Hk, S
        for t in (k_cache, v_cache):
            if t.dtype != q.dtype or not t.is_contiguous():
                raise ValueError("k_cache/v_cache must be contiguous, in q's dtype")
    else:
        total = int(np.sum(np.asarray(ctx_lens, dtype=np.int64)))
        Hk = int(opts.get("kv_heads") or H)
        for t in (k_cache, v_cache):
            if tuple(t.shape) != (Hk * total, d) or t.dtype != q.dtype:
                raise ValueError("k_cache/v_cache must be [kv_heads * sum(ctx_lens), d] in q's dtype")
    la_decode_ex(q, k_cache, v_cache, None if dev_lens else ctx_lens, B, H, d, scale, out, stream,
                 kind=kind, **opts)
    return out
