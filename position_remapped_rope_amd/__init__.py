"""Python binding of libprope (remapped-position RoPE attention on gfx950).

Argument marshalling only: every step of the computation runs in the HIP
library behind the C ABI declared in include/prope.h. PyTorch supplies device
memory and the current stream. If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["NOPE", "ROPE", "BIFOCAL", "PropeError", "lib", "lib_path", "rope_apply", "prefill", "prefill_queue",
           "prefill_bifocal_unfused", "bifocal_unfused_workspace_size", "decode", "decode_noalloc",
           "decode_workspace_size", "DECODE_SCRATCH_BYTES",
           "group_size", "status_string", "EXPORTED_SYMBOLS"]

NOPE, ROPE, BIFOCAL = 0, 1, 2
_MODES = {"nope": NOPE, "rope": ROPE, "bifocal": BIFOCAL}
REMOTE_ALIAS, REMOTE_INTERP = 0, 1
_REMOTE = {"alias": REMOTE_ALIAS, "interp": REMOTE_INTERP}
BF16, FP32 = 0, 1
DECODE_SCRATCH_BYTES = 16 << 20  # PROPE_DECODE_SCRATCH_BYTES

EXPORTED_SYMBOLS = ("prope_attn_prefill", "prope_attn_prefill_queued", "prope_prefill_queue_size",
                    "prope_attn_prefill_bifocal_unfused",
                    "prope_bifocal_unfused_workspace_size", "prope_attn_decode", "prope_attn_decode_noalloc",
                    "prope_decode_workspace_size",
                    "prope_rope_apply", "prope_group_size", "prope_status_string", "prope_version")

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree libprope.so, or the build PROPE_LIB_PATH names (e.g. a host-sanitized copy)."""
    return os.environ.get("PROPE_LIB_PATH") or os.path.join(_HERE, "libprope.so")


class PropeError(RuntimeError):
    pass


class PropeParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("period", ctypes.c_int32),
                ("remap_scale", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("w_pretrained", ctypes.c_int32), ("remote_map", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("interp_scale", ctypes.c_double),
                ("alibi_slopes", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libprope.so (once). Raises PropeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise PropeError(f"{path} is missing: build it with `python -m position_remapped_rope_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.prope_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     ctypes.POINTER(PropeParams), vp]
    L.prope_attn_prefill.restype = i32
    L.prope_attn_prefill_queued.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(PropeParams), vp, vp]
    L.prope_attn_prefill_queued.restype = i32
    L.prope_prefill_queue_size.argtypes = []
    L.prope_prefill_queue_size.restype = ctypes.c_size_t
    L.prope_attn_prefill_bifocal_unfused.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(PropeParams), vp, ctypes.c_size_t, vp]
    L.prope_attn_prefill_bifocal_unfused.restype = i32
    L.prope_bifocal_unfused_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.prope_bifocal_unfused_workspace_size.restype = ctypes.c_size_t
    L.prope_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                    ctypes.POINTER(PropeParams), vp, ctypes.c_size_t, vp]
    L.prope_attn_decode.restype = i32
    L.prope_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(PropeParams), vp]
    L.prope_attn_decode_noalloc.restype = i32
    L.prope_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    L.prope_decode_workspace_size.restype = ctypes.c_size_t
    L.prope_rope_apply.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_double, vp]
    L.prope_rope_apply.restype = i32
    L.prope_group_size.argtypes = [i64, i64]
    L.prope_group_size.restype = i32
    L.prope_status_string.argtypes = [i32]
    L.prope_status_string.restype = ctypes.c_char_p
    L.prope_version.argtypes = []
    L.prope_version.restype = i32
    _lib = L
    return L


def status_string(code: int) -> str:
    return lib().prope_status_string(code).decode()


def _check(code: int):
    if code != 0:
        raise PropeError(status_string(code))


def _params(mode, rope_base, period, remap_scale, window_left, softmax_scale, w_pretrained=0,
            remote_map="alias", interp_scale=0.0, alibi_slopes=None) -> PropeParams:
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    r = _REMOTE[remote_map] if isinstance(remote_map, str) else int(remote_map)
    return PropeParams(m, int(period), int(remap_scale), int(window_left), float(rope_base),
                       float(softmax_scale), int(w_pretrained), r, 0, float(interp_scale),
                       _ptr(alibi_slopes))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise PropeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise PropeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PropeError(f"{name} must be contiguous")


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _like(t, name, shape, dtype, device):
    """Check a caller-supplied output tensor: the C ABI cannot see buffer sizes."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device:
        raise PropeError(f"{name} must be {dtype} {list(shape)} on {device}, "
                         f"not {t.dtype} {list(t.shape)} on {t.device}")


def _slopes(alibi_slopes, Hq, device):
    import torch
    if alibi_slopes is None:
        return None
    _dev(alibi_slopes, "alibi_slopes")
    _like(alibi_slopes, "alibi_slopes", (Hq,), torch.float32, device)
    return alibi_slopes


# Work-queue buffers of the queued prefill, one per (device, stream): calls on
# one stream run in order and each leaves its queue zero for the next.
_queues = {}


def prefill_queue(device, stream: int):
    """The zero-filled work-queue buffer of prope_attn_prefill_queued for this (device, stream).

    Under HIP graph capture every call gets a buffer of its own, allocated (and
    zero-filled by a captured fill kernel) inside the capture: graphs captured on
    one stream may be replayed in any order or at the same time, so they must not
    share counters, and a cached buffer first created inside a capture would only
    be zeroed when the graph replays.
    """
    import torch
    n = int(lib().prope_prefill_queue_size())
    if torch.cuda.is_current_stream_capturing():
        return torch.zeros(n, dtype=torch.uint8, device=device)
    key = (torch.device(device).index, int(stream))
    buf = _queues.get(key)
    if buf is None:
        buf = torch.zeros(n, dtype=torch.uint8, device=device)
        _queues[key] = buf
    return buf


def group_size(L: int, w_pretrained: int) -> int:
    return lib().prope_group_size(int(L), int(w_pretrained))


def decode_workspace_size(B: int, Lmax: int, Hq: int, d: int) -> int:
    return lib().prope_decode_workspace_size(B, Lmax, Hq, d)


def rope_apply(x, pos, rope_base: float, out=None):
    """y = R_pos x for x [B,S,H,d] (bf16/fp32) and pos int32 [B,S]; out may be x."""
    import torch
    L = lib()
    _dev(x, "x"); _dev(pos, "pos")
    if pos.dtype != torch.int32 or x.dim() != 4 or tuple(pos.shape) != tuple(x.shape[:2]):
        raise PropeError("x must be [B,S,H,d] and pos int32 [B,S]")
    if pos.device != x.device:
        raise PropeError(f"pos must be on {x.device}")
    _like(out, "out", x.shape, x.dtype, x.device)
    y = torch.empty_like(x) if out is None else out
    _dev(y, "out")
    B, S, H, d = x.shape
    _check(L.prope_rope_apply(_ptr(x), _ptr(y), _ptr(pos), B, S, H, d, _dtype_code(x),
                              float(rope_base), _stream(x)))
    return y


def prefill(q, k, v, pos, mode="rope", rope_base: float = 1e4, period: int = 0,
            remap_scale: int = 1, window_left: int = -1, softmax_scale: float = 0.0,
            out=None, lse=None, return_lse: bool = False, w_pretrained: int = 0, remote_map="alias",
            schedule: str = "queue", interp_scale: float = 0.0, alibi_slopes=None):
    """Causal attention with RoPE fused under remapped ids (see include/prope.h).

    q [B,S,Hq,d], k/v [B,S,Hkv,d] unrotated; pos int32 [B,S] (None for NoPE).
    interp_scale: real remote scale s >= 1 of the interpolation map.
    alibi_slopes: float32 [Hq] device tensor of ALiBi slopes (nope/rope modes).
    schedule "queue" calls prope_attn_prefill_queued with this stream's queue
    buffer, "static" calls prope_attn_prefill; both give the same bits.
    Returns O [B,S,Hq,d] (and LSE float32 [B,Hq,S] if return_lse).
    """
    import torch
    L = lib()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (pos, "pos"), (out, "out"), (lse, "lse")):
        _dev(t, n)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise PropeError("k and v must be [B,S,Hkv,d] with q's dtype")
    if pos is not None and (pos.dtype != torch.int32 or tuple(pos.shape) != (B, S)):
        raise PropeError("pos must be int32 [B,S]")
    for t, n in ((k, "k"), (v, "v"), (pos, "pos")):
        if t is not None and t.device != q.device:
            raise PropeError(f"{n} must be on {q.device}")
    _like(out, "out", q.shape, q.dtype, q.device)
    _like(lse, "lse", (B, Hq, S), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    slopes = _slopes(alibi_slopes, Hq, q.device)
    p = _params(mode, rope_base, period, remap_scale, window_left, softmax_scale, w_pretrained, remote_map,
                interp_scale, slopes)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(pos), B, S, Hq, Hkv, d, _dtype_code(q),
            ctypes.byref(p))
    st = _stream(q)
    if schedule == "queue":
        _check(L.prope_attn_prefill_queued(*args, _ptr(prefill_queue(q.device, st)), st))
    elif schedule == "static":
        _check(L.prope_attn_prefill(*args, st))
    else:
        raise PropeError(f"schedule must be 'queue' or 'static', not {schedule!r}")
    return (o, lse) if return_lse else o


def bifocal_unfused_workspace_size(B: int, S: int, Hq: int, d: int, dtype_code: int = BF16) -> int:
    return lib().prope_bifocal_unfused_workspace_size(B, S, Hq, d, dtype_code)


def prefill_bifocal_unfused(q, k, v, pos, rope_base: float = 1e6, remap_scale: int = 1, window_left: int = -1,
                            softmax_scale: float = 0.0, out=None, lse=None, workspace=None,
                            return_lse: bool = False, w_pretrained: int = 0, remote_map="alias",
                            interp_scale: float = 0.0):
    """Bifocal prefill as three attention calls merged by Jet-Long Eq. (7) (see include/prope.h)."""
    import torch
    L = lib()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (pos, "pos"), (out, "out"), (lse, "lse"), (workspace, "workspace")):
        _dev(t, n)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise PropeError("k and v must be [B,S,Hkv,d] with q's dtype")
    if pos is None or pos.dtype != torch.int32 or tuple(pos.shape) != (B, S):
        raise PropeError("pos must be int32 [B,S]")
    for t, n in ((k, "k"), (v, "v"), (pos, "pos"), (workspace, "workspace")):
        if t is not None and t.device != q.device:
            raise PropeError(f"{n} must be on {q.device}")
    _like(out, "out", q.shape, q.dtype, q.device)
    _like(lse, "lse", (B, Hq, S), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    need = L.prope_bifocal_unfused_workspace_size(B, S, Hq, d, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    p = _params("bifocal", rope_base, 0, remap_scale, window_left, softmax_scale, w_pretrained, remote_map,
                interp_scale)
    _check(L.prope_attn_prefill_bifocal_unfused(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(pos),
                                                B, S, Hq, Hkv, d, _dtype_code(q), ctypes.byref(p),
                                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                _stream(q)))
    return (o, lse) if return_lse else o


def decode(q, k_cache, v_cache, kv_len, mode="bifocal", rope_base: float = 1e6,
           remap_scale: int = 1, window_left: int = -1, softmax_scale: float = 0.0,
           out=None, lse=None, workspace=None, return_lse: bool = False, w_pretrained: int = 0,
           remote_map="alias", interp_scale: float = 0.0, alibi_slopes=None, _noalloc: bool = False):
    """One decode step: q [B,Hq,d] base-rotated, caches [B,Lmax,Hkv,d], kv_len int32 [B]."""
    import torch
    L = lib()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_len, "kv_len"),
                 (out, "out"), (lse, "lse"), (workspace, "workspace")):
        _dev(t, n)
    B, Hq, d = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, Lmax, Hkv, d) or v_cache.shape != k_cache.shape:
        raise PropeError("caches must be [B,Lmax,Hkv,d]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise PropeError("k_cache and v_cache must have q's dtype")
    if kv_len.dtype != torch.int32 or tuple(kv_len.shape) != (B,):
        raise PropeError("kv_len must be int32 [B]")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (kv_len, "kv_len"), (workspace, "workspace")):
        if t is not None and t.device != q.device:
            raise PropeError(f"{n} must be on {q.device}")
    _like(out, "out", q.shape, q.dtype, q.device)
    _like(lse, "lse", (B, Hq), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    slopes = _slopes(alibi_slopes, Hq, q.device)
    p = _params(mode, rope_base, 0, remap_scale, window_left, softmax_scale, w_pretrained, remote_map,
                interp_scale, slopes)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(kv_len), B, Lmax, Hq, Hkv, d,
            _dtype_code(q), ctypes.byref(p))
    if _noalloc:
        if workspace is not None:
            raise PropeError("the no-allocation decode takes no workspace")
        _check(L.prope_attn_decode_noalloc(*args, _stream(q)))
        return (o, lse) if return_lse else o
    need = L.prope_decode_workspace_size(B, Lmax, Hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(L.prope_attn_decode(*args, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return (o, lse) if return_lse else o


def decode_noalloc(q, k_cache, v_cache, kv_len, out=None, lse=None, return_lse: bool = False, **kw):
    """decode() through prope_attn_decode_noalloc: the split-K partials live in the
    library's fixed device array (DECODE_SCRATCH_BYTES per device), so the call
    allocates no device memory when `out` (and `lse`, if wanted) are given."""
    return decode(q, k_cache, v_cache, kv_len, out=out, lse=lse, return_lse=return_lse, _noalloc=True, **kw)
