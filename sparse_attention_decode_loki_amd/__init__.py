"""Python binding of libloki.so (Loki decode-step sparse attention, gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
libloki.so (or, for calibrate, its host C++ code).  torch supplies device
memory and the current stream.  Importing this package does not load the
library; the first call does, and raises if libloki.so has not been built.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libloki.so")

LOKI_OK, LOKI_EINVAL, LOKI_EWORKSPACE, LOKI_EDEVICE, LOKI_EUNSUPPORTED = 0, -1, -2, -3, -4
LOKI_F32, LOKI_BF16 = 0, 1
PATH_AUTO, PATH_FUSED, PATH_SPLIT, PATH_UNION, PATH_SLICED = 0, 1, 2, 3, 4

# name -> (restype, argtypes); mirrors include/loki.h
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F64 = ctypes.c_double
_SIGS = {
    "loki_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "loki_abi_version": (ctypes.c_int, []),
    "loki_calibrate": (ctypes.c_int, [_P, ctypes.c_int64, _I, _P, _P]),
    "loki_kv_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "loki_decode_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "loki_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                   _P, _P, _P, ctypes.c_size_t, _P]),
    "loki_decode_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                      _P, _P, _P, ctypes.c_size_t, _I, _P]),
    "loki_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                        _I, _I, _P, _P, _P, ctypes.c_size_t, _I, _P]),
    "loki_decode_path": (ctypes.c_int, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "loki_scores": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P,
                                   ctypes.c_size_t, _P]),
    "loki_topk": (ctypes.c_int, [_P, _I, _I, _I, _I, _P, _P]),
    "loki_attend_indices": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _I,
                                           _I, _P, _P, ctypes.c_size_t, _P]),
    "loki_dense_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P,
                                         _P, ctypes.c_size_t, _P]),
    "loki_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _I, _P]),
    "loki_stream_read_shares": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _I, _I, _I, _P]),
    "loki_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                           _P, _P, _I, _P]),
    "loki_kv_append_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                           _F64, _P]),
    "loki_decode_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                        _F64, _P, _P, _P, ctypes.c_size_t, _I, _P]),
    "loki_decode_step_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                             _I, _I, _I, _F64, _P, _P, _P, ctypes.c_size_t, _I,
                                             _P]),
    "loki_dense_decode_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                              _I, _F64, _P, _P, ctypes.c_size_t, _P]),
}

_lib = None


class LokiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load(path: str | None = None):
    """Load libloki.so (once).  Raises FileNotFoundError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} not built; run python -m sparse_attention_decode_loki_amd.build_lib")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> list[str]:
    return list(_SIGS)


def status_string(status: int) -> str:
    return load().loki_status_string(int(status)).decode()


def _check(st: int, where: str):
    if st != LOKI_OK:
        raise LokiError(st, where)


# ------------------------------------------------------------ torch glue --

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return LOKI_F32
    if t.dtype == torch.bfloat16:
        return LOKI_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    """Reject a tensor the library could not use safely: the C ABI sees only
    pointers, so a wrong extent would become an out-of-bounds device access
    rather than an error.  Checks shape, dtype, contiguity and device."""
    if t is None:
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the cache on {device}")


def _on_gpu(t, name):
    """Last check of every call: its tensors (all on one device by then) are
    in device memory."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _need_q(q, cache):
    """q [cache.B, Hq, cache.D] in the cache dtype, Hq a multiple of cache.Hkv.
    Returns (B, Hq, D)."""
    if q is None or q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq, D = q.shape
    if Hq < 1 or Hq % cache.Hkv != 0:
        raise ValueError(f"q has {Hq} heads, not a multiple of the cache's {cache.Hkv} KV heads")
    _need(q, "q", cache.dtype, (cache.B, Hq, cache.D), cache.device)
    return B, Hq, D


def _need_P(P, cache):
    _need(P, "P", _torch().float32, (cache.Hkv, cache.D, cache.D), cache.device)


def _need_new(k_new, v_new, cache, step: bool):
    """New keys/values: [B, Hkv, D] for a decode step, [B, Hkv, T, D] for an
    append.  Returns T."""
    if k_new is None or k_new.dim() != (3 if step else 4):
        raise ValueError("k_new must be " + ("[B, Hkv, D]" if step else "[B, Hkv, T, D]"))
    shape = (cache.B, cache.Hkv, cache.D) if step else (cache.B, cache.Hkv, k_new.shape[2], cache.D)
    _need(k_new, "k_new", cache.dtype, shape, cache.device)
    _need(v_new, "v_new", cache.dtype, shape, cache.device)
    return 1 if step else shape[2]


def _out(out, shape, device, name="out"):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _need(out, name, torch.float32, shape, device)
    return out


def _idx(idx, shape, device):
    torch = _torch()
    if idx is None:
        return torch.empty(shape, dtype=torch.int32, device=device)
    _need(idx, "idx", torch.int32, shape, device)
    return idx


def _ws(workspace, device):
    if workspace is not None:
        _need(workspace, "workspace", device=device)
    return workspace


def _ws_bytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


class KVCache:
    """Device buffers of a Loki key/value cache with capacity S_max:
    k_slab [B, Hkv, S_max, d], k_rest [B, Hkv, S_max, D-d] (None if d == D),
    v [B, Hkv, S_max, D]; `length` counts the tokens appended so far."""

    def __init__(self, B, Hkv, S_max, D, d, dtype, device="cuda"):
        torch = _torch()
        self.B, self.Hkv, self.S_max, self.D, self.d = B, Hkv, S_max, D, d
        self.dtype = dtype
        self.k_slab = torch.zeros((B, Hkv, S_max, d), dtype=dtype, device=device)
        self.k_rest = (torch.zeros((B, Hkv, S_max, D - d), dtype=dtype, device=device)
                       if d < D else None)
        self.v = torch.zeros((B, Hkv, S_max, D), dtype=dtype, device=device)
        self.length = 0

    @property
    def device(self):
        return self.v.device


def calibrate(keys: np.ndarray):
    """PCA basis of sample keys (host).  keys [n, D] -> (P [D, D] float32,
    eigvals [D] float64), columns = principal axes, variance descending."""
    lib = load()
    k = np.ascontiguousarray(keys, dtype=np.float32)
    n, D = k.shape
    P = np.empty((D, D), dtype=np.float32)
    ev = np.empty(D, dtype=np.float64)
    _check(lib.loki_calibrate(k.ctypes.data, n, D, P.ctypes.data, ev.ctypes.data), "loki_calibrate")
    return P, ev


def append(cache: KVCache, k_new, v_new, P, pos: int | None = None,
           rope_base: float | None = None):
    """Rotate and store k_new/v_new [B, Hkv, T, D] at positions pos..pos+T-1
    (default: the cache's current length, which then advances).  With
    rope_base, each key is first given the rotary embedding of its position
    (loki_kv_append_rope)."""
    lib = load()
    T = _need_new(k_new, v_new, cache, step=False)
    _need_P(P, cache)
    _on_gpu(k_new, "k_new")
    at = cache.length if pos is None else pos
    args = (_ptr(k_new), _ptr(v_new), _ptr(P), _ptr(cache.k_slab), _ptr(cache.k_rest),
            _ptr(cache.v), cache.B, cache.Hkv, cache.D, cache.d, cache.S_max, at, T,
            _dtype_code(k_new))
    if rope_base is None:
        st = lib.loki_kv_append(*args, _stream(k_new))
    else:
        st = lib.loki_kv_append_rope(*args, float(rope_base), _stream(k_new))
    _check(st, "loki_kv_append")
    if pos is None or at + T > cache.length:
        cache.length = max(cache.length, at + T)


def workspace_size(B, Hq, S_max, D, k_max) -> int:
    """loki_decode_workspace_size: bytes of device workspace (same argument
    order as the C call)."""
    return int(load().loki_decode_workspace_size(B, Hq, S_max, D, k_max))


def alloc_workspace(B, Hq, S_max, D, k_max, device="cuda"):
    torch = _torch()
    n = max(workspace_size(B, Hq, S_max, D, k_max), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _decode_args(q, cache, P, k, S, out, idx, workspace, path):
    """Checked and allocated arguments shared by decode and DecodePlan."""
    B, Hq, D = _need_q(q, cache)
    _need_P(P, cache)
    S = cache.length if S is None else S
    kk = min(k, S)
    dev = cache.device
    out = _out(out, (B, Hq, D), dev)
    idx = _idx(idx, (B, Hq, kk), dev)
    workspace = _ws(workspace, dev)
    _on_gpu(q, "q")
    if workspace is None and path != PATH_FUSED:
        workspace = alloc_workspace(B, Hq, cache.S_max, D, kk, dev)
    head = (_ptr(q), _ptr(cache.k_slab), _ptr(cache.k_rest), _ptr(cache.v), _ptr(P),
            B, Hq, cache.Hkv, D, cache.d, S, cache.S_max, k, _dtype_code(q))
    tail = (_ptr(out), _ptr(idx), _ptr(workspace), _ws_bytes(workspace), path, _stream(q))
    return S, out, idx, workspace, head, tail


def decode(q, cache: KVCache, P, k: int, S: int | None = None, out=None, idx=None,
           workspace=None, path: int = PATH_AUTO, rope_base: float | None = None,
           q_pos: int | None = None):
    """One Loki decode step.  q [B, Hq, D] -> (out [B, Hq, D] float32,
    idx [B, Hq, min(k, S)] int32 ascending).  With rope_base the query is
    given the rotary embedding of position q_pos (default S - 1) first
    (loki_decode_rope; the cache must hold embedded keys)."""
    lib = load()
    S, out, idx, _ws_keep, head, tail = _decode_args(q, cache, P, k, S, out, idx, workspace, path)
    if rope_base is None:
        st = lib.loki_decode_ex(*head, *tail)
    else:
        st = lib.loki_decode_rope(*head, S - 1 if q_pos is None else q_pos, float(rope_base),
                                  *tail)
    _check(st, "loki_decode")
    return out, idx


# bytes of the library's own scratch behind decode_noalloc (one copy per GPU)
NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_noalloc(q, cache: KVCache, P, k: int, out, idx, S: int | None = None,
                   path: int = PATH_AUTO):
    """loki_decode_noalloc: decode_ex without a workspace (the split and
    union paths use the library's per-GPU scratch array).  out [B, Hq, D]
    float32 and idx [B, Hq, min(k, S)] int32 are the caller's; nothing is
    allocated here either."""
    lib = load()
    B, Hq, D = _need_q(q, cache)
    _need_P(P, cache)
    S = cache.length if S is None else S
    dev = cache.device
    _need(out, "out", _torch().float32, (B, Hq, D), dev)
    _need(idx, "idx", _torch().int32, (B, Hq, min(k, S)), dev)
    _on_gpu(q, "q")
    st = lib.loki_decode_noalloc(_ptr(q), _ptr(cache.k_slab), _ptr(cache.k_rest), _ptr(cache.v),
                                 _ptr(P), B, Hq, cache.Hkv, D, cache.d, S, cache.S_max, k,
                                 _dtype_code(q), _ptr(out), _ptr(idx), path, _stream(q))
    _check(st, "loki_decode_noalloc")
    return out, idx


def _step_args(q, k_new, v_new, cache, P, k, pos, out, idx, workspace, path):
    """Checked and allocated arguments shared by decode_step and StepPlan."""
    B, Hq, D = _need_q(q, cache)
    _need_new(k_new, v_new, cache, step=True)
    _need_P(P, cache)
    kk = min(k, pos + 1)
    dev = cache.device
    out = _out(out, (B, Hq, D), dev)
    idx = _idx(idx, (B, Hq, kk), dev)
    workspace = _ws(workspace, dev)
    _on_gpu(q, "q")
    if workspace is None and path != PATH_FUSED:
        workspace = alloc_workspace(B, Hq, cache.S_max, D, kk, dev)
    head = (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(P), _ptr(cache.k_slab), _ptr(cache.k_rest),
            _ptr(cache.v), B, Hq, cache.Hkv, D, cache.d, pos, cache.S_max, k, _dtype_code(q))
    tail = (_ptr(out), _ptr(idx), _ptr(workspace), _ws_bytes(workspace), path, _stream(q))
    return out, idx, workspace, head, tail


def decode_step(q, k_new, v_new, cache: KVCache, P, k: int, pos: int | None = None, out=None,
                idx=None, workspace=None, path: int = PATH_AUTO, rope_base: float | None = None):
    """Append k_new/v_new [B, Hkv, D] at `pos` (default: the cache length) and
    decode over pos + 1 tokens, in one call.  With rope_base the new key and
    the query are both embedded at pos (loki_decode_step_rope).  Returns
    (out, idx)."""
    lib = load()
    at = cache.length if pos is None else pos
    out, idx, _ws_keep, head, tail = _step_args(q, k_new, v_new, cache, P, k, at, out, idx,
                                                workspace, path)
    if rope_base is None:
        st = lib.loki_decode_step(*head, *tail)
    else:
        st = lib.loki_decode_step_rope(*head, float(rope_base), *tail)
    _check(st, "loki_decode_step")
    cache.length = max(cache.length, at + 1)
    return out, idx


def decode_path(B, Hq, Hkv, D, d, S, k, dtype="bf16", path=PATH_AUTO) -> int:
    """The path (PATH_FUSED, PATH_SPLIT or PATH_UNION) loki_decode_ex takes
    for these sizes and cache dtype ("bf16" or "f32")."""
    code = {"bf16": LOKI_BF16, "f32": LOKI_F32}[dtype]
    st = load().loki_decode_path(B, Hq, Hkv, D, d, S, k, code, path)
    if st < 0:
        raise LokiError(st, "loki_decode_path")
    return st


def scores(q, cache: KVCache, P, S: int | None = None, out=None, workspace=None):
    """Ranking scores [B, Hq, S] float32 (the low-rank pass alone)."""
    lib = load()
    B, Hq, D = _need_q(q, cache)
    _need_P(P, cache)
    S = cache.length if S is None else S
    dev = cache.device
    out = _out(out, (B, Hq, S), dev, "scores")
    workspace = _ws(workspace, dev)
    _on_gpu(q, "q")
    if workspace is None:
        workspace = alloc_workspace(B, Hq, cache.S_max, D, 1, dev)
    st = lib.loki_scores(_ptr(q), _ptr(cache.k_slab), _ptr(P), B, Hq, cache.Hkv, D, cache.d, S,
                         cache.S_max, _dtype_code(q), _ptr(out), _ptr(workspace),
                         _ws_bytes(workspace), _stream(q))
    _check(st, "loki_scores")
    return out


def topk(scores_2d, k: int, S: int | None = None, idx=None):
    """Top-k of each row of a float32 device matrix [rows, ld]; ascending ids."""
    torch = _torch()
    lib = load()
    if scores_2d is None or scores_2d.dim() != 2:
        raise ValueError("scores must be [rows, ld]")
    _need(scores_2d, "scores", torch.float32)
    rows, ld = scores_2d.shape
    S = ld if S is None else S
    if not 1 <= S <= ld:
        raise ValueError(f"S must be in [1, {ld}]")
    kk = min(k, S)
    idx = _idx(idx, (rows, kk), scores_2d.device)
    _on_gpu(scores_2d, "scores")
    st = lib.loki_topk(_ptr(scores_2d), rows, S, ld, k, _ptr(idx), _stream(scores_2d))
    _check(st, "loki_topk")
    return idx


def attend_indices(q, cache: KVCache, P, idx, S: int | None = None, out=None, workspace=None):
    """Exact attention over given ascending index rows idx [B, Hq, k] int32."""
    torch = _torch()
    lib = load()
    B, Hq, D = _need_q(q, cache)
    _need_P(P, cache)
    if idx is None or idx.dim() != 3:
        raise ValueError("idx must be [B, Hq, k]")
    k = idx.shape[-1]
    dev = cache.device
    _need(idx, "idx", torch.int32, (B, Hq, k), dev)
    S = cache.length if S is None else S
    out = _out(out, (B, Hq, D), dev)
    workspace = _ws(workspace, dev)
    _on_gpu(q, "q")
    if workspace is None:
        workspace = alloc_workspace(B, Hq, cache.S_max, D, k, dev)
    st = lib.loki_attend_indices(_ptr(q), _ptr(cache.k_slab), _ptr(cache.k_rest), _ptr(cache.v),
                                 _ptr(P), B, Hq, cache.Hkv, D, cache.d, S, cache.S_max, _ptr(idx),
                                 k, _dtype_code(q), _ptr(out), _ptr(workspace),
                                 _ws_bytes(workspace), _stream(q))
    _check(st, "loki_attend_indices")
    return out


def _dense_args(q, cache, P, S, out, workspace):
    B, Hq, D = _need_q(q, cache)
    _need_P(P, cache)
    S = cache.length if S is None else S
    dev = cache.device
    out = _out(out, (B, Hq, D), dev)
    workspace = _ws(workspace, dev)
    _on_gpu(q, "q")
    if workspace is None:
        workspace = alloc_workspace(B, Hq, cache.S_max, D, 1, dev)
    head = (_ptr(q), _ptr(cache.k_slab), _ptr(cache.k_rest), _ptr(cache.v), _ptr(P), B, Hq,
            cache.Hkv, D, cache.d, S, cache.S_max, _dtype_code(q))
    tail = (_ptr(out), _ptr(workspace), _ws_bytes(workspace), _stream(q))
    return S, out, workspace, head, tail


def dense_decode(q, cache: KVCache, P, S: int | None = None, out=None, workspace=None,
                 rope_base: float | None = None, q_pos: int | None = None):
    """Dense attention over all S tokens of the same rotated cache (the query
    embedded at q_pos, default S - 1, when rope_base is given)."""
    lib = load()
    S, out, _ws_keep, head, tail = _dense_args(q, cache, P, S, out, workspace)
    if rope_base is None:
        st = lib.loki_dense_decode(*head, *tail)
    else:
        st = lib.loki_dense_decode_rope(*head, S - 1 if q_pos is None else q_pos,
                                        float(rope_base), *tail)
    _check(st, "loki_dense_decode")
    return out


def stream_read(buf, sink, workgroups: int):
    """Measurement helper: read all of `buf` (a contiguous device tensor whose
    byte size is a multiple of 16) with the library's streaming-read probe;
    `sink` is a float32 device tensor of at least workgroups * 256 entries."""
    torch = _torch()
    _need(buf, "buf")
    _need(sink, "sink", torch.float32, device=buf.device)
    _on_gpu(buf, "buf")
    if sink.numel() < workgroups * 256:
        raise ValueError("sink needs workgroups * 256 floats")
    st = load().loki_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 workgroups, _stream(buf))
    _check(st, "loki_stream_read")


def stream_read_shares(buf, sink, workgroups: int, threads: int = 256, loads: int = 4):
    """Measurement helper: each of `workgroups` workgroups of `threads`
    threads reads its own contiguous share of `buf` (a contiguous device
    tensor whose byte size is a multiple of 16 * workgroups) with `loads`
    16-byte loads in flight per lane; `sink` is a float32 device tensor of at
    least workgroups * threads entries."""
    torch = _torch()
    _need(buf, "buf")
    _need(sink, "sink", torch.float32, device=buf.device)
    _on_gpu(buf, "buf")
    if sink.numel() < workgroups * threads:
        raise ValueError("sink needs workgroups * threads floats")
    st = load().loki_stream_read_shares(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                        workgroups, threads, loads, _stream(buf))
    _check(st, "loki_stream_read_shares")


# ------------------------------------------------- pre-marshalled calls --

class DecodePlan:
    """A decode call with every argument marshalled once, for loops that
    call loki_decode_ex repeatedly on the same buffers (q may be refilled in
    place between calls).  The stream is the current stream at creation."""

    def __init__(self, q, cache: KVCache, P, k: int, S: int | None = None, out=None, idx=None,
                 workspace=None, path: int = PATH_AUTO, rope_base: float | None = None,
                 q_pos: int | None = None):
        S, self.out, self.idx, workspace, head, tail = _decode_args(q, cache, P, k, S, out, idx,
                                                                    workspace, path)
        self._keep = (q, cache, P, workspace)
        if rope_base is None:
            self._fn = load().loki_decode_ex
            self._args = head + tail
        else:
            self._fn = load().loki_decode_rope
            self._args = head + (S - 1 if q_pos is None else q_pos, float(rope_base)) + tail

    def __call__(self):
        st = self._fn(*self._args)
        if st != LOKI_OK:
            raise LokiError(st, "loki_decode")
        return self.out, self.idx


class AppendPlan:
    """An append call marshalled once (fixed source buffers and position)."""

    def __init__(self, cache: KVCache, k_new, v_new, P, pos: int, rope_base: float | None = None):
        T = _need_new(k_new, v_new, cache, step=False)
        _need_P(P, cache)
        _on_gpu(k_new, "k_new")
        self._keep = (cache, k_new, v_new, P)
        args = (_ptr(k_new), _ptr(v_new), _ptr(P), _ptr(cache.k_slab), _ptr(cache.k_rest),
                _ptr(cache.v), cache.B, cache.Hkv, cache.D, cache.d, cache.S_max, pos, T,
                _dtype_code(k_new))
        if rope_base is None:
            self._fn = load().loki_kv_append
            self._args = args + (_stream(k_new),)
        else:
            self._fn = load().loki_kv_append_rope
            self._args = args + (float(rope_base), _stream(k_new))

    def __call__(self):
        st = self._fn(*self._args)
        if st != LOKI_OK:
            raise LokiError(st, "loki_kv_append")


class DensePlan:
    """A dense-baseline call marshalled once."""

    def __init__(self, q, cache: KVCache, P, S: int | None = None, out=None, workspace=None,
                 rope_base: float | None = None, q_pos: int | None = None):
        S, self.out, workspace, head, tail = _dense_args(q, cache, P, S, out, workspace)
        self._keep = (q, cache, P, workspace)
        if rope_base is None:
            self._fn = load().loki_dense_decode
            self._args = head + tail
        else:
            self._fn = load().loki_dense_decode_rope
            self._args = head + (S - 1 if q_pos is None else q_pos, float(rope_base)) + tail

    def __call__(self):
        st = self._fn(*self._args)
        if st != LOKI_OK:
            raise LokiError(st, "loki_dense_decode")
        return self.out


class StepPlan:
    """A decode-step call (append at `pos` + decode over pos + 1 tokens)
    marshalled once."""

    def __init__(self, q, k_new, v_new, cache: KVCache, P, k: int, pos: int, out=None, idx=None,
                 workspace=None, path: int = PATH_AUTO, rope_base: float | None = None):
        self.out, self.idx, workspace, head, tail = _step_args(q, k_new, v_new, cache, P, k, pos,
                                                               out, idx, workspace, path)
        self._keep = (q, k_new, v_new, cache, P, workspace)
        if rope_base is None:
            self._fn = load().loki_decode_step
            self._args = head + tail
        else:
            self._fn = load().loki_decode_step_rope
            self._args = head + (float(rope_base),) + tail

    def __call__(self):
        st = self._fn(*self._args)
        if st != LOKI_OK:
            raise LokiError(st, "loki_decode_step")
        return self.out, self.idx
