"""ctypes binding of libsinkattn.so (include/sinkattn.h): argument marshalling only.

Every function here checks tensor devices, dtypes, shapes and contiguity,
allocates outputs with torch when the caller passes none, and calls the C entry
point of the same name on torch's current stream.  All arithmetic runs in the
HIP kernels.  There is no fallback: if the shared library is missing the first
call raises ``SinkAttnUnavailable``.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SINKATTN_LIB", os.path.join(_HERE, "libsinkattn.so"))

F32, BF16 = 0, 1
RING, CONTIG = 0, 1
INTERLEAVED, HALF = 0, 1
DQK, DV = 192, 128

_ERRORS = {-1: "NULL_PTR", -2: "SHAPE", -3: "DTYPE", -4: "UNSUPPORTED", -5: "WORKSPACE",
           -6: "CAPACITY", -7: "ALIAS", -8: "HIP"}


class SinkAttnUnavailable(RuntimeError):
    pass


class SinkAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("sinkattn error %d (%s): %s" % (code, _ERRORS.get(code, "?"), msg))
        self.code = code


_lock = threading.Lock()
_lib = None


def _bind(lib):
    p, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    sig = {
        "sinkattn_abi_version": ([], i32),
        "sinkattn_status_string": ([i32], ctypes.c_char_p),
        "sinkattn_rope_partial": ([p, i32, i64, i32, i32, i32, p, f64, i32, p], i32),
        "sinkattn_prefill_swa": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, i32, p],
                                 i32),
        "sinkattn_prefill_global": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p],
                                    i32),
        "sinkattn_prefill_swa_rope": ([p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32,
                                       i32, f64, i32, p], i32),
        "sinkattn_decode_workspace_bytes": ([i32, i32, i32, i32, i32], sz),
        "sinkattn_decode": ([p, p, p, p, p, i32, i32, p, i32, p, p, i32, i32, i32, i32, i32, i32,
                             f32, i32, p, sz, i32, p], i32),
        "sinkattn_decode_noalloc": ([p, p, p, p, p, i32, i32, p, i32, p, p, i32, i32, i32, i32,
                                     i32, i32, f32, i32, i32, p], i32),
        "sinkattn_verify": ([p, p, p, p, p, i32, i32, p, i32, p, p, i32, i32, i32, i32, i32, i32,
                             i32, f32, i32, p, sz, i32, p], i32),
        "sinkattn_kv_append": ([p, p, p, p, i32, i32, p, p, i32, i32, i32, i32, i32, i32, p], i32),
        "sinkattn_advance_len": ([p, p, i32, i32, p], i32),
        "sinkattn_backward_workspace_bytes": ([i32, i32, i32], sz),
        "sinkattn_backward": ([p, p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                               f32, p, sz, i32, p], i32),
        "sinkattn_decode_fp8": ([p, p, p, p, p, i32, i32, p, i32, p, p, i32, i32, i32, i32, i32,
                                 i32, f32, f32, f32, i32, f64, i32, p, sz, p], i32),
        "sinkattn_verify_fp8": ([p, p, p, p, p, i32, i32, p, i32, p, p, p, i32, i32, i32, i32,
                                 i32, i32, i32, f32, f32, f32, i32, f64, i32, p, sz, p], i32),
        "sinkattn_kv_append_fp8": ([p, p, p, p, i32, i32, p, p, i32, i32, i32, i32, i32, f32, f32,
                                    p], i32),
        "sinkattn_prefill_global_rope": ([p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32,
                                          i32, f64, i32, p], i32),
        "sinkattn_decode_rope": ([p, p, p, p, p, i32, i32, p, i32, p, p, i32, i32, i32, i32, i32,
                                  i32, f32, i32, f64, i32, p, sz, i32, p], i32),
        "sinkattn_verify_rope": ([p, p, p, p, p, i32, i32, p, i32, p, p, p, i32, i32, i32, i32,
                                  i32, i32, i32, f32, i32, f64, i32, p, sz, i32, p], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def lib():
    """The loaded C library (raises SinkAttnUnavailable if it was not built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise SinkAttnUnavailable(
                        "libsinkattn.so not found at %s; build it with "
                        "`python -m sliding_window_sink_amd.build`" % LIB_PATH)
                _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


EXPORTED = ["sinkattn_abi_version", "sinkattn_status_string", "sinkattn_rope_partial",
            "sinkattn_prefill_swa", "sinkattn_prefill_swa_rope", "sinkattn_prefill_global", "sinkattn_decode_workspace_bytes",
            "sinkattn_decode", "sinkattn_verify", "sinkattn_kv_append",
            "sinkattn_prefill_global_rope", "sinkattn_decode_rope", "sinkattn_verify_rope",
            "sinkattn_advance_len", "sinkattn_decode_fp8", "sinkattn_verify_fp8",
            "sinkattn_kv_append_fp8", "sinkattn_backward_workspace_bytes", "sinkattn_backward",
            "sinkattn_decode_noalloc"]


def _check(rc: int):
    if rc != 0:
        raise SinkAttnError(rc, lib().sinkattn_status_string(rc).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise SinkAttnError(-3, "tensors must be bfloat16 or float32, got %s" % t.dtype)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise SinkAttnError(-1, "every tensor must live on the GPU")
        if not t.is_contiguous():
            raise SinkAttnError(-2, "every tensor must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _scale(scale):
    return 0.0 if scale is None else float(scale)


def abi_version() -> int:
    return int(lib().sinkattn_abi_version())


def rope_partial(x: torch.Tensor, pos: torch.Tensor, base: float, rope_dim: int = 64,
                 style: int = INTERLEAVED) -> torch.Tensor:
    """Partial RoPE in place on x [..., n_heads, head_dim]; pos int32 [n_tok]."""
    _dev(x, pos)
    if pos.dtype != torch.int32:
        raise SinkAttnError(-3, "pos must be int32")
    n_heads, head_dim = x.shape[-2], x.shape[-1]
    n_tok = x.numel() // max(1, n_heads * head_dim)
    if pos.numel() != n_tok:
        raise SinkAttnError(-2, "pos must hold one position per token")
    _check(lib().sinkattn_rope_partial(_ptr(x), _dtype_code(x), n_tok, n_heads, head_dim, rope_dim,
                                       _ptr(pos), float(base), int(style), _stream()))
    return x


def _lse_buffer(lse_out, B, Hq, T, device, return_lse):
    """The caller's lse tensor [B,Hq,T] fp32 (lse_out), a new one, or None."""
    if lse_out is not None:
        _dev(lse_out)
        if lse_out.shape != (B, Hq, T) or lse_out.dtype != torch.float32:
            raise SinkAttnError(-2, "lse_out must be float32 [B,Hq,T]")
        return lse_out
    return torch.empty((B, Hq, T), dtype=torch.float32, device=device) if return_lse else None


def _prefill(fn_name, q, k, v, sink, window, scale, out, return_lse, lse_out=None):
    _dev(q, k, v, sink, out)
    B, T, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    if k.shape != (B, T, Hkv, dqk) or v.shape[:3] != (B, T, Hkv) or sink.shape != (Hq,):
        raise SinkAttnError(-2, "q/k/v/sink shapes disagree")
    if sink.dtype != torch.float32 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise SinkAttnError(-3, "q, k, v share one dtype; sink is float32")
    o = out if out is not None else torch.empty((B, T, Hq, dv), dtype=q.dtype, device=q.device)
    if o.shape != (B, T, Hq, dv) or o.dtype != q.dtype:
        raise SinkAttnError(-2, "bad output tensor")
    lse = _lse_buffer(lse_out, B, Hq, T, q.device, return_lse)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), _ptr(lse), B, T, Hq, Hkv, dqk, dv]
    if fn_name == "sinkattn_prefill_swa":
        args.append(int(window))
    args += [_scale(scale), _dtype_code(q), _stream()]
    _check(getattr(lib(), fn_name)(*args))
    return (o, lse) if return_lse else o


def prefill_swa(q, k, v, sink, window: int = 128, scale=None, out=None, return_lse=False,
                lse_out=None):
    """Causal sliding-window prefill: q [B,T,Hq,192], k [B,T,Hkv,192], v [B,T,Hkv,128].
    lse_out: optional caller-owned fp32 [B,Hq,T] that receives lse (implies return_lse)."""
    return _prefill("sinkattn_prefill_swa", q, k, v, sink, window, scale, out,
                    return_lse or lse_out is not None, lse_out)


def prefill_swa_rope(q, k, v, sink, window: int = 128, base: float = 1e4, rope_dim: int = 64,
                     k_rot=None, scale=None, out=None, return_lse=False, lse_out=None):
    """SWA prefill with partial RoPE fused into the loads (q, k un-rotated and
    left untouched); k_rot, if given, receives the rotated k."""
    return_lse = return_lse or lse_out is not None
    _dev(q, k, v, sink, out, k_rot)
    B, T, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    if k.shape != (B, T, Hkv, dqk) or v.shape[:3] != (B, T, Hkv) or sink.shape != (Hq,):
        raise SinkAttnError(-2, "q/k/v/sink shapes disagree")
    if k_rot is not None and (k_rot.shape != k.shape or k_rot.dtype != k.dtype):
        raise SinkAttnError(-2, "k_rot must match k")
    o = out if out is not None else torch.empty((B, T, Hq, dv), dtype=q.dtype, device=q.device)
    lse = _lse_buffer(lse_out, B, Hq, T, q.device, return_lse)
    _check(lib().sinkattn_prefill_swa_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o), _ptr(lse),
                                           _ptr(k_rot), B, T, Hq, Hkv, dqk, dv, int(window),
                                           _scale(scale), int(rope_dim), float(base),
                                           _dtype_code(q), _stream()))
    return (o, lse) if return_lse else o


def prefill_global(q, k, v, sink, scale=None, out=None, return_lse=False, lse_out=None):
    """Causal full-context prefill (global-attention layer)."""
    return _prefill("sinkattn_prefill_global", q, k, v, sink, 0, scale, out,
                    return_lse or lse_out is not None, lse_out)


def prefill_global_rope(q, k, v, sink, base: float = 5e6, rope_dim: int = 64, k_rot=None,
                        scale=None, out=None, return_lse=False, lse_out=None):
    """Global prefill with partial RoPE fused (q, k un-rotated and left untouched).
    The rotated keys are written to k_rot (allocated here when not given), which
    is returned as the second element: (o, k_rot) or (o, lse, k_rot)."""
    _dev(q, k, v, sink, out, k_rot)
    B, T, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    if k.shape != (B, T, Hkv, dqk) or v.shape[:3] != (B, T, Hkv) or sink.shape != (Hq,):
        raise SinkAttnError(-2, "q/k/v/sink shapes disagree")
    if k_rot is None:
        k_rot = torch.empty_like(k)
    if k_rot.shape != k.shape or k_rot.dtype != k.dtype:
        raise SinkAttnError(-2, "k_rot must match k")
    o = out if out is not None else torch.empty((B, T, Hq, dv), dtype=q.dtype, device=q.device)
    return_lse = return_lse or lse_out is not None
    lse = _lse_buffer(lse_out, B, Hq, T, q.device, return_lse)
    _check(lib().sinkattn_prefill_global_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(o),
                                              _ptr(lse), _ptr(k_rot), B, T, Hq, Hkv, dqk, dv,
                                              _scale(scale), int(rope_dim), float(base),
                                              _dtype_code(q), _stream()))
    return (o, lse, k_rot) if return_lse else (o, k_rot)


def decode_workspace_bytes(B: int, Hq: int, n_q: int = 1, max_splits: int = 64, dv: int = DV) -> int:
    return int(lib().sinkattn_decode_workspace_bytes(B, Hq, dv, n_q, max_splits))


def _cached(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window, max_len_hint,
            num_splits, workspace, scale, out, verify, rope=None, k_rot=None):
    _dev(q, k_new, v_new, k_cache, v_cache, cache_len, sink, workspace, out, k_rot)
    if cache_len.dtype != torch.int32:
        raise SinkAttnError(-3, "cache_len must be int32")
    if verify:
        B, nq, Hq, dqk = q.shape
    else:
        B, Hq, dqk = q.shape
        nq = 1
    Bc, Hkv, cap, dk = k_cache.shape
    dv = v_cache.shape[3]
    if Bc != B or dk != dqk or v_cache.shape[:3] != (B, Hkv, cap) or sink.shape != (Hq,):
        raise SinkAttnError(-2, "cache / query shapes disagree")
    want_new = (B, nq, Hkv) if verify else (B, Hkv)
    if tuple(k_new.shape[:-1]) != want_new or tuple(v_new.shape[:-1]) != want_new:
        raise SinkAttnError(-2, "k_new/v_new shapes disagree")
    oshape = (B, nq, Hq, dv) if verify else (B, Hq, dv)
    o = out if out is not None else torch.empty(oshape, dtype=q.dtype, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    if k_rot is not None and (k_rot.shape != k_new.shape or k_rot.dtype != k_new.dtype):
        raise SinkAttnError(-2, "k_rot must match k_new")
    args = [_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), int(kind), cap,
            _ptr(cache_len), int(max_len_hint), _ptr(sink), _ptr(o)]
    if verify and rope is not None:
        args.append(_ptr(k_rot))
    args.append(B)
    if verify:
        args.append(nq)
    args += [Hq, Hkv, dqk, dv, int(window), _scale(scale)]
    if rope is not None:
        args += [int(rope[1]), float(rope[0])]
    args += [int(num_splits), ws_ptr, ws_bytes, _dtype_code(q), _stream()]
    if rope is None:
        fn = lib().sinkattn_verify if verify else lib().sinkattn_decode
    else:
        fn = lib().sinkattn_verify_rope if verify else lib().sinkattn_decode_rope
    _check(fn(*args))
    return o


def decode(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
           max_len_hint=None, num_splits=0, workspace=None, scale=None, out=None):
    """One decode step; also stores k_new/v_new into the cache at cache_len."""
    if max_len_hint is None:
        raise SinkAttnError(-2, "max_len_hint (host bound on cache_len) is required")
    return _cached(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window, max_len_hint,
                   num_splits, workspace, scale, out, verify=False)


def decode_noalloc(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
                   max_len_hint=None, num_splits=0, scale=None, out=None):
    """decode() whose split-K scratch is the library's fixed device array: the C
    call allocates nothing (pass `out` to keep the whole call allocation-free)."""
    if max_len_hint is None:
        raise SinkAttnError(-2, "max_len_hint (host bound on cache_len) is required")
    _dev(q, k_new, v_new, k_cache, v_cache, cache_len, sink, out)
    if cache_len.dtype != torch.int32:
        raise SinkAttnError(-3, "cache_len must be int32")
    B, Hq, dqk = q.shape
    Bc, Hkv, cap, dk = k_cache.shape
    dv = v_cache.shape[3]
    if Bc != B or dk != dqk or v_cache.shape[:3] != (B, Hkv, cap) or sink.shape != (Hq,):
        raise SinkAttnError(-2, "cache / query shapes disagree")
    if tuple(k_new.shape[:-1]) != (B, Hkv) or tuple(v_new.shape[:-1]) != (B, Hkv):
        raise SinkAttnError(-2, "k_new/v_new shapes disagree")
    o = out if out is not None else torch.empty((B, Hq, dv), dtype=q.dtype, device=q.device)
    _check(lib().sinkattn_decode_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                         _ptr(v_cache), int(kind), cap, _ptr(cache_len),
                                         int(max_len_hint), _ptr(sink), _ptr(o), B, Hq, Hkv,
                                         dqk, dv, int(window), _scale(scale), int(num_splits),
                                         _dtype_code(q), _stream()))
    return o


STATIC_SCRATCH_BYTES = 32 << 20  # SINKATTN_STATIC_SCRATCH_BYTES of include/sinkattn.h


def verify(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
           max_len_hint=None, num_splits=0, workspace=None, scale=None, out=None):
    """Multi-query verification; the caches are read-only."""
    if max_len_hint is None:
        raise SinkAttnError(-2, "max_len_hint (host bound on cache_len) is required")
    return _cached(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window, max_len_hint,
                   num_splits, workspace, scale, out, verify=True)


def decode_rope(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
                max_len_hint=None, base: float = 1e4, rope_dim: int = 64, num_splits=0,
                workspace=None, scale=None, out=None):
    """decode() with partial RoPE fused: q and k_new are un-rotated; the token is
    rotated at position cache_len[b] and its rotated k is stored in the cache."""
    if max_len_hint is None:
        raise SinkAttnError(-2, "max_len_hint (host bound on cache_len) is required")
    return _cached(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window, max_len_hint,
                   num_splits, workspace, scale, out, verify=False, rope=(base, rope_dim))


def verify_rope(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
                max_len_hint=None, base: float = 1e4, rope_dim: int = 64, k_rot=None,
                num_splits=0, workspace=None, scale=None, out=None):
    """verify() with partial RoPE fused: token t rotated at cache_len[b] + t; if
    k_rot is given it receives the rotated k_new (for a later kv_append)."""
    if max_len_hint is None:
        raise SinkAttnError(-2, "max_len_hint (host bound on cache_len) is required")
    return _cached(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window, max_len_hint,
                   num_splits, workspace, scale, out, verify=True, rope=(base, rope_dim),
                   k_rot=k_rot)


def kv_append(k_new, v_new, k_cache, v_cache, cache_len, kind=RING, n_accept=None):
    """Store tokens k_new/v_new [B,n,Hkv,d] at positions cache_len[b] + t."""
    _dev(k_new, v_new, k_cache, v_cache, cache_len, n_accept)
    B, n, Hkv, dqk = k_new.shape
    cap = k_cache.shape[2]
    dv = v_new.shape[3]
    if k_cache.dtype != k_new.dtype or v_cache.dtype != k_new.dtype or v_new.dtype != k_new.dtype:
        raise SinkAttnError(-3, "caches and new tokens share one dtype")
    _check(lib().sinkattn_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                    int(kind), cap, _ptr(cache_len), _ptr(n_accept), B, n, Hkv,
                                    dqk, dv, _dtype_code(k_new), _stream()))


def _cached_fp8(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window, max_len_hint,
                k_scale, v_scale, rope, num_splits, workspace, scale, out, verify, k_rot=None):
    _dev(q, k_new, v_new, k_cache, v_cache, cache_len, sink, workspace, out, k_rot)
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise SinkAttnError(-3, "E4M3 caches are uint8 tensors")
    if q.dtype != torch.bfloat16 or k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise SinkAttnError(-3, "q, k_new, v_new are bfloat16")
    if cache_len.dtype != torch.int32:
        raise SinkAttnError(-3, "cache_len must be int32")
    if max_len_hint is None:
        raise SinkAttnError(-2, "max_len_hint (host bound on cache_len) is required")
    if verify:
        B, nq, Hq, dqk = q.shape
    else:
        B, Hq, dqk = q.shape
        nq = 1
    Bc, Hkv, cap, dk = k_cache.shape
    dv = v_cache.shape[3]
    if Bc != B or dk != dqk or v_cache.shape[:3] != (B, Hkv, cap) or sink.shape != (Hq,):
        raise SinkAttnError(-2, "cache / query shapes disagree")
    want_new = (B, nq, Hkv) if verify else (B, Hkv)
    if tuple(k_new.shape[:-1]) != want_new or tuple(v_new.shape[:-1]) != want_new:
        raise SinkAttnError(-2, "k_new/v_new shapes disagree")
    if k_rot is not None and (k_rot.shape != k_new.shape or k_rot.dtype != k_new.dtype):
        raise SinkAttnError(-2, "k_rot must match k_new")
    oshape = (B, nq, Hq, dv) if verify else (B, Hq, dv)
    o = out if out is not None else torch.empty(oshape, dtype=q.dtype, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    rope_dim, base = (0, 0.0) if rope is None else (int(rope[1]), float(rope[0]))
    args = [_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), int(kind), cap,
            _ptr(cache_len), int(max_len_hint), _ptr(sink), _ptr(o)]
    if verify:
        args += [_ptr(k_rot), B, nq]
    else:
        args.append(B)
    args += [Hq, Hkv, dqk, dv, int(window), _scale(scale), float(k_scale), float(v_scale),
             rope_dim, base, int(num_splits), ws_ptr, ws_bytes, _stream()]
    fn = lib().sinkattn_verify_fp8 if verify else lib().sinkattn_decode_fp8
    _check(fn(*args))
    return o


def decode_fp8(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
               max_len_hint=None, k_scale=1.0, v_scale=1.0, rope=None, num_splits=0,
               workspace=None, scale=None, out=None):
    """decode() over E4M3 (uint8) caches with per-tensor scales; rope=(base, 64)
    fuses the partial RoPE, rope=None takes q / k_new as already rotated."""
    return _cached_fp8(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window,
                       max_len_hint, k_scale, v_scale, rope, num_splits, workspace, scale, out,
                       verify=False)


def verify_fp8(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind=RING, window=128,
               max_len_hint=None, k_scale=1.0, v_scale=1.0, rope=None, k_rot=None,
               num_splits=0, workspace=None, scale=None, out=None):
    """verify() over E4M3 (uint8) caches; the caches are read-only."""
    return _cached_fp8(q, k_new, v_new, k_cache, v_cache, cache_len, sink, kind, window,
                       max_len_hint, k_scale, v_scale, rope, num_splits, workspace, scale, out,
                       verify=True, k_rot=k_rot)


def kv_append_fp8(k_new, v_new, k_cache, v_cache, cache_len, kind=RING, n_accept=None,
                  k_scale=1.0, v_scale=1.0):
    """kv_append() into E4M3 (uint8) caches: bf16 rows quantized with the scales."""
    _dev(k_new, v_new, k_cache, v_cache, cache_len, n_accept)
    B, n, Hkv, dqk = k_new.shape
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise SinkAttnError(-3, "E4M3 caches are uint8 tensors")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise SinkAttnError(-3, "k_new, v_new are bfloat16")
    _check(lib().sinkattn_kv_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                        int(kind), k_cache.shape[2], _ptr(cache_len),
                                        _ptr(n_accept), B, n, Hkv, dqk, v_new.shape[3],
                                        float(k_scale), float(v_scale), _stream()))


def backward(q, k, v, o, dout, lse, sink, window: int = 0, scale=None, workspace=None,
             out=None):
    """Gradients (dq, dk, dv, dsink), fp32, of the causal prefill that produced o
    and lse (window >= 1: SWA, 0: global) for the upstream gradient dout."""
    _dev(q, k, v, o, dout, lse, sink, workspace)
    B, T, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    for t in (q, k, v, o, dout):
        if t.dtype != torch.bfloat16:
            raise SinkAttnError(-3, "q, k, v, o, dout are bfloat16")
    if o.shape != (B, T, Hq, dv) or dout.shape != o.shape or lse.shape != (B, Hq, T):
        raise SinkAttnError(-2, "o / dout / lse shapes disagree")
    need = int(lib().sinkattn_backward_workspace_bytes(B, T, Hq))
    if workspace is None:
        workspace = torch.empty(max(1, need // 4), dtype=torch.float32, device=q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    # dsink of an empty batch is a sum over no tokens: the library writes nothing
    # then, so a fresh dsink starts at zero in that case
    dq, dk, dvv, dsink = out if out is not None else (
        torch.empty(B, T, Hq, dqk, **f32), torch.empty(B, T, Hkv, dqk, **f32),
        torch.empty(B, T, Hkv, dv, **f32),
        torch.zeros(Hq, **f32) if B * T == 0 else torch.empty(Hq, **f32))
    _check(lib().sinkattn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                   _ptr(sink), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(dsink), B, T,
                                   Hq, Hkv, dqk, dv, int(window), _scale(scale), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _dtype_code(q), _stream()))
    return dq, dk, dvv, dsink


def advance_len(cache_len, n, n_accept=None):
    """cache_len[b] += min(n_accept[b], n) (n when n_accept is None), on the device."""
    _dev(cache_len, n_accept)
    if cache_len.dtype != torch.int32 or (n_accept is not None and n_accept.dtype != torch.int32):
        raise SinkAttnError(-3, "cache_len and n_accept are int32")
    _check(lib().sinkattn_advance_len(_ptr(cache_len), _ptr(n_accept), cache_len.numel(), int(n),
                                      _stream()))
    return cache_len


def default_scale(dqk: int = DQK) -> float:
    return 1.0 / math.sqrt(dqk)
