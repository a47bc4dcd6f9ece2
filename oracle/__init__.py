"""Plain fp64 CPU oracle for sink attention and partial RoPE.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``sliding_window_sink_amd`` and never imports it; the two
meet only at the seeded input generators, which hold none of the method's
arithmetic.

The arithmetic lives in ``sinkattn_oracle.c`` (plain C loops in double
precision, built with gcc).  This module compiles it on demand and marshals
numpy arrays through ctypes; on top it offers the per-entry-point views
(prefill, ring/contiguous decode, verify) that say which keys each query sees,
written from the definitions of the MiMo-V2-Flash Technical Report, Section 2.2
(sink softmax) and Section 2.1 / Table 1 (GQA, dims, partial RoPE).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sinkattn_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (OpenMP over query rows, no fast-math)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    d, i64, i32 = ctypes.c_double, ctypes.c_int64, ctypes.c_int
    p = ctypes.c_void_p
    lib.oracle_sink_attention.argtypes = [p, p, p, p, p, p, i64, i64, i32, i32, i32,
                                          i32, i64, d, p, p]
    lib.oracle_sink_attention.restype = i32
    lib.oracle_rope_partial.argtypes = [p, p, i64, i32, i32, i32, p, d, i32]
    lib.oracle_rope_partial.restype = i32
    lib.oracle_round_bf16.argtypes = [p, p, i64]
    lib.oracle_round_bf16.restype = None
    lib.oracle_sink_attention_bwd.argtypes = [p, p, p, p, p, p, p, i64, i64, i32, i32, i32,
                                              i32, i64, d, p, p, p, p]
    lib.oracle_sink_attention_bwd.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    return lib


def load_library(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            _lib = _bind(ctypes.CDLL(build()))
    return _lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor -> exact float64 copy
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads(lib=None) -> int:
    return int((lib or load_library()).oracle_num_threads())


def sink_attention(q, k, v, qpos, kpos, sink, window: int = 0, scale: float | None = None,
                   lib=None):
    """One sequence of sink attention (Section 2.2, all four equations).

    q [nq, hq, dqk], k [nk, hkv, dqk], v [nk, hkv, dv]; qpos [nq], kpos [nk]
    (negative kpos = empty slot); sink [hq]; window > 0 = sliding window of W
    keys including self, window <= 0 = global causal.  Returns (o [nq,hq,dv],
    lse [nq,hq]) in float64.
    """
    lib = lib or load_library()
    q, k, v, sink = _f64(q), _f64(k), _f64(v), _f64(sink)
    qpos, kpos = _i64(qpos), _i64(kpos)
    nq, hq, dqk = q.shape
    nk, hkv, dk = k.shape
    dv = v.shape[2]
    if dk != dqk or v.shape[:2] != (nk, hkv) or qpos.shape != (nq,) or kpos.shape != (nk,) \
            or sink.shape != (hq,):
        raise ValueError("oracle: inconsistent shapes")
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    o = np.zeros((nq, hq, dv), np.float64)
    lse = np.zeros((nq, hq), np.float64)
    rc = lib.oracle_sink_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(qpos), _ptr(kpos),
                                   _ptr(sink), nq, nk, hq, hkv, dqk, dv, int(window),
                                   float(scale), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_sink_attention failed (%d)" % rc)
    return o, lse


def sink_attention_bwd(q, k, v, qpos, kpos, sink, dout, window: int = 0,
                       scale: float | None = None, lib=None):
    """Gradients (dq, dk, dv, dsink) of sink_attention for the upstream gradient
    dout of o; same layouts as sink_attention (Section 2.2, chain rule)."""
    lib = lib or load_library()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    qpos, kpos, sink = _i64(qpos), _i64(kpos), _f64(sink)
    nq, hq, dqk = q.shape
    nk, hkv, dv = v.shape
    scale = 1.0 / np.sqrt(dqk) if scale is None else float(scale)
    dq, dk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dsink = np.empty(hq)
    rc = lib.oracle_sink_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(qpos), _ptr(kpos),
                                       _ptr(sink), _ptr(dout), nq, nk, hq, hkv, dqk, dv,
                                       int(window), scale, _ptr(dq), _ptr(dk), _ptr(dvv),
                                       _ptr(dsink))
    if rc != 0:
        raise ValueError("oracle_sink_attention_bwd failed (%d)" % rc)
    return dq, dk, dvv, dsink


def rope_partial(x, pos, base: float, rope_dim: int = 64, style: int = 0, lib=None):
    """Partial RoPE in fp64 on x [n_tok, n_heads, head_dim] (Section 2.1; RoFormer)."""
    lib = lib or load_library()
    x = _f64(x)
    pos = _i64(pos)
    n_tok, n_heads, head_dim = x.shape
    y = np.empty_like(x)
    rc = lib.oracle_rope_partial(_ptr(x), _ptr(y), n_tok, n_heads, head_dim, rope_dim,
                                 _ptr(pos), float(base), int(style))
    if rc != 0:
        raise ValueError("oracle_rope_partial failed (%d)" % rc)
    return y


def round_bf16_bits(x, lib=None) -> np.ndarray:
    """Round float64 values once (RNE) to bfloat16; returns uint16 bit patterns."""
    lib = lib or load_library()
    x = _f64(x)
    out = np.empty(x.shape, np.uint16)
    lib.oracle_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Entry-point views: which keys each query sees.  These only choose positions;
# the arithmetic is sink_attention above.
# ---------------------------------------------------------------------------

def prefill(q, k, v, sink, window: int = 0, scale=None, rows=None, lib=None):
    """Causal prefill of B sequences at positions 0..T-1.

    q [B,T,Hq,dqk], k [B,T,Hkv,dqk], v [B,T,Hkv,dv].  window > 0 = SWA.
    rows: optional index array of query tokens to evaluate (all if None); the
    result then holds only those rows.  Returns (o [B,R,Hq,dv], lse [B,R,Hq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T = q.shape[:2]
    rows = np.arange(T) if rows is None else _i64(rows)
    outs, lses = [], []
    for b in range(B):
        if window > 0 and len(rows) > 0:
            # only keys that some requested row can see are passed in
            lo = max(0, int(rows.min()) - window + 1)
        else:
            lo = 0
        hi = int(rows.max()) + 1 if len(rows) else 0
        kk, vv = k[b, lo:hi], v[b, lo:hi]
        o, lse = sink_attention(q[b, rows], kk, vv, rows, np.arange(lo, hi), sink,
                                window, scale, lib=lib)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def decode_or_verify(q, k_hist, v_hist, k_new, v_new, cache_len, sink, window: int = 0,
                     scale=None, lib=None):
    """Queries at positions L_b .. L_b+n-1 over the cached history plus new keys.

    q [B,n,Hq,dqk]; k_hist/v_hist: per-sequence arrays [L_b, Hkv, d] holding the
    keys at positions 0..L_b-1 (a list, one per sequence; with a window only the
    last W-1 rows matter); k_new/v_new [B,n,Hkv,d] at positions L_b..L_b+n-1.
    Query t sees history positions in its window and new tokens 0..t.
    Returns (o [B,n,Hq,dv], lse [B,n,Hq]).
    """
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    B, n = q.shape[:2]
    outs, lses = [], []
    for b in range(B):
        L = int(cache_len[b])
        kh, vh = _f64(k_hist[b]), _f64(v_hist[b])
        start = L - kh.shape[0]  # k_hist[b] may hold only the tail of the history
        kk = np.concatenate([kh, k_new[b]], 0)
        vv = np.concatenate([vh, v_new[b]], 0)
        kpos = np.arange(start, L + n)
        o, lse = sink_attention(q[b], kk, vv, np.arange(L, L + n), kpos, sink, window,
                                scale, lib=lib)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------------------
# FP8 KV cache.  The report runs inference in FP8 but does not give the format
# or the scaling of the attention cache.  Reading taken here: the OCP 8-bit
# floating point E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa
# bits; no infinities; S.1111.111 is NaN; largest finite value 448), one scale
# per tensor (cache value = code value * scale), and a quantizer that divides in
# IEEE fp32 and rounds that quotient once to the nearest E4M3 value, ties to the
# even code, saturating beyond +-448.
# ---------------------------------------------------------------------------

def fp8_e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code, from the format's definition (fp64, exact)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the finite non-negative values, codes 0x00 .. 0x7E in increasing order
_E4M3_TABLE = fp8_e4m3_decode(np.arange(0x7F))


def fp8_e4m3_encode(x) -> np.ndarray:
    """Nearest finite E4M3 code to each value (a search over the value table):
    ties go to the even code, magnitudes beyond 448 saturate to +-448, the sign
    of zero is kept.  NaN inputs are rejected."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("fp8_e4m3_encode: NaN input")
    a = np.abs(x).ravel()
    hi = np.clip(np.searchsorted(_E4M3_TABLE, a, side="left"), 0, len(_E4M3_TABLE) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_hi = np.abs(_E4M3_TABLE[hi] - a)
    d_lo = np.abs(a - _E4M3_TABLE[lo])
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= _E4M3_TABLE[-1], len(_E4M3_TABLE) - 1, pick)
    codes = pick.astype(np.uint8) | np.where(np.signbit(x.ravel()), 0x80, 0).astype(np.uint8)
    return codes.reshape(x.shape)


def fp8_quantize(x, scale: float) -> np.ndarray:
    """Cache codes of values x (each exactly representable in fp32, e.g. bf16)
    under a per-tensor scale: E4M3(fl32(x / scale))."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return fp8_e4m3_encode(q.astype(np.float64))


def fp8_dequantize(codes, scale: float) -> np.ndarray:
    """Cache values: code value * scale (fp64; exact for an fp32 scale)."""
    if hasattr(codes, "detach"):
        codes = codes.detach().cpu().numpy()
    return fp8_e4m3_decode(np.asarray(codes).view(np.uint8)) * float(np.float32(scale))
