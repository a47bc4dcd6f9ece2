"""The C-ABI library loads on the CPU, exports what include/sinkattn.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from sliding_window_sink_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, CAP, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7
P = ctypes.c_void_p
FAKE = [P((i + 1) << 36) for i in range(12)]  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.fail("libsinkattn.so is not built (python -m sliding_window_sink_amd.build)")
    return ops.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sinkattn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ops.EXPORTED) == names


def test_version_and_status_strings(lib):
    assert lib.sinkattn_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = lib.sinkattn_status_string(code)
        assert s and s != b"unknown status"
    assert lib.sinkattn_status_string(12345) == b"unknown status"


def test_workspace_bytes(lib):
    assert lib.sinkattn_decode_workspace_bytes(32, 64, 128, 1, 65) == 32 * 64 * 65 * 130 * 4
    assert lib.sinkattn_decode_workspace_bytes(4, 8, 128, 4, 1) == 0


def prefill(lib, *, q=FAKE[0], k=FAKE[1], v=FAKE[2], sink=FAKE[3], o=FAKE[4], lse=None, B=1,
            T=64, Hq=16, Hkv=2, dqk=192, dv=128, window=128, dtype=1, swa=True):
    if swa:
        return lib.sinkattn_prefill_swa(q, k, v, sink, o, lse, B, T, Hq, Hkv, dqk, dv, window,
                                        0.0, dtype, None)
    return lib.sinkattn_prefill_global(q, k, v, sink, o, lse, B, T, Hq, Hkv, dqk, dv, 0.0, dtype,
                                       None)


def test_prefill_validation(lib):
    assert prefill(lib, q=None) == NULL
    assert prefill(lib, sink=None) == NULL
    assert prefill(lib, dtype=7) == DTYPE
    assert prefill(lib, Hq=15) == SHAPE          # Hq % Hkv
    assert prefill(lib, Hkv=0) == SHAPE
    assert prefill(lib, dqk=128) == UNSUP
    assert prefill(lib, dv=192) == UNSUP
    assert prefill(lib, Hq=8, Hkv=2) == UNSUP    # bf16 needs groups of 8 heads
    assert prefill(lib, window=0) == SHAPE
    assert prefill(lib, T=-1) == SHAPE
    assert prefill(lib, B=0) == OK               # nothing to do, no HIP call
    assert prefill(lib, T=0, swa=False) == OK
    assert prefill(lib, B=0, q=None, o=None) == OK   # empty: pointers may be NULL
    # one sequence's q must fit 32-bit byte offsets except in the bf16 SWA kernel
    assert prefill(lib, T=87382, Hq=64, Hkv=8, swa=False) == SHAPE   # 2^31 + 2 bytes of bf16 q
    assert prefill(lib, T=43691, Hq=64, Hkv=8, dtype=0) == SHAPE     # fp32 SWA
    assert prefill(lib, T=87382, Hq=64, Hkv=8, window=200) == SHAPE  # window > 129: global kernel
    # o overlapping q
    assert prefill(lib, o=P(FAKE[0].value + 64)) == ALIAS
    assert prefill(lib, lse=P(FAKE[4].value + 8)) == ALIAS


def decode(lib, *, kind=0, cap=128, max_len=1000, B=2, Hq=16, Hkv=2, window=128, splits=0,
           ws=None, ws_bytes=0, dtype=1, o=FAKE[9], q=FAKE[0], cache_len=FAKE[5], k_cache=FAKE[3]):
    return lib.sinkattn_decode(q, FAKE[1], FAKE[2], k_cache, P(13 << 36), kind, cap,
                               cache_len, max_len, FAKE[6], o, B, Hq, Hkv, 192, 128, window, 0.0,
                               splits, ws, ws_bytes, dtype, None)


def test_decode_validation(lib):
    assert decode(lib, q=None) == NULL
    assert decode(lib, cache_len=None) == NULL
    assert decode(lib, kind=5) == UNSUP
    assert decode(lib, kind=0, cap=64) == CAP         # ring smaller than the window
    assert decode(lib, kind=0, window=0) == SHAPE
    assert decode(lib, kind=1, cap=1000, max_len=1000) == CAP  # decode writes index max_len
    assert decode(lib, kind=1, cap=4096, max_len=1000, splits=4) == WS
    assert decode(lib, kind=1, cap=4096, max_len=1000, splits=4, ws=FAKE[10],
                  ws_bytes=lib.sinkattn_decode_workspace_bytes(2, 16, 128, 1, 4) - 4) == WS
    assert decode(lib, max_len=-1) == SHAPE
    assert decode(lib, dtype=2) == DTYPE
    assert decode(lib, B=0) == OK
    assert decode(lib, kind=1, cap=5592406) == SHAPE   # cache rows past 32-bit offsets
    assert decode(lib, B=0, q=None, cache_len=None, o=None) == OK   # empty: NULL allowed
    assert decode(lib, o=P(FAKE[0].value + 2)) == ALIAS


def test_decode_noalloc_validation(lib):
    """The no-allocation decode validates like sinkattn_decode, and rejects an
    explicit split count whose scratch exceeds the fixed array (only cases that
    fail before any HIP call are run here)."""
    def dn(*, kind=1, cap=200000, max_len=131072, B=64, Hq=64, Hkv=4, window=0, splits=0,
           dtype=1, q=FAKE[0], cache_len=FAKE[5], o=FAKE[9]):
        return lib.sinkattn_decode_noalloc(q, FAKE[1], FAKE[2], FAKE[3], P(13 << 36), kind, cap,
                                           cache_len, max_len, FAKE[6], o, B, Hq, Hkv, 192, 128,
                                           window, 0.0, splits, dtype, None)
    per_split = lib.sinkattn_decode_workspace_bytes(64, 64, 128, 1, 2) // 2
    too_many = (32 << 20) // per_split + 1
    assert dn(splits=too_many) == WS
    assert dn(q=None) == NULL
    assert dn(cache_len=None) == NULL
    assert dn(kind=7) == UNSUP
    assert dn(kind=0, cap=64, window=128) == CAP
    assert dn(max_len=200000) == CAP
    assert dn(dtype=3) == DTYPE
    assert dn(Hq=62) == SHAPE
    assert dn(B=0) == OK
    assert dn(o=P(FAKE[0].value + 2)) == ALIAS


def test_verify_validation(lib):
    def verify(nq=4, Hq=64, Hkv=4, kind=1, cap=20000, max_len=16384):
        return lib.sinkattn_verify(FAKE[0], FAKE[1], FAKE[2], FAKE[3], P(13 << 36), kind, cap,
                                   FAKE[5], max_len, FAKE[6], FAKE[9], 2, nq, Hq, Hkv, 192, 128, 0,
                                   0.0, 1, None, 0, 1, None)
    assert verify(nq=0) == SHAPE
    assert verify(nq=9) == SHAPE
    assert verify(nq=5) == UNSUP                  # 5 * 16 columns > 64 on the bf16 path
    assert verify(max_len=20001) == CAP
    assert verify(kind=0, cap=100) == SHAPE       # ring needs a window >= 1 (window=0 here)


def test_prefill_swa_rope_validation(lib):
    f = lib.sinkattn_prefill_swa_rope
    def call(window=128, rope_dim=64, dtype=1, base=1e4, k_rot=None, Hq=16):
        return f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], None, k_rot, 1, 64, Hq, 2, 192, 128,
                 window, 0.0, rope_dim, base, dtype, None)
    assert call(window=130) == UNSUP
    assert call(rope_dim=32) == UNSUP
    assert call(dtype=0) == UNSUP
    assert call(rope_dim=63) == SHAPE
    assert call(base=0.0) == SHAPE
    assert call(window=0) == SHAPE
    assert call(k_rot=P(FAKE[1].value + 128)) == ALIAS   # k_rot over k
    assert call(Hq=15) == SHAPE           # Hq % Hkv != 0


def test_prefill_global_rope_validation(lib):
    f = lib.sinkattn_prefill_global_rope
    def call(rope_dim=64, dtype=1, base=5e6, k_rot=FAKE[7], Hq=16, B=1, T=64, o=FAKE[4]):
        return f(FAKE[0], FAKE[1], FAKE[2], FAKE[3], o, None, k_rot, B, T, Hq, 2, 192, 128, 0.0,
                 rope_dim, base, dtype, None)
    assert call(k_rot=None) == NULL                 # the attention reads k_rot back
    assert call(rope_dim=32) == UNSUP
    assert call(dtype=0) == UNSUP
    assert call(rope_dim=63) == SHAPE
    assert call(base=float("inf")) == SHAPE
    assert call(Hq=15) == SHAPE
    assert call(k_rot=P(FAKE[1].value + 64)) == ALIAS   # k_rot over k
    assert call(k_rot=P(FAKE[4].value + 64)) == ALIAS   # k_rot over o
    assert call(T=87382, Hq=64) == SHAPE               # q past 32-bit offsets
    assert call(B=0) == OK


def test_decode_verify_rope_validation(lib):
    def dec(rope_dim=64, base=1e4, dtype=1, B=2):
        return lib.sinkattn_decode_rope(FAKE[0], FAKE[1], FAKE[2], FAKE[3], P(13 << 36), 0, 128,
                                        FAKE[5], 1000, FAKE[6], FAKE[9], B, 16, 2, 192, 128, 128,
                                        0.0, rope_dim, base, 0, None, 0, dtype, None)
    assert dec(rope_dim=32) == UNSUP
    assert dec(dtype=0) == UNSUP
    assert dec(rope_dim=7) == SHAPE
    assert dec(base=-1.0) == SHAPE
    assert dec(B=0) == OK

    def ver(k_rot=None, rope_dim=64, nq=4):
        return lib.sinkattn_verify_rope(FAKE[0], FAKE[1], FAKE[2], FAKE[3], P(13 << 36), 0, 128,
                                        FAKE[5], 1000, FAKE[6], FAKE[9], k_rot, 2, nq, 16, 2, 192,
                                        128, 128, 0.0, rope_dim, 1e4, 0, None, 0, 1, None)
    assert ver(rope_dim=128) == UNSUP
    assert ver(nq=9) == SHAPE
    assert ver(k_rot=P(FAKE[1].value + 32)) == ALIAS   # k_rot over k_new
    assert ver(k_rot=P(FAKE[9].value + 32)) == ALIAS   # k_rot over o


def test_advance_len_validation(lib):
    f = lib.sinkattn_advance_len
    assert f(None, None, 4, 4, None) == NULL
    assert f(FAKE[0], None, -1, 4, None) == SHAPE
    assert f(FAKE[0], FAKE[1], 4, -1, None) == SHAPE
    assert f(FAKE[0], P(FAKE[0].value + 4), 4, 4, None) == ALIAS
    assert f(FAKE[0], FAKE[1], 0, 4, None) == OK   # nothing to do, no HIP call


def test_fp8_validation(lib):
    def dec(k_scale=0.5, v_scale=0.5, rope_dim=0, B=2, Hq=16):
        return lib.sinkattn_decode_fp8(FAKE[0], FAKE[1], FAKE[2], FAKE[3], P(13 << 36), 0, 128,
                                       FAKE[5], 1000, FAKE[6], FAKE[9], B, Hq, 2, 192, 128, 128,
                                       0.0, k_scale, v_scale, rope_dim, 1e4, 0, None, 0, None)
    assert dec(k_scale=0.0) == SHAPE
    assert dec(v_scale=float("nan")) == SHAPE
    assert dec(rope_dim=32) == UNSUP
    assert dec(Hq=15) == SHAPE
    assert dec(B=0) == OK

    def ver(k_rot=None, rope_dim=64):
        return lib.sinkattn_verify_fp8(FAKE[0], FAKE[1], FAKE[2], FAKE[3], P(13 << 36), 0, 128,
                                       FAKE[5], 1000, FAKE[6], FAKE[9], k_rot, 2, 4, 16, 2, 192,
                                       128, 128, 0.0, 1.0, 1.0, rope_dim, 1e4, 0, None, 0, None)
    assert ver(k_rot=FAKE[7], rope_dim=0) == SHAPE     # rotated keys need the fused RoPE
    assert ver(k_rot=P(FAKE[1].value + 32)) == ALIAS
    a = lib.sinkattn_kv_append_fp8
    assert a(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 0, 128, None, None, 2, 4, 8, 192, 128, 1.0, 1.0,
             None) == NULL
    assert a(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 0, 128, FAKE[4], None, 2, 4, 8, 192, 128, -1.0,
             1.0, None) == SHAPE
    assert a(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 0, 128, FAKE[4], None, 0, 4, 8, 192, 128, 1.0,
             1.0, None) == OK


def test_backward_validation(lib):
    ws_need = lib.sinkattn_backward_workspace_bytes(1, 64, 16)
    assert ws_need == 2 * 64 * 16 * 4
    def bwd(dtype=1, window=128, ws=FAKE[11], ws_bytes=ws_need, dq=FAKE[7], T=64, Hq=16,
            lse=FAKE[5]):
        return lib.sinkattn_backward(FAKE[0], FAKE[1], FAKE[2], FAKE[3], FAKE[4], lse, FAKE[6],
                                     dq, FAKE[8], FAKE[9], FAKE[10], 1, T, Hq, 2, 192, 128,
                                     window, 0.0, ws, ws_bytes, dtype, None)
    assert bwd(dtype=0) == UNSUP
    assert bwd(lse=None) == NULL
    assert bwd(window=-1) == SHAPE
    assert bwd(Hq=15) == SHAPE
    assert bwd(ws=None) == WS
    assert bwd(ws_bytes=ws_need - 4) == WS
    assert bwd(dq=P(FAKE[0].value + 64)) == ALIAS      # dq over q
    assert bwd(dq=P(FAKE[8].value + 64)) == ALIAS      # dq over dk
    assert bwd(T=0, ws=None, ws_bytes=0) == OK


def test_rope_and_append_validation(lib):
    r = lib.sinkattn_rope_partial
    assert r(None, 1, 10, 8, 192, 64, FAKE[1], 1e4, 0, None) == NULL
    assert r(FAKE[0], 1, 10, 8, 192, 63, FAKE[1], 1e4, 0, None) == SHAPE   # odd rope_dim
    assert r(FAKE[0], 1, 10, 8, 192, 256, FAKE[1], 1e4, 0, None) == SHAPE  # > head_dim
    assert r(FAKE[0], 1, 10, 8, 192, 64, FAKE[1], -1.0, 0, None) == SHAPE
    assert r(FAKE[0], 1, 10, 8, 192, 64, FAKE[1], 1e4, 2, None) == SHAPE
    assert r(FAKE[0], 9, 10, 8, 192, 64, FAKE[1], 1e4, 0, None) == DTYPE
    assert r(FAKE[0], 1, 0, 8, 192, 64, FAKE[1], 1e4, 0, None) == OK
    a = lib.sinkattn_kv_append
    assert a(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 0, 128, None, None, 2, 4, 8, 192, 128, 1,
             None) == NULL
    assert a(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 3, 128, FAKE[4], None, 2, 4, 8, 192, 128, 1,
             None) == UNSUP
    assert a(FAKE[0], FAKE[1], FAKE[2], FAKE[3], 0, 128, FAKE[4], None, 0, 4, 8, 192, 128, 1,
             None) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 8, 192)
    with pytest.raises(ops.SinkAttnError):
        ops.prefill_swa(q, q[:, :, :1], torch.zeros(1, 4, 1, 128), torch.zeros(8))
