"""Size limits and empty inputs on the GPU.

- The sliding-window bf16 prefill has no per-sequence limit (the persistent
  kernel re-bases its 32-bit offsets per run of tiles): a 100,000-token layer
  (q = 2.46 GB, past 2^31 bytes) is checked on sampled rows on both sides of the
  2^31-byte mark, plain and with RoPE fused.
- The global prefill addresses a sequence's q with 32-bit offsets: at the
  largest accepted length (T = 87381 with 64 query heads, q just under 2^31
  bytes) sampled rows are checked, plain and with RoPE fused.
- Empty batches and sequences: every entry point returns at once.
Oracle: MiMo-V2-Flash Technical Report, Section 2.2 sink softmax (and Section
2.1 RoPE), on sampled query rows with every key they see.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_close
from sliding_window_sink_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()
    yield
    torch.cuda.empty_cache()


def _print_case(*a):
    print("case:", *a, flush=True)


def _inputs(seed, T, Hq, Hkv):
    q = synth.device_normal(seed, (1, T, Hq, 192), device=DEV)
    k = synth.device_normal(seed + 1, (1, T, Hkv, 192), device=DEV)
    v = synth.device_normal(seed + 2, (1, T, Hkv, 128), device=DEV)
    sink = synth.device_normal(seed + 3, (Hq,), torch.float32, device=DEV)
    return q, k, v, sink


def _check_rows(o, q, k, v, sink, rows, window, base=None):
    s = sink.cpu()
    for t0 in rows:
        lo = max(0, t0 - window + 1) if window else 0
        kp = np.arange(lo, t0 + 1)
        qq, kk = q[0, t0:t0 + 1], k[0, lo:t0 + 1]
        if base is not None:
            qq = oracle.rope_partial(qq, [t0], base)
            kk = oracle.rope_partial(kk, kp, base)
        ref, _ = oracle.sink_attention(qq, kk, v[0, lo:t0 + 1], [t0], kp, s, window)
        assert_close(o[0, t0:t0 + 1], ref, torch.bfloat16, "row %d" % t0)


@pytest.mark.parametrize("rope", [False, True])
def test_swa_prefill_past_2gib_of_q(rope):
    T, Hq, Hkv, W = 100000, 64, 8, 128
    _print_case("SWA T=100000", "rope" if rope else "plain")
    q, k, v, sink = _inputs(7100, T, Hq, Hkv)
    assert q.numel() * 2 > 2 ** 31
    if rope:
        o = ops.prefill_swa_rope(q, k, v, sink, W, synth.BASE_SWA)
    else:
        o = ops.prefill_swa(q, k, v, sink, window=W)
    torch.cuda.synchronize()
    last = (2 ** 31) // (Hq * 192 * 2)  # rows past this one lie beyond 2^31 bytes of q
    rows = [0, 127, 128, last - 1, last, last + 1, 95999, T - 1]
    rows += sorted(np.random.default_rng(71).choice(T, 8, replace=False).tolist())
    _check_rows(o, q, k, v, sink, rows, W, synth.BASE_SWA if rope else None)


@pytest.mark.parametrize("rope", [False, True])
def test_global_prefill_at_the_size_limit(rope):
    Hq, Hkv = 64, 4
    T = (2 ** 31 - 1) // (Hq * 192 * 2)  # 87381: the longest accepted sequence
    _print_case("global T=%d" % T, "rope" if rope else "plain")
    q, k, v, sink = _inputs(7200, T, Hq, Hkv)
    if rope:
        o, _ = ops.prefill_global_rope(q, k, v, sink, synth.BASE_GA)
    else:
        o = ops.prefill_global(q, k, v, sink)
    torch.cuda.synchronize()
    _check_rows(o, q, k, v, sink, [0, 40000, T - 2, T - 1], 0,
                synth.BASE_GA if rope else None)
    del q, k, v, o
    z = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.SinkAttnError):  # one token more does not fit
        ops.prefill_global(z(1, T + 1, Hq, 192), z(1, T + 1, Hkv, 192), z(1, T + 1, Hkv, 128),
                           sink)


def test_empty_inputs():
    _print_case("empty inputs")
    z = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device=DEV)
    sink = torch.zeros(64, dtype=torch.float32, device=DEV)
    for B, T in ((0, 100), (1, 0)):
        q, k, v = z(B, T, 64, 192), z(B, T, 8, 192), z(B, T, 8, 128)
        assert ops.prefill_swa(q, k, v, sink, window=128).shape == (B, T, 64, 128)
        assert ops.prefill_swa_rope(q, k, v, sink, 128, 1e4).shape == (B, T, 64, 128)
        assert ops.prefill_global(q, k, v, sink).shape == (B, T, 64, 128)
        o, lse = ops.prefill_global(q, k, v, sink, return_lse=True)
        dq, dk, dv, dsink = ops.backward(q, k, v, o, z(B, T, 64, 128), lse, sink, 128)
        assert dq.shape == q.shape and torch.count_nonzero(dsink) == 0
    cl = torch.zeros(0, dtype=torch.int32, device=DEV)
    kc, vc = z(0, 8, 128, 192), z(0, 8, 128, 128)
    o = ops.decode(z(0, 64, 192), z(0, 8, 192), z(0, 8, 128), kc, vc, cl, sink, ops.RING, 128, 0)
    assert o.shape == (0, 64, 128)
    o = ops.verify(z(0, 4, 64, 192), z(0, 4, 8, 192), z(0, 4, 8, 128), kc, vc, cl, sink,
                   ops.RING, 128, 0)
    assert o.shape == (0, 4, 64, 128)
    ops.kv_append(z(0, 4, 8, 192), z(0, 4, 8, 128), kc, vc, cl, ops.RING)
    torch.cuda.synchronize()
