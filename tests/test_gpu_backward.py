"""Backward of the causal sink-attention prefill on the GPU against the oracle.

Gradients with respect to q, k, v and the per-head sink logit (MiMo-V2-Flash
Technical Report, Section 2.2: the sink is learnable, so it gets a gradient:
dsink_h = -sum_i p_sink_i (dO_i . o_i)).  The oracle differentiates the fp64
definition (pinned by finite differences); the GPU path consumes the bf16
forward output o and its lse, so its D_i carries one bf16 rounding of o.

Small cases (several 32-token tiles, ragged tails, two sequences, a -inf sink
head) are compared element by element at the bf16 tolerance plus a relative
Frobenius bound; the T = 32768 SWA layer in the launch configuration the bench
times is checked on sampled query rows (dq) and key blocks (dk, dv) against
oracle slices that hold every query seeing those keys, and dsink against
-sum_i e^(sink - lse_i) (dO_i . o_i) evaluated in fp64 from the forward outputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_close, to64
from sliding_window_sink_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()


def _print_case(*a):
    print("case:", *a, flush=True)


def _rel_fro(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def _forward(q, k, v, sink, window):
    if window > 0:
        return ops.prefill_swa(q, k, v, sink, window=window, return_lse=True)
    return ops.prefill_global(q, k, v, sink, return_lse=True)


@pytest.mark.parametrize("B,T,Hq,Hkv,window", [
    (1, 100, 16, 2, 40),
    (2, 97, 8, 1, 128),
    (1, 300, 16, 2, 128),
    (1, 150, 32, 2, 0),     # global, 16 heads per KV head (two dq workgroups)
    (2, 333, 16, 1, 0),     # global, three 128-key dK/dV blocks, ragged last block
    (3, 1, 8, 1, 0),        # global, one token: every tile and block ragged
    (1, 31, 8, 1, 128),     # windowed, one partial tile
    (1, 129, 64, 4, 0),     # global at the bench's head shape, one key past a block
    (1, 700, 8, 1, 512),    # W = 512 (the report's Table 2 ablation width)
])
def test_backward_vs_oracle(B, T, Hq, Hkv, window):
    _print_case("backward", B, T, Hq, Hkv, window)
    q, k, v, sink = synth.prefill_inputs(900 + T + window, B, T, Hq, Hkv, torch.bfloat16)
    sink[1] = float("-inf")
    g = synth.generator(77 + T)
    dout = synth.normal(g, (B, T, Hq, 128))
    qd, kd, vd, sd, gd = (t.to(DEV) for t in (q, k, v, sink, dout))
    o, lse = _forward(qd, kd, vd, sd, window)
    dq, dk, dv, dsink = ops.backward(qd, kd, vd, o, gd, lse, sd, window)
    torch.cuda.synchronize()
    pos = np.arange(T)
    ref_dsink = np.zeros(Hq)
    for b in range(B):
        rq, rk, rv, rs = oracle.sink_attention_bwd(q[b], k[b], v[b], pos, pos, sink, dout[b],
                                                   window)
        for name, got, ref in (("dq", dq[b], rq), ("dk", dk[b], rk), ("dv", dv[b], rv)):
            assert_close(got, ref, torch.bfloat16, "%s b=%d" % (name, b))
            assert _rel_fro(to64(got), ref) < 1e-2, (name, _rel_fro(to64(got), ref))
        ref_dsink += rs
    assert_close(dsink, ref_dsink, torch.bfloat16, "dsink")
    assert dsink[1].item() == 0.0  # a -inf sink takes no mass and gets no gradient


@pytest.mark.parametrize("sink_val,window", [(8.0, 128), (8.0, 0), (1e3, 128)])
def test_backward_sink_stress(sink_val, window):
    """A dominant sink (+8: most of the mass, so dsink carries most of the
    gradient) and an absorbing one (1e3: o = 0, so every gradient is exactly 0)."""
    _print_case("backward sink stress", sink_val, window)
    B, T, Hq, Hkv = 1, 260, 8, 1
    q, k, v, _ = synth.prefill_inputs(1234, B, T, Hq, Hkv, torch.bfloat16)
    sink = torch.full((Hq,), sink_val, dtype=torch.float32)
    dout = synth.normal(synth.generator(4321), (B, T, Hq, 128))
    qd, kd, vd, sd, gd = (t.to(DEV) for t in (q, k, v, sink, dout))
    o, lse = _forward(qd, kd, vd, sd, window)
    dq, dk, dv, dsink = ops.backward(qd, kd, vd, o, gd, lse, sd, window)
    torch.cuda.synchronize()
    if sink_val == 1e3:
        for x in (dq, dk, dv, dsink):
            assert torch.count_nonzero(x) == 0
        return
    pos = np.arange(T)
    rq, rk, rv, rs = oracle.sink_attention_bwd(q[0], k[0], v[0], pos, pos, sink, dout[0], window)
    for name, got, ref in (("dq", dq[0], rq), ("dk", dk[0], rk), ("dv", dv[0], rv),
                           ("dsink", dsink, rs)):
        assert_close(got, ref, torch.bfloat16, name)


def test_backward_deterministic():
    _print_case("backward determinism")
    q, k, v, sink = synth.prefill_inputs(31, 1, 200, 16, 2, torch.bfloat16)
    dout = synth.normal(synth.generator(32), (1, 200, 16, 128))
    qd, kd, vd, sd, gd = (t.to(DEV) for t in (q, k, v, sink, dout))
    o, lse = ops.prefill_swa(qd, kd, vd, sd, window=128, return_lse=True)
    r1 = ops.backward(qd, kd, vd, o, gd, lse, sd, 128)
    r2 = ops.backward(qd, kd, vd, o, gd, lse, sd, 128)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_backward_full_swa_layer_sampled():
    """T = 32768, 64 query / 8 KV heads, W = 128 (the headline layer shape)."""
    _print_case("backward full SWA layer")
    w = synth.WORKLOADS[2]
    B, T, Hq, Hkv, W = w.B, w.T, w.Hq, w.Hkv, w.window
    q, k, v, sink = synth.prefill_inputs(w.seed, B, T, Hq, Hkv, torch.bfloat16)
    dout = synth.normal(synth.generator(w.seed + 7), (B, T, Hq, 128))
    qd, kd, vd, sd, gd = (t.to(DEV) for t in (q, k, v, sink, dout))
    o, lse = ops.prefill_swa(qd, kd, vd, sd, window=W, return_lse=True)
    dq, dk, dv, dsink = ops.backward(qd, kd, vd, o, gd, lse, sd, W)
    torch.cuda.synchronize()
    # dq of sampled query tokens: the oracle over their windows
    for t0 in (0, 31, 4095, 20000, T - 1):
        lo = max(0, t0 - W + 1)
        rq, _, _, _ = oracle.sink_attention_bwd(q[0, t0:t0 + 1], k[0, lo:t0 + 1],
                                                v[0, lo:t0 + 1], [t0], np.arange(lo, t0 + 1),
                                                sink, dout[0, t0:t0 + 1], W)
        assert_close(dq[0, t0:t0 + 1], rq, torch.bfloat16, "dq token %d" % t0)
    # dk, dv of sampled key blocks: every query that sees them, and their windows
    for kb in (0, 4096, T - 32):
        qhi = min(T, kb + 32 + W - 1)
        klo = max(0, kb - W + 1)
        _, rk, rv, _ = oracle.sink_attention_bwd(q[0, kb:qhi], k[0, klo:qhi], v[0, klo:qhi],
                                                 np.arange(kb, qhi), np.arange(klo, qhi), sink,
                                                 dout[0, kb:qhi], W)
        sl = slice(kb - klo, kb - klo + 32)
        assert_close(dk[0, kb:kb + 32], rk[sl], torch.bfloat16, "dk block %d" % kb)
        assert_close(dv[0, kb:kb + 32], rv[sl], torch.bfloat16, "dv block %d" % kb)
    # dsink: -sum_i e^(sink - lse_i) (dO_i . o_i), fp64 from the forward outputs
    D = (to64(gd[0]) * to64(o[0])).sum(-1)                      # [T, Hq]
    ps = np.exp(sink.double().numpy()[None, :] - to64(lse[0]).T)  # [T, Hq]
    ref = -(ps * D).sum(0)
    assert_close(dsink, ref, torch.bfloat16, "dsink full layer")
