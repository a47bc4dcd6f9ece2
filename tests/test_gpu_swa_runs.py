"""The sliding-window prefill kernels compared with the oracle on EVERY output.

1. The headline layer at its full size (B=1, T=32768, 64 query / 8 KV heads,
   W=128, RoPE base 1e4 fused; MiMo-V2-Flash Technical Report, Section 2.2 and
   Table 1), launched exactly as the benchmark launches it, every one of the
   32768 x 64 x 128 outputs against the fp64 oracle; the rotated keys it writes
   in full against the standalone RoPE kernel (bit for bit) and the oracle.
2. The same layer through the plain (pre-rotated input) kernel, every output.
3. Smaller batches whose runs hold at least 7 tiles of 32 tokens each, so that
   the persistent kernel's next-tile prefetch, its 6-slot LDS ring of key blocks
   (which wraps after 6 blocks), the rotation tables of the next tiles and each
   run's first-block rotated-key write are all exercised: W = 128, 129 (the
   largest the kernel takes), 1 and 100, ragged last tiles, fused and plain.
   Every output is compared, lse included, and every output (o, lse, k_rot)
   sits inside a guard band that must come back untouched.

The oracle sees q and k rotated in fp64 and rounded once to bf16, which is what
the fused kernel is defined to compute (RoPE to bf16, then attention).
Tolerance: bf16 inputs, |d| <= 2e-2 + 1e-2 |oracle|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import Guarded, assert_close
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


def _rot_bf16(x, pos, base):
    """Oracle RoPE (fp64) of bf16 rows, rounded once to bf16 and widened back."""
    r = oracle.rope_partial(x, pos, base)
    return oracle.bf16_bits_to_f64(oracle.round_bf16_bits(r))


def _tiles_per_run(B, T, Hq, Hkv):
    """Tiles (32 query tokens) per run of the persistent SWA kernel: one run per
    compute unit over the (sequence, KV group, 8-head part) units, each run a
    contiguous range of tiles.  Mirrors the host launcher's plan so the cases
    below can assert that they really exercise long runs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = B * Hkv * ((Hq // Hkv) // 8)
    n_tiles = (T + 31) // 32
    runs = max(1, min(n_tiles, (cus + units - 1) // units))
    return (n_tiles + runs - 1) // runs


def _compare_rows(o, lse, q, k, v, sink, window, base, b=0, chunk=4096):
    """Every row of sequence b against the oracle, chunk by chunk (the oracle
    gets only the keys a chunk's rows can see).  base None: no RoPE."""
    T = q.shape[1]
    kpos_all = np.arange(T)
    kk = k[b] if base is None else _rot_bf16(k[b], kpos_all, base)
    worst = 0.0
    for c0 in range(0, T, chunk):
        rows = np.arange(c0, min(T, c0 + chunk))
        lo = max(0, c0 - window + 1)
        hi = rows[-1] + 1
        qq = q[b, c0:hi] if base is None else _rot_bf16(q[b, c0:hi], rows, base)
        ref_o, ref_lse = oracle.sink_attention(qq, kk[lo:hi], v[b, lo:hi], rows,
                                               np.arange(lo, hi), sink, window)
        worst = max(worst, assert_close(o[b, c0:hi], ref_o, torch.bfloat16,
                                        "o rows %d..%d" % (c0, hi - 1)))
        if lse is not None:
            assert_close(lse[b, :, c0:hi].transpose(0, 1), ref_lse, torch.bfloat16,
                         "lse rows %d..%d" % (c0, hi - 1))
    return worst


def _ulp_close(got_bits: np.ndarray, ref_f64: np.ndarray):
    """Rotated bf16 rows against the oracle's fp64 rotation: the kernels rotate
    in fp32 and round once to bf16, so each value is within one bf16 ulp of the
    exact one plus the fp32 rounding of the two products, which matters only
    when they cancel (|x0 c - x1 s| far below |x0|, |x1|): |d| <= 2^-8 |ref| +
    2e-6 for N(0,1) rows.  Almost all values equal the once-rounded oracle."""
    ref_bits = oracle.round_bf16_bits(ref_f64)
    got = oracle.bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref_f64)
    bad = err > 2.0 ** -8 * np.abs(ref_f64) + 2e-6
    assert not bad.any(), "%d rotated values off, worst %.3g" % (int(bad.sum()), float(err.max()))
    assert (got_bits == ref_bits).mean() > 0.99


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _device_inputs(w):
    q = synth.device_normal(w.seed, (w.B, w.T, w.Hq, 192), device=DEV)
    k = synth.device_normal(w.seed + 1, (w.B, w.T, w.Hkv, 192), device=DEV)
    v = synth.device_normal(w.seed + 2, (w.B, w.T, w.Hkv, 128), device=DEV)
    sink = synth.device_normal(w.seed + 3, (w.Hq,), torch.float32, device=DEV)
    return q, k, v, sink


def test_full_swa_prefill_rope_every_output():
    """The headline step in full: prefill_swa_rope at T = 32768 with the
    benchmark's inputs and launch (o and k_rot out, no lse)."""
    w = synth.WORKLOADS[2]
    _print_case("full SWA prefill + RoPE, every output", w.name)
    assert _tiles_per_run(w.B, w.T, w.Hq, w.Hkv) >= 7
    q, k, v, sink = _device_inputs(w)
    og = Guarded((w.B, w.T, w.Hq, 128), torch.bfloat16)
    kg = Guarded(tuple(k.shape), torch.bfloat16)
    ops.prefill_swa_rope(q, k, v, sink, w.window, w.base, k_rot=kg.t, out=og.t)
    torch.cuda.synchronize()
    og.assert_intact("o")
    kg.assert_intact("k_rot")
    # the rotated keys: bit for bit the standalone RoPE kernel's, and within the
    # fp32 rotation's bound of the oracle's fp64 rotation
    kr = k.clone()
    ops.rope_partial(kr, synth.positions(w.B, w.T).to(DEV), w.base)
    assert torch.equal(kg.t, kr), "k_rot differs from rope_partial(k)"
    del kr
    kh = k.cpu()
    _ulp_close(_bits(kg.t[0]), oracle.rope_partial(kh[0], np.arange(w.T), w.base))
    qh, vh, sh = q.cpu(), v.cpu(), sink.cpu()
    del q, k, v
    worst = _compare_rows(og.t.cpu(), None, qh, kh, vh, sh, w.window, w.base)
    print("full SWA prefill + RoPE: max|d| = %.4g over %d outputs" % (worst, og.t.numel()))


def test_full_swa_prefill_plain_every_output():
    """The plain kernel at the same size (inputs taken as already rotated)."""
    w = synth.WORKLOADS[2]
    _print_case("full SWA prefill plain, every output", w.name)
    q, k, v, sink = _device_inputs(w)
    og = Guarded((w.B, w.T, w.Hq, 128), torch.bfloat16)
    ops.prefill_swa(q, k, v, sink, window=w.window, out=og.t)
    torch.cuda.synchronize()
    og.assert_intact("o")
    qh, kh, vh, sh = q.cpu(), k.cpu(), v.cpu(), sink.cpu()
    del q, k, v
    worst = _compare_rows(og.t.cpu(), None, qh, kh, vh, sh, w.window, None)
    print("full SWA prefill plain: max|d| = %.4g" % worst)


RUN_CASES = [
    # B, T, Hq, Hkv, window
    (8, 2048, 64, 8, 128),   # 16 tiles per run: the LDS ring wraps twice
    (8, 1000, 64, 8, 129),   # the widest window the kernel takes; ragged last tile
    (8, 1024, 64, 8, 1),     # each query sees only itself
    (2, 3900, 64, 8, 100),   # window not a multiple of 32; ragged tail
    (1, 8192, 64, 8, 128),   # one sequence, 8 tiles per run
]


@pytest.mark.parametrize("B,T,Hq,Hkv,window", RUN_CASES)
def test_swa_prefill_long_runs(B, T, Hq, Hkv, window):
    _print_case("SWA long runs", B, T, Hq, Hkv, window)
    tpr = _tiles_per_run(B, T, Hq, Hkv)
    assert tpr >= 7, "case no longer exercises long runs (%d tiles per run)" % tpr
    q, k, v, sink = synth.prefill_inputs(7000 + T + window, B, T, Hq, Hkv, torch.bfloat16)
    qd, kd, vd, sd = (t.to(DEV) for t in (q, k, v, sink))
    # fused RoPE: o, lse, k_rot in guard bands
    og = Guarded((B, T, Hq, 128), torch.bfloat16)
    lg = Guarded((B, Hq, T), torch.float32)
    kg = Guarded((B, T, Hkv, 192), torch.bfloat16)
    ops.prefill_swa_rope(qd, kd, vd, sd, window, synth.BASE_SWA, k_rot=kg.t, out=og.t,
                         lse_out=lg.t)
    torch.cuda.synchronize()
    for g, name in ((og, "o"), (lg, "lse"), (kg, "k_rot")):
        g.assert_intact(name)
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k), "inputs must stay untouched"
    # bit for bit: standalone RoPE of q and k, then the plain kernel
    pos = synth.positions(B, T).to(DEV)
    qr, kr = qd.clone(), kd.clone()
    ops.rope_partial(qr, pos, synth.BASE_SWA)
    ops.rope_partial(kr, pos, synth.BASE_SWA)
    pg = Guarded((B, T, Hq, 128), torch.bfloat16)
    plg = Guarded((B, Hq, T), torch.float32)
    ops.prefill_swa(qr, kr, vd, sd, window=window, out=pg.t, lse_out=plg.t)
    torch.cuda.synchronize()
    pg.assert_intact("plain o")
    plg.assert_intact("plain lse")
    assert torch.equal(kg.t, kr), "k_rot differs from rope_partial(k)"
    assert torch.equal(og.t, pg.t) and torch.equal(lg.t, plg.t), "fused != rope + plain"
    o, lse = og.t.cpu(), lg.t.cpu()
    for b in range(B):
        _compare_rows(o, lse, q, k, v, sink, window, synth.BASE_SWA, b=b)
