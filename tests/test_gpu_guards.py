"""No entry point writes outside its outputs, and the caches change only where
the operation says.

Every output (o, lse, k_rot, the split-K workspace, the caches, the gradients,
RoPE's in-place rows) is passed as an interior view of a buffer whose bytes
start as 0xFF (NaN in bf16 and fp32); after the call the bytes before and after
the view must be unchanged.  Decode (MiMo-V2-Flash Technical Report, Section
2.3.1: one new token per step over a per-request cache) must change exactly the
one cache row of position P = cache_len[b] per (sequence, KV head) and nothing
else; verify must change no cache byte at all.  The values themselves are
checked against the oracle (Section 2.2) here as well.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import Guarded, assert_close, sink_for_half_mass
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


def _guarded_copy(x: torch.Tensor) -> Guarded:
    g = Guarded(tuple(x.shape), x.dtype)
    g.t.copy_(x.to(DEV))
    return g


def _bits(t: torch.Tensor) -> torch.Tensor:
    t = t.detach().cpu()
    return t.view(torch.int16) if t.element_size() == 2 else (
        t.view(torch.int32) if t.element_size() == 4 else t.view(torch.uint8))


def _assert_cache_rows(after, before, written, what):
    """after/before [B,Hkv,cap,d]; written: {b: slot}: that row of every KV head
    may differ, every other byte must be identical."""
    a, b0 = _bits(after), _bits(before)
    mask = torch.ones(a.shape[:3], dtype=torch.bool)
    for b, slot in written.items():
        mask[b, :, slot] = False
    diff = (a != b0).any(-1) & mask
    assert not bool(diff.any()), "%s: %d untouched cache rows changed, first at %s" % (
        what, int(diff.sum()), tuple(diff.nonzero()[0].tolist()))


@pytest.mark.parametrize("kind", [ops.RING, ops.CONTIG])
def test_decode_guards_and_untouched_slots(kind):
    _print_case("decode guards", kind)
    lens = [0, 1, 127, 128, 129, 700, 2049]
    cl = torch.tensor(lens, dtype=torch.int32)
    Hq, Hkv = 64, 4 if kind == ops.CONTIG else 8
    window = 128 if kind == ops.RING else 0
    layer = synth.cached_layer(synth.generator(901 + kind), cl, 1, Hq, Hkv, window,
                               torch.bfloat16)
    if kind == ops.CONTIG:
        layer.sink = torch.full((Hq,), sink_for_half_mass(1000), dtype=torch.float32)
    cap = 128 if kind == ops.RING else 2100
    fill = synth.fill_ring if kind == ops.RING else synth.fill_contig
    kc0, vc0 = fill(layer, cl, cap, Hkv)
    kg, vg = _guarded_copy(kc0), _guarded_copy(vc0)
    B = len(lens)
    og = Guarded((B, Hq, 128), torch.bfloat16)
    ws = None
    if kind == ops.CONTIG:
        ws = Guarded((ops.decode_workspace_bytes(B, Hq, 1, 7) // 4,), torch.float32)
    ops.decode(layer.q[:, 0].to(DEV), layer.k_new[:, 0].to(DEV), layer.v_new[:, 0].to(DEV),
               kg.t, vg.t, cl.to(DEV), layer.sink.to(DEV), kind, window, max(lens),
               num_splits=7 if ws is not None else 0, workspace=None if ws is None else ws.t,
               out=og.t)
    torch.cuda.synchronize()
    for g, name in ((og, "o"), (kg, "k_cache"), (vg, "v_cache")) + \
            (((ws, "workspace"),) if ws is not None else ()):
        g.assert_intact(name)
    ref = oracle.decode_or_verify(layer.q, layer.k_hist, layer.v_hist, layer.k_new,
                                  layer.v_new, cl, layer.sink, window)[0]
    assert_close(og.t[:, None], ref, torch.bfloat16, "decode o")
    slots = {b: (L % cap if kind == ops.RING else L) for b, L in enumerate(lens)}
    _assert_cache_rows(kg.t, kc0, slots, "k_cache")
    _assert_cache_rows(vg.t, vc0, slots, "v_cache")
    kc, vc = kg.t.cpu(), vg.t.cpu()
    for b, s in slots.items():
        assert torch.equal(kc[b, :, s], layer.k_new[b, 0])
        assert torch.equal(vc[b, :, s], layer.v_new[b, 0])


@pytest.mark.parametrize("kind", [ops.RING, ops.CONTIG])
def test_verify_rope_guards_read_only(kind):
    _print_case("verify guards", kind)
    lens = [0, 3, 126, 130, 1500]
    cl = torch.tensor(lens, dtype=torch.int32)
    nq, Hq = 4, 64
    Hkv = 8 if kind == ops.RING else 4
    window = 128 if kind == ops.RING else 0
    base = synth.BASE_SWA if kind == ops.RING else synth.BASE_GA
    layer = synth.cached_layer(synth.generator(911 + kind), cl, nq, Hq, Hkv, window,
                               torch.bfloat16)
    cap = 128 if kind == ops.RING else 1600
    fill = synth.fill_ring if kind == ops.RING else synth.fill_contig
    kc0, vc0 = fill(layer, cl, cap, Hkv)
    kg, vg = _guarded_copy(kc0), _guarded_copy(vc0)
    B = len(lens)
    og = Guarded((B, nq, Hq, 128), torch.bfloat16)
    krg = Guarded((B, nq, Hkv, 192), torch.bfloat16)
    ws = Guarded((ops.decode_workspace_bytes(B, Hq, nq, 64) // 4,), torch.float32)
    ops.verify_rope(layer.q.to(DEV), layer.k_new.to(DEV), layer.v_new.to(DEV), kg.t, vg.t,
                    cl.to(DEV), layer.sink.to(DEV), kind, window, max(lens), base=base,
                    k_rot=krg.t, num_splits=0, workspace=ws.t, out=og.t)
    torch.cuda.synchronize()
    for g, name in ((og, "o"), (krg, "k_rot"), (kg, "k_cache"), (vg, "v_cache"),
                    (ws, "workspace")):
        g.assert_intact(name)
    _assert_cache_rows(kg.t, kc0, {}, "k_cache")
    _assert_cache_rows(vg.t, vc0, {}, "v_cache")
    # oracle: q and the new keys rotated at positions P..P+nq-1
    qr = np.stack([oracle.rope_partial(layer.q[b], np.arange(L, L + nq), base)
                   for b, L in enumerate(lens)])
    kr = np.stack([oracle.rope_partial(layer.k_new[b], np.arange(L, L + nq), base)
                   for b, L in enumerate(lens)])
    ref = oracle.decode_or_verify(qr, layer.k_hist, layer.v_hist, kr, layer.v_new, cl,
                                  layer.sink, window)[0]
    assert_close(og.t, ref, torch.bfloat16, "verify o")
    assert_close(krg.t, kr, torch.bfloat16, "k_rot")


def test_kv_append_guards():
    _print_case("kv_append guards")
    g = synth.generator(921)
    B, n, Hkv, cap = 3, 4, 2, 128
    cl = torch.tensor([0, 126, 300], dtype=torch.int32)
    nacc = torch.tensor([4, 2, 0], dtype=torch.int32)
    kn, vn = synth.normal(g, (B, n, Hkv, 192)), synth.normal(g, (B, n, Hkv, 128))
    kc0 = synth.normal(g, (B, Hkv, cap, 192))
    vc0 = synth.normal(g, (B, Hkv, cap, 128))
    kg, vg = _guarded_copy(kc0), _guarded_copy(vc0)
    ops.kv_append(kn.to(DEV), vn.to(DEV), kg.t, vg.t, cl.to(DEV), ops.RING, nacc.to(DEV))
    torch.cuda.synchronize()
    kg.assert_intact("k_cache")
    vg.assert_intact("v_cache")
    ke, ve = kc0.clone(), vc0.clone()
    for b in range(B):
        for t in range(int(nacc[b])):
            s = (int(cl[b]) + t) % cap
            ke[b, :, s], ve[b, :, s] = kn[b, t], vn[b, t]
    assert torch.equal(kg.t.cpu(), ke) and torch.equal(vg.t.cpu(), ve)


def test_rope_in_place_guards():
    _print_case("rope guards")
    g = synth.generator(931)
    x = synth.normal(g, (77, 9, 192))
    xg = _guarded_copy(x)
    pos = torch.arange(1000, 1077, dtype=torch.int32)
    ops.rope_partial(xg.t, pos.to(DEV), synth.BASE_SWA)
    torch.cuda.synchronize()
    xg.assert_intact("x")
    ref = oracle.rope_partial(x, pos.numpy(), synth.BASE_SWA)
    assert_close(xg.t, ref, torch.bfloat16, "rope")


@pytest.mark.parametrize("window", [0, 128, 512])
def test_prefill_guards(window):
    _print_case("prefill guards", window)
    B, T, Hq, Hkv = 2, 333, 16, 2
    q, k, v, sink = synth.prefill_inputs(941 + window, B, T, Hq, Hkv, torch.bfloat16)
    og = Guarded((B, T, Hq, 128), torch.bfloat16)
    lg = Guarded((B, Hq, T), torch.float32)
    args = [t.to(DEV) for t in (q, k, v, sink)]
    if window:
        ops.prefill_swa(*args, window=window, out=og.t, lse_out=lg.t)
    else:
        ops.prefill_global(*args, out=og.t, lse_out=lg.t)
    torch.cuda.synchronize()
    og.assert_intact("o")
    lg.assert_intact("lse")
    ref_o, ref_lse = oracle.prefill(q, k, v, sink, window)
    assert_close(og.t, ref_o, torch.bfloat16, "o")
    assert_close(lg.t.permute(0, 2, 1), ref_lse, torch.bfloat16, "lse")


def test_global_rope_guards():
    _print_case("global rope guards")
    B, T, Hq, Hkv = 1, 300, 16, 1
    q, k, v, sink = synth.prefill_inputs(951, B, T, Hq, Hkv, torch.bfloat16)
    og = Guarded((B, T, Hq, 128), torch.bfloat16)
    lg = Guarded((B, Hq, T), torch.float32)
    kg = Guarded((B, T, Hkv, 192), torch.bfloat16)
    ops.prefill_global_rope(*[t.to(DEV) for t in (q, k, v, sink)], synth.BASE_GA, k_rot=kg.t,
                            out=og.t, lse_out=lg.t)
    torch.cuda.synchronize()
    for g_, name in ((og, "o"), (lg, "lse"), (kg, "k_rot")):
        g_.assert_intact(name)
    pos = np.arange(T)
    qr = oracle.rope_partial(q[0], pos, synth.BASE_GA)[None]
    kr = oracle.rope_partial(k[0], pos, synth.BASE_GA)[None]
    ref_o, _ = oracle.prefill(qr, kr, v, sink, 0)
    assert_close(og.t, ref_o, torch.bfloat16, "o")


@pytest.mark.parametrize("window", [128, 0])
def test_backward_guards(window):
    _print_case("backward guards", window)
    B, T, Hq, Hkv = 1, 200, 16, 2
    q, k, v, sink = synth.prefill_inputs(961 + window, B, T, Hq, Hkv, torch.bfloat16)
    dout = synth.normal(synth.generator(962), (B, T, Hq, 128))
    qd, kd, vd, sd = (t.to(DEV) for t in (q, k, v, sink))
    if window:
        o, lse = ops.prefill_swa(qd, kd, vd, sd, window=window, return_lse=True)
    else:
        o, lse = ops.prefill_global(qd, kd, vd, sd, return_lse=True)
    gs = [Guarded((B, T, Hq, 192), torch.float32), Guarded((B, T, Hkv, 192), torch.float32),
          Guarded((B, T, Hkv, 128), torch.float32), Guarded((Hq,), torch.float32)]
    ws = Guarded((ops.lib().sinkattn_backward_workspace_bytes(B, T, Hq) // 4,), torch.float32)
    ops.backward(qd, kd, vd, o, dout.to(DEV), lse, sd, window, workspace=ws.t,
                 out=tuple(g.t for g in gs))
    torch.cuda.synchronize()
    for g_, name in zip(gs + [ws], ("dq", "dk", "dv", "dsink", "workspace")):
        g_.assert_intact(name)
    dq, dk, dv, ds = oracle.sink_attention_bwd(q[0], k[0], v[0], np.arange(T), np.arange(T),
                                               sink, dout[0], window)
    for got, ref, name in ((gs[0].t[0], dq, "dq"), (gs[1].t[0], dk, "dk"), (gs[2].t[0], dv, "dv")):
        err = np.abs(got.cpu().double().numpy() - ref)
        assert np.all(err <= 2e-2 + 1e-2 * np.abs(ref)), (name, float(err.max()))
    # dsink sums -e^(sink - lse_i) (dO_i . o_i) over every token; the kernels use
    # the forward's bf16 o, whose rounding adds up over the tokens, so it is
    # checked tightly against that sum evaluated in fp64 from the forward outputs
    # and loosely (1% relative, Frobenius) against the exact oracle gradient
    got = gs[3].t.cpu().double().numpy()
    ps = np.exp(sink.double().numpy()[None, :] - lse[0].cpu().double().numpy().T)  # [T, Hq]
    dd = (o[0].cpu().double() * dout[0].double()).sum(-1).numpy()                  # [T, Hq]
    ref_fwd = -(ps * dd).sum(0)
    assert np.all(np.abs(got - ref_fwd) <= 2e-2 + 1e-2 * np.abs(ref_fwd)), (got, ref_fwd)
    assert np.linalg.norm(got - ds) <= 1e-2 * np.linalg.norm(ds), (got, ds)


def test_decode_fp8_guards_and_untouched_slots():
    _print_case("decode fp8 guards")
    ks, vs = 0.011, 0.0073
    lens = [0, 5, 128, 1000]
    cl = torch.tensor(lens, dtype=torch.int32)
    B, Hq, Hkv, cap = len(lens), 64, 4, 1100
    g = synth.generator(971)
    layer = synth.cached_layer(g, cl, 1, Hq, Hkv, 0, torch.bfloat16)
    kc0 = torch.zeros(B, Hkv, cap, 192, dtype=torch.uint8)
    vc0 = torch.zeros(B, Hkv, cap, 128, dtype=torch.uint8)
    for b, L in enumerate(lens):
        kc0[b, :, :L] = torch.from_numpy(oracle.fp8_quantize(layer.k_hist[b], ks)).permute(1, 0, 2)
        vc0[b, :, :L] = torch.from_numpy(oracle.fp8_quantize(layer.v_hist[b], vs)).permute(1, 0, 2)
    kg, vg = _guarded_copy(kc0), _guarded_copy(vc0)
    og = Guarded((B, Hq, 128), torch.bfloat16)
    ws = Guarded((ops.decode_workspace_bytes(B, Hq, 1, 64) // 4,), torch.float32)
    ops.decode_fp8(layer.q[:, 0].to(DEV), layer.k_new[:, 0].to(DEV), layer.v_new[:, 0].to(DEV),
                   kg.t, vg.t, cl.to(DEV), layer.sink.to(DEV), ops.CONTIG, 0, max(lens), ks, vs,
                   workspace=ws.t, out=og.t)
    torch.cuda.synchronize()
    for g_, name in ((og, "o"), (kg, "k_cache"), (vg, "v_cache"), (ws, "workspace")):
        g_.assert_intact(name)
    slots = {b: L for b, L in enumerate(lens)}
    _assert_cache_rows(kg.t, kc0, slots, "k_cache")
    _assert_cache_rows(vg.t, vc0, slots, "v_cache")
    kc = kg.t.cpu()
    for b, L in enumerate(lens):
        want = torch.from_numpy(oracle.fp8_quantize(layer.k_new[b, 0], ks))
        assert torch.equal(kc[b, :, L], want)
    kh = [oracle.fp8_dequantize(torch.from_numpy(oracle.fp8_quantize(x, ks)), ks)
          for x in layer.k_hist]
    vh = [oracle.fp8_dequantize(torch.from_numpy(oracle.fp8_quantize(x, vs)), vs)
          for x in layer.v_hist]
    ref = oracle.decode_or_verify(layer.q, kh, vh, layer.k_new, layer.v_new, cl, layer.sink, 0)[0]
    assert_close(og.t[:, None], ref, torch.bfloat16, "fp8 decode o")
    assert math.isfinite(float(og.t.float().abs().max()))
