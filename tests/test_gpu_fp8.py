"""E4M3 (FP8) KV caches on the GPU against the oracle.

The report runs inference in FP8 (MiMo-V2-Flash Technical Report, Section 4.6)
without defining the cache format; the oracle's reading is OCP E4M3 with one
scale per tensor and a quantizer E4M3(fl32(x / scale)) (ties to even,
saturating).  Checks:
  - kv_append_fp8 stores exactly the oracle's codes (incl. saturating and
    subnormal values);
  - decode_fp8 stores the new token's codes exactly and its output matches the
    oracle over the dequantized cache (new tokens at bf16) at the bf16
    tolerance, ring and contiguous, split and unsplit, with and without the
    fused RoPE; fused == unfused bit for bit;
  - verify_fp8 (token-wave kernel, up to 64 columns) likewise, caches untouched.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_close, sink_for_half_mass
from sliding_window_sink_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
KS, VS = 0.011, 0.0073   # per-tensor scales: N(0,1) data spans ~[-400, 400] codes


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()


def _print_case(*a):
    print("case:", *a, flush=True)


def _codes(x, scale):
    return torch.from_numpy(oracle.fp8_quantize(x, scale).view(np.uint8))


def _fp8_caches(layer, cl, kind, cap, Hkv):
    """uint8 caches holding the oracle's codes of the history, and the history
    the oracle attends to (dequantized codes)."""
    B = len(cl)
    kc = torch.zeros(B, Hkv, cap, 192, dtype=torch.uint8)
    vc = torch.zeros(B, Hkv, cap, 128, dtype=torch.uint8)
    kh, vh = [], []
    for b in range(B):
        L = int(cl[b])
        kb, vb = layer.k_hist[b], layer.v_hist[b]   # rows of positions L - len .. L-1
        n = kb.shape[0]
        kcode, vcode = _codes(kb, KS), _codes(vb, VS)
        for i in range(n):
            p = L - n + i
            slot = p % cap if kind == ops.RING else p
            kc[b, :, slot] = kcode[i]
            vc[b, :, slot] = vcode[i]
        kh.append(oracle.fp8_dequantize(kcode.numpy(), KS))
        vh.append(oracle.fp8_dequantize(vcode.numpy(), VS))
    return kc.to(DEV), vc.to(DEV), kh, vh


@pytest.mark.parametrize("kind", [ops.RING, ops.CONTIG])
def test_kv_append_fp8_codes(kind):
    _print_case("kv_append_fp8", kind)
    g = synth.generator(77)
    B, n, Hkv, cap = 3, 5, 2, 128 if kind == ops.RING else 400
    cl = torch.tensor([0, 126, 390], dtype=torch.int32)
    nacc = torch.tensor([5, 2, 0], dtype=torch.int32)
    kn = synth.normal(g, (B, n, Hkv, 192))
    vn = synth.normal(g, (B, n, Hkv, 128))
    kn[0, 0, 0, :8] = torch.tensor([1e4, -1e4, 5.0, -5.0, 1e-6, -1e-6, 4.9e-3, 0.0])
    vn[0, 1, 1, :4] = torch.tensor([3.3, -3.3, 2e-5, -0.0])
    kc = torch.zeros(B, Hkv, cap, 192, dtype=torch.uint8, device=DEV)
    vc = torch.zeros(B, Hkv, cap, 128, dtype=torch.uint8, device=DEV)
    ops.kv_append_fp8(kn.to(DEV), vn.to(DEV), kc, vc, cl.to(DEV), kind, nacc.to(DEV), KS, VS)
    kc, vc = kc.cpu(), vc.cpu()
    ke, ve = torch.zeros_like(kc), torch.zeros_like(vc)
    for b in range(B):
        for t in range(int(nacc[b])):
            p = int(cl[b]) + t
            slot = p % cap if kind == ops.RING else p
            if kind == ops.CONTIG and p >= cap:
                continue
            ke[b, :, slot] = _codes(kn[b, t], KS)
            ve[b, :, slot] = _codes(vn[b, t], VS)
    assert torch.equal(kc, ke) and torch.equal(vc, ve)


@pytest.mark.parametrize("kind,Hq,Hkv,window,splits,rope", [
    (ops.RING, 64, 8, 128, 0, False),
    (ops.RING, 64, 8, 128, 0, True),
    (ops.CONTIG, 64, 4, 0, 0, False),
    (ops.CONTIG, 64, 4, 0, 1, True),
    (ops.CONTIG, 64, 4, 0, 7, True),
])
def test_decode_fp8(kind, Hq, Hkv, window, splits, rope):
    _print_case("decode fp8", kind, Hq, Hkv, window, splits, rope)
    base = synth.BASE_SWA if window else synth.BASE_GA
    cl = torch.tensor([0, 1, 31, 127, 128, 700, 2049], dtype=torch.int32)
    layer = synth.cached_layer(synth.generator(1500 + Hkv + rope), cl, 1, Hq, Hkv, window,
                               torch.bfloat16)
    if not window:
        layer.sink = torch.full((Hq,), sink_for_half_mass(1000), dtype=torch.float32)
    cap = 128 if kind == ops.RING else 2100
    B, max_len = len(cl), int(cl.max())
    ws = torch.empty(ops.decode_workspace_bytes(B, Hq, 1, 64) // 4, dtype=torch.float32,
                     device=DEV)
    cld, sd = cl.to(DEV), layer.sink.to(DEV)
    q0, k0, v0 = (layer.q[:, 0].to(DEV), layer.k_new[:, 0].to(DEV), layer.v_new[:, 0].to(DEV))
    kc, vc, kh, vh = _fp8_caches(layer, cl, kind, cap, Hkv)
    o = ops.decode_fp8(q0, k0, v0, kc, vc, cld, sd, kind, window, max_len, KS, VS,
                       rope=(base, 64) if rope else None, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    # oracle: (rotated) q and new token at bf16 over the dequantized history
    qo, ko = layer.q, layer.k_new
    if rope:
        qo = np.stack([oracle.rope_partial(layer.q[b], [int(cl[b])], base) for b in range(B)])
        ko = np.stack([oracle.rope_partial(layer.k_new[b], [int(cl[b])], base)
                       for b in range(B)])
    ref = oracle.decode_or_verify(qo, kh, vh, ko, layer.v_new, cl, layer.sink, window)[0]
    assert_close(o[:, None], ref, torch.bfloat16, "fp8 decode")
    kc, vc = kc.cpu(), vc.cpu()
    if not rope:  # the stored token: the oracle's codes of k_new / v_new
        for b, L in enumerate(cl.tolist()):
            slot = L % cap if kind == ops.RING else L
            assert torch.equal(kc[b, :, slot], _codes(layer.k_new[b, 0], KS))
            assert torch.equal(vc[b, :, slot], _codes(layer.v_new[b, 0], VS))
    else:  # fused RoPE == rope_partial then the un-fused E4M3 decode, bit for bit
        kc2, vc2, _, _ = _fp8_caches(layer, cl, kind, cap, Hkv)
        pos = cl.to(DEV)
        qr, kr = q0.clone(), k0.clone()
        ops.rope_partial(qr, pos, base)
        ops.rope_partial(kr, pos, base)
        o2 = ops.decode_fp8(qr, kr, v0, kc2, vc2, cld, sd, kind, window, max_len, KS, VS,
                            num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(kc, kc2.cpu()) and torch.equal(vc, vc2.cpu())


@pytest.mark.parametrize("kind,Hq,Hkv,window,nq", [
    (ops.RING, 64, 8, 128, 4),
    (ops.RING, 16, 2, 128, 2),
    (ops.CONTIG, 64, 4, 0, 4),
    (ops.CONTIG, 64, 4, 0, 1),
])
def test_verify_fp8(kind, Hq, Hkv, window, nq):
    _print_case("verify fp8", kind, Hq, Hkv, window, nq)
    base = synth.BASE_SWA if window else synth.BASE_GA
    cl = torch.tensor([0, 3, 126, 127, 128, 500, 1999], dtype=torch.int32)
    layer = synth.cached_layer(synth.generator(1600 + nq), cl, nq, Hq, Hkv, window,
                               torch.bfloat16)
    if not window:
        layer.sink = torch.full((Hq,), sink_for_half_mass(1000), dtype=torch.float32)
    cap = 128 if kind == ops.RING else 2000
    B, max_len = len(cl), int(cl.max())
    ws = torch.empty(ops.decode_workspace_bytes(B, Hq, nq, 64) // 4, dtype=torch.float32,
                     device=DEV)
    kc, vc, kh, vh = _fp8_caches(layer, cl, kind, cap, Hkv)
    kc0, vc0 = kc.clone(), vc.clone()
    k_rot = torch.empty(B, nq, Hkv, 192, dtype=torch.bfloat16, device=DEV)
    o = ops.verify_fp8(layer.q.to(DEV), layer.k_new.to(DEV), layer.v_new.to(DEV), kc, vc,
                       cl.to(DEV), layer.sink.to(DEV), kind, window, max_len, KS, VS,
                       rope=(base, 64), k_rot=k_rot, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(kc, kc0) and torch.equal(vc, vc0), "verify must not write the caches"
    qo, ko = [], []
    for b in range(B):
        pos = int(cl[b]) + np.arange(nq)
        qo.append(oracle.rope_partial(layer.q[b], pos, base))
        ko.append(oracle.rope_partial(layer.k_new[b], pos, base))
    ref = oracle.decode_or_verify(np.stack(qo), kh, vh, np.stack(ko), layer.v_new, cl,
                                  layer.sink, window)[0]
    assert_close(o, ref, torch.bfloat16, "fp8 verify")
    # the rotated keys match the oracle's RoPE to within one bf16 rounding
    kr, ko = k_rot.float().cpu().double().numpy(), np.stack(ko)
    assert np.all(np.abs(kr - ko) <= 2.0 ** -8 * np.abs(ko) + 1e-4)
