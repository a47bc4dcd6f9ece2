"""Partial RoPE fused into the global prefill, decode and verify kernels.

Each fused entry point must equal, bit for bit, the unfused sequence it
replaces (sinkattn_rope_partial on q and k / k_new at their positions, then the
plain entry point): same outputs, same cache contents, same rotated keys.  Each
is also compared with the oracle (fp64 RoPE, then fp64 attention) at the bf16
tolerance.  Positions are those of the MiMo-V2-Flash report, Section 2.1
(RoPE on the first 64 of 192 dims) with the Section 3.2 bases (1e4 for SWA
layers, 5e6 for global layers).
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
BASE_SWA, BASE_GLOBAL = 1e4, 5e6


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()


def _print_case(*a):
    print("case:", *a, flush=True)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


# ----------------------------------------------------------------------------- prefill

@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 300, 32, 2), (2, 97, 16, 1)])
def test_prefill_global_rope_fused(B, T, Hq, Hkv):
    _print_case("prefill global rope fused", B, T, Hq, Hkv)
    q, k, v, sink = synth.prefill_inputs(700 + T, B, T, Hq, Hkv, torch.bfloat16)
    qd, kd, vd, sd = (t.to(DEV) for t in (q, k, v, sink))
    o_f, lse_f, k_rot = ops.prefill_global_rope(qd, kd, vd, sd, BASE_GLOBAL, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k), "inputs must stay untouched"
    pos = synth.positions(B, T).to(DEV)
    qr, kr = qd.clone(), kd.clone()
    ops.rope_partial(qr, pos, BASE_GLOBAL)
    ops.rope_partial(kr, pos, BASE_GLOBAL)
    o_u, lse_u = ops.prefill_global(qr, kr, vd, sd, return_lse=True)
    assert torch.equal(_bits(k_rot), _bits(kr))
    assert torch.equal(_bits(o_f), _bits(o_u)) and torch.equal(lse_f, lse_u)
    qo = np.stack([oracle.rope_partial(q[b], np.arange(T), BASE_GLOBAL) for b in range(B)])
    ko = np.stack([oracle.rope_partial(k[b], np.arange(T), BASE_GLOBAL) for b in range(B)])
    ref_o, _ = oracle.prefill(qo, ko, v, sink, 0)
    assert_close(o_f, ref_o, torch.bfloat16, "fused rope global prefill")


# ----------------------------------------------------------------------------- decode / verify

def _fill(layer, cl, kind, cap, Hkv):
    fill = synth.fill_ring if kind == ops.RING else synth.fill_contig
    kc, vc = fill(layer, cl, cap, Hkv)
    return kc.to(DEV), vc.to(DEV)


def _rotated_new(layer, cl, base):
    """Unfused reference inputs: q and k_new rotated on the GPU at L_b + t."""
    B, nq = layer.q.shape[:2]
    pos = (cl.view(B, 1) + torch.arange(nq, dtype=torch.int32).view(1, nq)).reshape(-1)
    pos = pos.to(torch.int32).to(DEV)
    qr = layer.q.to(DEV).clone()
    kr = layer.k_new.to(DEV).clone()
    ops.rope_partial(qr.view(B * nq, *qr.shape[2:]), pos, base)
    ops.rope_partial(kr.view(B * nq, *kr.shape[2:]), pos, base)
    return qr, kr


def _oracle_rotated(layer, cl, base, window):
    B, nq = layer.q.shape[:2]
    qo, ko = [], []
    for b in range(B):
        p = int(cl[b]) + np.arange(nq)
        qo.append(oracle.rope_partial(layer.q[b], p, base))
        ko.append(oracle.rope_partial(layer.k_new[b], p, base))
    return oracle.decode_or_verify(np.stack(qo), layer.k_hist, layer.v_hist, np.stack(ko),
                                   layer.v_new, cl, layer.sink, window)[0]


@pytest.mark.parametrize("kind,Hq,Hkv,window,splits", [
    (ops.RING, 64, 8, 128, 0),       # SWA layer: 8 heads per KV head (16-column kernel)
    (ops.CONTIG, 64, 4, 0, 0),       # global layer, automatic split-K
    (ops.CONTIG, 64, 4, 0, 1),       # global layer, one chunk
])
def test_decode_rope_fused(kind, Hq, Hkv, window, splits):
    _print_case("decode rope fused", kind, Hq, Hkv, window, splits)
    base = BASE_SWA if window else BASE_GLOBAL
    cl = torch.tensor([0, 1, 31, 127, 128, 700, 2049], dtype=torch.int32)
    layer = synth.cached_layer(synth.generator(1200 + Hkv), cl, 1, Hq, Hkv, window,
                               torch.bfloat16)
    if not window:
        layer.sink = torch.full((Hq,), sink_for_half_mass(1000), dtype=torch.float32)
    cap = 128 if kind == ops.RING else 2100
    max_len = int(cl.max())
    B = len(cl)
    ws = None
    if kind == ops.CONTIG:
        ws = torch.empty(ops.decode_workspace_bytes(B, Hq, 1, 64) // 4, dtype=torch.float32,
                         device=DEV)
    cld, sd = cl.to(DEV), layer.sink.to(DEV)
    q0, k0, v0 = (layer.q[:, 0].to(DEV), layer.k_new[:, 0].to(DEV), layer.v_new[:, 0].to(DEV))

    kc_f, vc_f = _fill(layer, cl, kind, cap, Hkv)
    o_f = ops.decode_rope(q0, k0, v0, kc_f, vc_f, cld, sd, kind, window, max_len,
                          base=base, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(q0.cpu(), layer.q[:, 0]) and torch.equal(k0.cpu(), layer.k_new[:, 0])

    qr, kr = _rotated_new(layer, cl, base)
    kc_u, vc_u = _fill(layer, cl, kind, cap, Hkv)
    o_u = ops.decode(qr[:, 0].contiguous(), kr[:, 0].contiguous(), v0, kc_u, vc_u, cld, sd, kind,
                     window, max_len, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o_f), _bits(o_u))
    assert torch.equal(_bits(kc_f), _bits(kc_u)) and torch.equal(_bits(vc_f), _bits(vc_u))
    ref = _oracle_rotated(layer, cl, base, window)
    assert_close(o_f[:, None], ref, torch.bfloat16, "fused rope decode")


@pytest.mark.parametrize("kind,Hq,Hkv,window,nq", [
    (ops.RING, 64, 8, 128, 4),       # SWA verify: 32 columns
    (ops.RING, 16, 2, 128, 2),       # 16 columns (16-column kernel)
    (ops.CONTIG, 64, 4, 0, 4),       # global verify: 64 columns, split-K
    (ops.CONTIG, 64, 4, 0, 1),
])
def test_verify_rope_fused(kind, Hq, Hkv, window, nq):
    _print_case("verify rope fused", kind, Hq, Hkv, window, nq)
    base = BASE_SWA if window else BASE_GLOBAL
    cl = torch.tensor([0, 3, 126, 127, 128, 500, 1999], dtype=torch.int32)
    layer = synth.cached_layer(synth.generator(1300 + nq), cl, nq, Hq, Hkv, window,
                               torch.bfloat16)
    if not window:
        layer.sink = torch.full((Hq,), sink_for_half_mass(1000), dtype=torch.float32)
    cap = 128 if kind == ops.RING else 2000
    max_len = int(cl.max())
    B = len(cl)
    ws = None
    if kind == ops.CONTIG:
        ws = torch.empty(ops.decode_workspace_bytes(B, Hq, nq, 64) // 4, dtype=torch.float32,
                         device=DEV)
    cld, sd = cl.to(DEV), layer.sink.to(DEV)
    qd, kd, vd = layer.q.to(DEV), layer.k_new.to(DEV), layer.v_new.to(DEV)
    kc, vc = _fill(layer, cl, kind, cap, Hkv)
    kc0, vc0 = kc.clone(), vc.clone()
    k_rot = torch.empty_like(kd)
    o_f = ops.verify_rope(qd, kd, vd, kc, vc, cld, sd, kind, window, max_len, base=base,
                          k_rot=k_rot, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kc), _bits(kc0)) and torch.equal(_bits(vc), _bits(vc0)), \
        "verify must not write the caches"
    assert torch.equal(qd.cpu(), layer.q) and torch.equal(kd.cpu(), layer.k_new)
    qr, kr = _rotated_new(layer, cl, base)
    o_u = ops.verify(qr, kr, vd, kc, vc, cld, sd, kind, window, max_len, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(k_rot), _bits(kr))
    assert torch.equal(_bits(o_f), _bits(o_u))
    ref = _oracle_rotated(layer, cl, base, window)
    assert_close(o_f, ref, torch.bfloat16, "fused rope verify")
