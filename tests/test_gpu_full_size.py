"""The workloads at their full sizes, launched the way bench.py times them,
checked against the oracle on sampled outputs.

Inputs are drawn as bench.py draws them (seeded N(0,1) on the device, the same
seeds), and the same entry points run: the fused-RoPE prefills, the fused-RoPE
decode / verify with the automatic split-K and a workspace for 256 splits, the
E4M3 decode over caches filled by kv_append_fp8, and the backward.  A whole
32K-token layer is out of the oracle's reach in seconds, so it evaluates sampled
query rows (prefill), sequences (decode / verify) or gradient rows one by one,
each with every key it sees (MiMo-V2-Flash Technical Report, Section 2.2; RoPE
of Section 2.1 applied by the oracle to the raw rows).  Tolerance: bf16 inputs,
|d| <= 2e-2 + 1e-2 |oracle|.
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
RNG = np.random.default_rng(20260)  # extra sampled rows / sequences (seeded)
FP8_K_SCALE, FP8_V_SCALE = 0.011, 0.0073  # the per-tensor scales bench.py uses


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()
    yield
    torch.cuda.empty_cache()


def _print_case(*a):
    print("case:", *a, flush=True)


def _rot_close(got, ref):
    """Rotated rows: the kernels round the fp32 rotation once to bf16."""
    g = to64(got)
    assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)


def _prefill_inputs(w):
    q = synth.device_normal(w.seed, (w.B, w.T, w.Hq, 192), device=DEV)
    k = synth.device_normal(w.seed + 1, (w.B, w.T, w.Hkv, 192), device=DEV)
    v = synth.device_normal(w.seed + 2, (w.B, w.T, w.Hkv, 128), device=DEV)
    sink = synth.device_normal(w.seed + 3, (w.Hq,), torch.float32, device=DEV)
    return q, k, v, sink


def test_full_swa_prefill_rope():
    """T = 32768, 64 Q / 8 KV heads, W = 128, RoPE base 1e4 fused (the headline)."""
    w = synth.WORKLOADS[2]
    _print_case("full SWA prefill", w.name)
    q, k, v, sink = _prefill_inputs(w)
    o = torch.empty(w.B, w.T, w.Hq, 128, dtype=torch.bfloat16, device=DEV)
    k_rot = torch.empty_like(k)
    ops.prefill_swa_rope(q, k, v, sink, w.window, w.base, k_rot=k_rot, out=o)
    torch.cuda.synchronize()
    s = sink.cpu()
    rows = [0, 1, 31, 32, 127, 128, 129, 4095, 16384, 20001, w.T - 1]
    for t0 in rows + sorted(RNG.choice(w.T, 16, replace=False).tolist()):
        lo = max(0, t0 - w.window + 1)
        kp = np.arange(lo, t0 + 1)
        qr = oracle.rope_partial(q[0, t0:t0 + 1], [t0], w.base)
        kr = oracle.rope_partial(k[0, lo:t0 + 1], kp, w.base)
        ref, _ = oracle.sink_attention(qr, kr, v[0, lo:t0 + 1], [t0], kp, s, w.window)
        assert_close(o[0, t0:t0 + 1], ref, torch.bfloat16, "SWA row %d" % t0)
    rows = np.array([0, 1, 127, 20000, w.T - 1])
    _rot_close(k_rot[0, rows], oracle.rope_partial(k[0, rows], rows, w.base))


def test_full_global_prefill_rope():
    """T = 32768, 64 Q / 4 KV heads, causal over the whole context, RoPE base 5e6."""
    w = synth.WORKLOADS[3]
    _print_case("full global prefill", w.name)
    q, k, v, sink = _prefill_inputs(w)
    o = torch.empty(w.B, w.T, w.Hq, 128, dtype=torch.bfloat16, device=DEV)
    k_rot = torch.empty_like(k)
    ops.prefill_global_rope(q, k, v, sink, w.base, k_rot=k_rot, out=o)
    torch.cuda.synchronize()
    s = sink.cpu()
    kr_all = oracle.rope_partial(k[0], np.arange(w.T), w.base)
    v_all = v[0].cpu()
    rows = [0, 31, 1000, 16383, w.T - 1]
    for t0 in rows + sorted(RNG.choice(w.T, 6, replace=False).tolist()):
        qr = oracle.rope_partial(q[0, t0:t0 + 1], [t0], w.base)
        ref, _ = oracle.sink_attention(qr, kr_all[:t0 + 1], v_all[:t0 + 1], [t0],
                                       np.arange(t0 + 1), s, 0)
        assert_close(o[0, t0:t0 + 1], ref, torch.bfloat16, "global row %d" % t0)
    rows = np.array([0, 5, 30000, w.T - 1])
    _rot_close(k_rot[0, rows], kr_all[rows])


def _decode_setup(fp8: bool):
    """The hybrid-block decode step's global layer and first ring layer, drawn as
    bench.py draws them (batch 32, contexts from [16K, 128K])."""
    w = synth.WORKLOADS[4]
    B, Hq = w.B, 64
    cl = synth.cache_lengths(synth.generator(w.seed), B, 16384, 131072)
    cap = 131072 + 8
    cdt = torch.uint8 if fp8 else torch.bfloat16
    zeros1 = torch.zeros(1, dtype=torch.int32, device=DEV)

    def fill(kc, vc, seed, n_tok):
        Hkv = kc.shape[1]
        if not fp8:
            synth.device_normal(seed, None, device=DEV, out=kc[0, :, :n_tok])
            synth.device_normal(seed + 1, None, device=DEV, out=vc[0, :, :n_tok])
            return
        kk = synth.device_normal(seed, (1, n_tok, Hkv, 192), device=DEV)
        vv = synth.device_normal(seed + 1, (1, n_tok, Hkv, 128), device=DEV)
        ops.kv_append_fp8(kk, vv, kc, vc, zeros1, ops.CONTIG if n_tok > 128 else ops.RING,
                          k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)

    layers = {}
    s0 = w.seed * 100  # ring layer 0
    r = dict(q=synth.device_normal(s0, (B, Hq, 192), device=DEV),
             kn=synth.device_normal(s0 + 1, (B, 8, 192), device=DEV),
             vn=synth.device_normal(s0 + 2, (B, 8, 128), device=DEV),
             kc=torch.empty(B, 8, 128, 192, dtype=cdt, device=DEV),
             vc=torch.empty(B, 8, 128, 128, dtype=cdt, device=DEV),
             sink=synth.device_normal(s0 + 5, (Hq,), torch.float32, device=DEV))
    for b in range(B):
        fill(r["kc"][b:b + 1], r["vc"][b:b + 1], s0 + 3000 + 2 * b, 128)
    layers["ring"] = r
    s0 = w.seed * 100 + 90
    gl = dict(q=synth.device_normal(s0, (B, Hq, 192), device=DEV),
              kn=synth.device_normal(s0 + 1, (B, 4, 192), device=DEV),
              vn=synth.device_normal(s0 + 2, (B, 4, 128), device=DEV),
              kc=torch.empty(B, 4, cap, 192, dtype=cdt, device=DEV),
              vc=torch.empty(B, 4, cap, 128, dtype=cdt, device=DEV),
              sink=synth.device_normal(s0 + 5, (Hq,), torch.float32, device=DEV))
    for b in range(B):
        fill(gl["kc"][b:b + 1], gl["vc"][b:b + 1], s0 + 1000 + 2 * b, int(cl[b]))
    layers["global"] = gl
    return cl, layers


def _history(cache, b, positions, slots, scale):
    """Rows [n, Hkv, d] (fp64) of sequence b at the given cache slots."""
    x = cache[b][:, slots].permute(1, 0, 2)
    if scale is None:
        return to64(x)
    return oracle.fp8_dequantize(x.cpu().numpy(), scale)


@pytest.mark.parametrize("fp8", [False, True])
def test_full_hybrid_decode(fp8):
    """One decode step of the global layer (split-K, automatic) and of a ring
    layer at batch 32 over contexts from [16K, 128K], RoPE fused; bf16 or E4M3
    caches.  Sampled sequences: the shortest, the longest and three more."""
    _print_case("full hybrid decode", "e4m3" if fp8 else "bf16")
    cl, layers = _decode_setup(fp8)
    B, Hq = cl.shape[0], 64
    cl_d, max_len = cl.to(DEV), int(cl.max())
    ws = torch.empty(ops.decode_workspace_bytes(B, Hq, 1, 256) // 4, dtype=torch.float32,
                     device=DEV)
    outs = {}
    for name, (kind, window, base) in (("global", (ops.CONTIG, 0, synth.BASE_GA)),
                                       ("ring", (ops.RING, 128, synth.BASE_SWA))):
        L = layers[name]
        if fp8:
            outs[name] = ops.decode_fp8(L["q"], L["kn"], L["vn"], L["kc"], L["vc"], cl_d,
                                        L["sink"], kind, window, max_len, FP8_K_SCALE,
                                        FP8_V_SCALE, rope=(base, 64), num_splits=0,
                                        workspace=ws)
        else:
            outs[name] = ops.decode_rope(L["q"], L["kn"], L["vn"], L["kc"], L["vc"], cl_d,
                                         L["sink"], kind, window, max_len, base=base,
                                         num_splits=0, workspace=ws)
    torch.cuda.synchronize()
    ks = FP8_K_SCALE if fp8 else None
    vs = FP8_V_SCALE if fp8 else None
    for b in sorted({int(cl.argmin()), int(cl.argmax()), 3, 17, 30}):
        P = int(cl[b])
        for name, (window, base) in (("global", (0, synth.BASE_GA)),
                                     ("ring", (128, synth.BASE_SWA))):
            L = layers[name]
            pos = np.arange(P - 127, P) if window else np.arange(P)
            slots = torch.as_tensor(pos % 128 if window else pos, device=DEV)
            kh = _history(L["kc"], b, pos, slots, ks)
            vh = _history(L["vc"], b, pos, slots, vs)
            qr = oracle.rope_partial(L["q"][b:b + 1], [P], base)
            kr = oracle.rope_partial(L["kn"][b:b + 1], [P], base)
            ref, _ = oracle.sink_attention(qr, np.concatenate([kh, kr]),
                                           np.concatenate([vh, to64(L["vn"][b:b + 1])]),
                                           [P], np.append(pos, P), L["sink"].cpu(), window)
            assert_close(outs[name][b:b + 1], ref, torch.bfloat16,
                         "%s layer, sequence %d (context %d)" % (name, b, P))
            if not fp8:  # the new token, rotated, now sits at slot P (P % 128 on the ring)
                slot = P % 128 if window else P
                _rot_close(L["kc"][b, :, slot][None], kr)


def test_full_verify():
    """Speculative verify of 1 + 3 tokens at batch 64, context 16384: the SWA ring
    layer and the global layer, RoPE fused, rotated draft keys written out."""
    w = synth.WORKLOADS[5]
    B, nq, Hq, L = w.B, w.T, 64, 16384
    _print_case("full verify", w.name)
    cap = L + 8
    cl = torch.full((B,), L, dtype=torch.int32)
    cl_d = cl.to(DEV)
    s0 = w.seed * 100
    swa = dict(q=synth.device_normal(s0, (B, nq, Hq, 192), device=DEV),
               kn=synth.device_normal(s0 + 1, (B, nq, 8, 192), device=DEV),
               vn=synth.device_normal(s0 + 2, (B, nq, 8, 128), device=DEV),
               kc=synth.device_normal(s0 + 3, (B, 8, 128, 192), device=DEV),
               vc=synth.device_normal(s0 + 4, (B, 8, 128, 128), device=DEV),
               sink=synth.device_normal(s0 + 5, (Hq,), torch.float32, device=DEV))
    gl = dict(q=synth.device_normal(s0 + 10, (B, nq, Hq, 192), device=DEV),
              kn=synth.device_normal(s0 + 11, (B, nq, 4, 192), device=DEV),
              vn=synth.device_normal(s0 + 12, (B, nq, 4, 128), device=DEV),
              kc=torch.empty(B, 4, cap, 192, dtype=torch.bfloat16, device=DEV),
              vc=torch.empty(B, 4, cap, 128, dtype=torch.bfloat16, device=DEV),
              sink=synth.device_normal(s0 + 15, (Hq,), torch.float32, device=DEV))
    synth.device_normal(s0 + 13, None, device=DEV, out=gl["kc"][:, :, :L])
    synth.device_normal(s0 + 14, None, device=DEV, out=gl["vc"][:, :, :L])
    ws = torch.empty(ops.decode_workspace_bytes(B, Hq, nq, 256) // 4, dtype=torch.float32,
                     device=DEV)
    kr_s, kr_g = torch.empty_like(swa["kn"]), torch.empty_like(gl["kn"])
    o_s = ops.verify_rope(swa["q"], swa["kn"], swa["vn"], swa["kc"], swa["vc"], cl_d,
                          swa["sink"], ops.RING, 128, L, base=synth.BASE_SWA, k_rot=kr_s)
    o_g = ops.verify_rope(gl["q"], gl["kn"], gl["vn"], gl["kc"], gl["vc"], cl_d, gl["sink"],
                          ops.CONTIG, 0, L, base=synth.BASE_GA, k_rot=kr_g, num_splits=0,
                          workspace=ws)
    torch.cuda.synchronize()
    qpos = np.arange(L, L + nq)
    for b in (0, 17, 40, B - 1):
        for lay, o, kr_out, window, base in ((swa, o_s, kr_s, 128, synth.BASE_SWA),
                                             (gl, o_g, kr_g, 0, synth.BASE_GA)):
            pos = np.arange(L - 127, L) if window else np.arange(L)
            slots = torch.as_tensor(pos % 128 if window else pos, device=DEV)
            kh = _history(lay["kc"], b, pos, slots, None)
            vh = _history(lay["vc"], b, pos, slots, None)
            qr = oracle.rope_partial(lay["q"][b], qpos, base)
            kr = oracle.rope_partial(lay["kn"][b], qpos, base)
            ref, _ = oracle.sink_attention(qr, np.concatenate([kh, kr]),
                                           np.concatenate([vh, to64(lay["vn"][b])]), qpos,
                                           np.concatenate([pos, qpos]), lay["sink"].cpu(),
                                           window)
            assert_close(o[b], ref, torch.bfloat16, "verify, window %d, sequence %d" % (window, b))
            _rot_close(kr_out[b], kr)


def test_full_global_backward_sampled():
    """Backward of the T = 32768 global layer (64 / 4 heads): dq of sampled query
    rows against the oracle over every key they see, and dsink against
    -sum_i e^(sink - lse_i) (dO_i . o_i) in fp64 from the forward outputs."""
    w = synth.WORKLOADS[3]
    _print_case("full global backward", w.name)
    q, k, v, sink = _prefill_inputs(w)
    dout = synth.device_normal(w.seed + 4, (w.B, w.T, w.Hq, 128), device=DEV)
    o, lse = ops.prefill_global(q, k, v, sink, return_lse=True)
    dq, dk, dv, dsink = ops.backward(q, k, v, o, dout, lse, sink, 0)
    torch.cuda.synchronize()
    del dk, dv
    s = sink.cpu()
    k_all, v_all = k[0].cpu(), v[0].cpu()
    for t0 in (0, 77, 9000, 24575, w.T - 1):
        rq, _, _, _ = oracle.sink_attention_bwd(q[0, t0:t0 + 1], k_all[:t0 + 1], v_all[:t0 + 1],
                                                [t0], np.arange(t0 + 1), s,
                                                dout[0, t0:t0 + 1], 0)
        assert_close(dq[0, t0:t0 + 1], rq, torch.bfloat16, "dq row %d" % t0)
    D = (to64(dout[0]) * to64(o[0])).sum(-1)                       # [T, Hq]
    ps = np.exp(s.double().numpy()[None, :] - to64(lse[0]).T)       # [T, Hq]
    assert_close(dsink, -(ps * D).sum(0), torch.bfloat16, "dsink full global layer")
