"""The self-speculative decoding loop at kernel level (MiMo-V2-Flash report,
Section 2.3.1 and Section 5: the main model verifies 1 + K draft tokens in one
pass; accepted tokens join the context).

Several iterations of, all stream-ordered on the device:
  verify_rope on an SWA ring layer and on a global contiguous layer (un-rotated
  q / k_new at positions L_b + t)  ->  a seeded acceptance count n_b in
  [1, nq]  ->  kv_append of the rotated keys (k_rot) and the values  ->
  advance_len.
Every verify output is compared with the oracle over a history the test keeps
itself (fp64 RoPE, accepted tokens appended); at the end the cached lengths and
every cache row must be exactly what the commits imply.
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


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()


def _bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("nq", [4, 2])
def test_speculative_loop(nq):
    print("case: speculative loop nq", nq, flush=True)
    g = synth.generator(4242 + nq)
    rng = np.random.default_rng(99 + nq)
    B, Hq, W, iters = 4, 16, 128, 6
    layers = {  # name: (kind, Hkv, window, base)
        "swa": (ops.RING, 2, W, synth.BASE_SWA),
        "ga": (ops.CONTIG, 1, 0, synth.BASE_GA),
    }
    L = [0, 5, 127, 300]
    cap_c = max(L) + nq * iters + 8
    st = {}
    for name, (kind, Hkv, window, base) in layers.items():
        cap = W if kind == ops.RING else cap_c
        kc = torch.zeros(B, Hkv, cap, 192, dtype=torch.bfloat16)
        vc = torch.zeros(B, Hkv, cap, 128, dtype=torch.bfloat16)
        hk, hv, bits = [], [], []
        for b in range(B):
            k = synth.normal(g, (L[b], Hkv, 192))
            v = synth.normal(g, (L[b], Hkv, 128))
            hk.append(k.double().numpy())
            hv.append(v.double().numpy())
            bits.append({p: k[p] for p in range(L[b])})
            for p in range(L[b]):
                slot = p % cap if kind == ops.RING else p
                kc[b, :, slot] = k[p]
                vc[b, :, slot] = v[p]
        sink = torch.linspace(-1.0, 3.0, Hq, dtype=torch.float32)
        st[name] = dict(kc=kc.to(DEV), vc=vc.to(DEV), hk=hk, hv=hv, bits=bits, cap=cap,
                        sink=sink, sink_d=sink.to(DEV))
    cl_d = torch.tensor(L, dtype=torch.int32, device=DEV)
    ws = torch.empty(ops.decode_workspace_bytes(B, Hq, nq, 16) // 4, dtype=torch.float32,
                     device=DEV)
    max_len = max(L)
    for it in range(iters):
        n_acc = rng.integers(1, nq + 1, size=B).astype(np.int32)
        n_acc_d = torch.from_numpy(n_acc).to(DEV)
        for name, (kind, Hkv, window, base) in layers.items():
            s = st[name]
            q = synth.normal(g, (B, nq, Hq, 192))
            kn = synth.normal(g, (B, nq, Hkv, 192))
            vn = synth.normal(g, (B, nq, Hkv, 128))
            k_rot = torch.empty(B, nq, Hkv, 192, dtype=torch.bfloat16, device=DEV)
            o = ops.verify_rope(q.to(DEV), kn.to(DEV), vn.to(DEV), s["kc"], s["vc"], cl_d,
                                s["sink_d"], kind, window, max_len, base=base, k_rot=k_rot,
                                workspace=ws if kind == ops.CONTIG else None)
            ops.kv_append(k_rot, vn.to(DEV), s["kc"], s["vc"], cl_d, kind, n_acc_d)
            # oracle over its own history
            qo, ko = [], []
            for b in range(B):
                pos = L[b] + np.arange(nq)
                qo.append(oracle.rope_partial(q[b], pos, base))
                ko.append(oracle.rope_partial(kn[b], pos, base))
            ref = oracle.decode_or_verify(np.stack(qo), s["hk"], s["hv"], np.stack(ko), vn,
                                          np.array(L), s["sink"], window)[0]
            assert_close(o, ref, torch.bfloat16, "verify %s iteration %d" % (name, it))
            kr = k_rot.cpu()
            for b in range(B):
                a = int(n_acc[b])
                s["hk"][b] = np.concatenate([s["hk"][b], ko[b][:a]], 0)
                s["hv"][b] = np.concatenate([s["hv"][b], vn[b, :a].double().numpy()], 0)
                for t in range(a):
                    s["bits"][b][L[b] + t] = kr[b, t]
        ops.advance_len(cl_d, nq, n_acc_d)
        for b in range(B):
            L[b] += int(n_acc[b])
        max_len += nq
    torch.cuda.synchronize()
    assert cl_d.cpu().tolist() == L
    for name, (kind, Hkv, window, base) in layers.items():
        s = st[name]
        kc, cap = s["kc"].cpu(), s["cap"]
        for b in range(B):
            lo = max(0, L[b] - cap) if kind == ops.RING else 0
            for p in range(lo, L[b]):
                slot = p % cap if kind == ops.RING else p
                assert torch.equal(_bits(kc[b, :, slot]), _bits(s["bits"][b][p])), (name, b, p)
