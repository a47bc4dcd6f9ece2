"""sinkattn_decode_noalloc: the decode step whose split-K scratch is the
library's fixed device array (for callers that cannot allocate), called through
the C ABI and compared bit for bit with sinkattn_decode given a caller
workspace of the same size, on two calls in a row, the second smaller (the
scratch still holds the first call's partial results), and against the oracle
(MiMo-V2-Flash Technical Report, Section 2.2 sink softmax; Section 2.3.1 one
new token per step over a per-request cache)."""
from __future__ import annotations

import pytest
import torch

import oracle
from gpu_helpers import assert_close, sink_for_half_mass
from sliding_window_sink_amd import ops, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    ops.lib()


def _call_pair(seed, lens, Hq, Hkv, cap, splits):
    print("case: noalloc decode", seed, lens, splits, flush=True)
    cl = torch.tensor(lens, dtype=torch.int32)
    layer = synth.cached_layer(synth.generator(seed), cl, 1, Hq, Hkv, 0, torch.bfloat16)
    layer.sink = torch.full((Hq,), sink_for_half_mass(max(lens) // 2), dtype=torch.float32)
    kc0, vc0 = synth.fill_contig(layer, cl, cap, Hkv)
    q, kn, vn = (layer.q[:, 0].to(DEV), layer.k_new[:, 0].to(DEV), layer.v_new[:, 0].to(DEV))
    sink, cld = layer.sink.to(DEV), cl.to(DEV)
    B = len(lens)
    # reference: the allocating entry point with a workspace as large as the scratch
    ws = torch.empty(ops.STATIC_SCRATCH_BYTES // 4, dtype=torch.float32, device=DEV)
    kc_r, vc_r = kc0.to(DEV), vc0.to(DEV)
    o_ref = ops.decode(q, kn, vn, kc_r, vc_r, cld, sink, ops.CONTIG, 0, max(lens),
                       num_splits=splits, workspace=ws)
    kc_n, vc_n = kc0.to(DEV), vc0.to(DEV)
    o_got = torch.full((B, Hq, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    ops.decode_noalloc(q, kn, vn, kc_n, vc_n, cld, sink, ops.CONTIG, 0, max(lens),
                       num_splits=splits, out=o_got)
    torch.cuda.synchronize()
    assert torch.equal(o_got, o_ref), "noalloc decode differs from decode with a workspace"
    # bitwise (the unused cache tails hold NaN)
    assert torch.equal(kc_n.view(torch.int16), kc_r.view(torch.int16)) and \
        torch.equal(vc_n.view(torch.int16), vc_r.view(torch.int16)), "caches differ"
    ref = oracle.decode_or_verify(layer.q, layer.k_hist, layer.v_hist, layer.k_new, layer.v_new,
                                  cl, layer.sink, 0)[0]
    assert_close(o_got[:, None], ref, torch.bfloat16, "noalloc decode vs oracle")


def test_noalloc_decode_two_calls():
    # first call: 8 long contexts, automatic split count (several splits)
    _call_pair(1201, [20000, 17, 9000, 19999, 4096, 1, 12000, 300], 64, 4, 20008, 0)
    # second call, smaller: 3 sequences, an explicit split count
    _call_pair(1202, [100, 5000, 2500], 64, 4, 5008, 5)


def test_noalloc_rejects_oversized_split():
    B, Hq = 64, 64
    per_split = ops.decode_workspace_bytes(B, Hq, 1, 2) // 2
    too_many = ops.STATIC_SCRATCH_BYTES // per_split + 1
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=DEV)
    with pytest.raises(ops.SinkAttnError) as e:
        ops.decode_noalloc(z(B, Hq, 192), z(B, 4, 192), z(B, 4, 128), z(B, 4, 300, 192),
                           z(B, 4, 300, 128), z(B, dt=torch.int32), z(Hq, dt=torch.float32),
                           ops.CONTIG, 0, 200, num_splits=too_many)
    assert e.value.code == -5
