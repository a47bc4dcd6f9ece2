"""HIP path vs the CPU oracle, element by element, on seeded inputs.

Sizes span several tiles (32 query tokens, 32 keys) with ragged tails.  Every
call goes through the C ABI (ctypes binding).  Tolerances: fp32 max|d| <= 1e-4;
bf16 |d| <= 2e-2 + 1e-2 |oracle|; RoPE within one bf16 ulp.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_close, sink_for_half_mass, to64
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


# ----------------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("style", [0, 1])
def test_rope_partial(dtype, style):
    _print_case("rope", dtype, style)
    g = synth.generator(11)
    n_tok, H = 300, 5
    x = synth.normal(g, (n_tok, H, 192), dtype)
    pos = torch.randint(0, 262144, (n_tok,), generator=g, dtype=torch.int64)
    pos[:4] = torch.tensor([0, 1, 131071, 262143])
    for base in (1e4, 5e6):
        xd = x.to(DEV)
        ops.rope_partial(xd, pos.to(torch.int32).to(DEV), base, 64, style)
        got = xd.cpu()
        ref = oracle.rope_partial(x, pos.numpy(), base, 64, style)
        assert torch.equal(got[..., 64:], x[..., 64:]), "dims >= 64 must be untouched"
        if dtype == torch.bfloat16:
            ref_bits = oracle.round_bf16_bits(ref)
            got_bits = got.view(torch.int16).numpy().view(np.uint16)
            # one ulp: compare as monotone integers
            def key(b):
                b = b.astype(np.int32)
                return np.where(b & 0x8000, -(b & 0x7FFF), b)
            diff = np.abs(key(got_bits) - key(ref_bits))
            assert diff.max() <= 1, "RoPE differs by %d bf16 ulps" % diff.max()
            assert (diff == 0).mean() > 0.99
        else:
            err = np.abs(got.double().numpy() - ref).max()
            assert err < 2e-6, err


# ----------------------------------------------------------------------------- prefill

def _prefill_case(B, T, Hq, Hkv, dtype, window, seed, sink_override=None, scale=None):
    q, k, v, sink = synth.prefill_inputs(seed, B, T, Hq, Hkv, dtype)
    if sink_override is not None:
        sink = torch.as_tensor(sink_override, dtype=torch.float32).expand(Hq).contiguous()
    fn = (lambda *a, **kw: ops.prefill_swa(*a, window=window, **kw)) if window > 0 else \
        ops.prefill_global
    o, lse = fn(q.to(DEV), k.to(DEV), v.to(DEV), sink.to(DEV), scale=scale, return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.prefill(q, k, v, sink, window, scale)
    return o, lse, ref_o, ref_lse, (q, k, v, sink)


PREFILL_CASES = [
    # B, T, Hq, Hkv, window
    (1, 300, 8, 1, 128),       # SWA: ragged tail, several tiles
    (2, 161, 16, 2, 128),      # two sequences, two KV groups
    (1, 257, 16, 1, 1),        # W = 1: only the query itself
    (1, 200, 8, 1, 33),        # window not a multiple of the tile
    (1, 700, 8, 1, 512),       # W = 512 (the report's Table 2 ablation width)
    (1, 230, 16, 1, 0),        # global, group of 16 (two workgroups per tile)
    (2, 97, 32, 2, 0),         # global, two sequences
    (1, 1, 8, 1, 128),         # a single token
]


@pytest.mark.parametrize("B,T,Hq,Hkv,window", PREFILL_CASES)
def test_prefill_bf16(B, T, Hq, Hkv, window):
    _print_case("prefill bf16", B, T, Hq, Hkv, window)
    o, lse, ref_o, ref_lse, _ = _prefill_case(B, T, Hq, Hkv, torch.bfloat16, window, 100 + T)
    assert_close(o, ref_o, torch.bfloat16, "o")
    assert_close(lse.permute(0, 2, 1), ref_lse, torch.bfloat16, "lse")


@pytest.mark.parametrize("B,T,Hq,Hkv,window", [(1, 300, 8, 1, 128), (1, 150, 16, 2, 0),
                                                (2, 70, 4, 2, 5)])
def test_prefill_f32(B, T, Hq, Hkv, window):
    _print_case("prefill f32", B, T, Hq, Hkv, window)
    o, lse, ref_o, ref_lse, _ = _prefill_case(B, T, Hq, Hkv, torch.float32, window, 200 + T)
    assert_close(o, ref_o, torch.float32, "o")
    assert_close(lse.permute(0, 2, 1), ref_lse, torch.float32, "lse")


@pytest.mark.parametrize("sink_val", [8.0, -math.inf, 1e3, -30.0])
@pytest.mark.parametrize("window", [128, 0])
def test_prefill_sink_stress(sink_val, window):
    """Sinks that dominate (+8, 1e3), vanish (-inf) or are negligible: only these
    make a dropped or double-counted sink visible at bf16 tolerance."""
    _print_case("prefill sink stress", sink_val, window)
    o, lse, ref_o, ref_lse, _ = _prefill_case(1, 260, 8, 1, torch.bfloat16, window, 300,
                                              sink_override=sink_val)
    assert_close(o, ref_o, torch.bfloat16, "o")
    if sink_val == 1e3:
        assert torch.count_nonzero(o) == 0
    if sink_val != -math.inf:
        assert_close(lse.permute(0, 2, 1), ref_lse, torch.bfloat16, "lse")


@pytest.mark.parametrize("T,Hq,Hkv,window", [(300, 16, 2, 128), (777, 8, 1, 128),
                                              (100, 16, 1, 1), (64, 8, 1, 129)])
def test_prefill_swa_rope_fused(T, Hq, Hkv, window):
    """Fused RoPE + SWA prefill equals rope_partial(q), rope_partial(k), then
    prefill_swa, bit for bit; the rotated k it writes equals rope_partial(k);
    and it matches the oracle on oracle-rotated inputs."""
    _print_case("prefill swa rope fused", T, Hq, Hkv, window)
    q, k, v, sink = synth.prefill_inputs(400 + T, 1, T, Hq, Hkv, torch.bfloat16)
    qd, kd, vd, sd = (t.to(DEV) for t in (q, k, v, sink))
    k_rot = torch.empty_like(kd)
    o_f, lse_f = ops.prefill_swa_rope(qd, kd, vd, sd, window, 1e4, k_rot=k_rot, return_lse=True)
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k), "inputs must stay untouched"
    pos = synth.positions(1, T).to(DEV)
    qr, kr = qd.clone(), kd.clone()
    ops.rope_partial(qr, pos, 1e4)
    ops.rope_partial(kr, pos, 1e4)
    o_u, lse_u = ops.prefill_swa(qr, kr, vd, sd, window=window, return_lse=True)
    assert torch.equal(k_rot, kr)
    assert torch.equal(o_f, o_u) and torch.equal(lse_f, lse_u)
    qo = oracle.rope_partial(q[0], np.arange(T), 1e4)[None]
    ko = oracle.rope_partial(k[0], np.arange(T), 1e4)[None]
    ref_o, _ = oracle.prefill(qo, ko, v, sink, window)
    assert_close(o_f, ref_o, torch.bfloat16, "fused rope prefill")


def test_prefill_zero_query_closed_form():
    """q = 0 makes every visible weight 1/(e^sink + |J|): a wrong window count
    or KV group shows up even in bf16."""
    _print_case("prefill q=0")
    T, Hq, Hkv, W = 200, 16, 2, 40
    q = torch.zeros(1, T, Hq, 192, dtype=torch.bfloat16)
    g = synth.generator(5)
    k = synth.normal(g, (1, T, Hkv, 192))
    j = torch.arange(T, dtype=torch.float64).view(1, T, 1, 1)
    gg = torch.arange(Hkv, dtype=torch.float64).view(1, 1, Hkv, 1)
    v = ((j % 50) * 0.02 + gg * 0.5).expand(1, T, Hkv, 128).to(torch.bfloat16).contiguous()
    sink = torch.linspace(-1, 2, Hq, dtype=torch.float32)
    o = ops.prefill_swa(q.to(DEV), k.to(DEV), v.to(DEV), sink.to(DEV), window=W)
    vv = v.double().numpy()[0]
    ref = np.zeros((T, Hq, 128))
    for i in range(T):
        lo = max(0, i - W + 1)
        for h in range(Hq):
            ref[i, h] = vv[lo:i + 1, h // (Hq // Hkv)].sum(0) / (math.exp(sink[h]) + i - lo + 1)
    assert_close(o[0], ref, torch.bfloat16, "q=0 closed form")


def test_swa_wide_window_equals_global():
    _print_case("W >= T == global")
    q, k, v, sink = synth.prefill_inputs(9, 1, 180, 16, 2, torch.bfloat16)
    args = [t.to(DEV) for t in (q, k, v, sink)]
    a = ops.prefill_swa(*args, window=180)
    b = ops.prefill_global(*args)
    c = ops.prefill_swa(*args, window=4096)
    assert torch.equal(a, b) and torch.equal(a, c)


def test_prefill_deterministic():
    _print_case("prefill determinism")
    q, k, v, sink = synth.prefill_inputs(10, 1, 333, 8, 1, torch.bfloat16)
    args = [t.to(DEV) for t in (q, k, v, sink)]
    a = ops.prefill_swa(*args, window=128)
    b = ops.prefill_swa(*args, window=128)
    assert torch.equal(a, b)


def test_prefill_config1_fp32_full():
    """The tiny fp32 workload in full: B=1, T=1024, 8 Q / 1 KV heads, W=128,
    partial RoPE (base 1e4) on q and k first, all through the C ABI."""
    _print_case("config1 full")
    w = synth.WORKLOADS[1]
    q, k, v, sink = synth.prefill_inputs(w.seed, w.B, w.T, w.Hq, w.Hkv, w.dtype)
    pos = synth.positions(w.B, w.T)
    qd, kd = q.to(DEV), k.to(DEV)
    ops.rope_partial(qd, pos.to(DEV), w.base)
    ops.rope_partial(kd, pos.to(DEV), w.base)
    o = ops.prefill_swa(qd, kd, v.to(DEV), sink.to(DEV), window=w.window)
    qr = oracle.rope_partial(q[0], pos.numpy(), w.base)[None]
    kr = oracle.rope_partial(k[0], pos.numpy(), w.base)[None]
    ref_o, _ = oracle.prefill(qr, kr, v, sink, w.window)
    err = assert_close(o, ref_o, torch.float32, "config 1")
    print("config 1 max|d| =", err)


# ----------------------------------------------------------------------------- decode / verify

def _layer(seed, cache_len, nq, Hq, Hkv, window, dtype=torch.bfloat16, sinks=None):
    g = synth.generator(seed)
    layer = synth.cached_layer(g, cache_len, nq, Hq, Hkv, window, dtype)
    if sinks is not None:
        layer.sink = torch.as_tensor(sinks, dtype=torch.float32).expand(Hq).contiguous()
    return layer


def _run_cached(layer, cache_len, kind, window, cap, Hkv, verify, num_splits=0, ws_splits=0,
                max_len=None):
    fill = synth.fill_ring if kind == ops.RING else synth.fill_contig
    kc, vc = fill(layer, cache_len, cap, Hkv)
    kc, vc = kc.to(DEV), vc.to(DEV)
    max_len = int(cache_len.max()) if max_len is None else max_len
    B, nq, Hq = layer.q.shape[:3]
    ws = None
    if ws_splits:
        nbytes = ops.decode_workspace_bytes(B, Hq, nq, ws_splits)
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    if verify:
        o = ops.verify(layer.q.to(DEV), layer.k_new.to(DEV), layer.v_new.to(DEV), kc, vc,
                       cache_len.to(DEV), layer.sink.to(DEV), kind, window, max_len, num_splits,
                       ws)
    else:
        o = ops.decode(layer.q[:, 0].to(DEV), layer.k_new[:, 0].to(DEV), layer.v_new[:, 0].to(DEV),
                       kc, vc, cache_len.to(DEV), layer.sink.to(DEV), kind, window, max_len,
                       num_splits, ws)
        o = o[:, None]
    torch.cuda.synchronize()
    return o, kc, vc


def _ref_cached(layer, cache_len, window):
    return oracle.decode_or_verify(layer.q, layer.k_hist, layer.v_hist, layer.k_new, layer.v_new,
                                   cache_len, layer.sink, window)[0]


RING_LENS = [0, 1, 5, 126, 127, 128, 129, 1000, 5000]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Hq,Hkv", [(64, 8), (16, 2)])
def test_decode_ring(dtype, Hq, Hkv):
    _print_case("decode ring", dtype, Hq, Hkv)
    cl = torch.tensor(RING_LENS, dtype=torch.int32)
    layer = _layer(21, cl, 1, Hq, Hkv, 128, dtype)
    o, kc, vc = _run_cached(layer, cl, ops.RING, 128, 128, Hkv, verify=False)
    assert_close(o, _ref_cached(layer, cl, 128), dtype, "ring decode")
    # the new token now sits in slot P % 128 (bit-exact copy)
    kc, vc = kc.cpu(), vc.cpu()
    for b, L in enumerate(RING_LENS):
        assert torch.equal(kc[b, :, L % 128], layer.k_new[b, 0])
        assert torch.equal(vc[b, :, L % 128], layer.v_new[b, 0])


@pytest.mark.parametrize("window", [100, 1])
def test_decode_ring_window_below_capacity(window):
    """A 128-slot ring under a narrower window: the one-token kernel reads every
    slot, so the slots behind the window (stale rows; here the oldest history row
    and NaN-poisoned slots never written) must stay out of the output."""
    _print_case("decode ring window below capacity", window)
    lens = [0, 1, window - 1, window, window + 1, 127, 128, 129, 1000]
    cl = torch.tensor(lens, dtype=torch.int32)
    layer = _layer(27 + window, cl, 1, 64, 8, window)
    o, kc, vc = _run_cached(layer, cl, ops.RING, window, 128, 8, verify=False)
    assert_close(o, _ref_cached(layer, cl, window), torch.bfloat16, "ring decode W < cap")
    kc = kc.cpu()
    for b, L in enumerate(lens):
        assert torch.equal(kc[b, :, L % 128], layer.k_new[b, 0])


def test_decode_ring_wide_window():
    """W = 512 (the width of the report's window-size ablation, Table 2) as a runtime
    parameter of the ring decode: up to 512 visible keys (the query included) over
    16 key blocks plus the new token."""
    _print_case("decode ring W512")
    lens = [0, 1, 300, 511, 512, 513, 3000]
    cl = torch.tensor(lens, dtype=torch.int32)
    layer = _layer(22, cl, 1, 16, 2, 512, torch.bfloat16)
    o, kc, vc = _run_cached(layer, cl, ops.RING, 512, 512, 2, verify=False)
    assert_close(o, _ref_cached(layer, cl, 512), torch.bfloat16, "ring decode W512")
    kc, vc = kc.cpu(), vc.cpu()
    for b, L in enumerate(lens):
        assert torch.equal(kc[b, :, L % 512], layer.k_new[b, 0])
        assert torch.equal(vc[b, :, L % 512], layer.v_new[b, 0])


@pytest.mark.parametrize("splits,ws", [(1, 0), (2, 2), (7, 7), (0, 64), (0, 0)])
def test_decode_contig_splits(splits, ws):
    """Global decode with the sink tuned to ~50% mass, several split counts:
    a sink dropped or added per split would fail."""
    _print_case("decode contig", splits, ws)
    cl = torch.tensor([0, 1, 31, 32, 33, 700, 2049, 3000], dtype=torch.int32)
    layer = _layer(31, cl, 1, 64, 4, 0, sinks=sink_for_half_mass(1500))
    o, kc, _ = _run_cached(layer, cl, ops.CONTIG, 0, 3100, 4, verify=False, num_splits=splits,
                           ws_splits=ws)
    assert_close(o, _ref_cached(layer, cl, 0), torch.bfloat16, "contig decode")
    kc = kc.cpu()
    for b, L in enumerate(cl.tolist()):
        assert torch.equal(kc[b, :, L], layer.k_new[b, 0])


def test_decode_split_invariance():
    _print_case("split invariance")
    cl = torch.tensor([4000, 100, 2500], dtype=torch.int32)
    layer = _layer(41, cl, 1, 32, 2, 0, sinks=sink_for_half_mass(2000))
    outs = []
    for s in (1, 2, 7, 16):
        o, _, _ = _run_cached(layer, cl, ops.CONTIG, 0, 4200, 2, verify=False, num_splits=s,
                              ws_splits=max(s, 2))
        outs.append(to64(o))
    for x in outs[1:]:
        assert np.abs(x - outs[0]).max() < 2e-2


def test_decode_contig_window():
    """A windowed layer over a contiguous cache: only the last W positions."""
    _print_case("contig window")
    cl = torch.tensor([10, 300, 1000], dtype=torch.int32)
    layer = _layer(51, cl, 1, 16, 2, 0)
    o, _, _ = _run_cached(layer, cl, ops.CONTIG, 128, 1100, 2, verify=False, num_splits=3,
                          ws_splits=3)
    assert_close(o, _ref_cached(layer, cl, 128), torch.bfloat16, "contig window")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_verify_ring(dtype):
    _print_case("verify ring", dtype)
    cl = torch.tensor([0, 3, 126, 127, 128, 500, 16384], dtype=torch.int32)
    layer = _layer(61, cl, 4, 64, 8, 128, dtype, sinks=None)
    kc0, vc0 = synth.fill_ring(layer, cl, 128, 8)
    o, kc, vc = _run_cached(layer, cl, ops.RING, 128, 128, 8, verify=True)
    assert_close(o, _ref_cached(layer, cl, 128), dtype, "ring verify")
    # verify never writes the cache
    assert torch.equal(kc.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       kc0.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def test_verify_ring_wide_window():
    """4-token verify over a W = 512 ring (token-wave mode, up to 516 keys per query)."""
    _print_case("verify ring W512")
    cl = torch.tensor([0, 2, 509, 510, 512, 700, 4096], dtype=torch.int32)
    layer = _layer(62, cl, 4, 64, 8, 512, torch.bfloat16)
    kc0, vc0 = synth.fill_ring(layer, cl, 512, 8)
    o, kc, vc = _run_cached(layer, cl, ops.RING, 512, 512, 8, verify=True)
    assert_close(o, _ref_cached(layer, cl, 512), torch.bfloat16, "ring verify W512")
    assert torch.equal(kc.cpu().view(torch.int16), kc0.view(torch.int16))


@pytest.mark.parametrize("splits,ws", [(1, 0), (0, 64), (5, 5)])
def test_verify_contig(splits, ws):
    _print_case("verify contig", splits, ws)
    cl = torch.tensor([0, 1, 1000, 2047, 2048], dtype=torch.int32)
    layer = _layer(71, cl, 4, 64, 4, 0, sinks=sink_for_half_mass(1000))
    o, _, _ = _run_cached(layer, cl, ops.CONTIG, 0, 2100, 4, verify=True, num_splits=splits,
                          ws_splits=ws)
    assert_close(o, _ref_cached(layer, cl, 0), torch.bfloat16, "contig verify")


@pytest.mark.parametrize("nq,splits", [(2, 0), (2, 3), (3, 1), (3, 0)])
def test_verify_contig_column_counts(nq, splits):
    """Verify of 2 and 3 tokens on a global layer (16 heads per KV head: 32 and 48
    (token, head) columns) -- the LDS-staged verify kernel with idle waves --
    over contexts that end on, just past and just before 32-key block edges."""
    _print_case("verify contig columns", nq, splits)
    cl = torch.tensor([0, 31, 32, 33, 95, 1000], dtype=torch.int32)
    layer = _layer(101 + nq, cl, nq, 64, 4, 0, sinks=sink_for_half_mass(1000))
    o, _, _ = _run_cached(layer, cl, ops.CONTIG, 0, 1040, 4, verify=True, num_splits=splits,
                          ws_splits=max(splits, 8))
    assert_close(o, _ref_cached(layer, cl, 0), torch.bfloat16, "contig verify columns")


@pytest.mark.parametrize("nq", [1, 2, 3, 8])
def test_verify_query_counts(nq):
    _print_case("verify nq", nq)
    cl = torch.tensor([5, 130, 900], dtype=torch.int32)
    layer = _layer(81 + nq, cl, nq, 16, 2, 128)
    o, _, _ = _run_cached(layer, cl, ops.RING, 128, 128, 2, verify=True)
    assert_close(o, _ref_cached(layer, cl, 128), torch.bfloat16, "verify nq")


def test_verify_equals_sequential_decodes():
    """verify(4) gives the rows of 4 decode steps that append one token each."""
    _print_case("verify == 4 decodes")
    cl = torch.tensor([200, 77], dtype=torch.int32)
    layer = _layer(91, cl, 4, 64, 8, 128)
    ov, kc, vc = _run_cached(layer, cl, ops.RING, 128, 128, 8, verify=True)
    kc0, vc0 = synth.fill_ring(layer, cl, 128, 8)
    kc, vc = kc0.to(DEV), vc0.to(DEV)
    rows = []
    for t in range(4):
        o = ops.decode(layer.q[:, t].contiguous().to(DEV), layer.k_new[:, t].contiguous().to(DEV),
                       layer.v_new[:, t].contiguous().to(DEV), kc, vc, (cl + t).to(DEV),
                       layer.sink.to(DEV), ops.RING, 128, int(cl.max()) + t)
        rows.append(to64(o))
    seq = np.stack(rows, 1)
    assert np.abs(seq - to64(ov)).max() < 2e-2


@pytest.mark.parametrize("kind", [ops.RING, ops.CONTIG])
def test_kv_append(kind):
    _print_case("kv_append", kind)
    g = synth.generator(7)
    B, n, Hkv, cap = 3, 5, 2, 128 if kind == ops.RING else 400
    cl = torch.tensor([0, 126, 390], dtype=torch.int32)
    nacc = torch.tensor([5, 2, 0], dtype=torch.int32)
    kn = synth.normal(g, (B, n, Hkv, 192))
    vn = synth.normal(g, (B, n, Hkv, 128))
    kc = torch.zeros(B, Hkv, cap, 192, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(B, Hkv, cap, 128, dtype=torch.bfloat16, device=DEV)
    ops.kv_append(kn.to(DEV), vn.to(DEV), kc, vc, cl.to(DEV), kind, nacc.to(DEV))
    kc, vc = kc.cpu(), vc.cpu()
    ke = torch.zeros_like(kc)
    ve = torch.zeros_like(vc)
    for b in range(B):
        for t in range(int(nacc[b])):
            p = int(cl[b]) + t
            slot = p % cap if kind == ops.RING else p
            if kind == ops.CONTIG and p >= cap:
                continue
            ke[b, :, slot] = kn[b, t]
            ve[b, :, slot] = vn[b, t]
    assert torch.equal(kc, ke) and torch.equal(vc, ve)


def test_kv_append_ring_keeps_last_cap():
    """Laying a whole prefill into a ring keeps only the last cap positions."""
    _print_case("ring from prefill")
    g = synth.generator(8)
    T, Hkv, cap = 300, 2, 128
    kn = synth.normal(g, (1, T, Hkv, 192))
    vn = synth.normal(g, (1, T, Hkv, 128))
    kc = torch.zeros(1, Hkv, cap, 192, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(1, Hkv, cap, 128, dtype=torch.bfloat16, device=DEV)
    ops.kv_append(kn.to(DEV), vn.to(DEV), kc, vc, torch.zeros(1, dtype=torch.int32, device=DEV),
                  ops.RING)
    kc = kc.cpu()
    for p in range(T - cap, T):
        assert torch.equal(kc[0, :, p % cap], kn[0, p])
