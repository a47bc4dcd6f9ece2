"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load_library()``
or a deliberately mutated copy) and raises AssertionError when the oracle
disagrees with what the pages and the mathematics fix:

- a library reduction: sink attention equals ordinary softmax attention over
  the keys plus one extra key whose logit is the sink and whose value is zero
  (torch's scaled_dot_product_attention in float64 on the CPU);
- sink = -inf is ordinary causal (or windowed) softmax attention, the "w/o
  sink" baseline of the report's Table 2;
- closed forms: q = 0 gives o_i = sum_{j in J_i} v_j / (e^sink + |J_i|); one
  key gives o = sigmoid(a - sink) v; n identical keys give o = n e^a /
  (e^sink + n e^a) * mean(v);
- invariants: attention mass + sink mass = 1; sink = 1e3 gives o = 0 exactly;
  W >= T equals global; |o| <= (1 - sink mass) max|v|;
- RoPE: rotation of (x_{2c} + i x_{2c+1}) by e^{i phi} with numpy complex
  arithmetic; pos = 0 is the identity; dims >= 64 untouched; shift invariance
  of q.k; the first two frequencies checked by hand values;
- bf16 rounding against torch's fp32 -> bf16 cast (round to nearest even).

No file here is imported by the HIP path; ``tests/test_oracle_pins.py`` runs
the pins against the real oracle, ``tests/test_oracle_mutants.py`` against
copies with planted mistakes (each must fail at least one pin).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

RNG_SEED = 12345


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _sdpa_augmented(q, k, v, sink, window, scale):
    """Sink attention via torch SDPA (fp64, CPU) on an augmented key set.

    q [T,Hq,d], k [T,Hkv,d], v [T,Hkv,dv] at positions 0..T-1.  One zero key
    and zero value are appended; its additive mask entry is sink_h, so its
    logit is exactly sink_h.  Invisible keys get -inf.  GQA by repeat.
    """
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq,T,d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)
    kt = torch.cat([kt, torch.zeros(Hq, 1, d, dtype=torch.float64)], 1)
    vt = torch.cat([vt, torch.zeros(Hq, 1, v.shape[2], dtype=torch.float64)], 1)
    i = torch.arange(T).view(T, 1)
    j = torch.arange(T).view(1, T)
    vis = (j <= i)
    if window > 0:
        vis = vis & (i - j < window)
    mask = torch.full((Hq, T, T + 1), -math.inf, dtype=torch.float64)
    mask[:, :, :T] = torch.where(vis, 0.0, -math.inf).to(torch.float64)
    mask[:, :, T] = torch.from_numpy(np.asarray(sink, np.float64)).view(Hq, 1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                         scale=scale)
    return o.permute(1, 0, 2).numpy()


def _run(lib, q, k, v, sink, window, scale=None, qpos=None, kpos=None):
    T = q.shape[0]
    qpos = np.arange(T) if qpos is None else qpos
    kpos = np.arange(k.shape[0]) if kpos is None else kpos
    return oracle.sink_attention(q, k, v, qpos, kpos, sink, window, scale, lib=lib)


def pin_sdpa_augmented(lib):
    for case, (T, Hq, Hkv, d, dv, window) in enumerate(
            [(1, 2, 1, 8, 4, 0), (7, 4, 2, 12, 6, 3), (37, 6, 3, 16, 8, 0),
             (37, 6, 3, 16, 8, 1), (40, 4, 1, 24, 16, 8), (29, 8, 2, 192, 128, 5)]):
        r = _rng(case)
        q = r.standard_normal((T, Hq, d))
        k = r.standard_normal((T, Hkv, d))
        v = r.standard_normal((T, Hkv, dv))
        sink = r.standard_normal(Hq) * 2.0
        sink[0] = 4.0  # make the sink term matter in at least one head
        scale = 1.0 / math.sqrt(d)
        o, _ = _run(lib, q, k, v, sink, window, scale)
        ref = _sdpa_augmented(q, k, v, sink, window, scale)
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-13), \
            ("sdpa", case, float(np.abs(o - ref).max()))


def pin_no_sink_is_softmax(lib):
    """sink = -inf removes the extra term: plain causal / windowed softmax."""
    T, Hq, Hkv, d, dv = 23, 4, 2, 16, 8
    r = _rng(10)
    q, k, v = r.standard_normal((T, Hq, d)), r.standard_normal((T, Hkv, d)), \
        r.standard_normal((T, Hkv, dv))
    sink = np.full(Hq, -np.inf)
    for window in (0, 4):
        o, lse = _run(lib, q, k, v, sink, window)
        qt = torch.from_numpy(q).permute(1, 0, 2)
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        if window == 0:
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        else:
            i = torch.arange(T).view(T, 1)
            j = torch.arange(T).view(1, T)
            m = (j <= i) & (i - j < window)
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
        ref = ref.permute(1, 0, 2).numpy()
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-13), ("nosink", window)
        # lse is the log of the plain softmax normaliser
        logits = np.einsum("thd,jhd->thj", q, np.repeat(k, Hq // Hkv, 1)) / math.sqrt(d)
        i = np.arange(T)[:, None]
        j = np.arange(T)[None, :]
        vis = (j <= i) & ((i - j < window) if window else True)
        logits = np.where(vis[:, None, :], logits, -np.inf)
        ref_lse = np.log(np.exp(logits).sum(-1))
        assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12), ("nosink-lse", window)


def pin_zero_query_closed_form(lib):
    """q = 0: every visible logit is 0, so o_i = sum_J v_j / (e^sink + |J_i|)."""
    T, Hq, Hkv, d, dv = 40, 6, 3, 8, 5
    group = Hq // Hkv
    q = np.zeros((T, Hq, d))
    r = _rng(20)
    k = r.standard_normal((T, Hkv, d))
    jj = np.arange(T)[:, None, None]
    gg = np.arange(Hkv)[None, :, None]
    cc = np.arange(dv)[None, None, :]
    v = (jj + 1) * 1e-3 + cc * 1e-6 + gg * 1.0   # position, dim and group all visible
    sink = np.array([0.0, 1.0, -2.0, 3.0, -np.inf, 0.5])
    for window in (0, 1, 3, 7, 64):
        o, lse = _run(lib, q, k, v, sink, window)
        for i in range(T):
            lo = 0 if window == 0 else max(0, i - window + 1)
            n = i - lo + 1
            for h in range(Hq):
                g = h // group
                es = 0.0 if sink[h] == -np.inf else math.exp(sink[h])
                ref = v[lo:i + 1, g].sum(0) / (es + n)
                assert np.allclose(o[i, h], ref, rtol=1e-13, atol=1e-15), \
                    ("q0", window, i, h)
                assert abs(lse[i, h] - math.log(es + n)) < 1e-12, ("q0-lse", window, i, h)


def pin_single_key_sigmoid(lib):
    """T = 1: o_0 = sigmoid(a_00 - sink) v_0 and lse = log(e^a + e^sink)."""
    r = _rng(30)
    d, dv = 192, 128
    for trial in range(5):
        q = r.standard_normal((1, 2, d))
        k = r.standard_normal((1, 1, d))
        v = r.standard_normal((1, 1, dv))
        sink = r.standard_normal(2) * 3
        scale = 1.0 / math.sqrt(d)
        o, lse = _run(lib, q, k, v, sink, 0, scale)
        for h in range(2):
            a = float(q[0, h] @ k[0, 0]) * scale
            sig = 1.0 / (1.0 + math.exp(-(a - sink[h])))
            assert np.allclose(o[0, h], sig * v[0, 0], rtol=1e-12, atol=1e-14), ("T1", h)
            assert abs(lse[0, h] - np.logaddexp(a, sink[h])) < 1e-12


def pin_identical_keys(lib):
    """n identical visible keys: each weight is e^a / (e^sink + n e^a)."""
    T, d, dv = 9, 16, 4
    r = _rng(40)
    q = r.standard_normal((T, 1, d))
    k = np.repeat(r.standard_normal((1, 1, d)), T, 0)
    v = r.standard_normal((T, 1, dv))
    sink = np.array([0.7])
    scale = 0.3
    for window in (0, 4):
        o, _ = _run(lib, q, k, v, sink, window, scale)
        for i in range(T):
            lo = 0 if window == 0 else max(0, i - window + 1)
            n = i - lo + 1
            a = float(q[i, 0] @ k[0, 0]) * scale
            w = math.exp(a) / (math.exp(sink[0]) + n * math.exp(a))
            ref = w * v[lo:i + 1, 0].sum(0)
            assert np.allclose(o[i, 0], ref, rtol=1e-12, atol=1e-14), ("ident", window, i)


def pin_mass_identity(lib):
    """With v = 1, o_i = sum_j s_ij, and sum_j s_ij + e^(sink - lse_i) = 1."""
    T, Hq, Hkv, d = 33, 4, 1, 24
    r = _rng(50)
    q, k = r.standard_normal((T, Hq, d)) * 2, r.standard_normal((T, Hkv, d))
    v = np.ones((T, Hkv, 3))
    sink = np.array([-1.0, 0.0, 2.5, 6.0])
    for window in (0, 5):
        o, lse = _run(lib, q, k, v, sink, window)
        sink_mass = np.exp(sink[None, :] - lse)
        assert np.allclose(o[..., 0] + sink_mass, 1.0, rtol=0, atol=1e-13), ("mass", window)
        assert np.allclose(o[..., 0], o[..., 2], rtol=0, atol=0)


def pin_large_sink_zero(lib):
    """A sink of 1e3 dwarfs every logit: o is exactly 0 and lse is the sink."""
    T, d = 12, 16
    r = _rng(60)
    q, k, v = r.standard_normal((T, 2, d)), r.standard_normal((T, 1, d)), \
        r.standard_normal((T, 1, 8))
    o, lse = _run(lib, q, k, v, np.array([1e3, 1e3]), 0)
    assert np.all(o == 0.0)
    assert np.allclose(lse, 1e3, rtol=0, atol=1e-9)


def pin_wide_window_is_global(lib):
    T, d = 17, 8
    r = _rng(70)
    q, k, v = r.standard_normal((T, 2, d)), r.standard_normal((T, 2, d)), \
        r.standard_normal((T, 2, 4))
    sink = np.array([0.2, -0.4])
    og, lg = _run(lib, q, k, v, sink, 0)
    for w in (T, T + 5, 1000):
        ow, lw = _run(lib, q, k, v, sink, w)
        assert np.array_equal(og, ow) and np.array_equal(lg, lw)
    ow, _ = _run(lib, q, k, v, sink, T - 1)
    assert not np.allclose(og, ow)  # a window shorter than T does cut keys


def pin_output_bound(lib):
    """|o_i| <= (1 - sink mass) * max_j |v_j| elementwise (a convex sub-mixture)."""
    T, d, dv = 30, 16, 6
    r = _rng(80)
    q, k, v = r.standard_normal((T, 3, d)), r.standard_normal((T, 3, d)), \
        r.standard_normal((T, 3, dv))
    sink = np.array([1.0, 3.0, -1.0])
    o, lse = _run(lib, q, k, v, sink, 6)
    sm = np.exp(sink[None, :] - lse)
    bound = (1.0 - sm)[..., None] * np.abs(v).max(0).max(0)[None, None, :]
    assert np.all(np.abs(o) <= bound + 1e-14)


def pin_views_consistent(lib):
    """The decode/verify view of the oracle equals the prefill view's rows.

    Query t at position L+t over history 0..L-1 plus new tokens 0..t is prefill
    row L+t; a ring's history (only the last W-1 rows) gives the same result
    under a window W.
    """
    T, Hq, Hkv, d, dv = 26, 4, 2, 16, 8
    r = _rng(90)
    q, k, v = r.standard_normal((1, T, Hq, d)), r.standard_normal((1, T, Hkv, d)), \
        r.standard_normal((1, T, Hkv, dv))
    sink = r.standard_normal(Hq)
    for window in (0, 5):
        op, lp = oracle.prefill(q, k, v, sink, window, lib=lib)
        for L, n in ((20, 1), (21, 4), (0, 3)):
            keep = L if window == 0 else min(L, window)
            o, lse = oracle.decode_or_verify(q[:, L:L + n], [k[0, L - keep:L]],
                                             [v[0, L - keep:L]], k[:, L:L + n],
                                             v[:, L:L + n], [L], sink, window, lib=lib)
            assert np.allclose(o, op[:, L:L + n], rtol=1e-13, atol=1e-14), (window, L, n)
            assert np.allclose(lse, lp[:, L:L + n], rtol=1e-13, atol=1e-13)
    rows = np.array([3, 11, 25])
    o_s, _ = oracle.prefill(q, k, v, sink, 5, rows=rows, lib=lib)
    assert np.allclose(o_s, op[:, rows], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- RoPE

def _rope(lib, x, pos, base, rope_dim=64, style=0):
    return oracle.rope_partial(x, pos, base, rope_dim, style, lib=lib)


def pin_rope_complex(lib):
    """Each pair (x_{2c}, x_{2c+1}) is the complex number x_{2c} + i x_{2c+1}
    multiplied by exp(i pos theta_c), theta_c = base^(-2c/64)."""
    r = _rng(100)
    n_tok, H, D = 11, 3, 192
    x = r.standard_normal((n_tok, H, D))
    pos = np.array([0, 1, 2, 7, 100, 1023, 4095, 32767, 65536, 131071, 262143])
    for base in (1e4, 6.4e5, 5e6):
        y = _rope(lib, x, pos, base)
        theta = np.power(base, -np.arange(32) * 2.0 / 64.0)
        rot = np.exp(1j * pos[:, None, None] * theta[None, None, :])
        z = (x[..., 0:64:2] + 1j * x[..., 1:64:2]) * rot
        # two libm's may round theta_c one ulp apart; the angle error then grows
        # with the position: |d phi| <= pos * 2^-52 * theta, times |x| <= 5
        tol = 1e-13 + 5 * 2.0 ** -52 * 2 * (pos[:, None, None] + 1.0)
        assert np.all(np.abs(y[..., 0:64:2] - z.real) <= tol), base
        assert np.all(np.abs(y[..., 1:64:2] - z.imag) <= tol), base
        assert np.array_equal(y[..., 64:], x[..., 64:])


def pin_rope_hand_values(lib):
    """theta_0 = 1 and theta_1 = base^(-1/32): at pos 1 the unit vector (1, 0)
    of pair c goes to (cos theta_c, sin theta_c)."""
    x = np.zeros((1, 1, 192))
    x[0, 0, 0] = 1.0
    x[0, 0, 2] = 1.0
    y = _rope(lib, x, np.array([1]), 1e4)
    assert abs(y[0, 0, 0] - math.cos(1.0)) < 1e-15 and abs(y[0, 0, 1] - math.sin(1.0)) < 1e-15
    t1 = 0.74989420933245582730  # 10^(-4/32), by hand
    assert abs(y[0, 0, 2] - math.cos(t1)) < 1e-15 and abs(y[0, 0, 3] - math.sin(t1)) < 1e-15


def pin_rope_identity_norm_shift(lib):
    r = _rng(110)
    x = r.standard_normal((5, 2, 192))
    y0 = _rope(lib, x, np.zeros(5, np.int64), 1e4)
    assert np.array_equal(y0, x)                       # pos 0: identity
    pos = np.array([3, 50, 999, 20000, 131000])
    y = _rope(lib, x, pos, 5e6)
    n0 = x[..., 0:64:2] ** 2 + x[..., 1:64:2] ** 2
    n1 = y[..., 0:64:2] ** 2 + y[..., 1:64:2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)  # pair norms preserved
    # q.k depends only on the position difference
    q = r.standard_normal((1, 1, 192))
    k = r.standard_normal((1, 1, 192))
    for base in (1e4, 5e6):
        for pq, pk, delta in ((10, 3, 1000), (500, 499, 77777), (7, 7, 123)):
            d0 = float((_rope(lib, q, np.array([pq]), base) * _rope(lib, k, np.array([pk]), base)).sum())
            d1 = float((_rope(lib, q, np.array([pq + delta]), base) *
                        _rope(lib, k, np.array([pk + delta]), base)).sum())
            assert abs(d0 - d1) < 1e-9, (base, pq, pk, delta)


def pin_rope_half_split(lib):
    """Half-split pairing is interleaved pairing under a fixed permutation."""
    r = _rng(120)
    x = r.standard_normal((4, 2, 192))
    pos = np.array([1, 9, 300, 77777])
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2), np.arange(64, 192)])
    yi = _rope(lib, x, pos, 1e4, style=0)
    xh = x[..., perm]            # half layout: xh[c] = x[2c], xh[c + 32] = x[2c + 1]
    yh = _rope(lib, xh, pos, 1e4, style=1)
    assert np.allclose(yh, yi[..., perm], rtol=0, atol=1e-13)


def pin_bf16_rounding(lib):
    """Rounding to bf16 equals torch's fp32 -> bf16 cast (RNE) on fp32 inputs."""
    r = _rng(130)
    vals = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (r.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-45, np.inf, -np.inf],
                 np.float32),
    ])
    # exact ties: 1 + (2k+1) * 2^-8 sit halfway between two bf16 values
    ties = (1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8).astype(np.float32)
    vals = np.concatenate([vals, ties, -ties])
    got = oracle.round_bf16_bits(vals.astype(np.float64), lib=lib)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nan = oracle.round_bf16_bits(np.array([np.nan]), lib=lib)
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


# ----------------------------------------------------------------------------- backward

def _bwd(lib, q, k, v, sink, dout, window, scale=None, qpos=None, kpos=None):
    T = q.shape[0]
    qpos = np.arange(T) if qpos is None else qpos
    kpos = np.arange(k.shape[0]) if kpos is None else kpos
    return oracle.sink_attention_bwd(q, k, v, qpos, kpos, sink, dout, window, scale, lib=lib)


def _loss(lib, q, k, v, sink, dout, window):
    o, _ = _run(lib, q, k, v, sink, window)
    return float((o * dout).sum())


def pin_bwd_finite_differences(lib):
    """Every gradient against central differences of the forward oracle's loss
    L = sum(dout * o) (fp64, h = 1e-6): windowed and global, a -inf sink head."""
    for window, seed in ((4, 0), (0, 1)):
        rng = _rng(40 + seed)
        T, Hq, Hkv, d, dv = 6, 4, 2, 5, 3
        q = rng.standard_normal((T, Hq, d))
        k = rng.standard_normal((T, Hkv, d))
        v = rng.standard_normal((T, Hkv, dv))
        sink = np.array([0.3, -1.2, -np.inf, 1.7])
        dout = rng.standard_normal((T, Hq, dv))
        dq, dk, dvv, dsink = _bwd(lib, q, k, v, sink, dout, window)
        h = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dvv), ("sink", sink, dsink)):
            flat, gflat = x.reshape(-1), g.reshape(-1)
            for idx in range(flat.size):
                if not np.isfinite(flat[idx]):
                    assert gflat[idx] == 0.0, (name, idx)
                    continue
                keep = flat[idx]
                flat[idx] = keep + h
                lp = _loss(lib, q, k, v, sink, dout, window)
                flat[idx] = keep - h
                lm = _loss(lib, q, k, v, sink, dout, window)
                flat[idx] = keep
                fd = (lp - lm) / (2 * h)
                assert abs(fd - gflat[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, gflat[idx])


def pin_bwd_torch_autograd(lib):
    """Against torch autograd (fp64) of the augmented softmax written with
    library ops: logits with an extra sink column, softmax, drop the column."""
    rng = _rng(50)
    T, Hq, Hkv, d, dv, window = 9, 4, 1, 6, 5, 5
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, dv))
    sink = rng.standard_normal(Hq)
    dout = rng.standard_normal((T, Hq, dv))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv, ts = (torch.tensor(x, requires_grad=True) for x in (q, k, v, sink))
    kk = tk.repeat_interleave(Hq // Hkv, 1)
    vv = tv.repeat_interleave(Hq // Hkv, 1)
    logits = torch.einsum("ihc,jhc->hij", tq, kk) * scale
    i = torch.arange(T).view(T, 1)
    j = torch.arange(T).view(1, T)
    vis = (j <= i) & (i - j < window)
    logits = logits.masked_fill(~vis, float("-inf"))
    aug = torch.cat([logits, ts.view(Hq, 1, 1).expand(Hq, T, 1)], 2)
    p = torch.softmax(aug, 2)[:, :, :T]
    o = torch.einsum("hij,jhc->ihc", p, vv)
    (o * torch.from_numpy(dout)).sum().backward()
    got = _bwd(lib, q, k, v, sink, dout, window)
    for g, t in zip(got, (tq, tk, tv, ts)):
        assert np.allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_bwd_no_sink_matches_softmax_attention(lib):
    """sink = -inf: dsink = 0 and dq, dk, dv are those of plain causal softmax
    attention (torch SDPA autograd, fp64)."""
    rng = _rng(60)
    T, Hq, Hkv, d, dv = 7, 2, 2, 4, 3
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, dv))
    dout = rng.standard_normal((T, Hq, dv))
    sink = np.full(Hq, -np.inf)
    tq, tk, tv = (torch.tensor(x.transpose(1, 0, 2).copy(), requires_grad=True)
                  for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    (o * torch.from_numpy(dout.transpose(1, 0, 2).copy())).sum().backward()
    dq, dk, dvv, dsink = _bwd(lib, q, k, v, sink, dout, 0)
    assert np.all(dsink == 0.0)
    for g, t in zip((dq, dk, dvv), (tq, tk, tv)):
        assert np.allclose(g, t.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
