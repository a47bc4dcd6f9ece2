"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
attention or RoPE arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any of the method's code.

Workloads follow the MiMo-V2-Flash Technical Report: Table 1 (SWA 64 query / 8
KV heads, GA 64 / 4, QK dim 192, V dim 128, window 128), Section 2.1 (RoPE on
the first 64 dims), Section 3.2 (RoPE bases 1e4 for SWA, 5e6 for GA after the
context extension) and Section 5.2 / Table 10 (16K-token contexts, batch 32-128
per node for speculative decoding).  No trained weights or datasets exist here:
activations are N(0,1) draws and sinks are N(0,1) scalars.

Every draw uses a CPU ``torch.Generator`` seeded per case; fp32 values are cast
to bf16 by round-to-nearest-even, so both sides see identical bits.
"""
from __future__ import annotations

import dataclasses

import torch

DQK = 192
DV = 128
WINDOW = 128
ROPE_DIM = 64
BASE_SWA = 1.0e4
BASE_GA = 5.0e6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "prefill_swa" | "prefill_global" | "decode_block" | "verify"
    B: int
    T: int             # prefill length or number of query tokens per sequence
    Hq: int
    Hkv: int
    dtype: torch.dtype
    window: int = WINDOW
    base: float = BASE_SWA
    seed: int = 0


# The five benchmark configurations (shapes from Table 1; contexts from
# Section 5.2 / Table 10 and the long-context range of Section 3).
WORKLOADS = {
    1: Workload("tiny_fp32_swa_T1024_8q1kv", "prefill_swa", 1, 1024, 8, 1, torch.float32,
                WINDOW, BASE_SWA, 1001),
    2: Workload("swa_prefill_bf16_T32768_64q8kv_W128", "prefill_swa", 1, 32768, 64, 8,
                torch.bfloat16, WINDOW, BASE_SWA, 1002),
    3: Workload("global_prefill_bf16_T32768_64q4kv", "prefill_global", 1, 32768, 64, 4,
                torch.bfloat16, 0, BASE_GA, 1003),
    4: Workload("hybrid_block_decode_bf16_B32_ctx16k-128k_5swa+1ga", "decode_block", 32, 1,
                64, 8, torch.bfloat16, WINDOW, BASE_SWA, 1004),
    5: Workload("spec_verify_bf16_B64_nq4_ctx16384_swa+ga", "verify", 64, 4, 64, 8,
                torch.bfloat16, WINDOW, BASE_SWA, 1005),
}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal(g: torch.Generator, shape, dtype=torch.bfloat16, std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 on the CPU, then cast (RNE) to ``dtype``."""
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype).contiguous()


def prefill_inputs(seed: int, B: int, T: int, Hq: int, Hkv: int, dtype=torch.bfloat16,
                   dqk: int = DQK, dv: int = DV):
    """q [B,T,Hq,dqk], k [B,T,Hkv,dqk], v [B,T,Hkv,dv], sink [Hq] (fp32)."""
    g = generator(seed)
    q = normal(g, (B, T, Hq, dqk), dtype)
    k = normal(g, (B, T, Hkv, dqk), dtype)
    v = normal(g, (B, T, Hkv, dv), dtype)
    sink = normal(g, (Hq,), torch.float32)
    return q, k, v, sink


def positions(B: int, T: int, start: int = 0) -> torch.Tensor:
    """int32 absolute positions start..start+T-1 for each of B sequences, flattened."""
    return torch.arange(start, start + T, dtype=torch.int32).repeat(B).contiguous()


def cache_lengths(g: torch.Generator, B: int, lo: int, hi: int) -> torch.Tensor:
    """Per-sequence cached lengths drawn uniformly from [lo, hi] (int32)."""
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


@dataclasses.dataclass
class CachedLayer:
    """One attention layer's decode/verify state.

    ``k_hist[b]`` / ``v_hist[b]`` hold the logical key/value history of sequence
    b: the rows for positions ``cache_len[b] - len .. cache_len[b] - 1``.  A ring
    layer keeps only the last ``window`` positions, a contiguous layer all of
    them.  ``k_new``/``v_new`` are the n new tokens, ``q`` their queries.
    """
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    sink: torch.Tensor
    k_hist: list
    v_hist: list
    window: int


def cached_layer(g: torch.Generator, cache_len: torch.Tensor, n: int, Hq: int, Hkv: int,
                 window: int, dtype=torch.bfloat16, dqk: int = DQK, dv: int = DV,
                 hist_rows: int | None = None) -> CachedLayer:
    """Draw one layer: q, new k/v, sink, then each sequence's history.

    window > 0: the history holds min(L, window) rows (a ring's live content);
    window <= 0: min(L, hist_rows or L) rows (all of a contiguous cache).
    """
    B = cache_len.shape[0]
    q = normal(g, (B, n, Hq, dqk), dtype)
    k_new = normal(g, (B, n, Hkv, dqk), dtype)
    v_new = normal(g, (B, n, Hkv, dv), dtype)
    sink = normal(g, (Hq,), torch.float32)
    k_hist, v_hist = [], []
    for b in range(B):
        L = int(cache_len[b])
        rows = min(L, window) if window > 0 else (L if hist_rows is None else min(L, hist_rows))
        k_hist.append(normal(g, (rows, Hkv, dqk), dtype))
        v_hist.append(normal(g, (rows, Hkv, dv), dtype))
    return CachedLayer(q, k_new, v_new, sink, k_hist, v_hist, window)


def fill_ring(layer: CachedLayer, cache_len: torch.Tensor, cap: int, Hkv: int,
              dqk: int = DQK, dv: int = DV, poison: bool = True):
    """Lay a ring layer's history out as [B,Hkv,cap,d]: position p sits in slot p % cap.

    Slots holding no live position are filled with NaN so that a read of one
    shows up in the output.
    """
    B = cache_len.shape[0]
    dt = layer.k_new.dtype
    fill = float("nan") if poison else 0.0
    kc = torch.full((B, Hkv, cap, dqk), fill, dtype=dt)
    vc = torch.full((B, Hkv, cap, dv), fill, dtype=dt)
    for b in range(B):
        L = int(cache_len[b])
        rows = layer.k_hist[b].shape[0]
        for r in range(rows):
            p = L - rows + r
            kc[b, :, p % cap] = layer.k_hist[b][r]
            vc[b, :, p % cap] = layer.v_hist[b][r]
    return kc, vc


def fill_contig(layer: CachedLayer, cache_len: torch.Tensor, cap: int, Hkv: int,
                dqk: int = DQK, dv: int = DV, poison: bool = True):
    """Lay a contiguous layer's history out as [B,Hkv,cap,d]: position p at index p.

    Rows at or beyond cache_len are NaN-poisoned (when ``poison``).
    """
    B = cache_len.shape[0]
    dt = layer.k_new.dtype
    fill = float("nan") if poison else 0.0
    kc = torch.full((B, Hkv, cap, dqk), fill, dtype=dt)
    vc = torch.full((B, Hkv, cap, dv), fill, dtype=dt)
    for b in range(B):
        L = int(cache_len[b])
        rows = layer.k_hist[b].shape[0]
        kc[b, :, L - rows:L] = layer.k_hist[b].permute(1, 0, 2)
        vc[b, :, L - rows:L] = layer.v_hist[b].permute(1, 0, 2)
    return kc, vc


def device_normal(seed: int, shape, dtype=torch.bfloat16, device="cuda", std: float = 1.0,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """N(0, std^2) drawn with a seeded generator ON the device (for buffers of
    gigabytes, where a CPU draw would take minutes), cast (RNE) to ``dtype``.
    Draws happen in slices of the leading dim so the fp32 temporary stays small."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=device)
    n0 = out.shape[0]
    per = max(1, (1 << 27) // max(1, out[0].numel()))
    for i in range(0, n0, per):
        j = min(n0, i + per)
        x = torch.randn(out[i:j].shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[i:j].copy_(x)
    return out
