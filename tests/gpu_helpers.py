"""Shared helpers of the GPU parity tests (tolerances, conversions)."""
from __future__ import annotations

import math

import numpy as np
import torch

# Tolerances stated for the hot path: fp32 inputs max|d| <= 1e-4; bf16 inputs
# with fp32 accumulation |d| <= 2e-2 + 1e-2 |oracle| elementwise.
F32_ATOL = 1e-4
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def assert_close(got: torch.Tensor, ref: np.ndarray, dtype, what: str = ""):
    g = to64(got)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), what + ": non-finite output"
    err = np.abs(g - ref)
    if dtype == torch.float32:
        worst = float(err.max()) if err.size else 0.0
        assert worst <= F32_ATOL, "%s: max|d| = %.3g > %.1g" % (what, worst, F32_ATOL)
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
        bad = err > bound
        if bad.any():
            idx = np.unravel_index(np.argmax(err - bound), err.shape)
            raise AssertionError("%s: %d elements out of tolerance, worst at %s: got %.5g ref %.5g"
                                 % (what, int(bad.sum()), idx, g[idx], ref[idx]))
    return float(err.max()) if err.size else 0.0


def sink_for_half_mass(n_keys: int) -> float:
    """A sink logit that takes about half of the softmax mass when the n_keys
    logits are q.k/sqrt(192) with q, k ~ N(0,1) (logits ~ N(0,1): E e^a = e^0.5)."""
    return math.log(max(1, n_keys)) + 0.5


# ----------------------------------------------------------------------------- guard bands
# Outputs handed to the library as interior views of a larger buffer whose
# margins (and interior) start as 0xFF bytes: NaN in bf16 and fp32.  After the
# call the margins must still hold exactly those bytes (no store outside the
# output), and any interior element the kernel failed to write stays NaN.
GUARD_BYTES = 64 << 10


class Guarded:
    def __init__(self, shape, dtype, device="cuda", margin: int = GUARD_BYTES):
        n = 1
        for s in shape:
            n *= int(s)
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.margin = margin
        self.buf = torch.full((self.nbytes + 2 * margin,), 255, dtype=torch.uint8, device=device)
        self.t = self.buf[margin:margin + self.nbytes].view(dtype).view(tuple(shape))

    def assert_intact(self, what: str = ""):
        lo = self.buf[:self.margin]
        hi = self.buf[self.margin + self.nbytes:]
        bad_lo = int((lo != 255).sum())
        bad_hi = int((hi != 255).sum())
        assert bad_lo == 0 and bad_hi == 0, \
            "%s: %d bytes before and %d bytes after the output were overwritten" % (
                what, bad_lo, bad_hi)
