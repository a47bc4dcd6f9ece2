"""MI355X (gfx950) sink attention: HIP kernels behind a C ABI, bound with ctypes.

Entry points (see include/sinkattn.h): ``rope_partial``, ``prefill_swa``,
``prefill_global``, ``decode``, ``verify``, ``kv_append``.  The shared library
is loaded on first use; nothing here computes on the CPU.
"""
from .ops import (BF16, CONTIG, F32, HALF, INTERLEAVED, RING, SinkAttnError,  # noqa: F401
                  SinkAttnUnavailable, abi_version, decode, decode_workspace_bytes,
                  default_scale, kv_append, prefill_global, prefill_swa, prefill_swa_rope,
                  rope_partial, verify)
