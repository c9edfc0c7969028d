"""Active-count buckets for graphs captured per bound on the active slots.

vLLM PR #32005 (its diff of the LoRA ops and the fused-MoE LoRA test)
sizes the fused kernel's LoRA grid axis by the number of active adapters
and captures one CUDA graph per specialisation of that number: no adapter,
the powers of two below the maximum, and the maximum.  Here the fused entry
points take that bound as `max_active_loras` (0 launches nothing), and these
two functions give the bucket set and the bucket a batch falls into; the host
knows a batch's adapters, so no device-to-host read is needed.  (One graph
captured with `max_active_loras = L` also serves every count, since the
kernels find the active slots on the device; the buckets only shrink the
launch.)
"""
from __future__ import annotations


def active_count_buckets(L: int) -> list:
    """0, the powers of two below L, and L: the bounds graphs are captured for."""
    if L < 1:
        raise ValueError("L >= 1")
    out = [0]
    b = 1
    while b < L:
        out.append(b)
        b *= 2
    out.append(L)
    return out


def bucket_for(n_active: int, L: int) -> int:
    """The smallest bucket holding n_active active slots."""
    if not 0 <= n_active <= L:
        raise ValueError(f"n_active must be in [0, {L}]")
    for b in active_count_buckets(L):
        if b >= n_active:
            return b
    raise AssertionError("unreachable")
