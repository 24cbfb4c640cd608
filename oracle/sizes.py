"""Closed-form KV-cache sizes (oracle; test infrastructure only).

Pins: the 70B GQA example of "DuoAttention: Dual Retrieval & Streaming Heads
Guide" (section "1. The Quadratic Prefill and Linear Decoding Bandwidth
Bottleneck"), the effective-context example of its section "2. DuoAttention
Cache Partitioning Mechanics", and the 512 MiB / 2 GiB example of "Attention
Variants and KV-Cache Compression" (section "MHA and GQA").
"""
from __future__ import annotations

from typing import Sequence


def kv_cache_bytes(L: int, n_kv: int, d_head: int, T: int, elem_bytes: int = 2) -> int:
    """Full KV cache of one sequence: keys and values (factor 2) of
    ``elem_bytes`` each, for every layer, KV head, head dimension and token.
    (DuoAttention guide, section 1, the KV Cache Size equation; the same product
    as 2*L*S*n_kv*d_h*b in "Attention Variants and KV-Cache Compression", "MHA and GQA".)"""
    return 2 * elem_bytes * L * n_kv * d_head * T


def duo_effective_context(R: float, T: int, S: int, W: int) -> float:
    """Average tokens kept per KV head when a fraction R of heads keeps all T
    tokens and the rest keep S sinks plus a W-token window (DuoAttention guide,
    section 2, the Effective Context per Head equation)."""
    return R * T + (1.0 - R) * (S + W)


def duo_cache_bytes(R: float, T: int, S: int, W: int, L: int, n_kv: int, d_head: int,
                    elem_bytes: int = 2) -> float:
    """Mixed-cache footprint: effective context times the per-token KV bytes of
    all layers and heads (DuoAttention guide, section 2, the Memory_Duo equation;
    the garbled subscripts there read as Memory_Duo and n_kv)."""
    return duo_effective_context(R, T, S, W) * 2 * elem_bytes * L * n_kv * d_head


def mixed_payload_bytes(mask: Sequence[Sequence[int]], B: int, T_cap: int, S: int, W: int,
                        d_head: int, elem_bytes: int) -> int:
    """K+V payload of a mixed cache with a per-layer, per-KV-head mask: a
    retrieval head reserves T_cap rows, a streaming head S+W rows (the two
    buffer kinds of the DuoAttention guide, section 2).  With every head a
    retrieval head this equals ``B * kv_cache_bytes``; with a fraction R of
    heads retrieval in every layer it equals ``B * duo_cache_bytes``."""
    rows = 0
    for layer in mask:
        for m in layer:
            rows += T_cap if m else (S + W)
    return rows * B * d_head * elem_bytes * 2


def local_global_bytes(H_kv: int, D: int, elem_bytes: int, L1: int, L2: int, T: int, W: int) -> int:
    """Layer-wise cache of a model with L1 sliding-window layers (window W) and
    L2 full-attention layers ("Attention Variants and Memory Efficiency",
    "Sliding-Window and Mixed Attention", the M^KV equation)."""
    return 2 * H_kv * D * elem_bytes * (L1 * min(T, W) + L2 * T)
