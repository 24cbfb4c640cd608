"""Simulation of the mixed KV cache's contents (oracle; test infrastructure only).

A retrieval head keeps every token in order (DuoAttention guide, section "2.
DuoAttention Cache Partitioning Mechanics": a full contiguous buffer, tokens 1
to T).  A streaming head first fills its S attention-sink entries and then a
rolling window of W entries whose oldest entry is evicted (same section, and
the head-separation simulation's append rule in "Implementation: Simulating
DuoAttention Head Separation in Python").  The window is a ring buffer whose
write slot is its own append count modulo W ("Attention Variants and Memory
Efficiency", "Sliding-Window and Mixed Attention").

Reading taken where the pages leave a step open: the physical slot of a
streaming head's entry is ``p`` for the sink part (p < S) and ``S + r`` for
ring slot ``r``; the ring's append count starts once the sinks are full, so
position p >= S lands in ring slot (p - S) mod W.

Pins: the ring example printed in "Sliding-Window and Mixed Attention"
(window 3, positions 0..4), hand-derived counts of the guide's simulation
(4 layers x 8 heads, 512 tokens, S=4, W=16, R=0.25), and brute-force
equality of the kept positions with the visible set of the newest query.
"""
from __future__ import annotations

from typing import Any, Dict, List, Optional, Tuple


class RingWindow:
    """Ring buffer of capacity W: slot = (append count) mod W."""

    def __init__(self, window_size: int):
        assert window_size >= 1
        self.window_size = window_size
        self.items: List[Optional[Tuple[int, Any]]] = [None] * window_size
        self.length = 0

    def append(self, position: int, payload: Any) -> int:
        slot = self.length % self.window_size
        self.items[slot] = (position, payload)
        self.length += 1
        return slot

    def ordered(self) -> List[Tuple[int, Any]]:
        """Entries still held, oldest first."""
        count = min(self.length, self.window_size)
        return [self.items[i % self.window_size] for i in range(self.length - count, self.length)]


class StreamingHeadCache:
    """S sink slots followed by a W-slot ring."""

    def __init__(self, sink: int, recent: int):
        assert sink >= 0 and recent >= 1
        self.S = sink
        self.W = recent
        self.sinks: List[Tuple[int, Any]] = []
        self.ring = RingWindow(recent)

    def append(self, position: int, payload: Any = None) -> int:
        """Store one token; returns the physical slot it was written to."""
        if len(self.sinks) < self.S:
            self.sinks.append((position, payload))
            return len(self.sinks) - 1
        return self.S + self.ring.append(position, payload)

    def slots(self) -> Dict[int, Tuple[int, Any]]:
        """physical slot -> (position, payload) for every occupied slot."""
        out = {i: e for i, e in enumerate(self.sinks)}
        for r, e in enumerate(self.ring.items):
            if e is not None:
                out[self.S + r] = e
        return out

    def positions(self) -> List[int]:
        return sorted(p for p, _ in self.slots().values())


class RetrievalHeadCache:
    """Every token, slot = position order."""

    def __init__(self):
        self.items: List[Tuple[int, Any]] = []

    def append(self, position: int, payload: Any = None) -> int:
        self.items.append((position, payload))
        return len(self.items) - 1

    def slots(self) -> Dict[int, Tuple[int, Any]]:
        return {i: e for i, e in enumerate(self.items)}

    def positions(self) -> List[int]:
        return [p for p, _ in self.items]


def make_head_cache(is_retrieval: bool, sink: int, recent: int):
    return RetrievalHeadCache() if is_retrieval else StreamingHeadCache(sink, recent)


def kept_positions(T: int, is_retrieval: bool, sink: int, recent: int) -> List[int]:
    """Positions a head still holds after tokens 0..T-1 were appended, found by
    running the cache (not by a formula)."""
    c = make_head_cache(is_retrieval, sink, recent)
    for p in range(T):
        c.append(p)
    return c.positions()


def slot_table(T: int, is_retrieval: bool, sink: int, recent: int) -> Dict[int, int]:
    """physical slot -> position after T appends (for bit-exact layout checks)."""
    c = make_head_cache(is_retrieval, sink, recent)
    for p in range(T):
        c.append(p)
    return {s: p for s, (p, _) in c.slots().items()}


class DuoKVManagerCounts:
    """Slot accounting of the guide's head-separation simulation: the first
    max(1, int(L*H*R)) heads, scanning layers then heads, that sit in a layer
    >= 1 at an even head index are retrieval heads; counts of held slots and of
    heads still holding a given token."""

    def __init__(self, num_layers: int, num_heads: int, sink: int, recent: int, ratio: float):
        self.L, self.H = num_layers, num_heads
        budget = max(1, int(num_layers * num_heads * ratio))
        self.mask: Dict[Tuple[int, int], int] = {}
        assigned = 0
        for l in range(num_layers):
            for h in range(num_heads):
                take = assigned < budget and l >= 1 and h % 2 == 0
                self.mask[(l, h)] = 1 if take else 0
                assigned += int(take)
        self.caches = {k: make_head_cache(bool(m), sink, recent) for k, m in self.mask.items()}

    def ingest(self, total_tokens: int) -> None:
        for t in range(total_tokens):
            for c in self.caches.values():
                c.append(t)

    def held_slots(self) -> int:
        return sum(len(c.slots()) for c in self.caches.values())

    def heads_holding(self, position: int) -> Tuple[int, int]:
        ret = sum(1 for k, c in self.caches.items() if self.mask[k] and position in c.positions())
        st = sum(1 for k, c in self.caches.items() if not self.mask[k] and position in c.positions())
        return ret, st
