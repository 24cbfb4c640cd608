"""Simulation of the mixed KV cache's contents (oracle; test infrastructure only).

A retrieval head keeps every token in order (DuoAttention guide, section "2.
DuoAttention Cache Partitioning Mechanics": one full, contiguous buffer of
all the tokens).  A streaming head keeps S attention-sink entries, filled
first, and after them a window of the W most recent entries in which a new
token replaces the oldest one (same section, and the append rule of the
guide's head-separation simulation in "Implementation: Simulating
DuoAttention Head Separation in Python").  "Attention Variants and Memory
Efficiency", "Sliding-Window and Mixed Attention" places window entries in a
circular buffer by their arrival count modulo the window size and keeps each
token's logical position beside it.

Reading taken where the pages leave a step open: a streaming head has S + W
physical slots.  The n-th token it receives (n = 0, 1, ...) goes to slot n
while n < S, and afterwards to slot S + ((n - S) mod W): the window's own
arrival count starts once the sinks are full.  Tokens arrive in position
order from position 0, so n is the token's position.

Every head here is a table slot -> (position, payload); what a head holds
and in what order is read off that table.

Pins: the circular-buffer example printed in "Sliding-Window and Mixed
Attention" (window 3, positions 0..4), hand-derived counts of the guide's
simulation (4 layers x 8 heads, 512 tokens, S=4, W=16, R=0.25), and
brute-force equality of the kept positions with the visible set of the
newest query.
"""
from __future__ import annotations

from typing import Any, Dict, List, Tuple


def streaming_slot(n: int, S: int, W: int) -> int:
    """Physical slot of the n-th token a streaming head receives."""
    return n if n < S else S + (n - S) % W


class _HeadTable:
    """Slot table of one head: slot -> (position, payload)."""

    def __init__(self):
        self.table: Dict[int, Tuple[int, Any]] = {}
        self.received = 0

    def slots(self) -> Dict[int, Tuple[int, Any]]:
        return dict(self.table)

    def positions(self) -> List[int]:
        """Held positions, ascending."""
        return sorted(p for p, _ in self.table.values())

    def ordered(self) -> List[Tuple[int, Any]]:
        """Held (position, payload) entries, oldest first."""
        return sorted(self.table.values(), key=lambda e: e[0])


class StreamingHeadCache(_HeadTable):
    """S sink slots, then a W-slot window."""

    def __init__(self, sink: int, recent: int):
        super().__init__()
        assert sink >= 0 and recent >= 1
        self.S, self.W = sink, recent

    def append(self, position: int, payload: Any = None) -> int:
        """Store one token; returns the physical slot it went to (the entry
        there before it, if any, is dropped)."""
        slot = streaming_slot(self.received, self.S, self.W)
        self.table[slot] = (position, payload)
        self.received += 1
        return slot


class RetrievalHeadCache(_HeadTable):
    """Every token; the n-th token received sits in slot n."""

    def append(self, position: int, payload: Any = None) -> int:
        slot = self.received
        self.table[slot] = (position, payload)
        self.received += 1
        return slot


def make_head_cache(is_retrieval: bool, sink: int, recent: int):
    return RetrievalHeadCache() if is_retrieval else StreamingHeadCache(sink, recent)


def _filled(T: int, is_retrieval: bool, sink: int, recent: int):
    c = make_head_cache(is_retrieval, sink, recent)
    for p in range(T):
        c.append(p)
    return c


def kept_positions(T: int, is_retrieval: bool, sink: int, recent: int) -> List[int]:
    """Positions a head still holds after tokens 0..T-1 were appended, found by
    running the cache (not by a formula)."""
    return _filled(T, is_retrieval, sink, recent).positions()


def slot_table(T: int, is_retrieval: bool, sink: int, recent: int) -> Dict[int, int]:
    """physical slot -> position after T appends (for bit-exact layout checks)."""
    return {s: p for s, (p, _) in _filled(T, is_retrieval, sink, recent).slots().items()}


class DuoKVManagerCounts:
    """Slot accounting of the guide's head-separation simulation.

    Which heads are retrieval heads: the simulation's budget is
    max(1, floor(L * H * R)) heads, and the heads eligible for it are those of
    layers 1 .. L-1 at even head indices, taken in (layer, head) order.  The
    mask is the first `budget` eligible heads.  Every head then receives the
    same token stream; the counts below are read off the heads' slot tables."""

    def __init__(self, num_layers: int, num_heads: int, sink: int, recent: int, ratio: float):
        self.L, self.H = num_layers, num_heads
        budget = max(1, int(num_layers * num_heads * ratio))
        eligible = [(l, h) for l in range(1, num_layers) for h in range(0, num_heads, 2)]
        chosen = set(eligible[:budget])
        self.mask: Dict[Tuple[int, int], int] = {(l, h): int((l, h) in chosen)
                                                  for l in range(num_layers) for h in range(num_heads)}
        self.caches = {k: make_head_cache(bool(m), sink, recent) for k, m in self.mask.items()}

    def ingest(self, total_tokens: int) -> None:
        for c in self.caches.values():
            for t in range(total_tokens):
                c.append(t)

    def held_slots(self) -> int:
        return sum(len(c.slots()) for c in self.caches.values())

    def heads_holding(self, position: int) -> Tuple[int, int]:
        """(retrieval heads, streaming heads) that still hold `position`."""
        holding = [k for k, c in self.caches.items() if position in c.positions()]
        ret = sum(self.mask[k] for k in holding)
        return ret, len(holding) - ret
