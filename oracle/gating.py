"""Head-gated blend of full and streaming attention, in float64 (oracle; test
infrastructure only).

What is computed.  "DuoAttention: Dual Retrieval & Streaming Heads Guide",
section 3 ("Automated Head Identification via Lightweight Optimization"),
item 2 (differentiable head gating): while heads are being identified, every
head carries a continuous gate alpha in [0, 1], and its output is alpha times
full attention plus (1 - alpha) times streaming attention, both taken over the
same queries, keys and values.  This module states that forward pass; the
gradient step and the sparsity penalty of item 3 are not part of it.

Readings where the page leaves the step open:
  * one gate per KV head, shared by the g query heads that read that KV head:
    the gate relaxes the retrieval/streaming role, and that role is a property
    of the KV head (guide, "Practical Deployment Checklist", GQA head-group
    consistency);
  * full attention is the causal mask; streaming attention is the sink + window
    mask with the same S and W the cache keeps (key j visible to the query at t
    iff j <= t and (j < S or j >= t - W + 1)), i.e. ``attention.visible``;
  * the forward runs over one whole sequence at positions 0 .. N-1 (no cache);
  * alpha is used as given: the blend is affine in alpha and nothing clips it.

Two routes, compared by the pins in ``tests/oracle_checks.py``: the numpy route
(``gated_forward``, through ``attention.prefill_full``) and a pure-Python
enumeration for tiny inputs (``gated_row_bruteforce``, through
``attention.attend_row_bruteforce``).  Both are pinned to a hand-derived value
(``tests/golden/gated_tiny.txt``), to torch's scaled_dot_product_attention at
alpha = 1 (causal) and alpha = 0 with S = 0 (a band mask), and to the
repeat_interleave expansion of GQA.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import attention as _att


def gate_of_query_heads(alpha: Sequence[float], n_q: int) -> np.ndarray:
    """The gate each query head uses: that of the KV head it reads."""
    n_kv = len(alpha)
    return np.array([float(alpha[_att.kv_head_of(h, n_q, n_kv)]) for h in range(n_q)], dtype=np.float64)


def blend(full, stream, a):
    """alpha * FullAttn + (1 - alpha) * StreamAttn (guide, section 3, item 2)."""
    return a * full + (1.0 - a) * stream


def gated_forward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, alpha: Sequence[float],
                  S: int, W: int, scale: float, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Q [n_q][N][d] (row = position), K, V [n_kv][N][d], alpha [n_kv].
    Returns [n_q][len(rows)][d] for the requested positions (all N by default)."""
    n_q = Q.shape[0]
    n_kv = K.shape[0]
    assert len(alpha) == n_kv
    full = _att.prefill_full(Q, K, V, [1] * n_kv, S, W, scale, rows)
    stream = _att.prefill_full(Q, K, V, [0] * n_kv, S, W, scale, rows)
    a = gate_of_query_heads(alpha, n_q)[:, None, None]
    return blend(full, stream, a)


def gated_row_bruteforce(q: List[float], keys: List[List[float]], values: List[List[float]],
                         t: int, alpha: float, S: int, W: int, scale: float) -> List[float]:
    """One query at position t over keys/values at positions 0 .. len(keys)-1,
    by enumerating the visibility rule (pure Python, tiny inputs)."""
    full = _att.attend_row_bruteforce(q, keys, values, t, True, S, W, scale)
    stream = _att.attend_row_bruteforce(q, keys, values, t, False, S, W, scale)
    return [blend(f, s, alpha) for f, s in zip(full, stream)]
