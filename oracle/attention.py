"""Masked softmax attention over a mixed KV cache, in float64 (oracle; test
infrastructure only).

What is computed (the plain definition; the GPU path must reach this result):

1. Head mapping.  Query head h reads KV head h // g with g = n_q / n_kv: the
   repeat_interleave expansion of "Attention Variants and Memory Efficiency",
   "Multi-Query and Grouped-Query Attention".  The retrieval/streaming role is
   a property of the KV head (DuoAttention guide, "Practical Deployment
   Checklist", GQA head-group consistency).
2. Visibility for a query at absolute position t (0-based).  Retrieval head:
   every key position j with 0 <= j <= t (guide, section 2: unrestricted access
   over the whole context).  Streaming head: 0 <= j <= t and (j < S or
   j >= t - W + 1): the S attention sinks plus the W most recent tokens, the
   query's own token included (guide, section 2; the window
   max(0, t-W+1) .. t of "Sliding-Window and Mixed Attention", read as exact).
3. Score s_j = scale * <q, k_j>, scale = 1/sqrt(d_head) (the pages state no
   scale; this is the standard one).
4. Softmax over the visible keys and the weighted sum of their values.
5. Chunked prefill.  Chunk row i sits at absolute position P + i, P = tokens
   already cached ("Attention Variants and KV-Cache Compression", "When Is Reuse
   Exact?"); its result is item 2-4 on the full sequence.  Read where the pages
   leave it open: the chunk attends over (cache before the chunk) plus the chunk,
   and only then is the chunk committed to the cache.

Two independent routes are provided and tested against each other:
  A. the cache route -- keys are what a simulated cache still holds
     (``oracle.cache``), with the visibility rule applied on their stored
     positions;
  B. the definition route -- every position 0..t is enumerated and the rule is
     applied directly (pure Python for tiny inputs, numpy for larger ones).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

from . import cache as _cache


# ---------------------------------------------------------------- definitions

def kv_head_of(h: int, n_q: int, n_kv: int) -> int:
    """KV head read by query head h under repeat_interleave(g) expansion."""
    assert n_q % n_kv == 0
    return h // (n_q // n_kv)


def visible(t: int, j: int, is_retrieval: bool, S: int, W: int) -> bool:
    """May the query at position t attend to the key at position j?"""
    if j < 0 or j > t:
        return False
    if is_retrieval:
        return True
    return j < S or j >= t - W + 1


def visible_matrix(t_rows: np.ndarray, positions: np.ndarray, is_retrieval: bool, S: int,
                   W: int) -> np.ndarray:
    """Vectorised ``visible``: bool [len(t_rows)][len(positions)]."""
    t = np.asarray(t_rows)[:, None]
    pos = np.asarray(positions)[None, :]
    ok = (pos >= 0) & (pos <= t)
    if not is_retrieval:
        ok &= (pos < S) | (pos >= t - W + 1)
    return ok


def visible_mask(t: int, positions: np.ndarray, is_retrieval: bool, S: int, W: int) -> np.ndarray:
    """``visible`` over an array of key positions for one query position."""
    return visible_matrix(np.array([t]), positions, is_retrieval, S, W)[0]


# ---------------------------------------------------------------- one query row

def attend_row(q: np.ndarray, keys: np.ndarray, values: np.ndarray, key_pos: Sequence[int],
               t: int, is_retrieval: bool, S: int, W: int, scale: float) -> np.ndarray:
    """Softmax attention of one query (position t) over the listed keys,
    keeping only the visible ones.  float64 throughout."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    vis = visible_mask(t, np.asarray(key_pos), is_retrieval, S, W)
    assert vis.any(), "a query always sees at least its own token"
    s = scale * (keys[vis] @ q)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ values[vis]


def softmax_weights(q, keys, key_pos, t, is_retrieval, S, W, scale):
    """(visible positions, weights) -- for invariant tests."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    kp = np.asarray(key_pos)
    vis = visible_mask(t, kp, is_retrieval, S, W)
    s = scale * (keys[vis] @ q)
    p = np.exp(s - s.max())
    return kp[vis], p / p.sum()


def attend_row_bruteforce(q: List[float], keys: List[List[float]], values: List[List[float]],
                          t: int, is_retrieval: bool, S: int, W: int, scale: float) -> List[float]:
    """Route B in pure Python: keys[j] / values[j] is the token at position j,
    for j = 0..t; enumerate, test visibility, softmax, sum."""
    scores = []
    for j in range(t + 1):
        if visible(t, j, is_retrieval, S, W):
            scores.append((j, scale * sum(a * b for a, b in zip(q, keys[j]))))
    top = max(s for _, s in scores)
    ws = [(j, math.exp(s - top)) for j, s in scores]
    z = sum(w for _, w in ws)
    d = len(values[0])
    return [sum(w * values[j][c] for j, w in ws) / z for c in range(d)]


# ---------------------------------------------------------------- decode step

def decode_step(q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: Sequence[int],
                S: int, W: int, scale: float, route: str = "cache") -> np.ndarray:
    """One decode step at context T = K.shape[1]: the query of every head sits
    at position T-1 and the cache holds tokens 0..T-1.

    q: [n_q][d]; K, V: [n_kv][T][d] (the full token stream, position = row);
    mask: [n_kv], 1 = retrieval.  Returns [n_q][d] float64.

    route "cache": keys are the positions the simulated cache still holds.
    route "definition": all positions 0..T-1 with the visibility rule.
    """
    n_q, d = q.shape
    n_kv, T, _ = K.shape
    out = np.zeros((n_q, d), dtype=np.float64)
    t = T - 1
    held = {}  # the keep set depends only on the head kind; simulate each kind once
    for h in range(n_q):
        k = kv_head_of(h, n_q, n_kv)
        ret = bool(mask[k])
        if route == "cache":
            if ret not in held:
                held[ret] = np.asarray(_cache.kept_positions(T, ret, S, W), dtype=np.int64)
            pos = held[ret]
        else:
            pos = np.arange(T, dtype=np.int64)
        out[h] = attend_row(q[h], K[k][pos], V[k][pos], pos, t, ret, S, W, scale)
    return out


def kept_rows(T: int, is_retrieval: bool, S: int, W: int) -> np.ndarray:
    """Kept positions after T appends, from the cache simulation, as an array."""
    return np.asarray(_cache.kept_positions(T, is_retrieval, S, W), dtype=np.int64)


# ---------------------------------------------------------------- prefill

def attend_rows(Q: np.ndarray, t_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                key_pos: np.ndarray, is_retrieval: bool, S: int, W: int, scale: float,
                block: int = 256) -> np.ndarray:
    """Rows of Q (query positions t_rows) against keys at positions key_pos:
    a dense score matrix, the visibility rule as a boolean mask, softmax along
    keys.  Processed in row blocks only to bound memory."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    kp = np.asarray(key_pos)
    out = np.empty((Q.shape[0], V.shape[1]), dtype=np.float64)
    for r0 in range(0, Q.shape[0], block):
        r1 = min(r0 + block, Q.shape[0])
        ok = visible_matrix(np.asarray(t_rows[r0:r1]), kp, is_retrieval, S, W)
        s = scale * (Q[r0:r1] @ K.T)
        s = np.where(ok, s, -np.inf)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r1] = p @ V
    return out


def prefill_full(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: Sequence[int],
                 S: int, W: int, scale: float, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Definition route for a whole sequence: Q [n_q][N][d] (row = position),
    K, V [n_kv][N][d].  Returns [n_q][len(rows)][d] for the requested positions
    (all N by default)."""
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((n_q, len(rows), d), dtype=np.float64)
    for h in range(n_q):
        k = kv_head_of(h, n_q, n_kv)
        hi = int(rows.max()) + 1 if len(rows) else 0
        out[h] = attend_rows(Q[h][rows], rows, K[k][:hi], V[k][:hi], np.arange(hi),
                             bool(mask[k]), S, W, scale)
    return out


def prefill_chunked(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mask: Sequence[int],
                    S: int, W: int, scale: float, chunk: int) -> np.ndarray:
    """Cache route for a whole sequence processed in chunks: each chunk attends
    over what the simulated cache holds plus the chunk itself (positions kept
    as original), then the chunk is committed and the cache evicts as it must.
    Returns [n_q][N][d]."""
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    out = np.empty((n_q, N, d), dtype=np.float64)
    caches = [_cache.make_head_cache(bool(mask[k]), S, W) for k in range(n_kv)]
    for P in range(0, N, chunk):
        C = min(chunk, N - P)
        for h in range(n_q):
            k = kv_head_of(h, n_q, n_kv)
            held = np.asarray(caches[k].positions(), dtype=np.int64)
            kp = np.concatenate([held, np.arange(P, P + C)])
            out[h, P:P + C] = attend_rows(Q[h, P:P + C], np.arange(P, P + C), K[k][kp], V[k][kp],
                                          kp, bool(mask[k]), S, W, scale)
        for k in range(n_kv):
            for p in range(P, P + C):
                caches[k].append(p)
    return out
