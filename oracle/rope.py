"""Rotary position embedding at each token's logical position (oracle; test
infrastructure only).

What is computed.  "Attention Variants and Memory Efficiency", "Sliding-Window
and Mixed Attention": a cached token's position information is its logical
position, not the ring-buffer slot it occupies; "What the Inference Runtime
Can Change": an attention kernel must apply the positional treatment the
checkpoint expects.  The pages name no positional encoding.  The reading
taken is the rotary position embedding published by Su et al., "RoFormer:
Enhanced Transformer with Rotary Position Embedding" (2021): pairs of
dimensions are rotated by an angle proportional to the position, pair i with
frequency theta^(-2i/d), so that the score of a rotated query and a rotated key
depends on their positions only through the difference.

Readings taken where the pages leave a step open:
  * pairing: dimension i with dimension i + d/2, i = 0 .. d/2 - 1 (the
    rotate-half layout of the LLaMA-family checkpoints whose shapes the
    workloads take; the paper pairs adjacent dimensions, which is the same
    rotation after a fixed permutation of the head dimension);
  * angle of pair i at position p: p * theta^(-2i/d); theta (the base) is a
    parameter of the cache (10000 in the paper);
  * a key is rotated at its logical position when it is stored, so a
    streaming head's ring slot never changes a key's rotation; a query is
    rotated at its own position (decode: the position of the token the step
    appends; prefill: P + i for chunk row i);
  * rotations are computed in float64.  The cache stores a rotated key
    rounded to its dtype (bf16: to nearest, ties to even); a query is used as
    rotated; in prefill the chunk's own keys are attended as rotated (before
    they are stored) and the held keys as stored.  Values are not rotated.

Pinned by tests/oracle_checks.py: unit vectors at position 1 for d = 8,
theta = 10^4 (frequencies 1, 0.1, 0.01, 0.001 exactly), the complex-number
form of the rotation, the relative-position property of scores, the bf16
rounding against torch's conversion, decode over the cache's slots
against the definition route over logical positions, and chunked prefill over
FP8 and INT4 rows against enumerations built from the complex-number
rotation, torch's bf16 rounding and torch's E4M3 conversion or rounding.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def inv_freq(d: int, theta: float) -> np.ndarray:
    """theta^(-2i/d) for i = 0 .. d/2 - 1, float64."""
    assert d % 2 == 0 and theta > 0
    return np.power(float(theta), -2.0 * np.arange(d // 2, dtype=np.float64) / d)


def rotate(X, positions, theta: float) -> np.ndarray:
    """X [..., n, d] at positions [n] -> rotated, float64.  For pair i,
    (x_i, x_{i+d/2}) -> (x_i cos a - x_{i+d/2} sin a, x_{i+d/2} cos a + x_i sin a)
    with a = position * theta^(-2i/d)."""
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[-1]
    h = d // 2
    a = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq(d, theta)[None, :]  # [n][d/2]
    c, s = np.cos(a), np.sin(a)
    lo, hi = X[..., :h], X[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits), ties to even,
    returned as float64 (normal range; the rows here never reach bf16's
    subnormals)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)  # np.rint rounds ties to even


def round_to(x, dtype: str) -> np.ndarray:
    """The cache dtype's rounding of float64 values: bf16, or float32."""
    if dtype == "bf16":
        return round_bf16(x)
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _low_bit_store(kv_format):
    """What a cache of low-bit rows keeps for float32 rows (None: as given)."""
    if kv_format == "fp8":
        from . import quant as _q
        return _q.stored_values
    if kv_format == "int4":
        from . import quant4 as _q4
        return _q4.stored_values_int4
    return None


def stored_keys(K, theta: float, dtype: str, kv_format=None) -> np.ndarray:
    """K [n_kv][T][d] (row = position) -> what the cache holds: each row
    rotated at its position and rounded to the cache dtype, float64.  With
    FP8 rows (oracle.quant) or INT4 rows (oracle.quant4) the rotated, rounded
    row is what is quantized."""
    K = np.asarray(K, dtype=np.float64)
    Ks = round_to(rotate(K, np.arange(K.shape[-2]), theta), dtype)
    store = _low_bit_store(kv_format)
    if store is not None:
        Ks = store(Ks.astype(np.float32))
    return Ks


def stored_values(V, kv_format=None) -> np.ndarray:
    """What the cache holds for value rows V (float32 inputs): as given, or
    the dequantized low-bit rows."""
    store = _low_bit_store(kv_format)
    if store is not None:
        return store(np.asarray(V, dtype=np.float32))
    return np.asarray(V, dtype=np.float64)


def decode_step_rope(q, K, V, mask: Sequence[int], S: int, W: int, scale: float, theta: float, dtype: str,
                     route: str = "cache", kv_format=None):
    """Decode at position T - 1 (T = K.shape[1]): the query q [n_q][d]
    rotated at T - 1 against the stored (rotated, rounded) keys and the
    stored values."""
    from . import attention as _att
    K = np.asarray(K, dtype=np.float64)
    T = K.shape[1]
    qr = rotate(np.asarray(q, dtype=np.float64)[:, None, :], [T - 1], theta)[:, 0, :]
    return _att.decode_step(qr, stored_keys(K, theta, dtype, kv_format), stored_values(V, kv_format), mask, S, W,
                            scale, route=route)


def prefill_chunked_rope(Q, K, V, mask: Sequence[int], S: int, W: int, scale: float, theta: float, dtype: str,
                         chunks, kv_format=None) -> np.ndarray:
    """Chunked prefill ([n_q][N][d], [n_kv][N][d]; N = sum(chunks)): chunk
    row i at position P + i attends, with its query rotated at P + i, over the
    held keys and values as stored and the chunk's own keys as rotated (its
    values as given); then the chunk is stored."""
    from . import attention as _att
    from . import cache as _cache
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    Qr = rotate(Q, np.arange(N), theta)
    Kr = rotate(K, np.arange(N), theta)
    Ks = stored_keys(K, theta, dtype, kv_format)
    Vs = stored_values(V.astype(np.float32) if kv_format else V, kv_format)
    out = np.empty((n_q, N, d), dtype=np.float64)
    heads = [_cache.make_head_cache(bool(mask[k]), S, W) for k in range(n_kv)]
    P = 0
    for C in chunks:
        C = int(min(C, N - P))
        for h in range(n_q):
            k = _att.kv_head_of(h, n_q, n_kv)
            held = np.asarray(heads[k].positions(), dtype=np.int64)
            kp = np.concatenate([held, np.arange(P, P + C)])
            keys = np.concatenate([Ks[k][held], Kr[k][P:P + C]])
            vals = np.concatenate([Vs[k][held], V[k][P:P + C]])
            out[h, P:P + C] = _att.attend_rows(Qr[h, P:P + C], np.arange(P, P + C), keys, vals, kp, bool(mask[k]),
                                               S, W, scale)
        for k in range(n_kv):
            for p in range(P, P + C):
                heads[k].append(p)
        P += C
    return out
