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

cos_sin_exact / rotate_exact (positions up to 2^31) are pinned by integer
angles (pair 0 at any base, and base 10^4 with d = 8 at positions that are
multiples of 1000) against the C library's cosine and sine, and by agreement
with rotate() at positions where float64 angles are exact to 1e-10.

Pinned by tests/oracle_checks.py: unit vectors at position 1 for d = 8,
theta = 10^4 (frequencies 1, 0.1, 0.01, 0.001 exactly), the complex-number
form of the rotation, the relative-position property of scores, the bf16
rounding against torch's conversion, decode over the cache's slots
against the definition route over logical positions, and chunked prefill over
FP8 and INT4 rows against enumerations built from the complex-number
rotation, torch's bf16 rounding and torch's E4M3 conversion or rounding.
"""
from __future__ import annotations

from decimal import Context, Decimal, localcontext
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


def _dec_pi(ctx):
    """pi in the context's precision from Machin's formula
    pi = 16 arctan(1/5) - 4 arctan(1/239), arctan(1/n) by its series."""
    def arctan_inv(n):
        x = ctx.divide(1, n)
        x2 = x * x
        term, total, k = x, x, 1
        eps = Decimal(10) ** (-(ctx.prec + 2))
        while True:
            term = -term * x2
            k += 2
            t = term / k
            if abs(t) < eps:
                return total
            total += t
    return 16 * arctan_inv(5) - 4 * arctan_inv(239)


def cos_sin_exact(p: int, i: int, d: int, theta: float, digits: int = 40):
    """(cos a, sin a) of the angle a = p * theta^(-2i/d) of pair i at position
    p, to about `digits` decimal digits, as Decimals: theta^(-2i/d) by
    Python's decimal power (correctly rounded in its context), a reduced
    modulo 2 pi with pi from Machin's formula, then the Taylor series of cosine
    and sine.  For positions where a float64 angle p * f is off by up to
    p * f * 2^-53 (about 2.4e-7 rad at p = 2^31)."""
    ctx = Context(prec=digits + 25)
    with localcontext(ctx) as c:
        f = Decimal(float(theta)) ** (Decimal(-2 * i) / Decimal(d))
        a = Decimal(int(p)) * f
        two_pi = 2 * _dec_pi(c)
        r = a - (a / two_pi).to_integral_value() * two_pi  # |r| <= pi
        r2 = r * r
        cos_t, sin_t = Decimal(1), r
        cs, sn, k = cos_t, sin_t, 0
        eps = Decimal(10) ** (-(digits + 20))
        while True:
            k += 2
            cos_t = -cos_t * r2 / ((k - 1) * k)
            sin_t = -sin_t * r2 / (k * (k + 1))
            cs += cos_t
            sn += sin_t
            if abs(cos_t) < eps and abs(sin_t) < eps:
                return +cs, +sn


def rotate_exact(X, positions, theta: float) -> np.ndarray:
    """rotate() with every angle from cos_sin_exact and every rotated value
    computed in decimal and rounded once to float64: X [n][d] (few rows)."""
    X = np.asarray(X, dtype=np.float64)
    n, d = X.shape
    h = d // 2
    out = np.empty_like(X)
    for r in range(n):
        for i in range(h):
            cs, sn = cos_sin_exact(int(positions[r]), i, d, theta)
            x, y = Decimal(float(X[r, i])), Decimal(float(X[r, i + h]))
            with localcontext(Context(prec=60)):
                out[r, i] = float(x * cs - y * sn)
                out[r, i + h] = float(y * cs + x * sn)
    return out


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
