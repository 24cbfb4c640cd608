"""FP8 (E4M3) key/value rows with one scale per row (oracle; test
infrastructure only).

What is computed.  "DuoAttention: Dual Retrieval & Streaming Heads Guide",
"Production Advantages and Deployment Considerations", item 2 (synergies with
low-bit quantization): FP8 or INT4 KV quantization stores each cache element
in 8 or 4 bits instead of 16 (a 2x to 4x smaller cache) and composes with the
head-level split.  "Attention Variants and KV-Cache Compression",
"Compressing an existing cache", and "Attention Variants and Memory
Efficiency", "What the Inference Runtime Can Change", describe cache
quantization as a change of the bytes per stored element that keeps the
attention rule.  The pages fix no format; the readings taken here:

  * the 8-bit format is E4M3 as defined by the OCP 8-bit floating-point
    specification: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    no infinities; exponent and mantissa all ones is NaN, so the largest
    finite magnitude is 1.75 * 2^8 = 448; subnormals are m * 2^-9, m = 1..7;
  * one scale per stored row (one token of one KV head; K and V rows
    separately): s = max_i |x_i| / 448, computed in float32 (a correctly
    rounded division), and element i is stored as the E4M3 value nearest to
    x_i / s (that quotient also computed in float32), ties to the even
    mantissa; a row of zeros has s = 0 and all codes 0;
  * attention over a quantized cache is attention over the dequantized rows
    code_value * s (exactly, in float64).  Queries, the new token's inputs
    and the outputs stay in the cache dtype (bf16).

Pinned by ``tests/oracle_checks.py``: the encoder against torch's
float8_e4m3fn cast on a dense sweep of float32 values (every tie and the
subnormal range included), the decoder against the same library on all 256
codes, the row quantizer against the format's error bound, and the chunked
prefill and decode routes, off the E4M3 grid and over several chunks, against
an enumeration over positions whose held rows are built with the library's
E4M3 conversion (a held row read as given fails that pin).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6   # smallest normal: 2^-6
E4M3_SUBNORMAL_QUANTUM = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8), in float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * E4M3_SUBNORMAL_QUANTUM
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def _round_half_even(y: np.ndarray) -> np.ndarray:
    """Nearest integer, ties to even (y >= 0, exact in float64)."""
    f = np.floor(y)
    r = y - f
    up = (r > 0.5) | ((r == 0.5) & (np.fmod(f, 2.0) == 1.0))
    return f + up


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code (uint8) of the value nearest to each float32 x, ties to even.
    Magnitudes from 448 up to (not including) 464 round to 448; larger ones are
    outside what the row quantizer can produce and raise."""
    a32 = np.asarray(x, dtype=np.float32)
    a = np.abs(a32.astype(np.float64))
    if np.any(~np.isfinite(a)) or np.any(a >= 464.0):
        raise ValueError("E4M3 encode: input outside the rounding range of the format")
    sign = np.signbit(a32).astype(np.int64)
    # quantum of the binade each magnitude falls in (subnormal binade: 2^-9)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ex = np.maximum(ex, E4M3_MIN_NORMAL_EXP)
    # floor(log2) of a float64 can be off by one next to a power of two; fix it
    ex = np.where(np.exp2(ex) > a, ex - 1, ex)
    ex = np.where(np.exp2(ex + 1) <= a, ex + 1, ex)
    ex = np.maximum(ex, E4M3_MIN_NORMAL_EXP)
    quantum = np.exp2(ex - 3.0)
    v = _round_half_even(a / quantum) * quantum  # exact: quantum is a power of two
    v = np.minimum(v, E4M3_MAX)
    # bits of v
    normal = v >= 2.0 ** E4M3_MIN_NORMAL_EXP
    with np.errstate(divide="ignore"):
        ev = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    ev = np.where(np.exp2(ev) > v, ev - 1, ev)
    mant_n = np.round((v / np.exp2(ev) - 1.0) * 8.0)
    bits_n = ((ev + 7).astype(np.int64) << 3) | mant_n.astype(np.int64)
    bits_s = np.round(v / E4M3_SUBNORMAL_QUANTUM).astype(np.int64)
    bits = np.where(normal, bits_n, bits_s)
    return ((sign << 7) | bits).astype(np.uint8)


def quantize_rows(X) -> tuple:
    """X float32 [..., d] -> (codes uint8 [..., d], scale float32 [...])."""
    X = np.asarray(X, dtype=np.float32)
    absmax = np.max(np.abs(X), axis=-1)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (X / safe[..., None]).astype(np.float32)  # float32 division, correctly rounded
    codes = e4m3_encode(q)
    codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize_rows(codes, scale) -> np.ndarray:
    """Rows as the attention sees them: code value * scale, in float64."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# ---------------------------------------------------------------- attention over FP8 rows

def stored_values(X) -> np.ndarray:
    """What a cache of FP8 rows holds for rows X (float32 [..., d]): the
    dequantized rows, in float64."""
    return dequantize_rows(*quantize_rows(X))


def decode_step_fp8(q, K, V, mask, S, W, scale):
    """Decode over a cache of FP8 rows: every held key and value is the stored
    (dequantized) row; q [n_q][d], K, V [n_kv][T][d] as float32 inputs."""
    from . import attention as _att
    return _att.decode_step(np.asarray(q, dtype=np.float64), stored_values(K), stored_values(V), mask, S, W, scale)


def prefill_chunked_fp8(Q, K, V, mask, S, W, scale, chunk):
    """Chunked prefill over a cache of FP8 rows (cache route, [n_q][N][d]):
    chunk rows attend over the held rows as stored (dequantized) plus the
    chunk's own rows as given; the chunk is then committed (quantized).
    `chunk` is one chunk length or the sequence of chunk lengths."""
    from . import attention as _att
    from . import cache as _cache
    Q = np.asarray(Q, dtype=np.float64)
    K64, V64 = np.asarray(K, dtype=np.float64), np.asarray(V, dtype=np.float64)
    Kq, Vq = stored_values(K), stored_values(V)
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    out = np.empty((n_q, N, d), dtype=np.float64)
    caches = [_cache.make_head_cache(bool(mask[k]), S, W) for k in range(n_kv)]
    lengths = [chunk] * ((N + chunk - 1) // chunk) if np.isscalar(chunk) else list(chunk)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    assert sum(lengths) >= N
    for P, C in zip(starts, lengths):
        C = int(min(C, N - P))
        for h in range(n_q):
            k = _att.kv_head_of(h, n_q, n_kv)
            held = np.asarray(caches[k].positions(), dtype=np.int64)
            kp = np.concatenate([held, np.arange(P, P + C)])
            keys = np.concatenate([Kq[k][held], K64[k][P:P + C]])
            vals = np.concatenate([Vq[k][held], V64[k][P:P + C]])
            out[h, P:P + C] = _att.attend_rows(Q[h, P:P + C], np.arange(P, P + C), keys, vals, kp,
                                               bool(mask[k]), S, W, scale)
        for k in range(n_kv):
            for p in range(P, P + C):
                caches[k].append(p)
    return out
