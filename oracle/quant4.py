"""INT4 key/value rows with one scale per row (oracle; test infrastructure
only).

What is computed.  "DuoAttention: Dual Retrieval & Streaming Heads Guide",
"Production Advantages and Deployment Considerations", item 2 (synergies with
low-bit quantization): INT4 KV quantization keeps each cache element in 4
bits instead of 16, a 4x smaller cache, on top of the head-level split;
"Attention Variants and Memory Efficiency", "What the Inference Runtime Can
Change": cache precision changes the bytes per stored element, not the
attention rule.  The pages fix no INT4 format; the readings taken here:

  * levels: a 4-bit code n (0..15) stands for the integer n - 8, the sixteen
    levels -8 .. 7 (offset binary);
  * one scale per stored row (one token of one KV head; K and V rows
    separately), the row being the quantization group:
    s = max_i |x_i| / 7 in float32 (a correctly rounded division); element i
    is stored as c_i, the integer nearest to x_i / s (that quotient also in
    float32), ties to even, kept within -7 .. 7, as the code n_i = c_i + 8
    (level -8 is never produced); a row of zeros has s = 0 and every c_i = 0;
  * two codes per byte: element 2k in the low nibble of byte k, element
    2k + 1 in the high nibble;
  * attention over the cache is attention over c_i * s (exactly, in float64).
    Queries, new-token inputs and outputs stay in the cache dtype (bf16).

Pinned by ``tests/oracle_checks.py``: the level table and hand-worked rows
(scale, ties to even, code bytes) from ``tests/golden/int4_rows.txt``; the
quantizer against torch's round-half-to-even and the half-step error bound;
rows already on the grid coming back exactly; and the decode and chunked
prefill routes against enumerations over positions whose held rows are built
independently.
"""
from __future__ import annotations

import numpy as np

INT4_OFFSET = 8     # code n stands for the level n - 8
INT4_QMAX = 7.0     # largest level magnitude the quantizer uses


def int4_levels() -> np.ndarray:
    """Level of each code 0..15 (int64)."""
    return np.arange(16, dtype=np.int64) - INT4_OFFSET


def quantize_rows_int4(X) -> tuple:
    """X float32 [..., d] -> (codes uint8 [..., d] in 0..15, scale float32 [...])."""
    X = np.asarray(X, dtype=np.float32)
    absmax = np.max(np.abs(X), axis=-1)
    scale = (absmax / np.float32(INT4_QMAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    quot = (X / safe[..., None]).astype(np.float32)                  # float32 division, correctly rounded
    c = np.rint(quot.astype(np.float64))                              # nearest integer, ties to even
    c = np.clip(c, -INT4_QMAX, INT4_QMAX)
    c = np.where(scale[..., None] > 0, c, 0.0)
    return (c + INT4_OFFSET).astype(np.uint8), scale


def pack_nibbles(codes) -> np.ndarray:
    """codes uint8 [..., d] (0..15, d even) -> bytes uint8 [..., d / 2]:
    element 2k in the low nibble of byte k, element 2k + 1 in the high one."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    """The inverse of pack_nibbles."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def dequantize_rows_int4(codes, scale) -> np.ndarray:
    """Rows as the attention sees them: level * scale, in float64."""
    lv = int4_levels()[np.asarray(codes, dtype=np.int64)]
    return lv.astype(np.float64) * np.asarray(scale, dtype=np.float64)[..., None]


def stored_values_int4(X) -> np.ndarray:
    """What a cache of INT4 rows holds for rows X (float32 [..., d]), in float64."""
    return dequantize_rows_int4(*quantize_rows_int4(X))


# ---------------------------------------------------------------- attention over INT4 rows

def decode_step_int4(q, K, V, mask, S, W, scale):
    """Decode over a cache of INT4 rows: every held key and value is the
    stored row; q [n_q][d], K, V [n_kv][T][d] as float32 inputs."""
    from . import attention as _att
    return _att.decode_step(np.asarray(q, dtype=np.float64), stored_values_int4(K), stored_values_int4(V), mask, S,
                            W, scale)


def prefill_chunked_int4(Q, K, V, mask, S, W, scale, chunk):
    """Chunked prefill over a cache of INT4 rows (cache route, [n_q][N][d]):
    chunk rows attend over the held rows as stored plus the chunk's own rows as
    given; the chunk is then committed (quantized).  `chunk` is one chunk
    length or the sequence of chunk lengths."""
    from . import attention as _att
    from . import cache as _cache
    Q = np.asarray(Q, dtype=np.float64)
    K64, V64 = np.asarray(K, dtype=np.float64), np.asarray(V, dtype=np.float64)
    Ks, Vs = stored_values_int4(K), stored_values_int4(V)
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    out = np.empty((n_q, N, d), dtype=np.float64)
    heads = [_cache.make_head_cache(bool(mask[k]), S, W) for k in range(n_kv)]
    lengths = [chunk] * ((N + chunk - 1) // chunk) if np.isscalar(chunk) else list(chunk)
    P = 0
    for C in lengths:
        C = int(min(C, N - P))
        for h in range(n_q):
            k = _att.kv_head_of(h, n_q, n_kv)
            held = np.asarray(heads[k].positions(), dtype=np.int64)
            kp = np.concatenate([held, np.arange(P, P + C)])
            keys = np.concatenate([Ks[k][held], K64[k][P:P + C]])
            vals = np.concatenate([Vs[k][held], V64[k][P:P + C]])
            out[h, P:P + C] = _att.attend_rows(Q[h, P:P + C], np.arange(P, P + C), keys, vals, kp,
                                               bool(mask[k]), S, W, scale)
        for k in range(n_kv):
            for p in range(P, P + C):
                heads[k].append(p)
        P += C
    return out
