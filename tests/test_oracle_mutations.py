"""Plant plausible mistakes into the oracle (on the CPU) and check that at
least one pin catches each of them."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import cache as Cc
from oracle import gating as G
from oracle import paging as PG
from oracle import rope as RP
from oracle import quant as QZ
from oracle import quant4 as Q4
from oracle import sizes as Z
from tests import oracle_checks as OC


def _window_too_wide(t_rows, positions, is_retrieval, S, W):
    t = np.asarray(t_rows)[:, None]; pos = np.asarray(positions)[None, :]
    ok = (pos >= 0) & (pos <= t)
    if not is_retrieval:
        ok &= (pos < S) | (pos >= t - W)          # W+1 recent tokens
    return ok


def _sinks_off_by_one(t_rows, positions, is_retrieval, S, W):
    t = np.asarray(t_rows)[:, None]; pos = np.asarray(positions)[None, :]
    ok = (pos >= 0) & (pos <= t)
    if not is_retrieval:
        ok &= (pos <= S) | (pos >= t - W + 1)      # S+1 sinks
    return ok


def _no_causal(t_rows, positions, is_retrieval, S, W):
    t = np.asarray(t_rows)[:, None]; pos = np.asarray(positions)[None, :] + 0 * t
    ok = pos >= 0
    if not is_retrieval:
        ok &= (pos < S) | (pos >= t - W + 1)
    return ok


def _wrong_scalar_window(t, j, is_retrieval, S, W):
    if j < 0 or j > t:
        return False
    return is_retrieval or j < S or j > t - W + 1  # W-1 recent tokens


def _head_mod(h, n_q, n_kv):
    return h % n_kv                                # transposed GQA mapping


def _attend_no_scale(q, keys, values, key_pos, t, is_retrieval, S, W, scale):
    return _orig_attend_row(q, keys, values, key_pos, t, is_retrieval, S, W, 1.0)


def _attend_sign(q, keys, values, key_pos, t, is_retrieval, S, W, scale):
    return _orig_attend_row(q, keys, values, key_pos, t, is_retrieval, S, W, -scale)


_orig_attend_row = A.attend_row


def _ring_slot_by_position(n, S, W):
    return n if n < S else S + n % W               # window indexed by absolute position


def _blend_swapped(full, stream, a):
    return (1.0 - a) * full + a * stream          # gate applied to the wrong attention


def _gate_by_query_mod(alpha, n_q):
    n_kv = len(alpha)
    return np.array([float(alpha[h % n_kv]) for h in range(n_q)])  # transposed gate mapping


def _round_half_up(y):
    return np.floor(y + 0.5)                       # ties away from even


def _quantize_rows_256(X):
    X = np.asarray(X, dtype=np.float32)
    scale = (np.max(np.abs(X), axis=-1) / np.float32(256.0)).astype(np.float32)  # wrong range
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    return QZ.e4m3_encode((X / safe[..., None]).astype(np.float32)), scale


def _kv_bytes_one_factor(L, n_kv, d_head, T, elem_bytes=2):
    return elem_bytes * L * n_kv * d_head * T      # dropped K+V factor


def _fork_copies_all(self, src, dst):
    n = self.count[src]
    pages = []
    for pg in self.rows[src]:                      # every page copied: no sharing
        c = PG._Page(self.P)
        c.slots = list(pg.slots)
        pages.append(c)
    self.rows[dst] = pages
    self.count[dst] = n


def _fork_shares_partial(self, src, dst):
    self.rows[dst] = list(self.rows[src])          # the partly filled page shared too
    self.count[dst] = self.count[src]


def _pages_floor(self, n):
    return n // self.P                             # a partial page not counted


_orig_rotate = RP.rotate


def _rope_adjacent_pairs(X, positions, theta):
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # pairs (2i, 2i+1)
    inv = np.argsort(perm)
    return _orig_rotate(X[..., perm], positions, theta)[..., inv]


def _rope_sign(X, positions, theta):
    return _orig_rotate(X, -np.asarray(positions, dtype=np.float64), theta)  # turned the other way


def _rope_freq(d, theta):
    return np.power(float(theta), -1.0 * np.arange(d // 2, dtype=np.float64) / d)  # exponent -i/d


def _bf16_half_up(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.floor(m * 256.0 + 0.5), e - 8)  # ties away from even


def _decode_query_unrotated(q, K, V, mask, S, W, scale, theta, dtype, route="cache"):
    K = np.asarray(K, dtype=np.float64)
    return A.decode_step(np.asarray(q, dtype=np.float64), RP.stored_keys(K, theta, dtype),
                         np.asarray(V, dtype=np.float64), mask, S, W, scale, route=route)


def _fp8_prefill_held_as_given(Q, K, V, mask, S, W, scale, chunk):
    # held rows read unquantized: every key and value as given
    Q = np.asarray(Q, dtype=np.float64)
    K64, V64 = np.asarray(K, dtype=np.float64), np.asarray(V, dtype=np.float64)
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    out = np.empty((n_q, N, d))
    lengths = [chunk] * ((N + chunk - 1) // chunk) if np.isscalar(chunk) else list(chunk)
    P = 0
    for C in lengths:
        C = int(min(C, N - P))
        for h in range(n_q):
            k = A.kv_head_of(h, n_q, n_kv)
            kp = np.asarray(Cc.kept_positions(P, bool(mask[k]), S, W) + list(range(P, P + C)), dtype=np.int64)
            out[h, P:P + C] = A.attend_rows(Q[h, P:P + C], np.arange(P, P + C), K64[k][kp], V64[k][kp], kp,
                                            bool(mask[k]), S, W, scale)
        P += C
    return out


_orig_prefill_rope = RP.prefill_chunked_rope


def _rope_fp8_held_unquantized(Q, K, V, mask, S, W, scale, theta, dtype, chunks, kv_format=None):
    return _orig_prefill_rope(Q, K, V, mask, S, W, scale, theta, dtype, chunks, kv_format=None)  # FP8 dropped


_orig_q4 = Q4.quantize_rows_int4


def _int4_ties_up(X):
    X = np.asarray(X, dtype=np.float32)
    scale = (np.max(np.abs(X), axis=-1) / np.float32(7.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    c = np.floor((X / safe[..., None]).astype(np.float32).astype(np.float64) + 0.5)  # ties rounded up
    c = np.where(scale[..., None] > 0, np.clip(c, -7, 7), 0.0)
    return (c + 8).astype(np.uint8), scale


def _int4_scale_8(X):
    X = np.asarray(X, dtype=np.float32)
    codes, _ = _orig_q4(X)
    scale = (np.max(np.abs(X), axis=-1) / np.float32(8.0)).astype(np.float32)  # wrong range
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    c = np.clip(np.rint((X / safe[..., None]).astype(np.float32).astype(np.float64)), -7, 7)
    return (np.where(scale[..., None] > 0, c, 0.0) + 8).astype(np.uint8), scale


def _int4_nibbles_swapped(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] << 4) | c[..., 1::2]).astype(np.uint8)  # element 2k in the high nibble


def _int4_levels_offset7():
    return np.arange(16, dtype=np.int64) - 7


def _int4_prefill_held_as_given(Q, K, V, mask, S, W, scale, chunk):
    Q = np.asarray(Q, dtype=np.float64)
    K64, V64 = np.asarray(K, dtype=np.float64), np.asarray(V, dtype=np.float64)
    n_q, N, d = Q.shape
    n_kv = K.shape[0]
    out = np.empty((n_q, N, d))
    lengths = [chunk] * ((N + chunk - 1) // chunk) if np.isscalar(chunk) else list(chunk)
    P = 0
    for C in lengths:
        C = int(min(C, N - P))
        for h in range(n_q):
            k = A.kv_head_of(h, n_q, n_kv)
            kp = np.asarray(Cc.kept_positions(P, bool(mask[k]), S, W) + list(range(P, P + C)), dtype=np.int64)
            out[h, P:P + C] = A.attend_rows(Q[h, P:P + C], np.arange(P, P + C), K64[k][kp], V64[k][kp], kp,
                                            bool(mask[k]), S, W, scale)   # held rows as given
        P += C
    return out


def _cos_sin_double_reduction(p, i, d, theta, digits=40):
    # the angle reduced with a float64 2 pi, as a kernel might: off by ~1e-7 rad at 2^31
    from decimal import Decimal
    f = float(theta) ** (-2.0 * i / d)
    a = float(p) * f
    r = a - round(a / (2 * np.pi)) * (2 * np.pi)
    return Decimal(np.cos(r)), Decimal(np.sin(r))


MUTATIONS = {
    "window_too_wide": (A, "visible_matrix", _window_too_wide),
    "sinks_off_by_one": (A, "visible_matrix", _sinks_off_by_one),
    "no_causal": (A, "visible_matrix", _no_causal),
    "scalar_window_narrow": (A, "visible", _wrong_scalar_window),
    "gqa_mod_mapping": (A, "kv_head_of", _head_mod),
    "dropped_scale": (A, "attend_row", _attend_no_scale),
    "flipped_sign": (A, "attend_row", _attend_sign),
    "ring_by_position": (Cc, "streaming_slot", _ring_slot_by_position),
    "kv_bytes_factor": (Z, "kv_cache_bytes", _kv_bytes_one_factor),
    "gate_swapped": (G, "blend", _blend_swapped),
    "gate_mod_mapping": (G, "gate_of_query_heads", _gate_by_query_mod),
    "e4m3_ties_up": (QZ, "_round_half_even", _round_half_up),
    "fp8_scale_range": (QZ, "quantize_rows", _quantize_rows_256),
    "fork_copies_all": (PG.PagedRows, "fork", _fork_copies_all),
    "fork_shares_partial": (PG.PagedRows, "fork", _fork_shares_partial),
    "pages_floor": (PG.PagedRows, "pages_needed", _pages_floor),
    "rope_adjacent_pairs": (RP, "rotate", _rope_adjacent_pairs),
    "rope_sign": (RP, "rotate", _rope_sign),
    "rope_freq": (RP, "inv_freq", _rope_freq),
    "bf16_half_up": (RP, "round_bf16", _bf16_half_up),
    "rope_query_unrotated": (RP, "decode_step_rope", _decode_query_unrotated),
    "fp8_held_as_given": (QZ, "prefill_chunked_fp8", _fp8_prefill_held_as_given),
    "rope_fp8_held_unquantized": (RP, "prefill_chunked_rope", _rope_fp8_held_unquantized),
    "int4_ties_up": (Q4, "quantize_rows_int4", _int4_ties_up),
    "int4_scale_range": (Q4, "quantize_rows_int4", _int4_scale_8),
    "int4_nibbles_swapped": (Q4, "pack_nibbles", _int4_nibbles_swapped),
    "int4_levels_offset": (Q4, "int4_levels", _int4_levels_offset7),
    "int4_held_as_given": (Q4, "prefill_chunked_int4", _int4_prefill_held_as_given),
    "rope_exact_double_reduction": (RP, "cos_sin_exact", _cos_sin_double_reduction),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    owner, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(owner, attr, fn)
    bad = OC.failing_checks()
    assert bad, f"planted mistake {name} went unnoticed"
