"""Checks that pin the oracle to facts outside itself.

Each ``check_*`` raises AssertionError on failure.  They are run one by one by
``test_oracle_pins.py`` and, with mistakes planted into the oracle, by
``test_oracle_mutations.py`` (every planted mistake must trip at least one).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import oracle
from oracle import attention as A
from oracle import cache as Cc
from oracle import gating as G
from oracle import paging as PG
from oracle import rope as RP
from oracle import quant as QZ
from oracle import quant4 as Q4
from oracle import sizes as Z

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ sizes

def check_printed_kv_sizes():
    for name, L, n_kv, d, T, e, want in _golden_lines("kv_sizes.txt"):
        got = Z.kv_cache_bytes(int(L), int(n_kv), int(d), int(T), int(e))
        assert got == int(want), (name, got, want)


def check_effective_context():
    kv = {k: v for k, v in _golden_lines("effective_context.txt")}
    got = Z.duo_effective_context(float(kv["R"]), int(kv["T"]), int(kv["S"]), int(kv["W"]))
    assert abs(got - float(kv["tokens"])) < 1e-9, got


def check_mixed_payload_closed_forms():
    # All-retrieval mask -> the full-cache formula of the guide's section 1.
    mask = [[1] * 8 for _ in range(80)]
    assert Z.mixed_payload_bytes(mask, 1, 128000, 64, 1024, 128, 2) == 41943040000
    # R = 2/8 in every layer -> the Memory_Duo formula of the guide's section 2.
    mask = [[1, 1, 0, 0, 0, 0, 0, 0] for _ in range(80)]
    got = Z.mixed_payload_bytes(mask, 1, 128000, 64, 1024, 128, 2)
    assert got == Z.duo_cache_bytes(0.25, 128000, 64, 1024, 80, 8, 128, 2) == 10753146880
    # Local/global layer formula reduces to the uniform one with L1 = 0.
    assert Z.local_global_bytes(8, 128, 2, 0, 32, 4096, 1024) == Z.kv_cache_bytes(32, 8, 128, 4096, 2)
    # ...and counts min(T, W) tokens for windowed layers.
    assert Z.local_global_bytes(8, 128, 2, 32, 0, 4096, 1024) == Z.kv_cache_bytes(32, 8, 128, 1024, 2)


# ------------------------------------------------------------------ cache placement

def check_ring_example():
    # The printed circular-buffer example: window 3, positions 0..4 with values
    # 10 p, held oldest first as [(2, 20), (3, 30), (4, 40)].  A streaming head
    # with no sinks is exactly that window.
    lines = _golden_lines("ring_window3.txt")
    kv = {ln[0]: ln[1:] for ln in lines}
    W = int(kv["window_size"][0])
    h = Cc.StreamingHeadCache(0, W)
    slots = [h.append(p, 10 * p) for p in map(int, kv["appended"])]
    want = [tuple(int(x) for x in s.strip("()").split(",")) for s in kv["ordered"]]
    assert h.ordered() == want, h.ordered()
    # arrival count modulo the window: slots 0, 1, 2, 0, 1
    assert slots == [0, 1, 2, 0, 1]
    assert h.slots() == {0: (3, 30), 1: (4, 40), 2: (2, 20)}


def check_streaming_composition():
    # A streaming head = the guide's append rule (sinks fill first, later tokens go
    # to the window) composed with the window of "Sliding-Window and Mixed
    # Attention" (an S = 0 head, pinned by the printed example above) fed only the
    # tokens that arrive after the sinks are full.
    for S, W, T in [(2, 3, 11), (4, 5, 23), (1, 4, 9), (3, 3, 3), (5, 2, 4), (3, 4, 30)]:
        h = Cc.StreamingHeadCache(S, W)
        window = Cc.StreamingHeadCache(0, W)
        for p in range(T):
            h.append(p, p)
            if p >= S:
                window.append(p, p)
        slots = h.slots()
        for i in range(min(S, T)):
            assert slots[i] == (i, i)
        for r, e in window.slots().items():
            assert slots[S + r] == e, (S, W, T, r)
        assert len(slots) == min(T, S + W)
    # Hand-derived: S = 2, W = 3, positions 0..7.  Positions 0, 1 are sinks;
    # 2, 3, 4 fill window slots 2, 3, 4; 5, 6, 7 then replace 2, 3, 4 in turn.
    h = Cc.StreamingHeadCache(2, 3)
    assert [h.append(p) for p in range(8)] == [0, 1, 2, 3, 4, 2, 3, 4]
    assert {s: p for s, (p, _) in h.slots().items()} == {0: 0, 1: 1, 2: 5, 3: 6, 4: 7}


def check_simulation_counts():
    # The guide's simulation: 4 layers x 8 heads, S=4, W=16, R=0.25, 512 tokens,
    # needle at 240.  Hand-derived: 8 retrieval heads (layers 1 and 2, even heads)
    # hold 512 slots each, 24 streaming heads hold 4 + 16 slots each.
    m = Cc.DuoKVManagerCounts(4, 8, 4, 16, 0.25)
    m.ingest(512)
    assert sum(m.mask.values()) == 8
    assert [k for k, v in m.mask.items() if v] == [(1, 0), (1, 2), (1, 4), (1, 6), (2, 0), (2, 2), (2, 4), (2, 6)]
    held = m.held_slots()
    assert held == 8 * 512 + 24 * 20 == 4576
    dense = 512 * 32
    assert round(dense / held, 2) == 3.58
    assert round((1 - held / dense) * 100, 2) == 72.07
    assert m.heads_holding(240) == (8, 0)
    assert m.heads_holding(3) == (8, 24)     # a sink token survives everywhere
    assert m.heads_holding(500) == (8, 24)   # a recent token survives everywhere
    assert m.heads_holding(495) == (8, 0)    # 17th most recent: just evicted


def check_keep_set_is_visible_set():
    # Route A (what a simulated cache keeps after T appends) equals route B
    # (positions the newest query may see, by the visibility rule), every T.
    for S, W in [(0, 1), (0, 3), (1, 1), (2, 3), (4, 5), (3, 1)]:
        for T in range(1, 3 * (S + W) + 2):
            kept = Cc.kept_positions(T, False, S, W)
            vis = [j for j in range(T) if A.visible(T - 1, j, False, S, W)]
            assert kept == vis, (S, W, T, kept, vis)
            assert len(kept) == min(T, S + W)
            assert Cc.kept_positions(T, True, S, W) == list(range(T))


# ------------------------------------------------------------------ attention values

def check_hand_cases():
    # T=3, d=1, q=1, all keys 0 -> uniform weights over what is visible.
    q = np.array([1.0]); K = np.zeros((3, 1)); V = np.array([[1.0], [2.0], [4.0]])
    pos = [0, 1, 2]
    assert abs(A.attend_row(q, K, V, pos, 2, True, 0, 1, 1.0)[0] - 7 / 3) < 1e-15
    assert abs(A.attend_row(q, K, V, pos, 2, False, 1, 1, 1.0)[0] - 5 / 2) < 1e-15
    assert abs(A.attend_row(q, K, V, pos, 2, False, 2, 1, 1.0)[0] - 7 / 3) < 1e-15
    assert abs(A.attend_row(q, K, V, pos, 2, False, 0, 2, 1.0)[0] - 3.0) < 1e-15
    # d=4, scale 1/2: scores 0 and ln 2 -> weights 1/3, 2/3 (pins sign and scale).
    q = np.array([1.0, 0, 0, 0]); K = np.array([[0.0, 0, 0, 0], [2 * math.log(2), 0, 0, 0]])
    V = np.array([[3.0, 0, 0, 0], [6.0, 0, 0, 0]])
    o = A.attend_row(q, K, V, [0, 1], 1, True, 0, 1, 0.5)
    assert abs(o[0] - 5.0) < 1e-12, o


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def check_bruteforce_agrees():
    # Route A (cache + numpy) vs route B (pure-Python enumeration), tiny inputs.
    rng_seed = 7
    for (n_q, n_kv, d, S, W, T) in [(2, 2, 3, 1, 2, 6), (4, 2, 2, 2, 3, 9), (3, 1, 4, 0, 2, 5), (2, 2, 1, 3, 1, 8)]:
        q = _rand((n_q, d), rng_seed); K = _rand((n_kv, T, d), rng_seed + 1); V = _rand((n_kv, T, d), rng_seed + 2)
        rng_seed += 3
        for mask in ([1] * n_kv, [0] * n_kv, [(k + 1) % 2 for k in range(n_kv)]):
            got = A.decode_step(q, K, V, mask, S, W, 0.7, route="cache")
            for h in range(n_q):
                k = h // (n_q // n_kv)
                ref = A.attend_row_bruteforce(list(q[h]), K[k].tolist(), V[k].tolist(), T - 1,
                                              bool(mask[k]), S, W, 0.7)
                assert np.allclose(got[h], ref, atol=1e-12, rtol=0), (h, mask, got[h], ref)


def _sdpa(Qh, Kh, Vh, attn_mask=None, is_causal=False, enable_gqa=False):
    import torch.nn.functional as F
    return F.scaled_dot_product_attention(torch.from_numpy(Qh), torch.from_numpy(Kh), torch.from_numpy(Vh),
                                          attn_mask=attn_mask, is_causal=is_causal,
                                          enable_gqa=enable_gqa).numpy()


def check_library_special_cases():
    N, d = 37, 8
    for n_q, n_kv in [(4, 4), (6, 2)]:
        Q = _rand((n_q, N, d), 11); K = _rand((n_kv, N, d), 12); V = _rand((n_kv, N, d), 13)
        scale = 1.0 / math.sqrt(d)
        # All heads retrieval == causal attention (torch SDPA, float64 CPU, GQA by the library).
        got = A.prefill_full(Q, K, V, [1] * n_kv, 4, 5, scale)
        ref = _sdpa(Q[None], K[None], V[None], is_causal=True, enable_gqa=(n_q != n_kv))[0]
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
        # Streaming with S + W >= N is full causal attention too.
        got = A.prefill_full(Q, K, V, [0] * n_kv, 10, N - 10, scale)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
        # Streaming with S = 0 is a pure sliding window of W keys: band mask from tril differences.
        W = 6
        band = torch.ones(N, N, dtype=torch.bool).tril() & ~torch.ones(N, N, dtype=torch.bool).tril(-W)
        got = A.prefill_full(Q, K, V, [0] * n_kv, 0, W, scale)
        ref = _sdpa(Q[None], K[None], V[None], attn_mask=band, enable_gqa=(n_q != n_kv))[0]
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
        # Decode step (newest query only) agrees with the last row of the same library result.
        dec = A.decode_step(Q[:, -1], K, V, [0] * n_kv, 0, W, scale)
        assert np.allclose(dec, ref[:, -1], atol=1e-12, rtol=0)


def check_softmax_invariants():
    rng = np.random.default_rng(5)
    for _ in range(20):
        T = int(rng.integers(1, 60)); d = 5; S = int(rng.integers(0, 6)); W = int(rng.integers(1, 9))
        q = rng.standard_normal(d); K = rng.standard_normal((T, d)) * 3; V = rng.standard_normal((T, d))
        for ret in (True, False):
            pos, w = A.softmax_weights(q, K, np.arange(T), T - 1, ret, S, W, 0.5)
            assert abs(w.sum() - 1.0) < 1e-12 and (w >= 0).all()
            o = A.attend_row(q, K, V, np.arange(T), T - 1, ret, S, W, 0.5)
            lo = V[pos].min(axis=0); hi = V[pos].max(axis=0)
            assert (o >= lo - 1e-12).all() and (o <= hi + 1e-12).all()
            # Shuffling the key order (ring slots are out of order) changes nothing.
            perm = rng.permutation(T)
            o2 = A.attend_row(q, K[perm], V[perm], np.arange(T)[perm], T - 1, ret, S, W, 0.5)
            assert np.allclose(o, o2, atol=1e-12, rtol=0)


def check_chunk_invariance():
    # Chunked prefill through a cache that evicts == one pass over the whole sequence.
    n_q, n_kv, N, d, S, W = 4, 2, 45, 6, 3, 7
    Q = _rand((n_q, N, d), 21); K = _rand((n_kv, N, d), 22); V = _rand((n_kv, N, d), 23)
    for mask in ([1, 0], [0, 0], [1, 1]):
        ref = A.prefill_full(Q, K, V, mask, S, W, 0.4)
        for C in (1, 7, 8, 16, N):
            got = A.prefill_chunked(Q, K, V, mask, S, W, 0.4, C)
            assert np.allclose(got, ref, atol=1e-12, rtol=0), (mask, C)


def check_gqa_expansion():
    # Result == the same computation on K/V expanded with repeat_interleave (one KV head per query head).
    n_q, n_kv, T, d, S, W = 8, 2, 30, 4, 2, 5
    q = _rand((n_q, d), 31); K = _rand((n_kv, T, d), 32); V = _rand((n_kv, T, d), 33)
    mask = [1, 0]
    got = A.decode_step(q, K, V, mask, S, W, 0.3)
    g = n_q // n_kv
    Ke = torch.from_numpy(K).repeat_interleave(g, dim=0).numpy()
    Ve = torch.from_numpy(V).repeat_interleave(g, dim=0).numpy()
    me = torch.tensor(mask).repeat_interleave(g).tolist()
    ref = A.decode_step(q, Ke, Ve, me, S, W, 0.3)
    assert np.allclose(got, ref, atol=1e-13, rtol=0)
    # And against the library's own GQA handling (causal SDPA, all retrieval, newest row).
    Qf = _rand((n_q, T, d), 34); Qf[:, -1] = q
    lib = _sdpa(Qf[None], K[None], V[None], is_causal=True, enable_gqa=True)[0][:, -1]
    got = A.decode_step(q, K, V, [1, 1], S, W, 1 / math.sqrt(d))
    assert np.allclose(got, lib, atol=1e-12, rtol=0)


# ------------------------------------------------------------------ head-gated forward

def check_gated_hand_case():
    # golden/gated_tiny.txt: the hand-derived blend on N=3, d=1, S=1, W=1.
    Q = np.ones((1, 3, 1)); K = np.zeros((1, 3, 1)); V = np.array([[[1.0], [2.0], [4.0]]])
    keys = K[0].tolist(); vals = V[0].tolist()
    for a_s, t_s, num, den in _golden_lines("gated_tiny.txt"):
        alpha, t, want = float(a_s), int(t_s), int(num) / int(den)
        got = G.gated_forward(Q, K, V, [alpha], 1, 1, 1.0, rows=np.array([t]))[0, 0, 0]
        assert abs(got - want) < 1e-15, (alpha, t, got, want)
        got_b = G.gated_row_bruteforce([1.0], keys, vals, t, alpha, 1, 1, 1.0)[0]
        assert abs(got_b - want) < 1e-15, (alpha, t, got_b, want)


def check_gated_library_endpoints():
    # alpha = 1 is causal attention and alpha = 0 (S = 0) a band of W keys: torch SDPA,
    # float64 CPU; a mixed per-KV-head gate blends the two library results per query head.
    N, d, W = 29, 8, 5
    for n_q, n_kv in [(3, 3), (8, 2)]:
        Q = _rand((n_q, N, d), 41); K = _rand((n_kv, N, d), 42); V = _rand((n_kv, N, d), 43)
        scale = 1.0 / math.sqrt(d)
        gqa = n_q != n_kv
        causal = _sdpa(Q[None], K[None], V[None], is_causal=True, enable_gqa=gqa)[0]
        band = torch.ones(N, N, dtype=torch.bool).tril() & ~torch.ones(N, N, dtype=torch.bool).tril(-W)
        window = _sdpa(Q[None], K[None], V[None], attn_mask=band, enable_gqa=gqa)[0]
        assert np.allclose(G.gated_forward(Q, K, V, [1.0] * n_kv, 0, W, scale), causal, atol=1e-12, rtol=0)
        assert np.allclose(G.gated_forward(Q, K, V, [0.0] * n_kv, 0, W, scale), window, atol=1e-12, rtol=0)
        alpha = [0.125 + 0.25 * k for k in range(n_kv)]
        got = G.gated_forward(Q, K, V, alpha, 0, W, scale)
        g = n_q // n_kv
        for h in range(n_q):
            a = alpha[h // g]
            assert np.allclose(got[h], a * causal[h] + (1 - a) * window[h], atol=1e-12, rtol=0), h


def check_gated_bruteforce_agrees():
    # numpy route vs pure-Python enumeration on tiny inputs, with sinks.
    seed = 51
    for (n_q, n_kv, d, S, W, N) in [(2, 2, 3, 1, 2, 7), (4, 2, 2, 2, 3, 9), (3, 1, 2, 0, 1, 5)]:
        Q = _rand((n_q, N, d), seed); K = _rand((n_kv, N, d), seed + 1); V = _rand((n_kv, N, d), seed + 2)
        alpha = list(np.random.default_rng(seed).uniform(0, 1, n_kv))
        seed += 3
        got = G.gated_forward(Q, K, V, alpha, S, W, 0.6)
        for h in range(n_q):
            k = h // (n_q // n_kv)
            for t in range(N):
                ref = G.gated_row_bruteforce(list(Q[h, t]), K[k, :t + 1].tolist(), V[k, :t + 1].tolist(),
                                             t, alpha[k], S, W, 0.6)
                assert np.allclose(got[h, t], ref, atol=1e-12, rtol=0), (h, t)


def check_gated_gqa_expansion():
    # Result == the same forward on K/V and gates expanded with repeat_interleave.
    n_q, n_kv, N, d, S, W = 8, 2, 21, 4, 2, 4
    Q = _rand((n_q, N, d), 61); K = _rand((n_kv, N, d), 62); V = _rand((n_kv, N, d), 63)
    alpha = [0.3, 0.9]
    got = G.gated_forward(Q, K, V, alpha, S, W, 0.5)
    g = n_q // n_kv
    Ke = torch.from_numpy(K).repeat_interleave(g, dim=0).numpy()
    Ve = torch.from_numpy(V).repeat_interleave(g, dim=0).numpy()
    ae = torch.tensor(alpha, dtype=torch.float64).repeat_interleave(g).tolist()
    ref = G.gated_forward(Q, Ke, Ve, ae, S, W, 0.5)
    assert np.allclose(got, ref, atol=1e-13, rtol=0)


# ------------------------------------------------------------------ FP8 rows

def _e4m3_sweep():
    """float32 inputs covering every E4M3 rounding decision: each representable
    magnitude, each midpoint between neighbours (the ties), points just off the
    midpoints, the subnormal range and values past 448 up to the overflow edge."""
    vals = np.unique(np.abs(QZ.e4m3_decode(np.arange(0, 127, dtype=np.uint8))))  # finite magnitudes
    mids = (vals[:-1] + vals[1:]) / 2.0
    ulp = np.float32(2.0 ** -20)
    pts = np.concatenate([vals, mids, mids * (1 + ulp), mids * (1 - ulp), [448.0, 450.0, 463.5],
                          np.linspace(0, 2.0 ** -6, 1000), np.linspace(0, 463.9, 20000)])
    pts = pts.astype(np.float32)
    return np.concatenate([pts, -pts])


def check_e4m3_against_library():
    # Encoder == torch's float8_e4m3fn cast (round to nearest, ties to even) on the sweep.
    x = _e4m3_sweep()
    got = QZ.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref), int(np.sum(got != ref))
    # Decoder == the library's conversion back to float on all 256 codes.
    c = np.arange(256, dtype=np.uint8)
    d = QZ.e4m3_decode(c)
    dl = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    assert np.all((d == dl) | (np.isnan(d) & np.isnan(dl)))


def check_fp8_row_quantizer():
    rng = np.random.default_rng(71)
    X = (rng.standard_normal((300, 64)) * np.exp(rng.uniform(-8, 8, (300, 1)))).astype(np.float32)
    X[5] = 0.0
    codes, scale = QZ.quantize_rows(X)
    # scale = max |x| / 448 in float32; the zero row keeps scale 0 and codes 0
    assert np.array_equal(scale, (np.max(np.abs(X), axis=1) / np.float32(448.0)).astype(np.float32))
    assert scale[5] == 0 and not codes[5].any()
    R = QZ.dequantize_rows(codes, scale)
    x64 = X.astype(np.float64)
    # the largest element of every nonzero row takes magnitude code 0x7E (448)
    nz = scale > 0
    big = np.argmax(np.abs(X), axis=1)
    assert np.all((codes[np.arange(300), big][nz] & 0x7F) == 0x7E)
    # error within half a quantum of the E4M3 binade of x / s (plus the float32 rounding of x / s)
    t = np.where(nz[:, None], np.abs(x64) / np.where(nz, scale, 1)[:, None].astype(np.float64), 0)
    e = np.maximum(np.floor(np.log2(np.maximum(t, 2.0 ** -6))), -6)
    half_quantum = np.exp2(e - 4) * scale[:, None]
    assert np.all(np.abs(R - x64) <= half_quantum * (1 + 2.0 ** -20) + np.abs(x64) * 2.0 ** -23)
    # rows already on the E4M3 grid times a power-of-two scale come back exactly
    grid = QZ.e4m3_decode(rng.integers(0, 126, (10, 64)).astype(np.uint8)).astype(np.float32)
    grid[:, 0] = 448.0
    c2, s2 = QZ.quantize_rows(grid * np.float32(0.25))
    assert np.array_equal(QZ.dequantize_rows(c2, s2), grid.astype(np.float64) * 0.25)


def check_fp8_attention_routes():
    # Rows already on the E4M3 grid times a power-of-two scale are stored exactly,
    # so the FP8 routes reduce to the native ones; with a single chunk nothing is
    # held and prefill sees only the chunk, as given.
    rng = np.random.default_rng(81)
    n_q, n_kv, N, d, S, W = 4, 2, 23, 8, 2, 5
    codes = rng.integers(0, 126, (n_kv, N, d)).astype(np.uint8)
    K = (QZ.e4m3_decode(codes) * 0.5).astype(np.float32); K[..., 0] = 224.0
    V = (QZ.e4m3_decode(rng.integers(0, 126, (n_kv, N, d)).astype(np.uint8)) * 0.25).astype(np.float32)
    V[..., 0] = 112.0
    Q = rng.standard_normal((n_q, N, d)) * 0.05
    for mask in ([1, 0], [0, 1]):
        ref = A.prefill_full(Q, K, V, mask, S, W, 0.3)
        for C in (1, 5, N):
            assert np.allclose(QZ.prefill_chunked_fp8(Q, K, V, mask, S, W, 0.3, C), ref, atol=1e-12, rtol=0)
        assert np.allclose(QZ.decode_step_fp8(Q[:, -1], K, V, mask, S, W, 0.3), ref[:, -1], atol=1e-12, rtol=0)
    # Off the grid, a single chunk still equals full attention on the exact rows,
    # while decode sees the stored rows.
    K2 = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    V2 = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    ref = A.prefill_full(Q, K2, V2, [1, 0], S, W, 0.3)
    assert np.allclose(QZ.prefill_chunked_fp8(Q, K2, V2, [1, 0], S, W, 0.3, N), ref, atol=1e-12, rtol=0)
    dq = A.decode_step(Q[:, -1], QZ.stored_values(K2), QZ.stored_values(V2), [1, 0], S, W, 0.3)
    assert np.allclose(QZ.decode_step_fp8(Q[:, -1], K2, V2, [1, 0], S, W, 0.3), dq, atol=1e-12, rtol=0)


def _fp8_stored_by_library(X):
    """What a row-scaled E4M3 cache holds for float32 rows X, built with
    torch's float8_e4m3fn conversion: s = max|x| / 448 and x / s in float32,
    the cast, then code value * s (a zero row stays zero)."""
    X = np.asarray(X, dtype=np.float32)
    s = (np.max(np.abs(X), axis=-1) / np.float32(448.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = np.ascontiguousarray((X / safe[..., None]).astype(np.float32))
    v = torch.from_numpy(y).to(torch.float8_e4m3fn).double().numpy()
    return np.where(s[..., None] > 0, v * s[..., None].astype(np.float64), 0.0)


def _chunked_by_enumeration(Qrows, held_k, given_k, held_v, given_v, mask, S, W, scale, chunks):
    """Chunk row t = P + i enumerates positions 0..t: a key or value at
    j < P (cached before the chunk) is taken from held_*, one at j >= P
    (the chunk's own) from given_*; softmax in pure Python."""
    n_q, N, d = Qrows.shape
    n_kv = given_k.shape[0]
    out = np.empty((n_q, N, d))
    P = 0
    for C in chunks:
        for h in range(n_q):
            k = A.kv_head_of(h, n_q, n_kv)
            for t in range(P, P + C):
                keys = [(held_k[k][j] if j < P else given_k[k][j]).tolist() for j in range(t + 1)]
                vals = [(held_v[k][j] if j < P else given_v[k][j]).tolist() for j in range(t + 1)]
                out[h, t] = A.attend_row_bruteforce(Qrows[h, t].tolist(), keys, vals, t, bool(mask[k]), S, W, scale)
        P += C
    return out


def check_fp8_prefill_held_rows():
    # Off the E4M3 grid and over several chunks: a chunk row sees every key and
    # value cached before its chunk as stored (code value x row scale) and the
    # chunk's own as given.  Expected values by enumeration over positions with
    # the library's E4M3 conversion; decode sees every held row as stored.
    rng = np.random.default_rng(91)
    n_q, n_kv, N, d, S, W = 4, 2, 23, 8, 2, 5
    chunks = [5, 7, 4, 7]
    K = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    V = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    Q = rng.standard_normal((n_q, N, d))
    Ks, Vs = _fp8_stored_by_library(K), _fp8_stored_by_library(V)
    K64, V64 = K.astype(np.float64), V.astype(np.float64)
    for mask in ([1, 0], [0, 1]):
        want = _chunked_by_enumeration(Q, Ks, K64, Vs, V64, mask, S, W, 0.35, chunks)
        got = QZ.prefill_chunked_fp8(Q, K, V, mask, S, W, 0.35, chunks)
        assert np.allclose(got, want, atol=1e-12, rtol=0), float(np.abs(got - want).max())
        # not vacuous: reading the held rows as given moves the result
        as_given = _chunked_by_enumeration(Q, K64, K64, V64, V64, mask, S, W, 0.35, chunks)
        assert np.abs(as_given - want).max() > 1e-3
        # decode at T = N: the query's own row was appended first, so it too is as stored
        kv = [A.kv_head_of(h, n_q, n_kv) for h in range(n_q)]
        dq = np.stack([A.attend_row_bruteforce(Q[h, N - 1].tolist(), Ks[kv[h]].tolist(), Vs[kv[h]].tolist(), N - 1,
                                               bool(mask[kv[h]]), S, W, 0.35) for h in range(n_q)])
        got_d = QZ.decode_step_fp8(Q[:, N - 1], K, V, mask, S, W, 0.35)
        assert np.allclose(got_d, dq, atol=1e-12, rtol=0), float(np.abs(got_d - dq).max())


def _rotate_by_complex(X, positions, theta):
    """Pair (x_i, x_(i + d/2)) as x_i + j x_(i + d/2), times exp(j p theta^(-2i/d))."""
    X = np.asarray(X, dtype=np.float64)
    h = X.shape[-1] // 2
    f = np.array([theta ** (-(2.0 * i) / X.shape[-1]) for i in range(h)])
    z = (X[..., :h] + 1j * X[..., h:]) * np.exp(1j * np.asarray(positions, dtype=np.float64)[:, None] * f[None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def check_rope_fp8_prefill_held_rows():
    # Rotary positions over FP8 rows, several chunks: a held key is the key
    # rotated at its position, rounded to bf16 and then stored as FP8; a held
    # value is stored as FP8; the chunk's own keys are rotated but not rounded,
    # its values as given; the query is rotated at its own position.
    rng = np.random.default_rng(92)
    n_q, n_kv, N, d, S, W, theta = 4, 2, 21, 8, 2, 4, 1e4
    chunks = [6, 1, 9, 5]
    K = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    V = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    Q = rng.standard_normal((n_q, N, d))
    pos = np.arange(N)
    Kr = _rotate_by_complex(K, pos, theta)
    Kb = torch.from_numpy(Kr.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(Kb.astype(np.float64), RP.round_bf16(Kr))  # one rounding, float64 -> bf16
    Ks, Vs = _fp8_stored_by_library(Kb), _fp8_stored_by_library(V)
    Qr = _rotate_by_complex(Q, pos, theta)
    for mask in ([1, 0], [0, 1]):
        want = _chunked_by_enumeration(Qr, Ks, Kr, Vs, V.astype(np.float64), mask, S, W, 0.35, chunks)
        got = RP.prefill_chunked_rope(Q, K, V, mask, S, W, 0.35, theta, "bf16", chunks, kv_format="fp8")
        assert np.allclose(got, want, atol=1e-9, rtol=0), float(np.abs(got - want).max())
        as_given = _chunked_by_enumeration(Qr, Kr, Kr, V.astype(np.float64), V.astype(np.float64), mask, S, W,
                                           0.35, chunks)
        assert np.abs(as_given - want).max() > 1e-3


# ------------------------------------------------------------------ INT4 rows

def check_int4_golden_rows():
    # the level table and rows worked by hand (tests/golden/int4_rows.txt)
    lines = [ln for ln in open(os.path.join(GOLDEN, "int4_rows.txt")) if ln.strip() and not ln.startswith("#")]
    levels = [int(v) for v in lines[0].split()[1:]]
    assert Q4.int4_levels().tolist() == levels == list(range(-8, 8))
    assert np.array_equal(Q4.unpack_nibbles(Q4.pack_nibbles(np.arange(16, dtype=np.uint8))), np.arange(16))
    for ln in lines[1:]:
        x, sc, lv, by = [part.split() for part in ln[4:].split("|")]
        codes, scale = Q4.quantize_rows_int4(np.array([float(v) for v in x], dtype=np.float32)[None])
        assert scale[0] == np.float32(float(sc[0])), (x, scale)
        assert Q4.int4_levels()[codes[0].astype(np.int64)].tolist() == [int(v) for v in lv], (x, codes)
        assert [f"{b:02x}" for b in Q4.pack_nibbles(codes[0])] == by, (x, Q4.pack_nibbles(codes[0]))
        assert np.array_equal(Q4.unpack_nibbles(Q4.pack_nibbles(codes)), codes)


def _int4_stored_by_library(X):
    """What a row-scaled INT4 cache holds for float32 rows X, built with
    torch's round (half to even): s = max|x| / 7 and x / s in float32."""
    X = np.asarray(X, dtype=np.float32)
    s = (np.max(np.abs(X), axis=-1) / np.float32(7.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = np.ascontiguousarray((X / safe[..., None]).astype(np.float32))
    c = torch.round(torch.from_numpy(y)).clamp(-7, 7).double().numpy()
    return np.where(s[..., None] > 0, c * s[..., None].astype(np.float64), 0.0)


def check_int4_row_quantizer():
    rng = np.random.default_rng(73)
    X = (rng.standard_normal((400, 64)) * np.exp(rng.uniform(-8, 8, (400, 1)))).astype(np.float32)
    X[3] = 0.0
    X[7, :] = np.resize(np.array([7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5], np.float32), 64)  # s = 1: ties
    codes, scale = Q4.quantize_rows_int4(X)
    assert np.array_equal(scale, (np.max(np.abs(X), axis=1) / np.float32(7.0)).astype(np.float32))
    assert scale[3] == 0 and np.all(codes[3] == 8)
    assert codes.min() >= 1 and codes.max() <= 15            # level -8 never produced
    R = Q4.dequantize_rows_int4(codes, scale)
    assert np.array_equal(R, _int4_stored_by_library(X))    # torch's rounding, independently
    # within half a step (plus the float32 rounding of x / s)
    x64 = X.astype(np.float64)
    assert np.all(np.abs(R - x64) <= scale[:, None].astype(np.float64) * (0.5 + 2.0 ** -20))
    # the largest element of every nonzero row takes level +-7
    big = np.argmax(np.abs(X), axis=1)
    nz = scale > 0
    assert np.all(np.abs(Q4.int4_levels()[codes[np.arange(400), big].astype(np.int64)][nz]) == 7)
    # rows on the grid (levels times a power of two, a level 7 in each) come back exactly
    lv = rng.integers(-7, 8, (10, 64)).astype(np.float64)
    lv[:, 0] = 7
    grid = (lv * 0.25).astype(np.float32)
    c2, s2 = Q4.quantize_rows_int4(grid)
    assert np.all(s2 == np.float32(0.25)) and np.array_equal(Q4.dequantize_rows_int4(c2, s2), lv * 0.25)


def check_int4_attention_routes():
    rng = np.random.default_rng(83)
    n_q, n_kv, N, d, S, W = 4, 2, 23, 8, 2, 5
    # on the grid the INT4 routes are the native ones
    lvk = rng.integers(-7, 8, (n_kv, N, d)).astype(np.float64); lvk[..., 0] = 7
    lvv = rng.integers(-7, 8, (n_kv, N, d)).astype(np.float64); lvv[..., 0] = -7
    K, V = (lvk * 0.5).astype(np.float32), (lvv * 0.125).astype(np.float32)
    Q = rng.standard_normal((n_q, N, d)) * 0.3
    for mask in ([1, 0], [0, 1]):
        ref = A.prefill_full(Q, K, V, mask, S, W, 0.3)
        for C in (1, 5, N):
            assert np.allclose(Q4.prefill_chunked_int4(Q, K, V, mask, S, W, 0.3, C), ref, atol=1e-12, rtol=0)
        assert np.allclose(Q4.decode_step_int4(Q[:, -1], K, V, mask, S, W, 0.3), ref[:, -1], atol=1e-12, rtol=0)
    # off the grid, over several chunks: held rows as stored, the chunk's own as given
    chunks = [5, 7, 4, 7]
    K2 = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    V2 = rng.standard_normal((n_kv, N, d)).astype(np.float32)
    Ks, Vs = _int4_stored_by_library(K2), _int4_stored_by_library(V2)
    K64, V64 = K2.astype(np.float64), V2.astype(np.float64)
    for mask in ([1, 0], [0, 1]):
        want = _chunked_by_enumeration(Q, Ks, K64, Vs, V64, mask, S, W, 0.35, chunks)
        got = Q4.prefill_chunked_int4(Q, K2, V2, mask, S, W, 0.35, chunks)
        assert np.allclose(got, want, atol=1e-12, rtol=0), float(np.abs(got - want).max())
        assert np.abs(_chunked_by_enumeration(Q, K64, K64, V64, V64, mask, S, W, 0.35, chunks) - want).max() > 1e-3
        kv = [A.kv_head_of(h, n_q, n_kv) for h in range(n_q)]
        dq = np.stack([A.attend_row_bruteforce(Q[h, N - 1].tolist(), Ks[kv[h]].tolist(), Vs[kv[h]].tolist(), N - 1,
                                               bool(mask[kv[h]]), S, W, 0.35) for h in range(n_q)])
        got_d = Q4.decode_step_int4(Q[:, N - 1], K2, V2, mask, S, W, 0.35)
        assert np.allclose(got_d, dq, atol=1e-12, rtol=0), float(np.abs(got_d - dq).max())
    # rotary positions over INT4 rows: held keys rotated, rounded to bf16, then stored
    theta, chunks = 1e4, [6, 1, 9, 7]
    Kr = _rotate_by_complex(K2, np.arange(N), theta)
    Kb = torch.from_numpy(Kr.astype(np.float32)).to(torch.bfloat16).float().numpy()
    Qr = _rotate_by_complex(Q, np.arange(N), theta)
    want = _chunked_by_enumeration(Qr, _int4_stored_by_library(Kb), Kr, _int4_stored_by_library(V2), V64, [1, 0], S,
                                   W, 0.35, chunks)
    got = RP.prefill_chunked_rope(Q, K2, V2, [1, 0], S, W, 0.35, theta, "bf16", chunks, kv_format="int4")
    assert np.allclose(got, want, atol=1e-9, rtol=0), float(np.abs(got - want).max())


# ------------------------------------------------------------------ paged rows

def check_paging_closed_forms():
    P = 256
    # rows that never share: each holds ceil(n / P) pages (a ragged batch
    # allocates per request, not the padded B * ceil(max n / P))
    lens = [1, 255, 256, 257, 1000, 0, 4096]
    m = PG.PagedRows(P, 10_000, len(lens))
    for b, n in enumerate(lens):
        if n:
            m.append(b, n)
    assert m.pages_in_use() == 1 + 1 + 1 + 2 + 4 + 0 + 16
    assert m.pages_in_use() < len(lens) * (4096 // P)
    # a prefix of n tokens forked from row 0 to rows 1..k, then row r appends
    # m_r: floor(n/P) shared pages + each row's own ceil((n + m_r)/P) - floor(n/P)
    for n in (0, 100, 256, 600, 1024):
        ms = [0, 5, 300, 1, 700]
        m = PG.PagedRows(P, 10_000, len(ms))
        if n:
            m.append(0, n)
        for r in range(1, len(ms)):
            m.fork(0, r)
        for r, mr in enumerate(ms):
            if mr:
                m.append(r, mr)
        want = n // P + sum(-(-(n + mr) // P) - n // P for mr in ms)
        assert m.pages_in_use() == want, (n, m.pages_in_use(), want)
        for r in range(1, len(ms)):
            assert m.shared_pages(0, r) == n // P
        # every row holds the prefix (from row 0) and then its own tokens
        for r, mr in enumerate(ms):
            assert m.content(r) == [(0, p) for p in range(n)] + [(r, p) for p in range(n, n + mr)]
        # resets return everything
        for r in range(len(ms)):
            m.reset(r)
        assert m.pages_in_use() == 0 and m.free_pages() == 10_000


def check_paging_capacity():
    m = PG.PagedRows(256, 3, 2)
    m.append(0, 600)                         # 3 pages
    before = (m.pages_in_use(), list(m.count))
    for grow in ([(1, 1)], [(0, 200)], [(0, 1), (1, 1)]):
        try:
            m.append_rows(grow)
            raise AssertionError("grew past the pool")
        except MemoryError:
            pass
        assert (m.pages_in_use(), list(m.count)) == before
    m.append(0, 168)                         # fills page 3 exactly: no new page
    assert m.pages_in_use() == 3 and m.count[0] == 768
    try:
        m.fork(0, 1)                         # all pages full: shared, nothing copied
    except MemoryError:
        raise AssertionError("a fork of full pages needs no page")
    assert m.pages_in_use() == 3 and m.shared_pages(0, 1) == 3


# ------------------------------------------------------------------ rotary positions

def check_rope_unit_vectors():
    # d = 8, theta = 10^4: pair frequencies 10^(-i) = 1, 0.1, 0.01, 0.001.  At
    # position p, unit vector e_i (i < 4) turns into cos(p f_i) e_i + sin(p f_i) e_(i+4)
    # and e_(i+4) into -sin(p f_i) e_i + cos(p f_i) e_(i+4).
    f = [1.0, 0.1, 0.01, 0.001]
    for p in (1, 7, 1000):
        R = RP.rotate(np.eye(8), [p] * 8, 1e4)     # row i: unit vector e_i at position p
        for i in range(4):
            want = np.zeros(8)
            want[i], want[i + 4] = math.cos(p * f[i]), math.sin(p * f[i])
            assert np.allclose(R[i], want, atol=1e-12), (p, i, R[i])
            want = np.zeros(8)
            want[i], want[i + 4] = -math.sin(p * f[i]), math.cos(p * f[i])
            assert np.allclose(R[i + 4], want, atol=1e-12), (p, i + 4, R[i + 4])
    X = np.random.default_rng(3).standard_normal((5, 16))
    assert np.array_equal(RP.rotate(X, [0] * 5, 5e5), X)  # position 0: no rotation


def check_rope_complex_form():
    # pair (x_i, x_(i+d/2)) as the complex number x_i + j x_(i+d/2), multiplied
    # by exp(j p f_i) with f_i = theta^(-2i/d)
    rng = np.random.default_rng(4)
    d, theta = 64, 5e5
    X = rng.standard_normal((3, 9, d))
    pos = np.array([0, 1, 2, 63, 64, 1000, 4095, 70000, 131071])
    z = X[..., : d // 2] + 1j * X[..., d // 2:]
    f = np.array([theta ** (-(2.0 * i) / d) for i in range(d // 2)])
    w = z * np.exp(1j * pos[:, None] * f[None, :])
    want = np.concatenate([w.real, w.imag], axis=-1)
    assert np.allclose(RP.rotate(X, pos, theta), want, atol=1e-9, rtol=0)


def check_rope_relative_positions():
    # scores of rotated queries and keys depend only on the position difference
    rng = np.random.default_rng(5)
    d = 128
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    def score(pq, pk):
        return float(RP.rotate(q[None], [pq], 1e4)[0] @ RP.rotate(k[None], [pk], 1e4)[0])
    for pq, pk in ((10, 3), (5000, 4990), (7, 7), (2, 9)):
        for shift in (1, 100, 65536):
            assert abs(score(pq, pk) - score(pq + shift, pk + shift)) < 1e-9
        assert abs(score(pq, pk) - float(q @ RP.rotate(k[None], [pk - pq], 1e4)[0])) < 1e-9


def check_rope_exact_integer_angles():
    # Integer angles, whose cosine and sine the C library gives after an exact
    # reduction: pair 0 turns by p (frequency 1 at any base); with base 10^4
    # and d = 8 the frequencies are 10^(-i), so at a multiple of 1000 every
    # pair's angle p / 10^i is an integer.
    p_big = (2 ** 31 - 1) // 1000 * 1000
    for p in (1, 7, 123456789, 2 ** 31 - 1):
        cs, sn = RP.cos_sin_exact(p, 0, 128, 5e5)
        assert abs(float(cs) - math.cos(p)) < 2e-16 and abs(float(sn) - math.sin(p)) < 2e-16, p
    for p in (1000, 5_000_000, p_big):
        for i in range(4):
            n = p // 10 ** i
            cs, sn = RP.cos_sin_exact(p, i, 8, 1e4)
            assert abs(float(cs) - math.cos(n)) < 2e-16 and abs(float(sn) - math.sin(n)) < 2e-16, (p, i)


def check_rope_exact_matches_float64_at_small_positions():
    # below 2^17 a float64 angle p * f is off by at most p * 2^-53 < 2e-11
    X = np.random.default_rng(9).standard_normal((3, 16))
    pos = [0, 4095, 131071]
    assert np.allclose(RP.rotate_exact(X, pos, 5e5), RP.rotate(X, pos, 5e5), atol=1e-10, rtol=0)


def check_bf16_rounding_against_library():
    mags = 10.0 ** np.random.default_rng(8).uniform(-3, 3, 20000)
    ties = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -9, 255.5, 0.0]  # halfway cases
    x = np.concatenate([np.random.default_rng(6).standard_normal(20000) * mags, ties])
    x32 = x.astype(np.float32)                      # float32-representable values: no double rounding
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(RP.round_bf16(x32.astype(np.float64)), want)


def check_rope_cache_route_uses_logical_positions():
    # a streaming head's ring holds keys rotated at their own positions: the
    # decode over the cache's slots equals the visibility rule over positions
    rng = np.random.default_rng(7)
    n_q, n_kv, T, d, S, W = 4, 2, 40, 16, 3, 8
    q = rng.standard_normal((n_q, d))
    K, V = rng.standard_normal((n_kv, T, d)), rng.standard_normal((n_kv, T, d))
    for mask in ([1, 0], [0, 0]):
        a = RP.decode_step_rope(q, K, V, mask, S, W, 0.25, 1e4, "f32", route="cache")
        b = RP.decode_step_rope(q, K, V, mask, S, W, 0.25, 1e4, "f32", route="definition")
        assert np.allclose(a, b, atol=1e-12)
    # chunked prefill with rotary positions: every chunking gives the same rows
    # up to the rounding of the held keys (a single chunk holds none)
    Q = rng.standard_normal((n_q, T, d))
    one = RP.prefill_chunked_rope(Q, K, V, [1, 0], S, W, 0.25, 1e4, "f32", [T])
    many = RP.prefill_chunked_rope(Q, K, V, [1, 0], S, W, 0.25, 1e4, "f32", [7, 1, 20, 12])
    assert np.allclose(one, many, atol=1e-5)
    # the last row of a prefill is a decode step at that position
    dec = RP.decode_step_rope(q, K, V, [1, 0], S, W, 0.25, 1e4, "f32")
    Q2 = Q.copy()
    Q2[:, T - 1] = q
    pre = RP.prefill_chunked_rope(Q2, K, V, [1, 0], S, W, 0.25, 1e4, "f32", [T - 1, 1])
    assert np.allclose(pre[:, T - 1], dec, atol=1e-12)
    # FP8 rows: the cache's decode equals the FP8 route over keys rotated and
    # rounded to bf16 beforehand (with the query rotated at T - 1)
    qr = RP.rotate(q[:, None, :], [T - 1], 1e4)[:, 0, :]
    Kb = RP.round_bf16(RP.rotate(K, np.arange(T), 1e4)).astype(np.float32)
    want = QZ.decode_step_fp8(qr, Kb, V.astype(np.float32), [1, 0], S, W, 0.25)
    got = RP.decode_step_rope(q, K, V.astype(np.float32), [1, 0], S, W, 0.25, 1e4, "bf16", kv_format="fp8")
    assert np.allclose(got, want, atol=1e-12)


ALL_CHECKS = [
    check_printed_kv_sizes, check_effective_context, check_mixed_payload_closed_forms,
    check_ring_example, check_streaming_composition, check_simulation_counts, check_keep_set_is_visible_set,
    check_hand_cases, check_bruteforce_agrees, check_library_special_cases,
    check_softmax_invariants, check_chunk_invariance, check_gqa_expansion,
    check_gated_hand_case, check_gated_library_endpoints, check_gated_bruteforce_agrees,
    check_gated_gqa_expansion, check_e4m3_against_library, check_fp8_row_quantizer,
    check_fp8_attention_routes, check_fp8_prefill_held_rows, check_rope_fp8_prefill_held_rows,
    check_int4_golden_rows, check_int4_row_quantizer, check_int4_attention_routes,
    check_paging_closed_forms, check_paging_capacity,
    check_rope_unit_vectors, check_rope_complex_form, check_rope_relative_positions,
    check_bf16_rounding_against_library, check_rope_cache_route_uses_logical_positions,
    check_rope_exact_integer_angles, check_rope_exact_matches_float64_at_small_positions,
]


def failing_checks():
    bad = []
    for c in ALL_CHECKS:
        try:
            c()
        except Exception:  # a failed assertion, or a planted mistake that crashes a check
            bad.append(c.__name__)
    return bad
