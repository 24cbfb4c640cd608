"""Head-gated forward parity: libduo's duo_gated_attention against the fp64
oracle (oracle.gating: alpha * causal + (1 - alpha) * sink+window attention)."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import gating as OG
from tests.gpu_util import check_close, need_gpu, say, stored


def _inputs(B, n_q, n_kv, d, N, seed, sink_rows=0):
    Q = WL.normal_f32((B, n_q, N, d), seed)
    K = WL.normal_f32((B, n_kv, N, d), seed + 1)
    V = WL.normal_f32((B, n_kv, N, d), seed + 2)
    K[:, :, :sink_rows] *= np.float32(4.0)
    return Q, K, V


def _run(Q, K, V, alpha, S, W, dtype):
    import head_wise_kv_amd as H
    Qd, Kd, Vd = (WL.to_torch(x, dtype).cuda() for x in (Q, K, V))
    a = torch.tensor(np.asarray(alpha, dtype=np.float32), device="cuda")
    out = H.gated_attention(Qd, Kd, Vd, a, S, W)
    torch.cuda.synchronize()
    return out


def _oracle(Q, K, V, alpha, S, W, dtype, rows=None):
    q64, k64, v64 = stored(Q, dtype), stored(K, dtype), stored(V, dtype)
    scale = 1.0 / np.sqrt(Q.shape[-1])
    return np.stack([OG.gated_forward(q64[b], k64[b], v64[b], alpha, S, W, scale, rows=rows)
                     for b in range(Q.shape[0])])


def _gates(n_kv, seed):
    # the endpoints 0 and 1 always appear (pure streaming / pure full attention)
    a = np.random.default_rng(seed).uniform(0.0, 1.0, n_kv).astype(np.float32)
    a[0] = 1.0
    if n_kv > 1:
        a[1] = 0.0
    return a


GRID = [(dt, d, g) for dt in ("bf16", "f32") for d in (64, 128) for g in (1, 2, 3, 4, 8)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g", GRID)
def test_gated_grid(dtype, d, g):
    """Every dtype x d x group size (odd g takes one query head per work item):
    N spans several 64-key tiles and row tiles with a ragged tail; S=5 (a sink
    tile shared with window keys), W=70 (the window edge crosses tiles)."""
    need_gpu()
    n_kv = 3
    N = 333 if dtype == "bf16" else 150
    say("gated grid", dtype, d, g, N)
    Q, K, V = _inputs(2, n_kv * g, n_kv, d, N, seed=900 + 10 * g + d, sink_rows=5)
    alpha = _gates(n_kv, g + d)
    out = _run(Q, K, V, alpha, 5, 70, dtype)
    check_close(out, _oracle(Q, K, V, alpha, 5, 70, dtype), dtype, f"gated {dtype} d{d} g{g}")


EDGES = [
    # (N, S, W): one token; window covers everything; no sinks; a one-token
    # window; sinks past one tile; sinks longer than the sequence; tile-exact N
    (1, 4, 16), (200, 64, 1024), (300, 0, 50), (260, 3, 1), (400, 70, 64), (90, 128, 8), (256, 64, 64),
]


@pytest.mark.gpu
@pytest.mark.parametrize("N,S,W", EDGES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_edges(N, S, W, dtype):
    need_gpu()
    say("gated edge", N, S, W, dtype)
    Q, K, V = _inputs(1, 8, 2, 128, N, seed=N + S + W)
    alpha = np.array([0.3, 0.85], dtype=np.float32)
    out = _run(Q, K, V, alpha, S, W, dtype)
    check_close(out, _oracle(Q, K, V, alpha, S, W, dtype), dtype, f"gated edge N{N} S{S} W{W}")


@pytest.mark.gpu
def test_gated_long_window_boundary():
    """S=64, W=1024 over 5,000 tokens (the LLaMA-3-8B layer's heads at reduced
    length): rows around the window's first full reach and the row tiles' edges."""
    need_gpu()
    N, S, W = 5000, 64, 1024
    say("gated long")
    Q, K, V = _inputs(1, 8, 2, 128, N, seed=4242)
    alpha = np.array([0.6, 0.1], dtype=np.float32)
    out = _run(Q, K, V, alpha, S, W, "bf16")
    rows = np.unique(np.concatenate([np.arange(0, 70), np.arange(1020, 1100), np.arange(1150, 1220),
                                     np.arange(2550, 2600), np.arange(N - 70, N)]))
    check_close(out[:, :, rows], _oracle(Q, K, V, alpha, S, W, "bf16", rows=rows), "bf16", "gated long")


@pytest.mark.gpu
def test_gated_repeatable_and_endpoints():
    """Bitwise-repeatable; a gate of 1 on every head gives causal attention and
    a gate of 0 the sink+window attention (each against the oracle), and a
    gate of 1/2 lies halfway between the two library results."""
    need_gpu()
    import head_wise_kv_amd as H
    say("gated repeat/endpoints")
    N, S, W = 700, 16, 96
    Q, K, V = _inputs(2, 8, 4, 64, N, seed=31)
    Qd, Kd, Vd = (WL.to_torch(x, "bf16").cuda() for x in (Q, K, V))
    gate = lambda x: torch.full((4,), x, dtype=torch.float32, device="cuda")
    o1 = H.gated_attention(Qd, Kd, Vd, gate(1.0), S, W)
    o0 = H.gated_attention(Qd, Kd, Vd, gate(0.0), S, W)
    oh = H.gated_attention(Qd, Kd, Vd, gate(0.5), S, W)
    oh2 = H.gated_attention(Qd, Kd, Vd, gate(0.5), S, W)
    torch.cuda.synchronize()
    assert torch.equal(oh.view(torch.int16), oh2.view(torch.int16))
    check_close(o1, _oracle(Q, K, V, [1.0] * 4, S, W, "bf16"), "bf16", "gate 1")
    check_close(o0, _oracle(Q, K, V, [0.0] * 4, S, W, "bf16"), "bf16", "gate 0")
    mid = 0.5 * (o1.float() + o0.float())
    assert float((oh.float() - mid).abs().max()) <= 2 * 2 ** -8 * float(mid.abs().max() + 1)


@pytest.mark.gpu
def test_llama3_8b_gated_32k():
    """Gated-forward workload at full size: n_q=32, n_kv=8, d=128, bf16, one
    32,768-token sequence, S=64, W=1024, seeded gates; sampled rows of every
    head (the first tile, the window's first full reach, row-tile edges, the end)."""
    need_gpu()
    import head_wise_kv_amd as H
    w = WL.WORKLOADS["llama3_8b_gated_32k"]
    say(w.name)
    Q = WL.stacked_rows_f32(w, 0, WL.TENSOR_Q, w.n_q, 0, w.T)
    K = WL.stacked_rows_f32(w, 0, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, 0, WL.TENSOR_V, w.n_kv, 0, w.T)
    alpha = WL.gate_values(w, 0)
    Qd, Kd, Vd = (WL.to_torch(x, w.dtype).cuda() for x in (Q, K, V))
    out = H.gated_attention(Qd, Kd, Vd, torch.from_numpy(alpha).cuda(), w.S, w.W, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(1085, 1092), [127, 128, 4095, 4096, 16383],
                                     rng.integers(0, w.T, 12), np.arange(w.T - 4, w.T)]))
    ref = _oracle(Q, K, V, alpha, w.S, w.W, w.dtype, rows=rows)
    check_close(out[:, :, rows], ref, w.dtype, w.name)


@pytest.mark.gpu
def test_gated_errors():
    need_gpu()
    import head_wise_kv_amd as H
    say("gated errors")
    q = torch.zeros(1, 4, 10, 96, dtype=torch.bfloat16, device="cuda")
    a = torch.zeros(2, dtype=torch.float32, device="cuda")
    with pytest.raises(H.DuoError) as e:
        H.gated_attention(q, q[:, :2].contiguous(), q[:, :2].contiguous(), a, 1, 4)
    assert e.value.code == H.DUO_EUNSUPPORTED
    q = torch.zeros(1, 4, 10, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        H.gated_attention(q, k, k, a, 1, 0)
    assert e.value.code == H.DUO_EINVAL
    with pytest.raises(ValueError):
        H.gated_attention(q, k, k, a[:1].contiguous(), 1, 4)


def _draw_gated(seed):
    r = np.random.default_rng(seed)
    dtype = str(r.choice(["bf16", "bf16", "f32"]))
    d = int(r.choice([64, 128]))
    n_kv = int(r.integers(1, 5))
    g = int(r.choice([1, 2, 3, 4, 5, 8]))   # any group size, odd ones included
    B = int(r.integers(1, 3))
    N = int(r.integers(1, 900 if dtype == "bf16" else 300))
    S = int(r.choice([0, 1, 7, 64]))
    W = int(r.choice([1, 5, 64, 300]))
    alpha = r.uniform(0.0, 1.0, n_kv).astype(np.float32)
    alpha[r.random(n_kv) < 0.25] = 0.0
    alpha[r.random(n_kv) < 0.25] = 1.0
    return dtype, d, n_kv, g, B, N, S, W, alpha


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(24))
def test_gated_random_config(seed):
    """Seeded random shapes: dtype, d, group size (odd included), batch,
    sequence length (one token up), sinks, windows and gates (0 and 1
    included), against the oracle."""
    need_gpu()
    dtype, d, n_kv, g, B, N, S, W, alpha = _draw_gated(8000 + seed)
    say("gated random", dtype, d, n_kv, g, B, N, S, W)
    Q, K, V = _inputs(B, n_kv * g, n_kv, d, N, seed=8100 + seed, sink_rows=min(S, 4))
    out = _run(Q, K, V, alpha, S, W, dtype)
    check_close(out, _oracle(Q, K, V, alpha, S, W, dtype), dtype, f"gated random {seed}")
