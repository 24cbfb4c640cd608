"""Fused append + decode (duo_decode_append) against the fp64 oracle, and its
cache state against the same tokens appended by duo_append."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests.gpu_util import check_close, need_gpu, oracle_decode, say, stored


def _steps_case(B, n_q, n_kv, d, dtype, T0, steps, S, W, mask, seed, check_every=1):
    """Fill T0 tokens with duo_append, then run `steps` fused steps; every
    `check_every`-th output is compared with the oracle at its context length.
    Returns the fused cache and the K/V tensors used."""
    from head_wise_kv_amd import DuoCache
    T = T0 + steps
    K = WL.normal_f32((B, n_kv, T, d), seed)
    V = WL.normal_f32((B, n_kv, T, d), seed + 1)
    Q = WL.normal_f32((B, n_q, T, d), seed + 2)
    K[:, :, :S] *= np.float32(4.0)
    c = DuoCache(1, B, n_q, n_kv, d, T, S, W, dtype, [mask])
    Kd, Vd = WL.to_torch(K, dtype).cuda(), WL.to_torch(V, dtype).cuda()
    Qd = WL.to_torch(Q, dtype).cuda()
    if T0:
        c.append(0, Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    Ks, Vs, Qs = stored(K, dtype), stored(V, dtype), stored(Q, dtype)
    scale = 1.0 / np.sqrt(d)
    for i in range(steps):
        t = T0 + i  # position of the appended token (and of the query)
        out = c.decode_append(0, Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous(),
                              Qd[:, :, t].contiguous(), scale=scale)
        assert c.seq_len(0) == t + 1
        if i % check_every == 0 or i == steps - 1:
            torch.cuda.synchronize()
            ref = oracle_decode(Qs[:, :, t], Ks[:, :, :t + 1], Vs[:, :, :t + 1], mask, S, W, scale)
            check_close(out, ref, dtype, f"step t={t}")
    return c, Kd, Vd


@pytest.mark.gpu
@pytest.mark.parametrize("T0", [0, 3, 19, 20, 21, 57])
def test_decode_append_each_step(T0):
    """From an empty cache, inside the sinks, at S+W-1, S+W (first eviction) and
    past it: 24 fused steps, each checked (S=4, W=16; ring fills and wraps)."""
    need_gpu()
    say("decode_append steps T0", T0)
    _steps_case(2, 8, 4, 64, "bf16", T0, 24, 4, 16, [1, 0, 1, 0], seed=300 + T0)


GRID = [(dt, d, g) for dt in ("bf16", "f32") for d in (64, 128) for g in (1, 2, 3, 4, 6, 8)] + [("bf16", 128, 16)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g", GRID)
def test_decode_append_grid(dtype, d, g):
    """Every built dtype x d x g across the ring-full boundary and a ragged tile tail."""
    need_gpu()
    say("decode_append grid", dtype, d, g)
    _steps_case(2, 3 * g, 3, d, dtype, 690, 6, 4, 16, [1, 0, 0], seed=11 * g + d, check_every=2)


@pytest.mark.gpu
def test_decode_append_cache_matches_append():
    """After fused steps the cache holds exactly the bytes and positions that
    duo_append of the same tokens writes (bit-exact)."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("decode_append cache state")
    B, n_q, n_kv, d, S, W = 2, 8, 4, 128, 4, 16
    mask = [1, 0, 0, 1]
    c, Kd, Vd = _steps_case(B, n_q, n_kv, d, "bf16", 5, 40, S, W, mask, seed=77, check_every=10)
    ref = DuoCache(1, B, n_q, n_kv, d, 45, S, W, "bf16", [mask])
    for t in range(45):
        ref.append(0, Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous())
    torch.cuda.synchronize()
    for h in range(n_kv):
        k1, v1, p1 = c.read_head(0, h)
        k2, v2, p2 = ref.read_head(0, h)
        held = 45 if mask[h] else S + W
        assert torch.equal(k1[:, :held].view(torch.int16), k2[:, :held].view(torch.int16)), f"K head {h}"
        assert torch.equal(v1[:, :held].view(torch.int16), v2[:, :held].view(torch.int16)), f"V head {h}"
        if p1 is not None:
            assert np.array_equal(np.asarray(p1), np.asarray(p2)), f"pos head {h}"


@pytest.mark.gpu
def test_decode_append_no_sinks_window_one():
    """S=0, W=1: a streaming head holds one token, which every step evicts."""
    need_gpu()
    say("decode_append S0 W1")
    _steps_case(1, 4, 2, 64, "bf16", 2, 8, 0, 1, [1, 0], seed=41)


@pytest.mark.gpu
def test_gqa70b_decode_append_128k_layer():
    """70B GQA shape at full size (T=128000, S=64, W=1024): positions 0..T-2
    filled, then the fused step appends position T-1 and decodes it."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["gqa70b_decode_128k"]
    layer = 3
    say(w.name, "fused layer", layer)
    mask = WL.retrieval_mask(w, layer)
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask])
    K = WL.stacked_rows_f32(w, layer, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, layer, WL.TENSOR_V, w.n_kv, 0, w.T)
    Q = WL.stacked_rows_f32(w, layer, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0]
    Kt, Vt = WL.to_torch(K, w.dtype).cuda(), WL.to_torch(V, w.dtype).cuda()
    c.append(0, Kt[:, :, : w.T - 1].contiguous(), Vt[:, :, : w.T - 1].contiguous())
    out = c.decode_append(0, Kt[:, :, w.T - 1:].contiguous(), Vt[:, :, w.T - 1:].contiguous(),
                          WL.to_torch(Q, w.dtype).cuda(), scale=w.scale)
    ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask, w.S, w.W, w.scale)
    check_close(out, ref, w.dtype, f"{w.name} fused layer {layer}")


@pytest.mark.gpu
def test_decode_append_errors_leave_state_unchanged():
    need_gpu()
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("decode_append errors")
    c = DuoCache(1, 1, 4, 2, 64, 3, 1, 2, "bf16", [[1, 0]])
    k = torch.zeros(1, 2, 1, 64, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        c.decode_append(0, k, k, q)
    assert c.seq_len(0) == 3
    with pytest.raises(H.DuoError) as e:
        c.decode_append(0, k, k, q)
    assert e.value.code == H.DUO_ECAPACITY and c.seq_len(0) == 3
    with pytest.raises(H.DuoError) as e:
        c.decode_append(1, k, k, q)
    assert e.value.code == H.DUO_EINVAL
