"""Decode parity: libduo's duo_decode against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from tests.gpu_util import check_close, need_gpu, oracle_decode, say, stored


def _decode_case(B, n_q, n_kv, d, dtype, T, S, W, mask, seed, pattern=None, sink_scale=4.0, layer_count=1):
    from head_wise_kv_amd import DuoCache
    K = WL.normal_f32((B, n_kv, T, d), seed)
    V = WL.normal_f32((B, n_kv, T, d), seed + 1)
    Q = WL.normal_f32((B, n_q, d), seed + 2)
    K[:, :, :S] *= np.float32(sink_scale)
    c = DuoCache(layer_count, B, n_q, n_kv, d, T, S, W, dtype, [mask] * layer_count)
    Kd, Vd = WL.to_torch(K, dtype).cuda(), WL.to_torch(V, dtype).cuda()
    p = 0
    for n in (pattern or [T]):
        c.append(layer_count - 1, Kd[:, :, p:p + n].contiguous(), Vd[:, :, p:p + n].contiguous())
        p += n
    out = c.decode(layer_count - 1, WL.to_torch(Q, dtype).cuda())
    torch.cuda.synchronize()
    ref = oracle_decode(stored(Q, dtype), stored(K, dtype), stored(V, dtype), mask, S, W, 1.0 / np.sqrt(d))
    return out, ref


@pytest.mark.gpu
def test_tiny_decode_workload():
    """1 layer, n_q=4, n_kv=2, d=64, fp32, T=512, head 0 retrieval, head 1 streaming (S=4, W=64)."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["tiny_decode"]
    say(w.name)
    mask = WL.retrieval_mask(w, 0)
    K = WL.stacked_rows_f32(w, 0, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, 0, WL.TENSOR_V, w.n_kv, 0, w.T)
    Q = WL.stacked_rows_f32(w, 0, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0]
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask])
    c.append(0, WL.to_torch(K, w.dtype).cuda(), WL.to_torch(V, w.dtype).cuda())
    out = c.decode(0, WL.to_torch(Q, w.dtype).cuda(), scale=w.scale)
    ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask, w.S, w.W, w.scale)
    check_close(out, ref, w.dtype, w.name)


GRID = []
for dtype in ("bf16", "f32"):
    for d in (64, 128):
        for g in (1, 2, 3, 4, 5, 6, 7, 8):
            GRID.append((dtype, d, g))
# groups above 8 run only where the scores use the matrix cores (bf16, d = 128)
GRID += [("bf16", 128, 12), ("bf16", 128, 16)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g", GRID)
@pytest.mark.parametrize("T", [1, 3, 9, 21, 37, 700, 1500])
def test_decode_grid(dtype, d, g, T):
    """Edge lengths around S=4, W=16: T < S, S <= T < S+W, T = S+W+1, ring wrap,
    several tiles and a ragged tail, in every built dtype x d x g."""
    need_gpu()
    n_kv = 4
    mask = [1, 0, 1, 0]
    say("grid", dtype, d, g, T)
    out, ref = _decode_case(2, n_kv * g, n_kv, d, dtype, T, 4, 16, mask, seed=T * 100 + g * 10 + d)
    check_close(out, ref, dtype, f"grid {dtype} d{d} g{g} T{T}")


@pytest.mark.gpu
@pytest.mark.parametrize("mask", [[1, 1], [0, 0]])
def test_decode_uniform_masks(mask):
    """All retrieval (full causal attention) and all streaming (sinks + window)."""
    need_gpu()
    say("uniform", mask)
    out, ref = _decode_case(1, 8, 2, 128, "bf16", 5000, 32, 256, mask, seed=5)
    check_close(out, ref, "bf16", f"mask {mask}")


@pytest.mark.gpu
def test_decode_after_ragged_appends():
    """Cache filled by appends of mixed sizes, including bulk appends larger than W."""
    need_gpu()
    say("ragged appends")
    out, ref = _decode_case(3, 16, 4, 128, "bf16", 2000, 5, 64, [0, 1, 0, 0], seed=9,
                            pattern=[1, 2, 300, 1, 77, 1000, 619])
    check_close(out, ref, "bf16", "ragged")


@pytest.mark.gpu
def test_decode_single_head_many_partials():
    """One retrieval head spread over every work item: the combine kernel merges
    one partial per compute unit."""
    need_gpu()
    say("single head, many partials")
    out, ref = _decode_case(1, 8, 1, 128, "bf16", 300000, 4, 64, [1], seed=11, sink_scale=1.0)
    check_close(out, ref, "bf16", "many partials")


@pytest.mark.gpu
def test_decode_repeated_calls_bitwise_equal():
    """The workspace keeps no state between calls: the same decode twice gives
    the same bits."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("repeat")
    B, n_q, n_kv, d, T = 1, 8, 2, 128, 70000
    K = WL.normal_f32((B, n_kv, T, d), 21)
    V = WL.normal_f32((B, n_kv, T, d), 22)
    Q = WL.normal_f32((B, n_q, d), 23)
    c = DuoCache(1, B, n_q, n_kv, d, T, 8, 128, "bf16", [[1, 0]])
    c.append(0, WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda())
    q = WL.to_torch(Q, "bf16").cuda()
    o1 = c.decode(0, q).clone()
    o2 = c.decode(0, q).clone()
    assert torch.equal(o1, o2)


@pytest.mark.gpu
def test_llama3_8b_decode_b8_32k():
    """LLaMA-3-8B-shaped layer, batch 8, T=32768, S=32, W=1024, 2/8 retrieval, sink keys x4 (full size)."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["llama3_8b_decode_b8_32k"]
    say(w.name)
    mask = WL.retrieval_mask(w, 0)
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask])
    K = WL.stacked_rows_f32(w, 0, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, 0, WL.TENSOR_V, w.n_kv, 0, w.T)
    Q = WL.stacked_rows_f32(w, 0, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0]
    c.append(0, WL.to_torch(K, w.dtype).cuda(), WL.to_torch(V, w.dtype).cuda())
    out = c.decode(0, WL.to_torch(Q, w.dtype).cuda(), scale=w.scale)
    ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask, w.S, w.W, w.scale)
    check_close(out, ref, w.dtype, w.name)


def _full_model_layer(w, layer):
    """One layer of a decode-with-append workload at its full per-layer shape:
    fill positions 0..T-2, append position T-1 (one token), decode."""
    from head_wise_kv_amd import DuoCache
    mask = WL.retrieval_mask(w, layer)
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask])
    K = WL.stacked_rows_f32(w, layer, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, layer, WL.TENSOR_V, w.n_kv, 0, w.T)
    Q = WL.stacked_rows_f32(w, layer, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0]
    Kt, Vt = WL.to_torch(K, w.dtype).cuda(), WL.to_torch(V, w.dtype).cuda()
    c.append(0, Kt[:, :, : w.T - 1].contiguous(), Vt[:, :, : w.T - 1].contiguous())
    c.append(0, Kt[:, :, w.T - 1:].contiguous(), Vt[:, :, w.T - 1:].contiguous())
    out = c.decode(0, WL.to_torch(Q, w.dtype).cuda(), scale=w.scale)
    ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask, w.S, w.W, w.scale)
    return out, ref


@pytest.mark.gpu
@pytest.mark.parametrize("layer", [0, 79])
def test_gqa70b_decode_128k_layer(layer):
    """70B GQA shape: n_q=64, n_kv=8, d=128, bf16, T=128000, S=64, W=1024, 2/8 retrieval; append 1 + decode."""
    need_gpu()
    w = WL.WORKLOADS["gqa70b_decode_128k"]
    say(w.name, "layer", layer)
    out, ref = _full_model_layer(w, layer)
    check_close(out, ref, w.dtype, f"{w.name} layer {layer}")


@pytest.mark.gpu
@pytest.mark.parametrize("layer", [31])
def test_mha7b_decode_128k_layer(layer):
    """7B MHA shape: n_q=n_kv=32, d=128, bf16, T=131072, S=64, W=1024, 16/32 retrieval; append 1 + decode."""
    need_gpu()
    w = WL.WORKLOADS["mha7b_decode_128k"]
    say(w.name, "layer", layer)
    out, ref = _full_model_layer(w, layer)
    check_close(out, ref, w.dtype, f"{w.name} layer {layer}")


@pytest.mark.gpu
def test_error_paths_leave_state_unchanged():
    need_gpu()
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("errors")
    c = DuoCache(2, 1, 4, 2, 64, 10, 2, 4, "bf16", [[1, 0], [0, 0]])
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.decode(0, q)
    assert e.value.code == H.DUO_EEMPTY
    k = torch.zeros(1, 2, 11, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.append(0, k, k)
    assert e.value.code == H.DUO_ECAPACITY
    assert c.seq_len(0) == 0
    c.append(0, k[:, :, :10].contiguous(), k[:, :, :10].contiguous())
    assert c.seq_len(0) == 10
    with pytest.raises(H.DuoError) as e:
        c.append(0, k[:, :, :1].contiguous(), k[:, :, :1].contiguous())
    assert e.value.code == H.DUO_ECAPACITY and c.seq_len(0) == 10
    with pytest.raises(H.DuoError) as e:
        c.append(5, k, k)
    assert e.value.code == H.DUO_EINVAL
    import ctypes
    rc = H.lib.duo_decode(c._h, 0, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()), 1.0,
                          ctypes.c_void_p(c.workspace.data_ptr()), 16, None)
    assert rc == H.DUO_EWORKSPACE
    assert c.seq_len(1) == 0
