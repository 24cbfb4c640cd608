"""The decode step in the launch configuration the bench times, for the two
full-model workloads: one HIP graph of a fused decode-append per layer.

  * 70B GQA shape: 80 layers at 128,000 tokens, layers 0, 41 and 79 checked;
  * 7B MHA shape: 32 layers at 131,072 tokens, layers 0, 15 and 31 checked.

The checked layers hold the seeded host inputs (the others are filled on the
device, as the bench fills them); after one replay their outputs are
compared with the fp64 oracle.  A second replay is the next step (the
kernels read each row's token count when they run): with the same new token
fed again it attends over T + 1 positions, checked on the first checked
layer, and duo_cache_sync then reports T + 1 tokens in every layer."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests.gpu_util import check_close, need_gpu, oracle_decode, say, stored

CASES = {"gqa70b_decode_128k": (0, 41, 79), "mha7b_decode_128k": (0, 15, 31)}


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(CASES))
def test_full_model_graph_step(name):
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS[name]
    sampled = CASES[name]
    L, T = w.L, w.T
    say(w.name, f"{L}-layer graph step, layers {sampled} checked")
    mask = WL.mask_table(w, L)
    c = DuoCache(L, w.B, w.n_q, w.n_kv, w.d, T + 1, w.S, w.W, w.dtype, mask)
    host = {}
    buf_k = torch.empty(w.B, w.n_kv, T, w.d, dtype=torch.bfloat16, device="cuda")
    buf_v = torch.empty_like(buf_k)
    q = torch.empty(L, w.B, w.n_q, w.d, dtype=torch.bfloat16, device="cuda")
    k_new = torch.empty(L, w.B, w.n_kv, 1, w.d, dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    for layer in range(L):
        if layer in sampled:
            K = WL.stacked_rows_f32(w, layer, WL.TENSOR_K, w.n_kv, 0, T)
            V = WL.stacked_rows_f32(w, layer, WL.TENSOR_V, w.n_kv, 0, T)
            Q = WL.stacked_rows_f32(w, layer, WL.TENSOR_Q, w.n_q, T - 1, T)[:, :, 0]
            host[layer] = (K, V, Q)
            buf_k.copy_(WL.to_torch(K, w.dtype))
            buf_v.copy_(WL.to_torch(V, w.dtype))
            q[layer].copy_(WL.to_torch(Q, w.dtype))
            say(f"layer {layer}: host inputs uploaded")
        else:
            WL.device_fill_normal(buf_k, WL.device_seed(w, layer, WL.TENSOR_K))
            WL.device_fill_normal(buf_v, WL.device_seed(w, layer, WL.TENSOR_V))
            WL.device_fill_normal(q[layer], WL.device_seed(w, layer, WL.TENSOR_Q))
        c.append(layer, buf_k[:, :, : T - 1].contiguous(), buf_v[:, :, : T - 1].contiguous())
        # the step's new token of this layer (position T - 1) kept for the graph
        k_new[layer].copy_(buf_k[:, :, T - 1:])
        v_new[layer].copy_(buf_v[:, :, T - 1:])
    del buf_k, buf_v
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for layer in range(L):
            c.decode_append(layer, k_new[layer], v_new[layer], q[layer], out=out[layer], scale=w.scale)
    graph.replay()
    torch.cuda.synchronize()
    for layer in sampled:
        K, V, Q = host[layer] if layer == sampled[0] else host.pop(layer)
        ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask[layer], w.S, w.W,
                            w.scale)
        check_close(out[layer], ref, w.dtype, f"{w.name} {L}-layer graph, layer {layer}")
        del K, V
    out.zero_()
    graph.replay()  # the next step: position T holds the same new token again
    torch.cuda.synchronize()
    K, V, Q = host.pop(sampled[0])
    K = np.concatenate([K, K[:, :, T - 1:]], axis=2)
    V = np.concatenate([V, V[:, :, T - 1:]], axis=2)
    ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask[sampled[0]], w.S, w.W,
                        w.scale)
    check_close(out[sampled[0]], ref, w.dtype, f"{w.name} {L}-layer graph, next step, layer {sampled[0]}")
    assert np.isfinite(out.float().cpu().numpy()).all()
    c.sync()
    assert all(c.seq_len(layer) == T + 1 for layer in range(L))
