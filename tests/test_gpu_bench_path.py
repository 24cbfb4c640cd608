"""The decode step in the launch configuration the bench times: the 70B GQA
shape, 80 layers at 128,000 tokens, one HIP graph of 80 fused
decode-appends.  Three layers hold the seeded host inputs (the others are
filled on the device, as the bench fills them); after one replay those three
layers' outputs are checked against the fp64 oracle, and a second replay must
reproduce the first bit for bit."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests.gpu_util import check_close, need_gpu, oracle_decode, say, stored

SAMPLED = (0, 41, 79)


@pytest.mark.gpu
def test_gqa70b_80_layer_graph_step():
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["gqa70b_decode_128k"]
    L, T = w.L, w.T
    say(w.name, "80-layer graph step")
    mask = WL.mask_table(w, L)
    c = DuoCache(L, w.B, w.n_q, w.n_kv, w.d, T, w.S, w.W, w.dtype, mask)
    host = {}
    buf_k = torch.empty(w.B, w.n_kv, T, w.d, dtype=torch.bfloat16, device="cuda")
    buf_v = torch.empty_like(buf_k)
    q = torch.empty(L, w.B, w.n_q, w.d, dtype=torch.bfloat16, device="cuda")
    for layer in range(L):
        if layer in SAMPLED:
            K = WL.stacked_rows_f32(w, layer, WL.TENSOR_K, w.n_kv, 0, T)
            V = WL.stacked_rows_f32(w, layer, WL.TENSOR_V, w.n_kv, 0, T)
            Q = WL.stacked_rows_f32(w, layer, WL.TENSOR_Q, w.n_q, T - 1, T)[:, :, 0]
            host[layer] = (K, V, Q)
            buf_k.copy_(WL.to_torch(K, w.dtype))
            buf_v.copy_(WL.to_torch(V, w.dtype))
            q[layer].copy_(WL.to_torch(Q, w.dtype))
        else:
            WL.device_fill_normal(buf_k, WL.device_seed(w, layer, WL.TENSOR_K))
            WL.device_fill_normal(buf_v, WL.device_seed(w, layer, WL.TENSOR_V))
            WL.device_fill_normal(q[layer], WL.device_seed(w, layer, WL.TENSOR_Q))
        c.append(layer, buf_k[:, :, : T - 1].contiguous(), buf_v[:, :, : T - 1].contiguous())
        # the step's new token of this layer (position T - 1) kept for the graph
        if layer == 0:
            k_new = torch.empty(L, w.B, w.n_kv, 1, w.d, dtype=torch.bfloat16, device="cuda")
            v_new = torch.empty_like(k_new)
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
    first = out.clone()
    for layer in SAMPLED:
        K, V, Q = host[layer]
        ref = oracle_decode(stored(Q, w.dtype), stored(K, w.dtype), stored(V, w.dtype), mask[layer], w.S, w.W,
                            w.scale)
        check_close(out[layer], ref, w.dtype, f"80-layer graph, layer {layer}")
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    assert np.isfinite(out.float().cpu().numpy()).all()
