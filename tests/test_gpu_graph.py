"""HIP graph capture: a captured duo_decode_append / duo_decode replays the
same launches with the same arguments, so every replay must give the eager
call's output and leave the same cache, bit for bit.  Replays are separated
by unrelated eager work and synchronisations, and the cases include a step
that starts a new page (the captured launches then include the page-table
write) and rotary positions."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import rope as RP
from tests.gpu_util import check_close, need_gpu, say, stored

CASES = [
    # (page_rows, rope_theta, kv_format, T before the captured step)
    (0, 0.0, None, 700),
    (256, 0.0, None, 512),       # the captured step's token starts page 2
    (256, 10000.0, None, 512),
    (0, 0.0, "fp8", 300),
    (256, 10000.0, "fp8", 256),
]


def _pair(page_rows, theta, kvf, B, n_q, n_kv, d, T_cap, S, W, mask):
    from head_wise_kv_amd import DuoCache
    kw = dict(kv_format=kvf, rope_theta=theta)
    if page_rows:
        kw.update(page_rows=page_rows, n_pages=B * (-(-T_cap // page_rows)))
    return [DuoCache(2, B, n_q, n_kv, d, T_cap, S, W, "bf16", [mask, mask[::-1]], **kw) for _ in range(2)]


@pytest.mark.gpu
@pytest.mark.parametrize("page_rows,theta,kvf,T", CASES)
def test_graph_replays_match_eager(page_rows, theta, kvf, T):
    need_gpu()
    say("graph replay", page_rows, theta, kvf, T)
    B, n_q, n_kv, d, S, W = 2, 16, 4, 128, 4, 64
    mask = [1, 0, 1, 0]
    T_cap = T + 1
    K = WL.normal_f32((B, n_kv, T_cap, d), 2100 + T)
    V = WL.normal_f32((B, n_kv, T_cap, d), 2101 + T)
    Q = WL.normal_f32((B, n_q, d), 2102 + T)
    Kd, Vd = WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda()
    q = WL.to_torch(Q, "bf16").cuda()
    kn, vn = Kd[:, :, T:].contiguous(), Vd[:, :, T:].contiguous()
    eager, captured = _pair(page_rows, theta, kvf, B, n_q, n_kv, d, T_cap, S, W, mask)
    for c in (eager, captured):
        for layer in range(2):
            c.append(layer, Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
    torch.cuda.synchronize()
    want = [eager.decode_append(layer, kn, vn, q) for layer in range(2)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(q) for _ in range(2)]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for layer in range(2):
            captured.decode_append(layer, kn, vn, q, out=outs[layer])
    for rep in range(4):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for layer in range(2):
            assert torch.equal(outs[layer].view(torch.int16), want[layer].view(torch.int16)), (rep, layer)
        # unrelated eager work between replays
        x = torch.randn(4096, 1024, device="cuda")
        float((x @ x.T).sum())
        torch.cuda.synchronize()
    for layer in range(2):
        for h in range(n_kv):
            a, b = eager.read_head(layer, h), captured.read_head(layer, h)
            held = T + 1  # positions past a row's count on its last page are never written
            assert torch.equal(a[0][:, :held].view(torch.uint8), b[0][:, :held].view(torch.uint8)), (layer, h)
            assert torch.equal(a[1][:, :held].view(torch.uint8), b[1][:, :held].view(torch.uint8)), (layer, h)
            if a[2] is not None:
                assert torch.equal(a[2], b[2]), (layer, h)
    # the replayed result against the oracle (layer 0)
    if kvf is None:
        Ks, Vs = stored(K, "bf16"), stored(V, "bf16")
        for b in range(B):
            if theta:
                ref = RP.decode_step_rope(stored(Q[b], "bf16"), Ks[b], Vs[b], mask, S, W, d ** -0.5, theta, "bf16")
            else:
                from oracle import attention as OA
                ref = OA.decode_step(stored(Q[b], "bf16"), Ks[b], Vs[b], mask, S, W, d ** -0.5)
            check_close(outs[0][b], ref, "bf16", f"graph replay row {b}")
