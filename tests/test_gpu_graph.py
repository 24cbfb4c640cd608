"""HIP graph capture: the kernels read each row's token count from the
device when they run, so a captured duo_decode_append replays as the next
generation step (at the next position), and a captured duo_append appends at
the next positions.  Each replay is checked bit for bit against the same step
made eagerly on a twin cache (its inputs copied into the captured buffers
first), the final caches against each other, the host counts after
duo_cache_sync, and the outputs against the fp64 oracle.  Replays are
separated by unrelated eager work and synchronisations.  A replay that finds
no room stores nothing, does not advance, and is reported by duo_cache_sync."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import rope as RP
from tests.gpu_util import check_close, need_gpu, say, stored

CASES = [
    # (page_rows, rope_theta, kv_format, T held before the first captured step)
    (0, 0.0, None, 700),
    (256, 0.0, None, 509),       # the replays cross into page 2
    (256, 10000.0, None, 510),
    (0, 0.0, "fp8", 300),
    (256, 10000.0, "fp8", 253),
    (0, 10000.0, None, 65),      # the streaming heads' S + W = 68 slots fill during the replays
    (0, 0.0, "int4", 300),
    (512, 10000.0, "int4", 1021),  # INT4 rows in 512-row pages, crossing into page 2
]
STEPS = 6
B, N_Q, N_KV, D, S, W = 2, 16, 4, 128, 4, 64


def _caches(page_rows, theta, kvf, T_cap, mask, L=2):
    from head_wise_kv_amd import DuoCache
    kw = dict(kv_format=kvf, rope_theta=theta)
    if page_rows:
        kw.update(page_rows=page_rows, n_pages=B * (-(-T_cap // page_rows)))
    return [DuoCache(L, B, N_Q, N_KV, D, T_cap, S, W, "bf16", [mask, mask[::-1]][:L], **kw) for _ in range(2)]


def _same_cache(a, b, layers, held):
    for layer in range(layers):
        for h in range(N_KV):
            x, y = a.read_head(layer, h), b.read_head(layer, h)
            n = min(held, x[0].shape[1])
            assert torch.equal(x[0][:, :n].view(torch.uint8), y[0][:, :n].view(torch.uint8)), (layer, h)
            assert torch.equal(x[1][:, :n].view(torch.uint8), y[1][:, :n].view(torch.uint8)), (layer, h)
            if x[2] is not None:
                assert torch.equal(x[2], y[2]), (layer, h)


def _unrelated_work():
    x = torch.randn(2048, 1024, device="cuda")
    float((x @ x.T).sum())
    torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.parametrize("page_rows,theta,kvf,T", CASES)
def test_graph_replays_are_successive_steps(page_rows, theta, kvf, T):
    need_gpu()
    say("graph replay", page_rows, theta, kvf, T)
    mask = [1, 0, 1, 0]
    T_cap = T + STEPS
    K = WL.normal_f32((B, N_KV, T_cap, D), 2100 + T)
    V = WL.normal_f32((B, N_KV, T_cap, D), 2101 + T)
    Q = WL.normal_f32((STEPS, B, N_Q, D), 2102 + T)
    Kd, Vd = WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda()
    Qd = WL.to_torch(Q, "bf16").cuda()
    eager, captured = _caches(page_rows, theta, kvf, T_cap, mask)
    for c in (eager, captured):
        for layer in range(2):
            c.append(layer, Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
    # the captured step's inputs and outputs live in fixed buffers
    kn = torch.empty(B, N_KV, 1, D, dtype=torch.bfloat16, device="cuda")
    vn, q = torch.empty_like(kn), torch.empty(B, N_Q, D, dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty_like(q) for _ in range(2)]
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for layer in range(2):
            captured.decode_append(layer, kn, vn, q, out=outs[layer])
    for layer in range(2):
        # pages for the replays: the capture counted (and took the page of) the first step
        captured.reserve(layer, STEPS - 1)
    for i in range(STEPS):
        p = T + i
        kn.copy_(Kd[:, :, p:p + 1])
        vn.copy_(Vd[:, :, p:p + 1])
        q.copy_(Qd[i])
        for o in outs:
            o.zero_()
        graph.replay()
        want = [eager.decode_append(layer, Kd[:, :, p:p + 1].contiguous(), Vd[:, :, p:p + 1].contiguous(), Qd[i])
                for layer in range(2)]
        torch.cuda.synchronize()
        if i == 0:
            # the same plan as the eager call: the same launch, bit for bit.  Later
            # replays keep the work split planned at capture (its last item of
            # each head covers the rows added since), where an eager call re-plans,
            # so their fp32 partial sums may be added in another order.
            for layer in range(2):
                assert torch.equal(outs[layer].view(torch.int16), want[layer].view(torch.int16)), layer
        for layer in range(2):
            got = outs[layer].clone()
            for b in range(B):
                check_close(got[b], _oracle_step(K, V, Q, i, b, T + i, [mask, mask[::-1]][layer], theta, kvf), "bf16",
                            f"graph replay {i} layer {layer} row {b}")
        _unrelated_work()
    captured.sync()
    for layer in range(2):
        for b in range(B):
            assert captured.row_len(layer, b) == T + STEPS
    _same_cache(eager, captured, 2, T + STEPS)


def _oracle_step(K, V, Q, i, b, p, mask, theta, kvf):
    """The fused step at position p (query Q[i, b]) over positions 0..p."""
    from oracle import quant as OQ
    q = stored(Q[i, b], "bf16")
    Kb = stored(K[b, :, :p + 1], "bf16")
    Vb = stored(V[b, :, :p + 1], "bf16")
    if theta:
        return RP.decode_step_rope(q, Kb, Vb.astype(np.float32) if kvf else Vb, mask, S, W, D ** -0.5, theta, "bf16",
                                   kv_format=kvf)
    if kvf == "fp8":
        return OQ.decode_step_fp8(q, Kb.astype(np.float32), Vb.astype(np.float32), mask, S, W, D ** -0.5)
    if kvf == "int4":
        from oracle import quant4 as OQ4
        return OQ4.decode_step_int4(q, Kb.astype(np.float32), Vb.astype(np.float32), mask, S, W, D ** -0.5)
    return OA.decode_step(q, Kb, Vb, mask, S, W, D ** -0.5)


@pytest.mark.gpu
@pytest.mark.parametrize("page_rows", [0, 256])
def test_captured_bulk_append_advances(page_rows):
    need_gpu()
    say("captured append", page_rows)
    mask = [0, 1, 1, 0]
    T, n, R = 250, 3, 4
    T_cap = T + n * R
    K = WL.normal_f32((B, N_KV, T_cap, D), 2200)
    V = WL.normal_f32((B, N_KV, T_cap, D), 2201)
    Kd, Vd = WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda()
    eager, captured = _caches(page_rows, 0.0, None, T_cap, mask, L=1)
    for c in (eager, captured):
        c.append(0, Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
    kb = torch.empty(B, N_KV, n, D, dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        captured.append(0, kb, vb)
    captured.reserve(0, n * (R - 1))  # the capture counted the first append
    for i in range(R):
        p = T + n * i
        kb.copy_(Kd[:, :, p:p + n])
        vb.copy_(Vd[:, :, p:p + n])
        graph.replay()
        eager.append(0, Kd[:, :, p:p + n].contiguous(), Vd[:, :, p:p + n].contiguous())
        torch.cuda.synchronize()
    captured.sync()
    assert captured.seq_len(0) == T_cap
    _same_cache(eager, captured, 1, T_cap)


@pytest.mark.gpu
@pytest.mark.parametrize("page_rows", [0, 256])
def test_replay_without_room_stores_nothing(page_rows):
    need_gpu()
    say("replay without room", page_rows)
    import head_wise_kv_amd as H
    mask = [1, 0, 1, 0]
    # contiguous: T_cap is reached after 2 replays; paged: page 0 (positions
    # 0..255) is full after 2 replays and no further page is reserved
    T = 254
    T_cap = T + 2 if page_rows == 0 else 1024
    K = WL.normal_f32((B, N_KV, T + 5, D), 2300)
    V = WL.normal_f32((B, N_KV, T + 5, D), 2301)
    Q = WL.normal_f32((B, N_Q, D), 2302)
    Kd, Vd, q = WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda(), WL.to_torch(Q, "bf16").cuda()
    c, _ = _caches(page_rows, 0.0, None, T_cap, mask, L=1)
    c.append(0, Kd[:, :, :T].contiguous(), Vd[:, :, :T].contiguous())
    kn = torch.empty(B, N_KV, 1, D, dtype=torch.bfloat16, device="cuda")
    vn = torch.empty_like(kn)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        c.decode_append(0, kn, vn, q, out=out)
    snap = None
    for i in range(4):
        kn.copy_(Kd[:, :, T + i:T + i + 1])
        vn.copy_(Vd[:, :, T + i:T + i + 1])
        graph.replay()
        torch.cuda.synchronize()
        if i == 1:
            snap = [c.read_head(0, h) for h in range(N_KV)]
            c.sync()
            assert c.seq_len(0) == T + 2
        if i >= 2:
            # the row is full: the step attends to its token but stores nothing
            Ks, Vs = stored(K[:, :, :T + 3], "bf16"), stored(V[:, :, :T + 3], "bf16")
            Ks[:, :, T + 2] = stored(K[:, :, T + i], "bf16")  # this replay's token, in the position after the held ones
            Vs[:, :, T + 2] = stored(V[:, :, T + i], "bf16")
            for b in range(B):
                ref = OA.decode_step(stored(Q[b], "bf16"), Ks[b], Vs[b], mask, S, W, D ** -0.5)
                check_close(out[b], ref, "bf16", f"full row, replay {i} row {b}")
    with pytest.raises(H.DuoError) as e:
        c.sync()
    assert e.value.code == H.DUO_ECAPACITY
    assert c.seq_len(0) == T + 2
    for h in range(N_KV):
        after = c.read_head(0, h)
        for x, y in zip(after, snap[h]):
            if x is not None:
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), h
    c.sync()  # the flag was cleared by the report
