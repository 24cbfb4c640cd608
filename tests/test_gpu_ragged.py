"""Ragged batches: batch rows that hold different token counts, grown with
duo_append_row / duo_prefill_chunk_row / duo_append and decoded together.
Every row is checked against the fp64 oracle on that row alone (rows are
independent sequences), and the cache state bit-exactly."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import cache as OC
from oracle import quant as OQ
from tests.gpu_util import check_close, need_gpu, say, stored


def _rows(B, n_kv, N, d, seed, n_q):
    K = WL.normal_f32((B, n_kv, N, d), seed)
    V = WL.normal_f32((B, n_kv, N, d), seed + 1)
    Q = WL.normal_f32((B, n_q, N, d), seed + 2)
    return K, V, Q


def _ref_decode(Q, K, V, b, t, mask, S, W, d, dtype, fp8):
    """Oracle output of row b for the query at position t over positions 0..t."""
    q = stored(Q[b, :, t], dtype)
    Ks, Vs = stored(K[b, :, :t + 1], dtype), stored(V[b, :, :t + 1], dtype)
    if fp8:
        return OQ.decode_step_fp8(q, Ks.astype(np.float32), Vs.astype(np.float32), mask, S, W, d ** -0.5)
    return OA.decode_step(q, Ks, Vs, mask, S, W, d ** -0.5)


def _check_rows_cache(c, K, V, lens, mask, S, W, dtype):
    st_k, st_v = WL.to_torch(K, dtype), WL.to_torch(V, dtype)
    for h in range(K.shape[1]):
        Kc, Vc, pos = c.read_head(0, h)
        for b, n in enumerate(lens):
            for slot, p in OC.slot_table(n, bool(mask[h]), S, W).items():
                assert torch.equal(Kc[b, slot], st_k[b, h, p]) and torch.equal(Vc[b, slot], st_v[b, h, p]), (h, b, slot)
                if pos is not None:
                    assert int(pos[b, slot]) == p, (h, b, slot)


CASES = [("bf16", 128, 4, None), ("bf16", 64, 8, None), ("f32", 64, 1, None), ("bf16", 128, 8, "fp8"),
         ("bf16", 128, 1, "fp8")]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g,kvf", CASES)
def test_ragged_decode(dtype, d, g, kvf):
    """Rows of 1, 17, 300, 2,049 and 64 tokens in one decode; each row's
    query at its own position."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("ragged decode", dtype, d, g, kvf)
    lens = [1, 17, 300, 2049, 64]
    B, n_kv, S, W = len(lens), 4, 4, 64
    mask = [1, 0, 1, 0]
    n_q = n_kv * g
    N = max(lens)
    K, V, Q = _rows(B, n_kv, N, d, 900 + d + g, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, dtype, [mask], kv_format=kvf)
    Kd, Vd, Qd = (WL.to_torch(x, dtype).cuda() for x in (K, V, Q))
    for b, n in enumerate(lens):
        c.append_row(0, b, Kd[b:b + 1, :, :n].contiguous(), Vd[b:b + 1, :, :n].contiguous())
        assert c.row_len(0, b) == n
    q = torch.stack([Qd[b, :, n - 1] for b, n in enumerate(lens)]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        ref = _ref_decode(Q, K, V, b, n - 1, mask, S, W, d, dtype, kvf == "fp8")
        check_close(out[b], ref, dtype, f"ragged row {b} (len {n})")


@pytest.mark.gpu
@pytest.mark.parametrize("kvf", [None, "fp8"])
def test_ragged_decode_append_steps(kvf):
    """Fused steps over rows starting at 0 (empty), 5 and 30 tokens (S=4,
    W=16: the rows fill and wrap their rings at different steps); each step
    checked per row, the cache bit-exact at the end."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("ragged fused", kvf)
    start = [0, 5, 30]
    steps = 22
    B, n_q, n_kv, d, S, W = len(start), 8, 4, 128, 4, 16
    mask = [1, 0, 0, 1]
    N = max(start) + steps
    K, V, Q = _rows(B, n_kv, N, d, 950, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], kv_format=kvf)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    for b, n in enumerate(start):
        if n:
            c.append_row(0, b, Kd[b:b + 1, :, :n].contiguous(), Vd[b:b + 1, :, :n].contiguous())
    for i in range(steps):
        t = [n + i for n in start]  # each row's new position
        kn = torch.stack([Kd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        vn = torch.stack([Vd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        q = torch.stack([Qd[b, :, t[b]] for b in range(B)]).contiguous()
        out = c.decode_append(0, kn, vn, q)
        if i % 4 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            for b in range(B):
                ref = _ref_decode(Q, K, V, b, t[b], mask, S, W, d, "bf16", kvf == "fp8")
                check_close(out[b], ref, "bf16", f"ragged fused step {i} row {b}")
    torch.cuda.synchronize()
    lens = [n + steps for n in start]
    assert [c.row_len(0, b) for b in range(B)] == lens
    if kvf is None:
        _check_rows_cache(c, K, V, lens, mask, S, W, "bf16")
    else:
        Ks, Vs = stored(K, "bf16").astype(np.float32), stored(V, "bf16").astype(np.float32)
        for h in range(n_kv):
            kc, vc, _ = c.read_head(0, h)
            ksc, vsc = c.head_scales(0, h)
            for b, n in enumerate(lens):
                for slot, p in OC.slot_table(n, bool(mask[h]), S, W).items():
                    ck, sk = OQ.quantize_rows(Ks[b, h, p])
                    assert np.array_equal(kc[b, slot].numpy(), ck) and float(ksc[b, slot]) == float(sk), (h, b, slot)
                    cv, sv = OQ.quantize_rows(Vs[b, h, p])
                    assert np.array_equal(vc[b, slot].numpy(), cv) and float(vsc[b, slot]) == float(sv), (h, b, slot)


@pytest.mark.gpu
def test_append_all_rows_at_their_own_counts():
    """duo_append of 7 tokens to rows holding 3, 20 and 0 tokens puts each
    row's tokens at that row's positions."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("ragged append")
    B, n_q, n_kv, d, S, W = 3, 4, 2, 128, 2, 8
    mask = [1, 0]
    start = [3, 20, 0]
    N = 27
    K, V, _ = _rows(B, n_kv, N + 7, d, 970, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask])
    Kd, Vd = WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda()
    for b, n in enumerate(start):
        if n:
            c.append_row(0, b, Kd[b:b + 1, :, :n].contiguous(), Vd[b:b + 1, :, :n].contiguous())
    kn = torch.stack([Kd[b, :, n:n + 7] for b, n in enumerate(start)]).contiguous()
    vn = torch.stack([Vd[b, :, n:n + 7] for b, n in enumerate(start)]).contiguous()
    c.append(0, kn, vn)
    torch.cuda.synchronize()
    _check_rows_cache(c, K, V, [n + 7 for n in start], mask, S, W, "bf16")


@pytest.mark.gpu
@pytest.mark.parametrize("kvf", [None, "fp8"])
def test_prefill_rows_then_decode(kvf):
    """Row 1 prefilled in chunks of 200, row 2 in one chunk of 333, row 0 given
    5 tokens by append; the prefill outputs of each row against the oracle,
    then one decode of all three rows."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("ragged prefill", kvf)
    B, n_q, n_kv, d, S, W = 3, 8, 2, 128, 5, 40
    mask = [1, 0]
    plan = {0: None, 1: [200, 200, 137], 2: [333]}
    lens = [5, 537, 333]
    N = max(lens) + 1
    K, V, Q = _rows(B, n_kv, N, d, 990, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], kv_format=kvf)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    c.append_row(0, 0, Kd[0:1, :, :5].contiguous(), Vd[0:1, :, :5].contiguous())
    outs = {}
    for b in (1, 2):
        p, parts = 0, []
        for C in plan[b]:
            parts.append(c.prefill_chunk_row(0, b, Qd[b:b + 1, :, p:p + C].contiguous(),
                                             Kd[b:b + 1, :, p:p + C].contiguous(), Vd[b:b + 1, :, p:p + C].contiguous()))
            p += C
        outs[b] = torch.cat(parts, dim=2)
    torch.cuda.synchronize()
    assert [c.row_len(0, b) for b in range(B)] == lens
    for b in (1, 2):
        Qs, Ks, Vs = stored(Q[b, :, :lens[b]], "bf16"), stored(K[b, :, :lens[b]], "bf16"), stored(V[b, :, :lens[b]], "bf16")
        if kvf == "fp8":
            ref = OQ.prefill_chunked_fp8(Qs, Ks.astype(np.float32), Vs.astype(np.float32), mask, S, W, d ** -0.5, plan[b])
        else:
            ref = OA.prefill_full(Qs, Ks, Vs, mask, S, W, d ** -0.5)
        check_close(outs[b][0], ref, "bf16", f"prefill row {b}")
    # one more token per row, then a decode of all rows at their own positions
    kn = torch.stack([Kd[b, :, n:n + 1] for b, n in enumerate(lens)]).contiguous()
    vn = torch.stack([Vd[b, :, n:n + 1] for b, n in enumerate(lens)]).contiguous()
    c.append(0, kn, vn)
    q = torch.stack([Qd[b, :, n] for b, n in enumerate(lens)]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        ref = _ref_decode(Q, K, V, b, n, mask, S, W, d, "bf16", kvf == "fp8")
        check_close(out[b], ref, "bf16", f"decode after ragged prefill row {b}")


@pytest.mark.gpu
def test_ragged_errors():
    need_gpu()
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("ragged errors")
    c = DuoCache(1, 2, 4, 2, 64, 8, 1, 2, "bf16", [[1, 0]])
    one = torch.zeros(1, 2, 3, 64, dtype=torch.bfloat16, device="cuda")
    c.append_row(0, 1, one, one)
    q = torch.zeros(2, 4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.decode(0, q)                      # row 0 holds nothing
    assert e.value.code == H.DUO_EEMPTY
    with pytest.raises(H.DuoError) as e:
        c.seq_len(0)                        # rows differ
    assert e.value.code == H.DUO_EINVAL
    qq = torch.zeros(2, 4, 2, 64, dtype=torch.bfloat16, device="cuda")
    kk = torch.zeros(2, 2, 2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.prefill_chunk(0, qq, kk, kk)      # rows differ: one at a time
    assert e.value.code == H.DUO_EINVAL
    big = torch.zeros(1, 2, 6, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.append_row(0, 1, big, big)        # 3 + 6 > T_cap 8
    assert e.value.code == H.DUO_ECAPACITY and c.row_len(0, 1) == 3
    with pytest.raises(H.DuoError) as e:
        c.append_row(0, 2, one, one)        # no row 2
    assert e.value.code == H.DUO_EINVAL


@pytest.mark.gpu
def test_ragged_gqa70b_128k_layer():
    """70B GQA layer shape with four rows of 128,000, 20,000, 1,500 and 1
    tokens decoded in one launch (fused step), each row against the oracle."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["gqa70b_decode_128k"]
    lens = [128000, 20000, 1500, 1]
    layer = 2
    say(w.name, "ragged rows", lens)
    mask = WL.retrieval_mask(w, layer)
    B = len(lens)
    c = DuoCache(1, B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask])
    rows = []
    for b, n in enumerate(lens):
        wb = w.with_(index=w.index + 100 * (b + 1))  # a different seeded sequence per row
        K = WL.stacked_rows_f32(wb, layer, WL.TENSOR_K, w.n_kv, 0, n)
        V = WL.stacked_rows_f32(wb, layer, WL.TENSOR_V, w.n_kv, 0, n)
        Q = WL.stacked_rows_f32(wb, layer, WL.TENSOR_Q, w.n_q, n - 1, n)[:, :, 0]
        rows.append((K, V, Q))
        if n > 1:
            c.append_row(0, b, WL.to_torch(K[:, :, : n - 1], w.dtype).cuda(), WL.to_torch(V[:, :, : n - 1], w.dtype).cuda())
    kn = torch.cat([WL.to_torch(K[:, :, -1:], w.dtype) for K, _, _ in rows]).cuda().contiguous()
    vn = torch.cat([WL.to_torch(V[:, :, -1:], w.dtype) for _, V, _ in rows]).cuda().contiguous()
    q = torch.cat([WL.to_torch(Q, w.dtype) for _, _, Q in rows]).cuda().contiguous()
    out = c.decode_append(0, kn, vn, q, scale=w.scale)
    torch.cuda.synchronize()
    for b, (K, V, Q) in enumerate(rows):
        ref = OA.decode_step(stored(Q, w.dtype)[0], stored(K, w.dtype)[0], stored(V, w.dtype)[0], mask, w.S, w.W, w.scale)
        check_close(out[b], ref, w.dtype, f"ragged 70B row {b} (len {lens[b]})")


@pytest.mark.gpu
@pytest.mark.parametrize("page_rows,theta", [(0, 0.0), (256, 0.0), (256, 10000.0)])
def test_ragged_max_rows(page_rows, theta):
    """64 batch rows (the most a cache takes) of 1 to 2,016 tokens, grown in
    two rounds of per-row appends and decoded together: the decode's row
    table is full, and the longest rows split over several work items."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    from oracle import rope as RP
    say("ragged 64 rows", page_rows, theta)
    B, n_kv, g, d, S, W = 64, 2, 4, 128, 4, 32
    n_q = n_kv * g
    mask = [1, 0]
    lens = [1 + (37 * b * b + 11 * b) % 2016 for b in range(B)]
    N = max(lens)
    K, V, Q = _rows(B, n_kv, N, d, 2300, n_q)
    kw = dict(page_rows=page_rows, n_pages=sum(-(-n // page_rows) for n in lens)) if page_rows else {}
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], rope_theta=theta, **kw)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    for b, n in enumerate(lens):
        h = n // 2
        if h:
            c.append_row(0, b, Kd[b:b + 1, :, :h].contiguous(), Vd[b:b + 1, :, :h].contiguous())
        c.append_row(0, b, Kd[b:b + 1, :, h:n].contiguous(), Vd[b:b + 1, :, h:n].contiguous())
    if page_rows:
        assert c.free_pages(0) == 0
    q = torch.stack([Qd[b, :, n - 1] for b, n in enumerate(lens)]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        qs, Ks, Vs = stored(Q[b, :, n - 1], "bf16"), stored(K[b, :, :n], "bf16"), stored(V[b, :, :n], "bf16")
        if theta:
            ref = RP.decode_step_rope(qs, Ks, Vs, mask, S, W, d ** -0.5, theta, "bf16")
        else:
            ref = OA.decode_step(qs, Ks, Vs, mask, S, W, d ** -0.5)
        check_close(out[b], ref, "bf16", f"64 rows: row {b} (len {n})")
