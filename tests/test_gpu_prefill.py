"""Chunked-prefill parity: libduo's duo_prefill_chunk against the fp64 oracle
(definition route on the whole sequence), plus the cache it leaves behind."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import cache as OC
from tests.gpu_util import check_close, need_gpu, oracle_decode, say, stored


def _run_prefill(B, n_q, n_kv, d, dtype, N, S, W, mask, chunks, seed, sink_scale=1.0):
    from head_wise_kv_amd import DuoCache
    Q = WL.normal_f32((B, n_q, N, d), seed)
    K = WL.normal_f32((B, n_kv, N, d), seed + 1)
    V = WL.normal_f32((B, n_kv, N, d), seed + 2)
    K[:, :, :S] *= np.float32(sink_scale)
    Qd, Kd, Vd = (WL.to_torch(x, dtype).cuda() for x in (Q, K, V))
    c = DuoCache(1, B, n_q, n_kv, d, N + 1, S, W, dtype, [mask])
    outs = []
    p = 0
    for C in chunks:
        outs.append(c.prefill_chunk(0, Qd[:, :, p:p + C].contiguous(), Kd[:, :, p:p + C].contiguous(),
                                    Vd[:, :, p:p + C].contiguous()))
        p += C
    torch.cuda.synchronize()
    assert c.seq_len(0) == N
    out = torch.cat(outs, dim=2)
    return c, (Q, K, V), out


def _oracle_prefill(Q, K, V, mask, S, W, dtype, rows=None):
    q64, k64, v64 = stored(Q, dtype), stored(K, dtype), stored(V, dtype)
    d = Q.shape[-1]
    return np.stack([OA.prefill_full(q64[b], k64[b], v64[b], mask, S, W, 1.0 / np.sqrt(d), rows=rows)
                     for b in range(Q.shape[0])])


CASES = []
for dtype in ("bf16", "f32"):
    for d in (64, 128):
        # bf16 takes every group size the MFMA path packs differently: one head
        # per work item (g = 1, 3), two (g = 2, 6: three head groups), four
        # (g = 4), two head groups of four (g = 8)
        for g in ((1, 2, 3, 4, 6, 8) if dtype == "bf16" else (1, 3, 4)):
            CASES.append((dtype, d, g))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g", CASES)
@pytest.mark.parametrize("chunks", [[300], [1] * 5 + [64, 128, 103], [7] * 42 + [6], [129, 171]])
def test_prefill_grid(dtype, d, g, chunks):
    """Chunk sizes 1..300 (several query tiles, ragged tails, single-token chunks)
    with S=5, W=40: sinks inside the first chunk, windows crossing chunk edges."""
    need_gpu()
    N = sum(chunks)
    n_kv = 4
    mask = [1, 0, 0, 1]
    say("prefill grid", dtype, d, g, chunks[:3], N)
    c, (Q, K, V), out = _run_prefill(2, n_kv * g, n_kv, d, dtype, N, 5, 40, mask, chunks, seed=N + d + g, sink_scale=4.0)
    ref = _oracle_prefill(Q, K, V, mask, 5, 40, dtype)
    check_close(out, ref, dtype, f"prefill {dtype} d{d} g{g} {chunks[:3]}")
    # The cache after prefill holds what the oracle's cache simulation holds, bit for bit.
    st = WL.to_torch(K, dtype)
    for h in range(n_kv):
        Kc, _, pos = c.read_head(0, h)
        table = OC.slot_table(N, bool(mask[h]), 5, 40)
        for slot, position in table.items():
            assert torch.equal(Kc[:, slot], st[:, h, position])
            if pos is not None:
                assert (pos[:, slot] == position).all()


@pytest.mark.gpu
@pytest.mark.parametrize("mask", [[1, 1], [0, 0], [1, 0]])
def test_prefill_lambda_mask_long(mask):
    """S=64, W=1024, chunks of 4096 with a ragged last chunk: the sink+local band
    against ring slots that hold the previous chunk's tail."""
    need_gpu()
    N = 9000
    chunks = [4096, 4096, N - 8192]
    say("lambda long", mask)
    c, (Q, K, V), out = _run_prefill(1, 8, 2, 128, "bf16", N, 64, 1024, mask, chunks, seed=77)
    rows = np.unique(np.concatenate([np.arange(0, 80), np.arange(1000, 1100), np.arange(4090, 4200),
                                     np.arange(5100, 5140), np.arange(8180, 8300), np.arange(N - 60, N)]))
    ref = _oracle_prefill(Q, K, V, mask, 64, 1024, "bf16", rows=rows)
    check_close(out[:, :, rows], ref, "bf16", f"lambda {mask}")


@pytest.mark.gpu
def test_prefill_then_decode():
    """Prefill a prompt in chunks, then append one token and decode: the decode
    sees exactly the cache the prefill left behind."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    B, n_q, n_kv, d, S, W, N = 2, 16, 4, 128, 8, 100, 1500
    mask = [0, 1, 0, 0]
    say("prefill then decode")
    Q = WL.normal_f32((B, n_q, N + 1, d), 5)
    K = WL.normal_f32((B, n_kv, N + 1, d), 6)
    V = WL.normal_f32((B, n_kv, N + 1, d), 7)
    Qd, Kd, Vd = (WL.to_torch(x, "bf16").cuda() for x in (Q, K, V))
    c = DuoCache(1, B, n_q, n_kv, d, N + 1, S, W, "bf16", [mask])
    p = 0
    for C in (512, 512, 476):
        c.prefill_chunk(0, Qd[:, :, p:p + C].contiguous(), Kd[:, :, p:p + C].contiguous(), Vd[:, :, p:p + C].contiguous())
        p += C
    c.append(0, Kd[:, :, N:].contiguous(), Vd[:, :, N:].contiguous())
    out = c.decode(0, Qd[:, :, N].contiguous())
    ref = oracle_decode(stored(Q[:, :, N], "bf16"), stored(K, "bf16"), stored(V, "bf16"), mask, S, W, d ** -0.5)
    check_close(out, ref, "bf16", "prefill->decode")


@pytest.mark.gpu
@pytest.mark.timeout(400)
def test_llama3_8b_prefill_64k():
    """Chunked prefill workload at full size: n_q=32, n_kv=8, d=128, bf16,
    65,536 tokens in 16 chunks of 4,096, 2/8 retrieval, S=64, W=1024; every
    chunk's output checked on sampled rows of every head, and every row of
    chunks 0 and 15 for one retrieval and one streaming query head."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["llama3_8b_prefill_64k"]
    say(w.name)
    mask = WL.retrieval_mask(w, 0)
    N, C = w.T, w.chunk
    Q = WL.stacked_rows_f32(w, 0, WL.TENSOR_Q, w.n_q, 0, N)
    K = WL.stacked_rows_f32(w, 0, WL.TENSOR_K, w.n_kv, 0, N)
    V = WL.stacked_rows_f32(w, 0, WL.TENSOR_V, w.n_kv, 0, N)
    Qd, Kd, Vd = (WL.to_torch(x, w.dtype).cuda() for x in (Q, K, V))
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, N, w.S, w.W, w.dtype, [mask])
    rng = np.random.default_rng(3)
    q64, k64, v64 = stored(Q[0], w.dtype), stored(K[0], w.dtype), stored(V[0], w.dtype)
    for ci, p in enumerate(range(0, N, C)):
        out = c.prefill_chunk(0, Qd[:, :, p:p + C].contiguous(), Kd[:, :, p:p + C].contiguous(),
                              Vd[:, :, p:p + C].contiguous(), scale=w.scale)
        rows = np.unique(np.concatenate([[0, 1, 127, 128, 1022, 1023, 1024, C - 1], rng.integers(0, C, 8)]))
        got = out[0][:, rows].float().cpu().double().numpy()
        ref = OA.prefill_full(q64, k64, v64, mask, w.S, w.W, w.scale, rows=p + rows)
        check_close(torch.from_numpy(got), ref, w.dtype, f"{w.name} chunk {ci}")
        if ci in (0, N // C - 1):
            # every row of the first and the last chunk, for the first query
            # head of a retrieval KV head and of a streaming KV head
            for kvh in (int(np.argmax(mask == 1)), int(np.argmax(mask == 0))):
                h = kvh * w.g
                ref_h = OA.prefill_full(q64[h:h + 1], k64[kvh:kvh + 1], v64[kvh:kvh + 1], [mask[kvh]], w.S, w.W,
                                        w.scale, rows=p + np.arange(C))
                kind = "retrieval" if mask[kvh] else "streaming"
                check_close(out[0][h:h + 1], ref_h, w.dtype, f"{w.name} chunk {ci} all rows, {kind} head {h}")
    assert c.seq_len(0) == N


@pytest.mark.gpu
@pytest.mark.parametrize("d,chunks,page_rows", [(128, [36000, 34000], 0), (128, [36000, 34000], 256),
                                                (64, [20000, 20000], 0)])
def test_prefill_past_tile_table(d, chunks, page_rows):
    """Work items with more key tiles than the workgroup's descriptor table
    holds (1,024 tiles of 64 keys at d = 128, 512 at d = 64): the entries of
    passed tiles are refilled during the item; rows of the second chunk whose
    keys reach past the table (cache and chunk tiles both), checked against
    the oracle, contiguous and paged."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    N = sum(chunks)
    B, n_q, n_kv, S, W = 1, 4, 2, 16, 256
    mask = [1, 0]
    say("prefill past tile table", d, chunks, page_rows)
    Q = WL.normal_f32((B, n_q, N, d), 2100 + d)
    K = WL.normal_f32((B, n_kv, N, d), 2101 + d)
    V = WL.normal_f32((B, n_kv, N, d), 2102 + d)
    Qd, Kd, Vd = (WL.to_torch(x, "bf16").cuda() for x in (Q, K, V))
    kw = dict(page_rows=page_rows, n_pages=-(-N // page_rows)) if page_rows else {}
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], **kw)
    p = 0
    for C in chunks:
        out = c.prefill_chunk(0, Qd[:, :, p:p + C].contiguous(), Kd[:, :, p:p + C].contiguous(),
                              Vd[:, :, p:p + C].contiguous())
        p += C
    torch.cuda.synchronize()
    C, P0 = chunks[-1], N - chunks[-1]
    rng = np.random.default_rng(d)
    rows = np.unique(np.concatenate([np.arange(C - 64, C), [0, 1, 63, 64], rng.integers(0, C, 12)]))
    got = out[0][:, rows].float().cpu().double().numpy()
    ref = OA.prefill_full(stored(Q[0], "bf16"), stored(K[0], "bf16"), stored(V[0], "bf16"), mask, S, W,
                          d ** -0.5, rows=P0 + rows)
    check_close(torch.from_numpy(got), ref, "bf16", f"prefill past tile table d{d} pages {page_rows}")
