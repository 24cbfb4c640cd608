"""Caches of FP8 K/V rows (kv_format "fp8"): the stored codes and scales
bit-exact against the oracle's quantizer, and decode / fused decode-append /
chunked prefill against the fp64 oracle over the stored rows (oracle.quant)."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import cache as OC
from oracle import quant as OQ
from tests.gpu_util import check_close, need_gpu, say, stored


def _inputs(B, n_kv, N, d, seed, n_q=None, spread=1.0):
    K = WL.normal_f32((B, n_kv, N, d), seed)
    V = WL.normal_f32((B, n_kv, N, d), seed + 1)
    # rows of different magnitudes (a factor e^(2 spread) end to end), and a row of zeros
    K *= np.exp(np.linspace(-spread, spread, N, dtype=np.float32))[None, None, :, None]
    V[:, :, N // 3] = 0.0
    Q = WL.normal_f32((B, n_q, N, d), seed + 2) if n_q else None
    return K, V, Q


def _check_cache(c, K, V, mask, S, W, T):
    """Codes, scales and positions of every head against the oracle's
    quantizer applied to the stored (bf16) inputs, at the slots the cache
    simulation assigns."""
    Ks, Vs = stored(K, "bf16").astype(np.float32), stored(V, "bf16").astype(np.float32)
    for h in range(K.shape[1]):
        k_codes, v_codes, pos = c.read_head(0, h)
        k_sc, v_sc = c.head_scales(0, h)
        table = OC.slot_table(T, bool(mask[h]), S, W)
        for slot, p in table.items():
            ck, sk = OQ.quantize_rows(Ks[:, h, p])
            cv, sv = OQ.quantize_rows(Vs[:, h, p])
            assert np.array_equal(k_codes[:, slot].numpy(), ck), (h, slot, p)
            assert np.array_equal(v_codes[:, slot].numpy(), cv), (h, slot, p)
            assert np.array_equal(k_sc[:, slot].numpy(), sk) and np.array_equal(v_sc[:, slot].numpy(), sv), (h, slot)
            if pos is not None:
                assert (pos[:, slot] == p).all()


@pytest.mark.gpu
def test_fp8_append_bit_exact():
    """Appends of 1..37 tokens across the sinks, the ring's first fill and its
    wrap: codes (ties, subnormals, the 448 edge, a zero row) and scales equal
    the oracle's bit for bit."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("fp8 append")
    B, n_kv, d, S, W = 2, 4, 128, 3, 20
    mask = [1, 0, 1, 0]
    N = 120
    K, V, _ = _inputs(B, n_kv, N, d, 501, spread=6.0)
    c = DuoCache(1, B, 8, n_kv, d, N, S, W, "bf16", [mask], kv_format="fp8")
    Kd, Vd = WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda()
    p = 0
    for n in (1, 2, 37, 5, 1, 30, 44):
        c.append(0, Kd[:, :, p:p + n].contiguous(), Vd[:, :, p:p + n].contiguous())
        p += n
        torch.cuda.synchronize()
        _check_cache(c, K[:, :, :p], V[:, :, :p], mask, S, W, p)
    assert p == N


def _decode_case(B, n_q, n_kv, d, T, S, W, mask, seed):
    from head_wise_kv_amd import DuoCache
    K, V, Q = _inputs(B, n_kv, T, d, seed, n_q=n_q)
    c = DuoCache(1, B, n_q, n_kv, d, T, S, W, "bf16", [mask], kv_format="fp8")
    c.append(0, WL.to_torch(K, "bf16").cuda(), WL.to_torch(V, "bf16").cuda())
    q = Q[:, :, T - 1]
    out = c.decode(0, WL.to_torch(q, "bf16").cuda().contiguous())
    torch.cuda.synchronize()
    Ks, Vs, qs = stored(K, "bf16"), stored(V, "bf16"), stored(q, "bf16")
    ref = np.stack([OQ.decode_step_fp8(qs[b], Ks[b].astype(np.float32), Vs[b].astype(np.float32), mask, S, W,
                                       d ** -0.5) for b in range(B)])
    return out, ref


@pytest.mark.gpu
@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("T", [1, 7, 300, 2049])
def test_fp8_decode_grid(g, T):
    """Every group size; contexts from one token to several 256-row rounds with
    a ragged tail; retrieval and streaming heads."""
    need_gpu()
    say("fp8 decode", g, T)
    out, ref = _decode_case(2, 3 * g, 3, 128, T, 4, 64, [1, 0, 1], seed=600 + g + T)
    check_close(out, ref, "bf16", f"fp8 decode g{g} T{T}")


@pytest.mark.gpu
@pytest.mark.parametrize("T0", [0, 3, 19, 21])
def test_fp8_decode_append_steps(T0):
    """Fused steps on an FP8 cache: each output against the oracle, and the
    cache afterwards bit-exact (the new token is quantized as the append
    quantizes it)."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("fp8 decode_append", T0)
    B, n_q, n_kv, d, S, W = 2, 8, 4, 128, 4, 16
    mask = [1, 0, 1, 0]
    steps = 20
    T = T0 + steps
    K, V, Q = _inputs(B, n_kv, T, d, 700 + T0, n_q=n_q)
    c = DuoCache(1, B, n_q, n_kv, d, T, S, W, "bf16", [mask], kv_format="fp8")
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    if T0:
        c.append(0, Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    Ks, Vs, Qs = stored(K, "bf16"), stored(V, "bf16"), stored(Q, "bf16")
    for i in range(steps):
        t = T0 + i
        out = c.decode_append(0, Kd[:, :, t:t + 1].contiguous(), Vd[:, :, t:t + 1].contiguous(), Qd[:, :, t].contiguous())
        if i % 3 == 0 or i == steps - 1:
            torch.cuda.synchronize()
            ref = np.stack([OQ.decode_step_fp8(Qs[b, :, t], Ks[b, :, :t + 1].astype(np.float32),
                                               Vs[b, :, :t + 1].astype(np.float32), mask, S, W, d ** -0.5)
                            for b in range(B)])
            check_close(out, ref, "bf16", f"fp8 fused t={t}")
    torch.cuda.synchronize()
    _check_cache(c, K, V, mask, S, W, T)


@pytest.mark.gpu
@pytest.mark.parametrize("chunks", [[300], [64, 1, 129, 200], [17] * 12])
def test_fp8_prefill_chunked(chunks):
    """Chunked prefill on an FP8 cache: held rows read as stored, the chunk's
    own rows as given; then the cache (bit-exact) and one decode step."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    N = sum(chunks)
    say("fp8 prefill", chunks[:3], N)
    B, n_q, n_kv, d, S, W = 1, 8, 2, 128, 5, 40
    mask = [1, 0]
    K, V, Q = _inputs(B, n_kv, N + 1, d, 800 + N, n_q=n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N + 1, S, W, "bf16", [mask], kv_format="fp8")
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    outs, p = [], 0
    for C in chunks:
        outs.append(c.prefill_chunk(0, Qd[:, :, p:p + C].contiguous(), Kd[:, :, p:p + C].contiguous(),
                                    Vd[:, :, p:p + C].contiguous()))
        p += C
    out = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    Ks, Vs, Qs = stored(K, "bf16"), stored(V, "bf16"), stored(Q, "bf16")
    ref = OQ.prefill_chunked_fp8(Qs[0, :, :N], Ks[0, :, :N].astype(np.float32), Vs[0, :, :N].astype(np.float32),
                                 mask, S, W, d ** -0.5, chunks)
    check_close(out[0], ref, "bf16", f"fp8 prefill {chunks[:3]}")
    _check_cache(c, K[:, :, :N], V[:, :, :N], mask, S, W, N)
    c.append(0, Kd[:, :, N:].contiguous(), Vd[:, :, N:].contiguous())
    dec = c.decode(0, Qd[:, :, N].contiguous())
    torch.cuda.synchronize()
    refd = OQ.decode_step_fp8(Qs[0, :, N], Ks[0].astype(np.float32), Vs[0].astype(np.float32), mask, S, W, d ** -0.5)
    check_close(dec[0], refd, "bf16", "fp8 decode after prefill")


@pytest.mark.gpu
def test_fp8_gqa70b_decode_append_128k_layer():
    """70B GQA shape at full size on an FP8 cache: positions 0..T-2 appended,
    then the fused step at T-1, against the oracle over the stored rows."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["gqa70b_decode_128k"]
    layer = 5
    say(w.name, "fp8 fused layer", layer)
    mask = WL.retrieval_mask(w, layer)
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask], kv_format="fp8")
    K = WL.stacked_rows_f32(w, layer, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, layer, WL.TENSOR_V, w.n_kv, 0, w.T)
    Q = WL.stacked_rows_f32(w, layer, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0]
    Kt, Vt = WL.to_torch(K, w.dtype).cuda(), WL.to_torch(V, w.dtype).cuda()
    c.append(0, Kt[:, :, : w.T - 1].contiguous(), Vt[:, :, : w.T - 1].contiguous())
    out = c.decode_append(0, Kt[:, :, w.T - 1:].contiguous(), Vt[:, :, w.T - 1:].contiguous(),
                          WL.to_torch(Q, w.dtype).cuda(), scale=w.scale)
    torch.cuda.synchronize()
    Ks, Vs = stored(K, w.dtype).astype(np.float32), stored(V, w.dtype).astype(np.float32)
    ref = OQ.decode_step_fp8(stored(Q, w.dtype)[0], Ks[0], Vs[0], mask, w.S, w.W, w.scale)
    check_close(out[0], ref, w.dtype, f"{w.name} fp8 fused layer {layer}")


@pytest.mark.gpu
def test_fp8_errors():
    need_gpu()
    import ctypes
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("fp8 errors")
    with pytest.raises(H.DuoError) as e:
        DuoCache(1, 1, 4, 2, 128, 10, 1, 4, "f32", [[1, 0]], kv_format="fp8")
    assert e.value.code == H.DUO_EUNSUPPORTED
    c = DuoCache(1, 1, 4, 2, 128, 10, 1, 4, "bf16", [[1, 0]], kv_format="fp8")
    x = torch.zeros(1, 4, 3, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 2, 3, 128, dtype=torch.bfloat16, device="cuda")
    rc = H.lib.duo_prefill_chunk(c._h, 0, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(kv.data_ptr()),
                                 ctypes.c_void_p(kv.data_ptr()), 3, ctypes.c_void_p(x.data_ptr()), 0.1, None, 0, None)
    assert rc == H.DUO_EWORKSPACE and c.seq_len(0) == 0
