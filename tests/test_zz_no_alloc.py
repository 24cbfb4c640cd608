"""duo_decode_append_noalloc, through the C ABI, against duo_decode_append
with a caller workspace: two calls in a row on two caches (the second call's
cache smaller, so it writes fewer partial records into the library's scratch
than the first left behind), outputs and stored tokens bit for bit, outputs
also against the fp64 oracle; and a call that needs more scratch than the
library holds is refused without a state change."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as WL
from tests.gpu_util import check_close, need_gpu, oracle_decode, say, stored

CASES = [
    # B, n_q, n_kv, d, T (after the step), S, W, mask, seed
    (2, 16, 4, 128, 6000, 16, 256, [1, 0, 1, 0], 11),
    (1, 4, 2, 64, 300, 4, 32, [0, 1], 12),
]


def _noalloc(c, layer, k, v, q, out, scale):
    import head_wise_kv_amd as H
    return H.lib.duo_decode_append_noalloc(c._h, layer, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                           ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                           ctypes.c_float(scale), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    need_gpu()
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    for B, n_q, n_kv, d, T, S, W, mask, seed in CASES:
        say(f"noalloc B{B} n_q{n_q} n_kv{n_kv} d{d} T{T} S{S} W{W}")
        K = WL.normal_f32((B, n_kv, T, d), seed)
        V = WL.normal_f32((B, n_kv, T, d), seed + 100)
        Q = WL.normal_f32((B, n_q, d), seed + 200)
        Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
        caches = [DuoCache(1, B, n_q, n_kv, d, T, S, W, "bf16", [mask]) for _ in range(2)]
        for c in caches:
            c.append(0, Kd[:, :, : T - 1].contiguous(), Vd[:, :, : T - 1].contiguous())
        kn, vn = Kd[:, :, T - 1:].contiguous(), Vd[:, :, T - 1:].contiguous()
        scale = d ** -0.5
        ref_out = caches[0].decode_append(0, kn, vn, Qd, scale=scale)
        out = torch.empty_like(Qd)
        rc = _noalloc(caches[1], 0, kn, vn, Qd, out, scale)
        assert rc == H.DUO_OK, H.lib.duo_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert caches[1].seq_len(0) == T
        for h in range(n_kv):
            a, b = caches[0].read_head(0, h), caches[1].read_head(0, h)
            assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), h
            assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16)), h
            if a[2] is not None:
                assert torch.equal(a[2], b[2]), h
        ref = oracle_decode(stored(Q, "bf16"), stored(K, "bf16"), stored(V, "bf16"), mask, S, W, scale)
        check_close(out, ref, "bf16", f"noalloc B{B} d{d} T{T}")


@pytest.mark.gpu
def test_noalloc_refuses_more_than_its_scratch():
    need_gpu()
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("noalloc refusal")
    # 64 rows x 32 KV heads = 2,048 work items of 8 x 130 floats: more than 8 MiB
    B, n_q, n_kv, d, T = 64, 256, 32, 128, 4
    c = DuoCache(1, B, n_q, n_kv, d, T, 1, 2, "bf16", [[1] * 16 + [0] * 16])
    k = torch.ones(B, n_kv, 1, d, dtype=torch.bfloat16, device="cuda")
    c.append(0, k, k)
    q = torch.ones(B, n_q, d, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    rc = _noalloc(c, 0, k, k, q, out, d ** -0.5)
    assert rc == H.DUO_EWORKSPACE, rc
    assert b"scratch" in H.lib.duo_last_error()
    assert c.seq_len(0) == 1
    c.decode_append(0, k, k, q, out=out)  # the workspace call serves it
    torch.cuda.synchronize()
    assert c.seq_len(0) == 2
    assert torch.allclose(out.float(), torch.ones_like(out, dtype=torch.float32))
