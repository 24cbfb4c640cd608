"""Bit-exact cache placement on the GPU: after any sequence of appends, every
held slot holds exactly the input bytes of the position the oracle's cache
simulation puts there, and a streaming head's position array says so."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import cache as OC
from tests.gpu_util import need_gpu, say

PATTERNS = [
    (3, 5, [1] * 20),
    (3, 5, [7, 1, 13, 2]),
    (3, 5, [40]),
    (2, 4, [1, 30, 1, 1]),
    (0, 3, [1, 1, 1, 1, 1]),      # the printed ring example's shape (window 3, five appends)
    (0, 7, [20, 3]),
    (6, 1, [3, 3, 3, 2]),
    (64, 1024, [5000, 1, 1]),
    (4, 16, [3]),                 # fewer tokens than sinks
]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,W,pattern", PATTERNS)
def test_slot_placement_bit_exact(S, W, pattern, dtype):
    need_gpu()
    B, n_q, n_kv, d = 2, 8, 4, 64
    mask = [1, 0, 0, 1]
    T = sum(pattern)
    say("placement", dtype, S, W, pattern)
    K = WL.normal_f32((B, n_kv, T, d), seed=T * 7 + S)
    V = WL.normal_f32((B, n_kv, T, d), seed=T * 7 + S + 1)
    Kt, Vt = WL.to_torch(K, dtype), WL.to_torch(V, dtype)
    from head_wise_kv_amd import DuoCache
    c = DuoCache(1, B, n_q, n_kv, d, T, S, W, dtype, [mask])
    Kd, Vd = Kt.cuda(), Vt.cuda()
    p = 0
    for n in pattern:
        c.append(0, Kd[:, :, p:p + n].contiguous(), Vd[:, :, p:p + n].contiguous())
        p += n
    torch.cuda.synchronize()
    assert c.seq_len(0) == T
    for h in range(n_kv):
        ret = bool(mask[h])
        Kc, Vc, pos = c.read_head(0, h)
        table = OC.slot_table(T, ret, S, W)
        assert (pos is None) == ret
        for slot, position in table.items():
            assert torch.equal(Kc[:, slot].view(torch.int16 if dtype == "bf16" else torch.int32),
                               Kt[:, h, position].view(torch.int16 if dtype == "bf16" else torch.int32)), (h, slot)
            assert torch.equal(Vc[:, slot].view(torch.int16 if dtype == "bf16" else torch.int32),
                               Vt[:, h, position].view(torch.int16 if dtype == "bf16" else torch.int32)), (h, slot)
            if not ret:
                assert (pos[:, slot] == position).all(), (h, slot, pos[:, slot], position)
        if not ret:
            held = len(table)
            assert held == min(T, S + W)
