"""Random operation sequences on a paged cache: per-row appends, forks of one
row into an empty one, resets, and fused decode-append steps over all rows,
interleaved at random.  The host keeps each row's logical token sequence (ids
into one pool of seeded K/V rows); every fused step's output is checked
against the fp64 oracle over each row's sequence, and the page accounting
against the oracle's page model after every operation."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import paging as OP
from oracle import rope as RP
from tests.gpu_util import check_close, need_gpu, say, stored

P = 256


def _pages_ok(c, model, B):
    tables = [c.row_pages(0, b) for b in range(B)]
    for b in range(B):
        assert len(tables[b]) == model.pages_needed(model.count[b]), (b, tables[b], model.count[b])
    assert len({p for t in tables for p in t}) == model.pages_in_use()
    assert c.free_pages(0) == model.free_pages()
    for b1 in range(B):
        for b2 in range(b1 + 1, B):
            assert len(set(tables[b1]) & set(tables[b2])) == model.shared_pages(b1, b2)


@pytest.mark.gpu
@pytest.mark.parametrize("seed,theta,pr", [(0, 0.0, P), (1, 0.0, P), (2, 10000.0, P), (3, 0.0, P), (4, 500000.0, P),
                                           (5, 0.0, 128), (6, 10000.0, 128)])
def test_paged_random_ops(seed, theta, pr):
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("paged random ops", seed, theta, pr)
    rng = np.random.default_rng(100 + seed)
    B, n_kv, g, d, S, W = 4, 2, 4, 128, 4, 64
    n_q = n_kv * g
    mask = [1, 0]
    T_cap = 1400
    n_pages = 12 * (P // pr)  # tight: appends can be refused, and that must change nothing
    pool = 6000   # seeded K/V/Q rows that appends draw from
    Kp = WL.normal_f32((n_kv, pool, d), 4000 + seed)
    Vp = WL.normal_f32((n_kv, pool, d), 4001 + seed)
    Qp = WL.normal_f32((n_q, pool, d), 4002 + seed)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (Kp, Vp, Qp))
    c = DuoCache(1, B, n_q, n_kv, d, T_cap, S, W, "bf16", [mask], page_rows=pr, n_pages=n_pages, rope_theta=theta)
    model = OP.PagedRows(pr, n_pages, B)
    seqs = [[] for _ in range(B)]  # token ids per row
    next_id = 0
    n_checked = 0
    for step in range(60):
        op = rng.choice(["append", "append", "fork", "reset", "step", "step"])
        if op == "append":
            b = int(rng.integers(0, B))
            n = int(rng.integers(1, 500))
            ids = list(range(next_id, next_id + n))
            if next_id + n > pool or len(seqs[b]) + n > T_cap:
                continue
            k = Kd[:, next_id:next_id + n].unsqueeze(0).contiguous()
            v = Vd[:, next_id:next_id + n].unsqueeze(0).contiguous()
            try:
                model.append(b, n)
            except MemoryError:
                import head_wise_kv_amd as H
                with pytest.raises(H.DuoError) as e:
                    c.append_row(0, b, k, v)
                assert e.value.code == H.DUO_ECAPACITY
                assert c.row_len(0, b) == len(seqs[b])
                continue
            c.append_row(0, b, k, v)
            seqs[b] += ids
            next_id += n
        elif op == "fork":
            src = int(rng.integers(0, B))
            empty = [b for b in range(B) if b != src and not seqs[b]]
            if not empty:  # free a row to fork into
                dst = int(rng.choice([b for b in range(B) if b != src]))
                c.reset_row(0, dst)
                model.reset(dst)
                seqs[dst] = []
            else:
                dst = int(rng.choice(empty))
            try:
                model.fork(src, dst)
            except MemoryError:
                continue  # the library would refuse it too; the pool is checked below
            c.fork_row(0, src, dst)
            seqs[dst] = list(seqs[src])
        elif op == "reset":
            b = int(rng.integers(0, B))
            c.reset_row(0, b)
            model.reset(b)
            seqs[b] = []
        else:  # one fused step on every row
            if next_id + B > pool or any(len(s) + 1 > T_cap for s in seqs):
                continue
            try:
                model.append_rows([(b, 1) for b in range(B)])
            except MemoryError:
                continue
            ids = list(range(next_id, next_id + B))
            kn = Kd[:, next_id:next_id + B].transpose(0, 1).unsqueeze(2).contiguous()  # [B][n_kv][1][d]
            vn = Vd[:, next_id:next_id + B].transpose(0, 1).unsqueeze(2).contiguous()
            qn = Qd[:, next_id:next_id + B].transpose(0, 1).contiguous()               # [B][n_q][d]
            out = c.decode_append(0, kn, vn, qn)
            torch.cuda.synchronize()
            for b in range(B):
                seqs[b].append(ids[b])
                sel = np.asarray(seqs[b])
                q = stored(Qp[:, ids[b]], "bf16")
                Ks, Vs = stored(Kp[:, sel], "bf16"), stored(Vp[:, sel], "bf16")
                if theta:
                    ref = RP.decode_step_rope(q, Ks, Vs, mask, S, W, d ** -0.5, theta, "bf16")
                else:
                    ref = OA.decode_step(q, Ks, Vs, mask, S, W, d ** -0.5)
                check_close(out[b], ref, "bf16", f"seed {seed} step {step} row {b} (len {len(sel)})")
                n_checked += 1
            next_id += B
        torch.cuda.synchronize()
        assert [c.row_len(0, b) for b in range(B)] == [len(s) for s in seqs], step
        _pages_ok(c, model, B)
    assert n_checked > 0
