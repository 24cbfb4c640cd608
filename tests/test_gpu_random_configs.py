"""Seeded random configurations: the features combined in ways the targeted
tests do not list one by one -- dtype, d_head, group size, sink and window
sizes, retrieval masks, ragged rows grown by appends and per-row prefill
chunks, pages, rotary positions and FP8 or INT4 rows -- each followed by a
decode and two fused decode-append steps, every row checked against the fp64
oracle over its own sequence."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import quant as OQ
from oracle import quant4 as OQ4
from oracle import rope as RP
from tests.gpu_util import check_close, need_gpu, say, stored

N_CASES = 64


def _draw(seed):
    r = np.random.default_rng(seed)
    fp8 = bool(r.random() < 0.3)
    dtype = "bf16" if fp8 else str(r.choice(["bf16", "bf16", "f32"]))
    d = 128 if fp8 else int(r.choice([64, 128]))
    # any group size; above 8 only where the scores use the matrix cores
    g = int(r.choice([1, 2, 3, 4, 5, 6, 7, 8] + ([12, 16] if dtype == "bf16" and d == 128 else [])))
    n_kv = int(r.choice([1, 2, 3, 4]))
    mask = [int(x) for x in r.integers(0, 2, n_kv)]
    B = int(r.integers(1, 5))
    S = int(r.choice([0, 1, 4, 16]))
    W = int(r.choice([1, 8, 64, 200]))
    paged = bool(r.random() < 0.4)
    theta = float(r.choice([0.0, 0.0, 10000.0, 500000.0]))
    lens = [int(x) for x in r.integers(1, 700, B)]
    prefill = [bool(x) for x in r.random(B) < 0.5]  # rows grown by prefill chunks (else appends)
    kvf = ("int4" if r.random() < 0.5 else "fp8") if fp8 else None  # low-bit rows: half of them INT4
    return dict(fp8=fp8, kvf=kvf, dtype=dtype, d=d, g=g, n_kv=n_kv, mask=mask, B=B, S=S, W=W, paged=paged,
                theta=theta, lens=lens, prefill=prefill, seed=seed)


def _ref_decode(cfg, Q, K, V, b, t):
    """Oracle output of row b's query at position t over positions 0..t."""
    dt, d = cfg["dtype"], cfg["d"]
    q, Ks, Vs = stored(Q[b, :, t], dt), stored(K[b, :, :t + 1], dt), stored(V[b, :, :t + 1], dt)
    kvf = cfg["kvf"]
    if cfg["theta"]:
        return RP.decode_step_rope(q, Ks, Vs.astype(np.float32), cfg["mask"], cfg["S"], cfg["W"], d ** -0.5,
                                   cfg["theta"], dt, kv_format=kvf)
    if kvf == "int4":
        return OQ4.decode_step_int4(q, Ks.astype(np.float32), Vs.astype(np.float32), cfg["mask"], cfg["S"],
                                    cfg["W"], d ** -0.5)
    if cfg["fp8"]:
        return OQ.decode_step_fp8(q, Ks.astype(np.float32), Vs.astype(np.float32), cfg["mask"], cfg["S"], cfg["W"],
                                  d ** -0.5)
    return OA.decode_step(q, Ks, Vs, cfg["mask"], cfg["S"], cfg["W"], d ** -0.5)


def _ref_prefill(cfg, Q, K, V, b, n, chunks):
    dt, d = cfg["dtype"], cfg["d"]
    Qs, Ks, Vs = stored(Q[b, :, :n], dt), stored(K[b, :, :n], dt), stored(V[b, :, :n], dt)
    if cfg["theta"]:
        return RP.prefill_chunked_rope(Qs, Ks, Vs, cfg["mask"], cfg["S"], cfg["W"], d ** -0.5, cfg["theta"], dt,
                                       chunks, kv_format=cfg["kvf"])
    if cfg["kvf"] == "int4":
        return OQ4.prefill_chunked_int4(Qs, Ks.astype(np.float32), Vs.astype(np.float32), cfg["mask"], cfg["S"],
                                        cfg["W"], d ** -0.5, chunks)
    if cfg["fp8"]:
        return OQ.prefill_chunked_fp8(Qs, Ks.astype(np.float32), Vs.astype(np.float32), cfg["mask"], cfg["S"],
                                      cfg["W"], d ** -0.5, chunks)
    return OA.prefill_full(Qs, Ks, Vs, cfg["mask"], cfg["S"], cfg["W"], d ** -0.5)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_config(seed):
    need_gpu()
    from head_wise_kv_amd import DuoCache
    cfg = _draw(7000 + seed)
    say("random config", {k: v for k, v in cfg.items() if k not in ("lens", "prefill")}, cfg["lens"])
    dt, d, g, n_kv, B = cfg["dtype"], cfg["d"], cfg["g"], cfg["n_kv"], cfg["B"]
    n_q = n_kv * g
    steps = 2
    N = max(cfg["lens"]) + steps
    K = WL.normal_f32((B, n_kv, N, d), 3 * seed + 1)
    V = WL.normal_f32((B, n_kv, N, d), 3 * seed + 2)
    Q = WL.normal_f32((B, n_q, N, d), 3 * seed + 3)
    kw = dict(kv_format=cfg["kvf"], rope_theta=cfg["theta"])
    if cfg["paged"]:
        # the smallest page the row format allows: one decode round, 32 KB of stored K rows
        row_bytes = {"int4": d // 2, "fp8": d}.get(cfg["kvf"], d * (4 if dt == "f32" else 2))
        pr = max(64, 32768 // row_bytes)
        kw.update(page_rows=pr, n_pages=sum(-(-(n + steps) // pr) for n in cfg["lens"]))
    c = DuoCache(1, B, n_q, n_kv, d, N, cfg["S"], cfg["W"], dt, [cfg["mask"]], **kw)
    Kd, Vd, Qd = (WL.to_torch(x, dt).cuda() for x in (K, V, Q))
    rng = np.random.default_rng(seed)
    for b, n in enumerate(cfg["lens"]):
        # pieces of random length; prefill rows check every chunk's output
        p, chunks = 0, []
        while p < n:
            m = int(min(n - p, rng.integers(1, 400)))
            sl = (slice(b, b + 1), slice(None), slice(p, p + m))
            if cfg["prefill"][b]:
                out = c.prefill_chunk_row(0, b, Qd[sl].contiguous(), Kd[sl].contiguous(), Vd[sl].contiguous())
                chunks.append((p, m, out))
            else:
                c.append_row(0, b, Kd[sl].contiguous(), Vd[sl].contiguous())
            p += m
        assert c.row_len(0, b) == n
        if chunks:
            torch.cuda.synchronize()
            ref = _ref_prefill(cfg, Q, K, V, b, n, [m for _, m, _ in chunks])
            got = torch.cat([o[0] for _, _, o in chunks], dim=1)
            check_close(got, ref, dt, f"seed {seed} prefill row {b}")
    q = torch.stack([Qd[b, :, n - 1] for b, n in enumerate(cfg["lens"])]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for b, n in enumerate(cfg["lens"]):
        check_close(out[b], _ref_decode(cfg, Q, K, V, b, n - 1), dt, f"seed {seed} decode row {b} (len {n})")
    for i in range(steps):
        t = [n + i for n in cfg["lens"]]
        kn = torch.stack([Kd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        vn = torch.stack([Vd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        qn = torch.stack([Qd[b, :, t[b]] for b in range(B)]).contiguous()
        out = c.decode_append(0, kn, vn, qn)
        torch.cuda.synchronize()
        for b in range(B):
            check_close(out[b], _ref_decode(cfg, Q, K, V, b, t[b]), dt, f"seed {seed} fused step {i} row {b}")
