"""Paged retrieval rows and prefix sharing (page_rows > 0): batch rows take
pages from a per-layer pool as they grow; duo_cache_fork_row shares a row's
full pages with an empty row.  Outputs are checked against the fp64 oracle
over each row's logical sequence; the page accounting against the oracle's
page model (oracle.paging); the stored rows bit-exactly through the page
tables.  Page numbers themselves are the library's choice: the tests check
what is fixed (counts, sharing, content) and that the rest is valid (no page
held by two rows unless shared by a fork, no page outside the pool)."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import attention as OA
from oracle import cache as OC
from oracle import paging as OP
from oracle import quant as OQ
from tests.gpu_util import check_close, need_gpu, say, stored

P = 256


def _seq(B, n_kv, N, d, seed, n_q):
    K = WL.normal_f32((B, n_kv, N, d), seed)
    V = WL.normal_f32((B, n_kv, N, d), seed + 1)
    Q = WL.normal_f32((B, n_q, N, d), seed + 2)
    return K, V, Q


def _ref_decode(Q, K, V, b, t, mask, S, W, d, dtype, fp8):
    """Oracle output of row b's query at position t over positions 0..t of
    the row's logical sequence K[b], V[b]."""
    q = stored(Q[b, :, t], dtype)
    Ks, Vs = stored(K[b, :, :t + 1], dtype), stored(V[b, :, :t + 1], dtype)
    if fp8:
        return OQ.decode_step_fp8(q, Ks.astype(np.float32), Vs.astype(np.float32), mask, S, W, d ** -0.5)
    return OA.decode_step(q, Ks, Vs, mask, S, W, d ** -0.5)


def _check_pages(c, model, layer=0):
    """Page counts against the model; every page in the pool; a page held by
    two rows only where the model shares one."""
    B = model.B
    tables = [c.row_pages(layer, b) for b in range(B)]
    for b in range(B):
        assert len(tables[b]) == model.pages_needed(model.count[b]) == len(model.rows[b]), (b, tables[b])
        assert all(0 <= p < model.n_pages for p in tables[b])
        assert len(set(tables[b])) == len(tables[b])
    used = {p for t in tables for p in t}
    assert len(used) == model.pages_in_use()
    assert c.free_pages(layer) == model.free_pages()
    for b1 in range(B):
        for b2 in range(b1 + 1, B):
            assert len(set(tables[b1]) & set(tables[b2])) == model.shared_pages(b1, b2), (b1, b2)


def _check_rows(c, K, V, lens, mask, S, W, dtype, fp8):
    """Stored rows of every head bit-exact: the inputs (native rows) or the
    oracle's quantizer applied to them (FP8 rows), at the slots the cache
    simulation assigns (a paged head read through its row's page table)."""
    if fp8:
        Ks, Vs = stored(K, dtype).astype(np.float32), stored(V, dtype).astype(np.float32)
    else:
        st_k, st_v = WL.to_torch(K, dtype), WL.to_torch(V, dtype)
    for h in range(K.shape[1]):
        kc, vc, pos = c.read_head(0, h)
        ksc, vsc = c.head_scales(0, h) if fp8 else (None, None)
        for b, n in enumerate(lens):
            for slot, p in OC.slot_table(n, bool(mask[h]), S, W).items():
                if fp8:
                    ck, sk = OQ.quantize_rows(Ks[b, h, p])
                    cv, sv = OQ.quantize_rows(Vs[b, h, p])
                    assert np.array_equal(kc[b, slot].numpy(), ck) and float(ksc[b, slot]) == float(sk), (h, b, p)
                    assert np.array_equal(vc[b, slot].numpy(), cv) and float(vsc[b, slot]) == float(sv), (h, b, p)
                else:
                    assert torch.equal(kc[b, slot], st_k[b, h, p]) and torch.equal(vc[b, slot], st_v[b, h, p]), (h, b, p)
                if pos is not None:
                    assert int(pos[b, slot]) == p, (h, b, slot)


# (dtype, d, g, K/V row format, page rows): 256-row pages, and the smallest
# page each row format allows (one decode round)
CASES = [("bf16", 128, 4, None, P), ("bf16", 128, 8, None, P), ("bf16", 64, 2, None, P), ("f32", 128, 1, None, P),
         ("f32", 64, 8, None, P), ("bf16", 128, 8, "fp8", P), ("bf16", 128, 1, "fp8", P),
         ("bf16", 128, 8, None, 128), ("bf16", 128, 3, None, 128), ("f32", 128, 2, None, 64), ("f32", 64, 4, None, 128)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g,kvf,pr", CASES)
def test_paged_ragged_decode(dtype, d, g, kvf, pr):
    """Rows of 1, 255, 256, 600 and 2,049 tokens appended in pieces that cross
    page edges, decoded together: every row against the oracle, the pages
    against the model, the rows bit-exact."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("paged decode", dtype, d, g, kvf, pr)
    lens = [1, 255, 256, 600, 2049]
    B, n_kv, S, W = len(lens), 4, 4, 64
    mask = [1, 0, 1, 1]
    n_q = n_kv * g
    N = max(lens)
    n_pages = 20 * (P // pr)
    K, V, Q = _seq(B, n_kv, N, d, 1200 + d + g, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, dtype, [mask], kv_format=kvf, page_rows=pr, n_pages=n_pages)
    model = OP.PagedRows(pr, n_pages, B)
    Kd, Vd, Qd = (WL.to_torch(x, dtype).cuda() for x in (K, V, Q))
    for b, n in enumerate(lens):
        p = 0
        for piece in (100, 300, 1000, 10_000):
            m = min(piece, n - p)
            if m <= 0:
                break
            c.append_row(0, b, Kd[b:b + 1, :, p:p + m].contiguous(), Vd[b:b + 1, :, p:p + m].contiguous())
            model.append(b, m)
            p += m
        assert c.row_len(0, b) == n
    _check_pages(c, model)
    q = torch.stack([Qd[b, :, n - 1] for b, n in enumerate(lens)]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        check_close(out[b], _ref_decode(Q, K, V, b, n - 1, mask, S, W, d, dtype, kvf == "fp8"), dtype,
                    f"paged row {b} (len {n})")
    _check_rows(c, K, V, lens, mask, S, W, dtype, kvf == "fp8")


@pytest.mark.gpu
@pytest.mark.parametrize("kvf", [None, "fp8"])
def test_paged_decode_append_steps(kvf):
    """Fused steps over rows starting at 0, 250 and 511 tokens: the rows start
    new pages at different steps (the page enters the table before the launch
    that writes the token into it)."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("paged fused", kvf)
    start = [0, 250, 511]
    steps = 12
    B, n_q, n_kv, d, S, W = len(start), 16, 2, 128, 4, 16
    mask = [1, 0]
    N = max(start) + steps
    n_pages = 8
    K, V, Q = _seq(B, n_kv, N, d, 1300, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], kv_format=kvf, page_rows=P, n_pages=n_pages)
    model = OP.PagedRows(P, n_pages, B)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    for b, n in enumerate(start):
        if n:
            c.append_row(0, b, Kd[b:b + 1, :, :n].contiguous(), Vd[b:b + 1, :, :n].contiguous())
            model.append(b, n)
    for i in range(steps):
        t = [n + i for n in start]
        kn = torch.stack([Kd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        vn = torch.stack([Vd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        q = torch.stack([Qd[b, :, t[b]] for b in range(B)]).contiguous()
        out = c.decode_append(0, kn, vn, q)
        model.append_rows([(b, 1) for b in range(B)])
        torch.cuda.synchronize()
        for b in range(B):
            check_close(out[b], _ref_decode(Q, K, V, b, t[b], mask, S, W, d, "bf16", kvf == "fp8"), "bf16",
                        f"paged fused step {i} row {b}")
    _check_pages(c, model)
    _check_rows(c, K, V, [n + steps for n in start], mask, S, W, "bf16", kvf == "fp8")


PREFILL = [("bf16", 128, 4, None, P), ("bf16", 64, 8, None, P), ("f32", 64, 2, None, P), ("bf16", 128, 8, "fp8", P),
           ("bf16", 128, 4, None, 128), ("bf16", 128, 6, None, 128), ("f32", 128, 1, None, 64)]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g,kvf,pr", PREFILL)
def test_paged_prefill_chunked(dtype, d, g, kvf, pr):
    """Chunked prefill of two rows (chunks of 300, 1, 256 and 200 tokens:
    held rows on several pages, chunk edges inside pages), then one decode."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    chunks = [300, 1, 256, 200]
    N = sum(chunks)
    say("paged prefill", dtype, d, g, kvf, pr)
    B, n_kv, S, W = 2, 2, 5, 40
    mask = [1, 0]
    n_q = n_kv * g
    npg = 6 * (P // pr)
    K, V, Q = _seq(B, n_kv, N + 1, d, 1400 + d + g, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N + 1, S, W, dtype, [mask], kv_format=kvf, page_rows=pr, n_pages=npg)
    Kd, Vd, Qd = (WL.to_torch(x, dtype).cuda() for x in (K, V, Q))
    outs, p = [], 0
    for C in chunks:
        outs.append(c.prefill_chunk(0, Qd[:, :, p:p + C].contiguous(), Kd[:, :, p:p + C].contiguous(),
                                    Vd[:, :, p:p + C].contiguous()))
        p += C
    out = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    Qs, Ks, Vs = stored(Q, dtype), stored(K, dtype), stored(V, dtype)
    for b in range(B):
        if kvf == "fp8":
            ref = OQ.prefill_chunked_fp8(Qs[b, :, :N], Ks[b, :, :N].astype(np.float32),
                                         Vs[b, :, :N].astype(np.float32), mask, S, W, d ** -0.5, chunks)
        else:
            ref = OA.prefill_full(Qs[b, :, :N], Ks[b, :, :N], Vs[b, :, :N], mask, S, W, d ** -0.5)
        check_close(out[b], ref, dtype, f"paged prefill row {b}")
    model = OP.PagedRows(pr, npg, B)
    model.append_rows([(b, N) for b in range(B)])
    _check_pages(c, model)
    _check_rows(c, K[:, :, :N], V[:, :, :N], [N, N], mask, S, W, dtype, kvf == "fp8")
    c.append(0, Kd[:, :, N:].contiguous(), Vd[:, :, N:].contiguous())
    dec = c.decode(0, Qd[:, :, N].contiguous())
    torch.cuda.synchronize()
    for b in range(B):
        check_close(dec[b], _ref_decode(Q, K, V, b, N, mask, S, W, d, dtype, kvf == "fp8"), dtype,
                    f"paged decode after prefill, row {b}")


@pytest.mark.gpu
@pytest.mark.parametrize("paged,kvf", [(True, None), (True, "fp8"), (False, None), (False, "fp8")])
def test_prefix_fork(paged, kvf):
    """A 600-token prefix prefilled into row 0 and forked to rows 1-3 (two
    full pages shared, the partial third page copied, streaming slots
    copied); each row then continues with its own tokens (different counts)
    and all four decode together for a few fused steps.  Each row against the
    oracle over prefix + its own tokens; pages against the model; resets
    return the pages."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("prefix fork", paged, kvf)
    n = 600
    own = [0, 3, 300, 40]
    steps = 5
    B, n_q, n_kv, d, S, W = 4, 16, 4, 128, 4, 64
    mask = [1, 0, 0, 1]
    N = n + max(own) + steps
    n_pages = 16
    K, V, Q = _seq(B, n_kv, N, d, 1500, n_q)
    # row r's logical sequence: row 0's first n tokens, then its own
    K[1:, :, :n], V[1:, :, :n] = K[0, :, :n], V[0, :, :n]
    kw = dict(page_rows=P, n_pages=n_pages) if paged else {}
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], kv_format=kvf, **kw)
    model = OP.PagedRows(P, n_pages, B)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    for p0, C in ((0, 256), (256, 344)):
        c.prefill_chunk_row(0, 0, Qd[:1, :, p0:p0 + C].contiguous(), Kd[:1, :, p0:p0 + C].contiguous(),
                            Vd[:1, :, p0:p0 + C].contiguous())
    model.append(0, n)
    for r in range(1, B):
        c.fork_row(0, 0, r)
        model.fork(0, r)
        assert c.row_len(0, r) == n
    for r, m in enumerate(own):
        if m:
            c.append_row(0, r, Kd[r:r + 1, :, n:n + m].contiguous(), Vd[r:r + 1, :, n:n + m].contiguous())
            model.append(r, m)
    if paged:
        _check_pages(c, model)
        t0 = c.row_pages(0, 0)
        for r in range(1, B):
            assert c.row_pages(0, r)[:2] == t0[:2]  # the full pages are shared
    else:
        assert c.free_pages(0) == 0 and c.row_pages(0, 1) == []
    for i in range(steps):
        t = [n + m + i for m in own]
        kn = torch.stack([Kd[r, :, t[r]:t[r] + 1] for r in range(B)]).contiguous()
        vn = torch.stack([Vd[r, :, t[r]:t[r] + 1] for r in range(B)]).contiguous()
        q = torch.stack([Qd[r, :, t[r]] for r in range(B)]).contiguous()
        out = c.decode_append(0, kn, vn, q)
        model.append_rows([(r, 1) for r in range(B)])
        torch.cuda.synchronize()
        for r in range(B):
            check_close(out[r], _ref_decode(Q, K, V, r, t[r], mask, S, W, d, "bf16", kvf == "fp8"), "bf16",
                        f"fork step {i} row {r}")
    lens = [n + m + steps for m in own]
    _check_rows(c, K, V, lens, mask, S, W, "bf16", kvf == "fp8")
    if paged:
        _check_pages(c, model)
        for r in (1, 2, 3):
            c.reset_row(0, r)
            model.reset(r)
            assert c.row_len(0, r) == 0
            _check_pages(c, model)
        # a reset row starts again from nothing
        c.append_row(0, 2, Kd[2:3, :, :10].contiguous(), Vd[2:3, :, :10].contiguous())
        model.append(2, 10)
        _check_pages(c, model)


@pytest.mark.gpu
def test_paged_errors():
    """Pool limits: a call that would need more pages than are free fails with
    DUO_ECAPACITY and changes nothing; a fork of a partly filled page needs
    one; a reset frees; bad page configurations are rejected."""
    need_gpu()
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("paged errors")
    B, n_q, n_kv, d, S, W = 2, 4, 2, 128, 4, 16
    mask = [1, 0]
    for pr, npg in ((100, 4), (384, 4), (32, 4), (256, 0)):
        with pytest.raises(H.DuoError) as e:
            DuoCache(1, B, n_q, n_kv, d, 4096, S, W, "bf16", [mask], page_rows=pr, n_pages=npg)
        assert e.value.code == H.DUO_EINVAL, (pr, npg)
    with pytest.raises(H.DuoError) as e:  # below one decode round (128 bf16 rows of d 128)
        DuoCache(1, B, n_q, n_kv, d, 4096, S, W, "bf16", [mask], page_rows=64, n_pages=4)
    assert e.value.code == H.DUO_EUNSUPPORTED
    c = DuoCache(1, B, n_q, n_kv, d, 4096, S, W, "bf16", [mask], page_rows=P, n_pages=3)
    x = torch.randn(1, n_kv, 600, d, device="cuda").to(torch.bfloat16)
    c.append_row(0, 0, x, x)
    assert c.free_pages(0) == 0
    one = torch.zeros(1, n_kv, 1, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.append_row(0, 1, one, one)
    assert e.value.code == H.DUO_ECAPACITY and c.row_len(0, 1) == 0
    kb = torch.zeros(B, n_kv, 1, d, dtype=torch.bfloat16, device="cuda")
    qb = torch.zeros(B, n_q, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.DuoError) as e:
        c.decode_append(0, kb, kb, qb)
    assert e.value.code == H.DUO_ECAPACITY and c.row_len(0, 0) == 600
    with pytest.raises(H.DuoError) as e:
        c.fork_row(0, 0, 1)
    assert e.value.code == H.DUO_ECAPACITY and c.row_len(0, 1) == 0
    with pytest.raises(H.DuoError) as e:
        c.fork_row(0, 0, 0)
    assert e.value.code == H.DUO_EINVAL
    c.append_row(0, 0, one, one)  # position 600 is on page 2, already held
    assert c.row_len(0, 0) == 601 and c.free_pages(0) == 0
    c.reset_row(0, 0)
    assert c.free_pages(0) == 3 and c.row_len(0, 0) == 0
    c.fork_row(0, 0, 1)  # an empty source: nothing to share
    assert c.row_len(0, 1) == 0 and c.free_pages(0) == 3
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_paged_gqa70b_128k_layer():
    """70B GQA shape at full size with 256-row pages: positions 0..T-2
    appended, then the fused step at T-1 (the decode's items cut at round
    edges so that every round lies in one page), against the oracle."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    w = WL.WORKLOADS["gqa70b_decode_128k"]
    layer = 5
    say(w.name, "paged fused layer", layer)
    mask = WL.retrieval_mask(w, layer)
    n_pages = -(-w.T // P)
    c = DuoCache(1, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, [mask], page_rows=P, n_pages=n_pages)
    K = WL.stacked_rows_f32(w, layer, WL.TENSOR_K, w.n_kv, 0, w.T)
    V = WL.stacked_rows_f32(w, layer, WL.TENSOR_V, w.n_kv, 0, w.T)
    Q = WL.stacked_rows_f32(w, layer, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0]
    Kt, Vt = WL.to_torch(K, w.dtype).cuda(), WL.to_torch(V, w.dtype).cuda()
    c.append(0, Kt[:, :, : w.T - 1].contiguous(), Vt[:, :, : w.T - 1].contiguous())
    out = c.decode_append(0, Kt[:, :, w.T - 1:].contiguous(), Vt[:, :, w.T - 1:].contiguous(),
                          WL.to_torch(Q, w.dtype).cuda(), scale=w.scale)
    torch.cuda.synchronize()
    assert c.free_pages(0) == 0
    Ks, Vs = stored(K, w.dtype), stored(V, w.dtype)
    ref = OA.decode_step(stored(Q, w.dtype)[0], Ks[0], Vs[0], mask, w.S, w.W, w.scale)
    check_close(out[0], ref, w.dtype, f"{w.name} paged fused layer {layer}")


SHARED = [(8, 2, None, 0.0, False), (4, 4, None, 0.0, False), (4, 3, None, 10000.0, True),
          (8, 2, "fp8", 0.0, False), (8, 2, "int4", 0.0, True)]


@pytest.mark.gpu
@pytest.mark.parametrize("g,R,kvf,theta,exact", SHARED)
def test_shared_prefix_decode(g, R, kvf, theta, exact):
    """Rows forked from one prefix decode as a share group: the prefix's full
    pages are read once by shared work items that attend every row's queries
    to them, each row's own items take the rest, and the combine merges both.
    R rows forked from row 0 (one of them with no tokens of its own when the
    prefix is whole pages), plus an unrelated row; plain decodes and fused
    steps against the oracle, with the plan checked to use shared items."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    from oracle import quant4 as Q4
    from oracle import rope as RP
    say("shared prefix", g, R, kvf, theta, exact)
    pr = 512 if kvf == "int4" else P  # INT4 rounds are 512 rows: pages of >= 512
    B, n_kv, d, S, W = R + 1, 2, 128, 4, 64
    n_q = n_kv * g
    mask = [1, 0]
    n = 4 * pr if exact else 3 * pr + 37
    own = [5, 0 if exact else 9] + [40 * i for i in range(2, R)] + [n + 11]  # the last row is not a fork
    steps = 3
    N = n + max(own) + steps
    K, V, Q = _seq(B, n_kv, N, d, 2600 + g + R, n_q)
    K[1:R, :, :n], V[1:R, :, :n] = K[0, :, :n], V[0, :, :n]
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], kv_format=kvf, page_rows=pr,
                 n_pages=B * (-(-N // pr)), rope_theta=theta)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    c.append_row(0, 0, Kd[:1, :, :n].contiguous(), Vd[:1, :, :n].contiguous())
    for r in range(1, R):
        c.fork_row(0, 0, r)
    for r, m in enumerate(own):
        p0 = n if r < R else 0
        if m:
            c.append_row(0, r, Kd[r:r + 1, :, p0:p0 + m].contiguous(), Vd[r:r + 1, :, p0:p0 + m].contiguous())
    lens = [n + m if r < R else m for r, m in enumerate(own)]
    items, shared = c.decode_plan(0)
    assert shared > 0, (items, shared)

    def ref(r, t):
        q = stored(Q[r, :, t], "bf16")
        Ks, Vs = stored(K[r, :, :t + 1], "bf16"), stored(V[r, :, :t + 1], "bf16")
        if theta > 0:
            return RP.decode_step_rope(q, Ks, Vs, mask, S, W, d ** -0.5, theta, "bf16", kv_format=kvf)
        if kvf == "int4":
            return Q4.decode_step_int4(q, Ks.astype(np.float32), Vs.astype(np.float32), mask, S, W, d ** -0.5)
        if kvf == "fp8":
            return OQ.decode_step_fp8(q, Ks.astype(np.float32), Vs.astype(np.float32), mask, S, W, d ** -0.5)
        return OA.decode_step(q, Ks, Vs, mask, S, W, d ** -0.5)

    q = torch.stack([Qd[r, :, lens[r] - 1] for r in range(B)]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for r in range(B):
        check_close(out[r], ref(r, lens[r] - 1), "bf16", f"shared decode row {r}")
    for i in range(steps):
        t = [m + i for m in lens]
        kn = torch.stack([Kd[r, :, t[r]:t[r] + 1] for r in range(B)]).contiguous()
        vn = torch.stack([Vd[r, :, t[r]:t[r] + 1] for r in range(B)]).contiguous()
        q = torch.stack([Qd[r, :, t[r]] for r in range(B)]).contiguous()
        out = c.decode_append(0, kn, vn, q)
        torch.cuda.synchronize()
        for r in range(B):
            check_close(out[r], ref(r, t[r]), "bf16", f"shared step {i} row {r}")
    assert c.decode_plan(0)[1] > 0
