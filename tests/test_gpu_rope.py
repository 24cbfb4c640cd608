"""Rotary positions (rope_theta > 0): keys stored rotated at their logical
position, queries rotated at theirs.  Outputs against the fp64 oracle
(oracle.rope); stored keys against the oracle's rotated, rounded keys.

The kernels rotate keys (which the cache stores) in double precision and
round once to the cache dtype, as the oracle's float64 rotation is rounded, so
stored keys are compared bit for bit.  The two sides' angles agree to the last
bits of a double (the device's and the host's exp2, pow and sin/cos), so a
stored element can still differ by one step where the exact rotation lies that
close to a rounding boundary: never seen for bf16 (a step of 2^-8; allowed on
one element in a million), about once in a million for fp32 (a step of 2^-24;
allowed on ten in a million).  FP8 codes, quantized from the bf16 key, are
compared bit for bit.  Queries are rotated in float (they are attended, not
stored); the outputs carry that within the usual tolerance."""
import numpy as np
import pytest
import torch

import workloads as WL
from oracle import cache as OC
from oracle import rope as RP
from tests.gpu_util import check_close, need_gpu, say, stored

THETA = 10000.0


def _seq(B, n_kv, N, d, seed, n_q):
    K = WL.normal_f32((B, n_kv, N, d), seed)
    V = WL.normal_f32((B, n_kv, N, d), seed + 1)
    Q = WL.normal_f32((B, n_q, N, d), seed + 2)
    return K, V, Q


def _ref_decode(Q, K, V, b, t, mask, S, W, d, dtype, kvf, theta=THETA):
    """Oracle output of row b's query at position t over positions 0..t."""
    return RP.decode_step_rope(stored(Q[b, :, t], dtype), stored(K[b, :, :t + 1], dtype),
                               stored(V[b, :, :t + 1], dtype).astype(np.float32), mask, S, W, d ** -0.5, theta,
                               dtype, kv_format=kvf)


def _check_keys(c, K, V, lens, mask, S, W, dtype, theta=THETA):
    """Stored keys against the oracle's rotated, rounded keys (see the module
    note), values and positions bit-exact, at the simulated cache's slots."""
    st_v = WL.to_torch(V, dtype)
    want_k = RP.stored_keys(stored(K, dtype), theta, dtype)  # [B][n_kv][T][d], positions = rows
    step = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -23
    n_diff = n_all = 0
    for h in range(K.shape[1]):
        kc, vc, pos = c.read_head(0, h)
        for b, n in enumerate(lens):
            for slot, p in OC.slot_table(n, bool(mask[h]), S, W).items():
                got = kc[b, slot].double().numpy()
                want = want_k[b, h, p]
                diff = got != want
                if diff.any():
                    assert (np.abs(got - want)[diff] <= np.abs(want)[diff] * step).all(), (h, b, p)
                n_diff += int(diff.sum())
                n_all += diff.size
                assert torch.equal(vc[b, slot], st_v[b, h, p]), (h, b, p)
                if pos is not None:
                    assert int(pos[b, slot]) == p
    budget = 1e-6 if dtype == "bf16" else 1e-5
    assert n_diff <= budget * n_all, f"{n_diff} of {n_all} stored key elements off by one step"


def _check_fp8_keys(c, K, V, lens, mask, S, W, theta=THETA):
    """FP8 rows with rotary positions: K codes and scales are those of the
    oracle's rotated key rounded to bf16, V those of the value as given, bit
    for bit, at the simulated cache's slots."""
    from oracle import quant as OQ
    Kr = RP.stored_keys(stored(K, "bf16"), theta, "bf16").astype(np.float32)
    Vs = stored(V, "bf16").astype(np.float32)
    for h in range(K.shape[1]):
        kc, vc, pos = c.read_head(0, h)
        ksc, vsc = c.head_scales(0, h)
        for b, n in enumerate(lens):
            for slot, p in OC.slot_table(n, bool(mask[h]), S, W).items():
                ck, sk = OQ.quantize_rows(Kr[b, h, p])
                cv, sv = OQ.quantize_rows(Vs[b, h, p])
                assert np.array_equal(kc[b, slot].numpy(), ck) and float(ksc[b, slot]) == float(sk), (h, b, p)
                assert np.array_equal(vc[b, slot].numpy(), cv) and float(vsc[b, slot]) == float(sv), (h, b, p)


DECODE = [("bf16", 128, 8, None), ("bf16", 128, 1, None), ("bf16", 64, 4, None), ("f32", 128, 2, None),
          ("f32", 64, 1, None), ("bf16", 128, 8, "fp8"), ("bf16", 128, 2, "fp8")]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g,kvf", DECODE)
def test_rope_decode(dtype, d, g, kvf):
    """Rows of 1, 70, 2,049 and 5,000 tokens (S=4, W=64: rings wrapped many
    times, each key rotated at its logical position), decoded together."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("rope decode", dtype, d, g, kvf)
    lens = [1, 70, 2049, 5000]
    B, n_kv, S, W = len(lens), 2, 4, 64
    mask = [1, 0]
    n_q = n_kv * g
    N = max(lens)
    K, V, Q = _seq(B, n_kv, N, d, 1600 + d + g, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, dtype, [mask], kv_format=kvf, rope_theta=THETA)
    Kd, Vd, Qd = (WL.to_torch(x, dtype).cuda() for x in (K, V, Q))
    for b, n in enumerate(lens):
        for p0 in range(0, n, 1500):
            m = min(1500, n - p0)
            c.append_row(0, b, Kd[b:b + 1, :, p0:p0 + m].contiguous(), Vd[b:b + 1, :, p0:p0 + m].contiguous())
    q = torch.stack([Qd[b, :, n - 1] for b, n in enumerate(lens)]).contiguous()
    out = c.decode(0, q)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        check_close(out[b], _ref_decode(Q, K, V, b, n - 1, mask, S, W, d, dtype, kvf), dtype, f"rope row {b} len {n}")
    if kvf is None:
        _check_keys(c, K, V, lens, mask, S, W, dtype)
    else:
        _check_fp8_keys(c, K, V, lens, mask, S, W)


@pytest.mark.gpu
@pytest.mark.parametrize("kvf", [None, "fp8"])
def test_rope_decode_append_steps(kvf):
    """Fused steps: the new token's key is rotated at its position in the
    kernel, attended and stored; rows start at 0, 3 and 100 tokens."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    say("rope fused", kvf)
    start = [0, 3, 100]
    steps = 10
    B, n_q, n_kv, d, S, W = len(start), 16, 2, 128, 4, 16
    mask = [0, 1]
    N = max(start) + steps
    K, V, Q = _seq(B, n_kv, N, d, 1700, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N, S, W, "bf16", [mask], kv_format=kvf, rope_theta=THETA)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    for b, n in enumerate(start):
        if n:
            c.append_row(0, b, Kd[b:b + 1, :, :n].contiguous(), Vd[b:b + 1, :, :n].contiguous())
    for i in range(steps):
        t = [n + i for n in start]
        kn = torch.stack([Kd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        vn = torch.stack([Vd[b, :, t[b]:t[b] + 1] for b in range(B)]).contiguous()
        q = torch.stack([Qd[b, :, t[b]] for b in range(B)]).contiguous()
        out = c.decode_append(0, kn, vn, q)
        torch.cuda.synchronize()
        for b in range(B):
            check_close(out[b], _ref_decode(Q, K, V, b, t[b], mask, S, W, d, "bf16", kvf), "bf16",
                        f"rope fused step {i} row {b}")
    if kvf is None:
        _check_keys(c, K, V, [n + steps for n in start], mask, S, W, "bf16")
    else:
        _check_fp8_keys(c, K, V, [n + steps for n in start], mask, S, W)


PREFILL = [("bf16", 128, 4, None), ("bf16", 64, 8, None), ("f32", 128, 1, None), ("bf16", 128, 8, "fp8")]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,d,g,kvf", PREFILL)
def test_rope_prefill_chunked(dtype, d, g, kvf):
    """Chunked prefill (chunks 300, 1, 512, 250): each chunk row's query
    rotated at P + i; then a decode step."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    chunks = [300, 1, 512, 250]
    N = sum(chunks)
    say("rope prefill", dtype, d, g, kvf)
    B, n_kv, S, W = 2, 2, 5, 40
    mask = [1, 0]
    n_q = n_kv * g
    K, V, Q = _seq(B, n_kv, N + 1, d, 1800 + d + g, n_q)
    c = DuoCache(1, B, n_q, n_kv, d, N + 1, S, W, dtype, [mask], kv_format=kvf, rope_theta=THETA)
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
        ref = RP.prefill_chunked_rope(Qs[b, :, :N], Ks[b, :, :N], Vs[b, :, :N], mask, S, W, d ** -0.5, THETA, dtype,
                                      chunks, kv_format=kvf)
        check_close(out[b], ref, dtype, f"rope prefill row {b}")
    if kvf is None:
        _check_keys(c, K[:, :, :N], V[:, :, :N], [N, N], mask, S, W, dtype)
    else:
        _check_fp8_keys(c, K[:, :, :N], V[:, :, :N], [N, N], mask, S, W)
    c.append(0, Kd[:, :, N:].contiguous(), Vd[:, :, N:].contiguous())
    dec = c.decode(0, Qd[:, :, N].contiguous())
    torch.cuda.synchronize()
    for b in range(B):
        check_close(dec[b], _ref_decode(Q, K, V, b, N, mask, S, W, d, dtype, kvf), dtype, f"rope decode row {b}")


@pytest.mark.gpu
def test_rope_large_positions():
    """A 128k-token retrieval head with base 500,000: angles up to about
    1.3e5 radians (reduced in double precision), queries at the last
    position; and a paged cache with a forked prefix (shared pages hold keys
    rotated at the same logical positions in both rows)."""
    need_gpu()
    from head_wise_kv_amd import DuoCache
    theta = 500000.0
    T, d, S, W = 131072, 128, 64, 1024
    n_q, n_kv = 8, 2
    mask = [1, 0]
    say("rope large positions", T)
    K = WL.normal_f32((1, n_kv, T, d), 1900)
    V = WL.normal_f32((1, n_kv, T, d), 1901)
    Q = WL.normal_f32((1, n_q, d), 1902)  # the query at position T - 1
    c = DuoCache(1, 2, n_q, n_kv, d, T, S, W, "bf16", [mask], rope_theta=theta, page_rows=256, n_pages=1024)
    Kd, Vd, Qd = (WL.to_torch(x, "bf16").cuda() for x in (K, V, Q))
    c.append_row(0, 0, Kd[:, :, :T - 1].contiguous(), Vd[:, :, :T - 1].contiguous())
    c.fork_row(0, 0, 1)
    kn = torch.cat([Kd[:, :, T - 1:]] * 2).contiguous()
    vn = torch.cat([Vd[:, :, T - 1:]] * 2).contiguous()
    q = torch.cat([Qd] * 2).contiguous()
    out = c.decode_append(0, kn, vn, q)
    torch.cuda.synchronize()
    ref = RP.decode_step_rope(stored(Q[0], "bf16"), stored(K[0], "bf16"), stored(V[0], "bf16"), mask, S, W,
                              d ** -0.5, theta, "bf16")
    check_close(out[0], ref, "bf16", "rope 128k row 0")
    check_close(out[1], ref, "bf16", "rope 128k forked row 1")
    assert c.row_pages(0, 1)[:511] == c.row_pages(0, 0)[:511]


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float64)).astype(np.float32)
    return np.spacing(x).astype(np.float64)


@pytest.mark.gpu
@pytest.mark.parametrize("d,theta", [(128, 500000.0), (64, 10000.0)])
def test_rope_apply_up_to_largest_position(d, theta):
    """duo_rope_apply at positions up to 2^31 - 1, the largest a cache row can
    reach, against the exact rotation (oracle.rope.rotate_exact: decimal
    angles, reduced with a 40-digit pi).  float32 rows: every value within
    half a float32 step of the exact rotation (plus 1e-15 of the pair's size
    for the double arithmetic before the rounding); a float64 angle p * f
    would be off by up to ~2.4e-7 rad there, which shows as several float32
    steps.  bf16 rows: the exact rotation rounded once, bit for bit."""
    need_gpu()
    import head_wise_kv_amd as H
    C = 3
    p0 = [2 ** 31 - C, 2 ** 30 + 12345, 1_000_000_007, 0]
    B = len(p0)
    say("rope_apply", d, theta)
    X = WL.normal_f32((B, 1, C, d), 1950 + d)
    want = np.stack([RP.rotate_exact(X[b, 0], [p0[b] + c for c in range(C)], theta) for b in range(B)])[:, None]
    got = H.rope_apply(torch.from_numpy(X).cuda(), p0, theta).cpu().double().numpy()
    h = d // 2
    pair = np.sqrt(X[..., :h] ** 2 + X[..., h:] ** 2).astype(np.float64)
    pair = np.concatenate([pair, pair], axis=-1)
    err = np.abs(got - want)
    bound = 0.5 * _ulp32(want) + 1e-15 * pair
    say("rope_apply f32 max err", float(err.max()), "max err / bound", float((err / bound).max()))
    assert (err <= bound).all(), np.argwhere(err > bound)[:5]
    # bf16: the exact rotation of the bf16 inputs, rounded once to bf16
    Xb = stored(X, "bf16")
    want_b = np.stack([RP.rotate_exact(Xb[b, 0], [p0[b] + c for c in range(C)], theta) for b in range(B)])[:, None]
    got_b = H.rope_apply(WL.to_torch(X, "bf16").cuda(), p0, theta).cpu().double().numpy()
    assert np.array_equal(got_b, RP.round_bf16(want_b)), np.argwhere(got_b != RP.round_bf16(want_b))[:5]
    # in place, and the argument checks
    xt = torch.from_numpy(X).cuda()
    H.rope_apply(xt, p0, theta, out=xt)
    assert np.array_equal(xt.cpu().double().numpy(), got)
    for bad_p0 in ([2 ** 31 - C + 1, 0, 0, 0], [-1, 0, 0, 0]):
        with pytest.raises(H.DuoError) as e:
            H.rope_apply(torch.from_numpy(X).cuda(), bad_p0, theta)
        assert e.value.code == H.DUO_EINVAL


@pytest.mark.gpu
def test_rope_errors_and_workspace():
    """Bad bases are rejected; a prefill workspace too small for the rotated
    chunk is refused with DUO_EWORKSPACE (nothing enqueued, count unchanged)."""
    need_gpu()
    import ctypes
    import head_wise_kv_amd as H
    from head_wise_kv_amd import DuoCache
    say("rope errors")
    for bad in (-1.0, 0.5, 1.0, float("inf"), float("nan")):
        with pytest.raises(H.DuoError) as e:
            DuoCache(1, 1, 4, 2, 64, 100, 1, 4, "bf16", [[1, 0]], rope_theta=bad)
        assert e.value.code == H.DUO_EINVAL, bad
    c = DuoCache(1, 1, 4, 2, 64, 100, 1, 4, "bf16", [[1, 0]], rope_theta=THETA)
    need = ctypes.c_size_t()
    assert H.lib.duo_prefill_workspace_bytes(c._h, 1, 10, ctypes.byref(need)) == 0
    assert need.value >= (4 + 2) * 10 * 64 * 2
    x = torch.zeros(1, 4, 10, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(need.value - 256, dtype=torch.uint8, device="cuda")
    rc = H.lib.duo_prefill_chunk(c._h, 0, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(kv.data_ptr()),
                                 ctypes.c_void_p(kv.data_ptr()), 10, ctypes.c_void_p(x.data_ptr()), 0.1,
                                 ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert rc == H.DUO_EWORKSPACE and c.seq_len(0) == 0
