"""libduo on the CPU: it loads, exports every entry point of include/duo.h,
and its host-only logic (validation, layout sizes) is right.  No GPU work."""
import ctypes
import os
import re

import pytest

import head_wise_kv_amd as H
import workloads as WL
from oracle import sizes as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "duo.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(duo_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10, names
    assert set(names) == set(H.EXPORTS)
    lib = ctypes.CDLL(H.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", WL.ORDER)
def test_payload_matches_closed_form(name):
    w = WL.WORKLOADS[name]
    mask = WL.mask_table(w)
    T_cap = w.T
    _, ws, payload = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, T_cap, w.S, w.W, w.dtype, mask)
    assert payload == Z.mixed_payload_bytes(mask.tolist(), w.B, T_cap, w.S, w.W, w.d, w.elem_bytes)
    assert ws > 0


@pytest.mark.parametrize("name", ["gqa70b_decode_128k", "mha7b_decode_128k", "llama3_8b_prefill_64k"])
def test_fp8_payload_closed_form(name):
    """FP8 rows: one byte per element plus one fp32 scale per stored K and V row."""
    w = WL.WORKLOADS[name]
    mask = WL.mask_table(w)
    _, ws, payload = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask, "fp8")
    codes = Z.mixed_payload_bytes(mask.tolist(), w.B, w.T, w.S, w.W, w.d, 1)
    scales = Z.mixed_payload_bytes(mask.tolist(), w.B, w.T, w.S, w.W, 1, 4)
    assert payload == codes + scales
    _, ws_native, native = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask)
    assert payload < native * 0.52 and ws > ws_native


@pytest.mark.parametrize("name", ["gqa70b_decode_128k", "mha7b_decode_128k", "llama3_8b_prefill_64k"])
def test_int4_payload_closed_form(name):
    """INT4 rows: d / 2 bytes of codes plus one fp32 scale per stored K and V row."""
    w = WL.WORKLOADS[name]
    mask = WL.mask_table(w)
    _, ws, payload = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask, "int4")
    codes = Z.mixed_payload_bytes(mask.tolist(), w.B, w.T, w.S, w.W, w.d // 2, 1)
    scales = Z.mixed_payload_bytes(mask.tolist(), w.B, w.T, w.S, w.W, 1, 4)
    assert payload == codes + scales
    _, _, native = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask)
    assert payload * 3.7 < native < payload * 3.8   # 256 bytes against 64 + 4


def test_int4_pages_hold_a_decode_round():
    with pytest.raises(H.DuoError) as e:
        H.cache_bytes(1, 1, 8, 2, 128, 4096, 4, 8, "bf16", [[1, 0]], "int4", page_rows=256, n_pages=16)
    assert e.value.code == H.DUO_EUNSUPPORTED
    H.cache_bytes(1, 1, 8, 2, 128, 4096, 4, 8, "bf16", [[1, 0]], "int4", page_rows=512, n_pages=8)


def test_low_bit_rows_need_bf16_d128():
    for kvf in ("fp8", "int4"):
        for dtype, d in (("f32", 128), ("bf16", 64)):
            with pytest.raises(H.DuoError) as e:
                H.cache_bytes(1, 1, 8, 2, d, 64, 4, 8, dtype, [[1, 0]], kvf)
            assert e.value.code == H.DUO_EUNSUPPORTED


@pytest.mark.parametrize("kvf", [None, "fp8"])
def test_paged_payload_closed_form(kvf):
    """A paged cache's retrieval payload is its pools (n_pages * page_rows rows
    per retrieval head and layer) instead of B * T_cap rows; the streaming
    heads' part is unchanged."""
    w = WL.WORKLOADS["llama3_8b_decode_b8_32k"]
    mask = WL.mask_table(w)
    P, n_pages = 256, 300
    _, ws, paged = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask, kvf, P, n_pages)
    e = 1 if kvf == "fp8" else w.elem_bytes
    n_ret = int(mask.sum())
    n_str = mask.size - n_ret
    want = 2 * (n_ret * n_pages * P + w.B * n_str * (w.S + w.W)) * w.d * e
    if kvf == "fp8":
        want += 2 * (n_ret * n_pages * P + w.B * n_str * (w.S + w.W)) * 4
    assert paged == want
    # the same pool as the contiguous rows (n_pages * P = B * T_cap) holds the same payload
    _, _, same = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask, kvf, P, w.B * w.T // P)
    _, _, contiguous = H.cache_bytes(w.L, w.B, w.n_q, w.n_kv, w.d, w.T, w.S, w.W, w.dtype, mask, kvf)
    assert same == contiguous


def test_payload_reproduces_printed_examples():
    # 70B GQA, all heads retrieval: the printed 41,943,040,000 bytes.
    _, _, p = H.cache_bytes(80, 1, 64, 8, 128, 128000, 64, 1024, "bf16", [[1] * 8] * 80)
    assert p == 41943040000
    # 2 of 8 heads retrieval per layer: the Memory_Duo formula with R = 0.25.
    _, _, p = H.cache_bytes(80, 1, 64, 8, 128, 128000, 64, 1024, "bf16", [[1, 1, 0, 0, 0, 0, 0, 0]] * 80)
    assert p == Z.duo_cache_bytes(0.25, 128000, 64, 1024, 80, 8, 128, 2) == 10753146880
    # L=32, 4096 tokens, 8 KV heads of 128, 2-byte: 512 MiB; MHA (32 KV heads) 2 GiB.
    _, _, p = H.cache_bytes(32, 1, 32, 8, 128, 4096, 0, 1, "bf16", [[1] * 8] * 32)
    assert p == 536870912
    _, _, p = H.cache_bytes(32, 1, 32, 32, 128, 4096, 0, 1, "bf16", [[1] * 32] * 32)
    assert p == 2 * 1024 ** 3


BAD = [
    (dict(n_q=6, n_kv=4), H.DUO_EINVAL),
    (dict(d_head=96), H.DUO_EUNSUPPORTED),
    (dict(n_q=68, n_kv=4), H.DUO_EUNSUPPORTED),   # g = 17: above the 16 query columns of a matrix-core tile
    (dict(n_q=36, n_kv=4, dtype_code=0), H.DUO_EUNSUPPORTED),  # g = 9 on the vector ALU (fp32)
    (dict(n_q=36, n_kv=4, d_head=64), H.DUO_EUNSUPPORTED),     # g = 9 on the vector ALU (d_head 64)
    (dict(sink=-1), H.DUO_EINVAL),
    (dict(recent=0), H.DUO_EINVAL),
    (dict(T_cap=0), H.DUO_EINVAL),
    (dict(T_cap=2 ** 31 - 4096), H.DUO_EINVAL),              # within 4,096 of 2^31
    (dict(L=0), H.DUO_EINVAL),
    (dict(mask_value=2), H.DUO_EINVAL),
    (dict(dtype_code=7), H.DUO_EUNSUPPORTED),
    (dict(kv_format=5), H.DUO_EUNSUPPORTED),
    (dict(B=65), H.DUO_EUNSUPPORTED),                          # at most 64 batch rows
    (dict(kv_format=1, dtype_code=0), H.DUO_EUNSUPPORTED),   # FP8 rows need bf16
    (dict(kv_format=1, d_head=64), H.DUO_EUNSUPPORTED),      # FP8 rows are built for d_head 128
    (dict(page_rows=32, n_pages=4), H.DUO_EINVAL),           # pages of at least 64 rows
    (dict(page_rows=64, n_pages=4), H.DUO_EUNSUPPORTED),     # below a decode round (128 bf16 rows of d 128)
    (dict(page_rows=128, n_pages=4, kv_format=1), H.DUO_EUNSUPPORTED),  # FP8: a round is 256 rows
    (dict(page_rows=256, n_pages=4, kv_format=2), H.DUO_EUNSUPPORTED),  # INT4: a round is 512 rows
    (dict(page_rows=384, n_pages=4), H.DUO_EINVAL),          # a power of two
    (dict(page_rows=256, n_pages=0), H.DUO_EINVAL),          # an empty pool
    (dict(page_rows=-256, n_pages=4), H.DUO_EINVAL),
    (dict(rope_theta=-1.0), H.DUO_EINVAL),
    (dict(rope_theta=1.0), H.DUO_EINVAL),                    # a base must exceed 1
    (dict(rope_theta=float("nan")), H.DUO_EINVAL),
    (dict(rope_theta=float("inf")), H.DUO_EINVAL),
]


GOOD_GROUPS = [(g, dt, d) for g in (3, 5, 6, 7, 12, 16) for dt, d in ((H.DUO_BF16, 128),)] + \
              [(g, dt, d) for g in (3, 5, 6, 7) for dt, d in ((H.DUO_F32, 128), (H.DUO_F32, 64), (H.DUO_BF16, 64))]


@pytest.mark.parametrize("g,dtype_code,d_head", GOOD_GROUPS)
def test_group_sizes_accepted(g, dtype_code, d_head):
    """Any group size up to 16 where the scores run on the matrix cores (bf16,
    d_head 128), up to 8 on the vector ALU."""
    buf = (ctypes.c_uint8 * 4)(1, 0, 1, 0)
    cfg = H.duo_config(2, 1, 2 * g, 2, d_head, 100, 2, 8, dtype_code,
                       ctypes.cast(buf, ctypes.POINTER(ctypes.c_uint8)), 0, 0, 0, 0.0)
    a = ctypes.c_size_t()
    assert H.lib.duo_cache_bytes(ctypes.byref(cfg), ctypes.byref(a), None) == H.DUO_OK, H.lib.duo_last_error()


@pytest.mark.parametrize("over,code", BAD)
def test_validation_codes(over, code):
    base = dict(L=2, B=1, n_q=8, n_kv=4, d_head=128, T_cap=100, sink=2, recent=8)
    base.update({k: v for k, v in over.items() if k in base})
    n_mask = max(base["L"], 0) * base["n_kv"]
    mv = over.get("mask_value", 1)
    buf = (ctypes.c_uint8 * max(n_mask, 1))(*([mv] * max(n_mask, 1)))
    cfg = H.duo_config(base["L"], base["B"], base["n_q"], base["n_kv"], base["d_head"], base["T_cap"],
                       base["sink"], base["recent"], over.get("dtype_code", H.DUO_BF16),
                       ctypes.cast(buf, ctypes.POINTER(ctypes.c_uint8)), over.get("kv_format", 0),
                       over.get("page_rows", 0), over.get("n_pages", 0), over.get("rope_theta", 0.0))
    a = ctypes.c_size_t()
    rc = H.lib.duo_cache_bytes(ctypes.byref(cfg), ctypes.byref(a), None)
    assert rc == code, H.lib.duo_last_error()
    assert H.lib.duo_last_error()


def test_null_config_and_mask():
    assert H.lib.duo_cache_bytes(None, None, None) == H.DUO_EINVAL
    cfg = H.duo_config(1, 1, 4, 2, 64, 10, 1, 2, H.DUO_F32, None)
    assert H.lib.duo_cache_bytes(ctypes.byref(cfg), None, None) == H.DUO_EINVAL


def test_calls_on_null_handle_fail_cleanly():
    x = ctypes.c_int64()
    assert H.lib.duo_cache_seq_len(None, 0, ctypes.byref(x)) == H.DUO_EINVAL
    assert H.lib.duo_append(None, 0, None, None, 1, None) == H.DUO_EINVAL
    assert H.lib.duo_decode(None, 0, None, None, 1.0, None, 0, None) == H.DUO_EINVAL
    assert H.lib.duo_decode_append(None, 0, None, None, None, None, 1.0, None, 0, None) == H.DUO_EINVAL
    assert H.lib.duo_cache_head_scales(None, 0, 0, None, None, None) == H.DUO_EINVAL
    assert H.lib.duo_append_row(None, 0, 0, None, None, 1, None) == H.DUO_EINVAL
    assert H.lib.duo_prefill_chunk_row(None, 0, 0, None, None, None, 1, None, 1.0, None, 0, None) == H.DUO_EINVAL
    assert H.lib.duo_cache_row_len(None, 0, 0, ctypes.byref(x)) == H.DUO_EINVAL
    assert H.lib.duo_cache_reset_row(None, 0, 0) == H.DUO_EINVAL
    assert H.lib.duo_cache_fork_row(None, 0, 0, 1, None) == H.DUO_EINVAL
    assert H.lib.duo_cache_free_pages(None, 0, ctypes.byref(x)) == H.DUO_EINVAL
    assert H.lib.duo_cache_row_pages(None, 0, 0, None, 0, ctypes.byref(x)) == H.DUO_EINVAL
    sz = ctypes.c_size_t()
    assert H.lib.duo_prefill_workspace_bytes(None, 1, 10, ctypes.byref(sz)) == H.DUO_EINVAL
    H.lib.duo_cache_free(None)


GATED_BAD = [
    (dict(n_q=6, n_kv=4), H.DUO_EINVAL),
    (dict(B=0), H.DUO_EINVAL),
    (dict(d_head=96), H.DUO_EUNSUPPORTED),
    (dict(N=0), H.DUO_EINVAL),
    (dict(sink=-1), H.DUO_EINVAL),
    (dict(recent=0), H.DUO_EINVAL),
    (dict(N=2 ** 31 - 10, recent=64), H.DUO_EINVAL),
    (dict(dtype=7), H.DUO_EUNSUPPORTED),
    (dict(), H.DUO_EINVAL),  # valid shape, NULL tensors
]


@pytest.mark.parametrize("over,code", GATED_BAD)
def test_gated_validation_codes(over, code):
    """duo_gated_attention validates its shape and pointers before any launch."""
    base = dict(B=1, n_q=8, n_kv=4, d_head=128, N=100, sink=4, recent=16, dtype=H.DUO_BF16)
    base.update(over)
    shape = H.duo_gated_shape(base["B"], base["n_q"], base["n_kv"], base["d_head"], base["N"], base["sink"],
                              base["recent"], base["dtype"])
    rc = H.lib.duo_gated_attention(ctypes.byref(shape), None, None, None, None, None, 1.0, None)
    assert rc == code, H.lib.duo_last_error()
    assert H.lib.duo_last_error()
    assert H.lib.duo_gated_attention(None, None, None, None, None, None, 1.0, None) == H.DUO_EINVAL
